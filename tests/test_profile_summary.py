"""The kernel-source hash that marks when HBM counter figures were taken: prose edits keep
it, code edits change it."""
from post_weight_quantization_27_amd import profile_summary as P


def test_code_only_ignores_comments_and_spacing():
    a = "int f(int x) {\n  // doubles x\n  return 2 * x; /* fast */\n}\n"
    b = "/* header\n   text */\nint f(int x) {\n    return 2 * x;   // other words\n}"
    assert P.code_only(a) == P.code_only(b)


def test_code_only_sees_code_changes():
    a = "int f(int x) { return 2 * x; }"
    assert P.code_only(a) != P.code_only(a.replace("2", "3"))
    assert P.code_only(a) != P.code_only(a.replace("int x", "long x"))


def test_source_hash_is_stable():
    h = P.source_hash()
    assert len(h) == 16 and h == P.source_hash()
