"""Throughput of the layer-wise quantization path on one MI355X.

One step = every step of the path for every layer of the workload, on inputs already
resident in HBM: Hessian from X, damping, [act-order], H^-1 factor, GPTQ (INT4 packed +
fp16 scales), RTN, dequant of the GPTQ result, and the reconstruction MSE of both (through
the tokens, or through H where that product is the cheaper one).  The value is weights
quantized per second (sum of d_out * d_in over the layers / step).

The default workload is the 70B-shaped layer set (q 8192 -> 8192, gate/up 8192 -> 28672,
down 28672 -> 8192, 262144 bfloat16 tokens each), measured with act-order off (the line's
value) and on (a second object in the same line).

Prints ONE JSON line.  For each act-order setting: the value comes from K timed steps with
no events between the launches; per-call durations from K more steps with HIP events
recorded around every call on the stream it runs on (each layer has its own stream, which
the binding passes to libpwq); per-kernel durations from the library's own events around
its large kernels (pwq_profile_enable), one layer at a time.  The roofline object describes
the kernel with the most time per step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GPTQ INT4-g128 weights quantized/s per layer; XᵀX+update MFMA util"
PEAK = {"hbm": 8000.0, "mfma_f32": 157.3, "mfma_bf16": 2500.0}   # GB/s, TFLOP/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama70b")
    ap.add_argument("--layers", default="", help="comma-separated layer names (default: all)")
    ap.add_argument("--act-order", choices=("off", "on", "both"), default="both",
                    help="act-order off, on, or both (the line's value is the first; 'both' adds an act_order_on object)")
    ap.add_argument("--zero-point", action="store_true", help="the asymmetric form (a scale and a zero per group)")
    ap.add_argument("--streams", type=int, default=-1,
                    help="1: one stream per layer, 0: all on one stream, -1 (default): one stream per layer when every "
                         "layer has fewer than 4096 inputs (their factors are chains of small launches that other "
                         "layers' work can fill), else one stream (every step then fills the GPU by itself, and "
                         "sharing it only slows the longest chain)")
    ap.add_argument("--stagger", type=int, default=1,
                    help="1: the layer with the longest chain starts alone and the others once its Hessian is "
                         "formed (default), 0: all layers start together")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--awq-alphas", type=int, default=21,
                    help="grid size of the activation-aware scaling search timed per layer (0 to skip)")
    ap.add_argument("--matmul-tokens", default="1,16",
                    help="token counts at which Y = X What^T is timed on each layer's GPTQ output ('' to skip)")
    ap.add_argument("--cpu-layer", default="", help="layer the oracle baseline samples (default: the one with the "
                    "fewest inputs, then the fewest weights)")
    ap.add_argument("--cpu-rows", type=int, default=256, help="rows of W the oracle's column loop runs on")
    ap.add_argument("--prof-reps", type=int, default=2, help="steps per layer in the per-kernel timing pass")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (3 times), the reference for HBM traffic counters")
    return ap.parse_args()


class Layer:
    """Device-resident inputs and preallocated outputs of one layer."""

    def __init__(self, spec, torch, pwq, synth, act_order, zero_point=False):
        import numpy as np
        self.spec = spec
        dev = "cuda:0"
        W = synth.weight(spec)
        X = synth.x_full(spec, threads=16)
        self.W = torch.from_numpy(W).to(dev)
        if spec.x_dtype == synth.BF16:
            self.X = torch.from_numpy(X.view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            self.X = torch.from_numpy(X).to(dev)
        n, m = spec.d_in, spec.d_out
        self.H = torch.empty((n, n), dtype=torch.float32, device=dev)
        self.U = torch.empty((n, n), dtype=torch.float32, device=dev)
        self.info = torch.empty(1, dtype=torch.int32, device=dev)
        self.gq = {}
        self.rq = {}
        self.what = torch.empty((m, n), dtype=torch.float16, device=dev)
        self.mse = torch.empty(2, dtype=torch.float64, device=dev)
        self.lam = torch.zeros(1, dtype=torch.float32, device=dev)     # what damping adds to diag H
        self.act = act_order
        self.zp = zero_point
        # the reconstruction MSE through H (d_out x d_in^2) when that is cheaper than through
        # the tokens (n_tok x d_in x d_out bfloat16 MFMA)
        self.mse_h = mse_through_hessian(spec)
        del X, W


def mse_split_route(spec):
    # layers of at least 256 output tiles of 256 x 256: the library forms tr(dW H dW^T) as a
    # bfloat16 hi/lo split product over one triangle of H, about 3 d_out d_in^2 bfloat16 flops
    return -(-spec.d_out // 256) * -(-spec.d_in // 256) >= 256


def mse_through_hessian(spec):
    # split route: cheaper than the token route (2 n_tok d_in d_out bfloat16 flops) from
    # n_tok >= 1.5 (d_in + 256) on; taken from n_tok >= 2 d_in (70B q, k, v, o, gate, up, down).
    # Smaller layers form it on float32 MFMA, a sixteenth of the bfloat16 rate, but the token
    # route reaches only part of its peak on small contractions: measured, the float32 route
    # is the faster one from n_tok = 10 d_in on (GPT-2's 768-input layers)
    if mse_split_route(spec):
        return spec.n_tok >= 2 * spec.d_in
    return spec.n_tok >= 10 * spec.d_in


def run_step(L, pwq, timers=None, after_hessian=None, parts="all"):
    """One pass of the whole path over one layer.  timers: dict name -> list of (start, end) events;
    after_hessian: called once the Hessian's kernels are enqueued.  parts: "all", or the two
    halves that do not depend on each other: "rtn" (round-to-nearest and its error, which need
    only W and X) and "gptq" (everything else)."""
    import torch
    s = L.spec

    def t(name):
        if timers is None:
            return None
        e0 = torch.cuda.Event(enable_timing=True)
        e0.record()
        timers.setdefault(name, []).append([e0, None])
        return name

    def done(name):
        if name is None:
            return
        e1 = torch.cuda.Event(enable_timing=True)
        e1.record()
        timers[name][-1][1] = e1

    rq = pwq.rtn_quantize_zp if L.zp else pwq.rtn_quantize
    if parts == "rtn":
        k = t("rtn_quantize"); rq(L.W, s.bits, s.group_size, want_codes=False, out=L.rq); done(k)
        k = t("recon_mse")
        pwq.recon_mse(L.X, L.W, L.rq["scales"], s.bits, s.group_size, packed=L.rq["packed"], mse=L.mse[1:2],
                      zeros=L.rq.get("zeros"))
        done(k)
        return
    k = t("hessian_accumulate"); L.H.zero_(); pwq.hessian_accumulate(L.X, L.H); done(k)
    if after_hessian is not None:
        after_hessian()
    k = t("hessian_damp"); pwq.hessian_damp(L.H, s.damp, lambda_out=L.lam); done(k)
    perm = None
    if L.act:
        k = t("act_order_perm"); perm = pwq.act_order_perm(L.H); done(k)
    k = t("chol_inverse_upper"); pwq.chol_inverse_upper(L.H, perm, U=L.U, info=L.info); done(k)
    k = t("gptq_quantize_layer")
    gq = pwq.gptq_quantize_layer_zp if L.zp else pwq.gptq_quantize_layer
    gq(L.W, L.U, L.info, s.bits, s.group_size, s.block_size, perm=perm, want_codes=False, want_packed=True, out=L.gq)
    done(k)
    if parts == "all":
        k = t("rtn_quantize"); rq(L.W, s.bits, s.group_size, want_codes=False, out=L.rq); done(k)
    k = t("dequant")
    if L.zp:
        pwq.dequant_zp(L.gq["scales"], L.gq["zeros"], s.d_in, s.bits, s.group_size, packed=L.gq["packed"],
                       g_idx=L.gq.get("g_idx"), out=L.what)
    else:
        pwq.dequant(L.gq["scales"], s.d_in, s.bits, s.group_size, packed=L.gq["packed"], g_idx=L.gq.get("g_idx"),
                    out=L.what)
    done(k)
    k = t("recon_mse")
    if L.mse_h:
        # H is damped by now: its damping is taken off as the shift
        pwq.recon_mse_hessian(L.H, s.n_tok, L.W, L.gq["scales"], s.bits, s.group_size, packed=L.gq["packed"],
                              g_idx=L.gq.get("g_idx"), zeros=L.gq.get("zeros"), shift=L.lam, mse=L.mse[0:1])
        if parts == "all":
            pwq.recon_mse_hessian(L.H, s.n_tok, L.W, L.rq["scales"], s.bits, s.group_size, packed=L.rq["packed"],
                                  zeros=L.rq.get("zeros"), shift=L.lam, mse=L.mse[1:2])
    else:
        pwq.recon_mse(L.X, L.W, L.gq["scales"], s.bits, s.group_size, packed=L.gq["packed"], g_idx=L.gq.get("g_idx"),
                      mse=L.mse[0:1], zeros=L.gq.get("zeros"))
        if parts == "all":
            pwq.recon_mse(L.X, L.W, L.rq["scales"], s.bits, s.group_size, packed=L.rq["packed"], mse=L.mse[1:2],
                          zeros=L.rq.get("zeros"))
    done(k)


def work_of(name, spec, zero_point=False):
    """(peak key, algorithmic amount of one call on one layer, unit).  Contractions count
    the flops the method needs (not what the kernels execute); codec passes the bytes they
    must move."""
    m, n, N = spec.d_out, spec.d_in, spec.n_tok
    xb = 4 if spec.x_dtype == "f32" else 2
    wb = 4 if spec.w_dtype == "f32" else 2
    ng = 1 if spec.group_size == 0 else -(-n // spec.group_size)
    pg = 4 if zero_point else 2                  # bytes per group: scale (and zero)
    if name == "hessian_accumulate":            # symmetric X^T X: upper triangle + diagonal
        # float32 X with >= 1024 tokens and d_in >= 256 runs as four bfloat16 products
        bf = xb == 2 or (n >= 256 and N >= 1024)
        return ("mfma_bf16" if bf else "mfma_f32"), N * n * (n + 1), "flop"
    if name == "chol_inverse_upper":            # Cholesky n^3/3 + triangular inverse n^3/3
        return "mfma_f32", 2 * n ** 3 / 3, "flop"
    if name == "gptq_quantize_layer":           # trailing products + in-block rank-1 updates
        return "mfma_f32", m * n * (n - spec.block_size) + m * n * (spec.block_size - 1), "flop"
    if name == "recon_mse":                     # two calls (GPTQ and RTN)
        if mse_through_hessian(spec):           # 2 m n^2 each (dW H), bfloat16 split or float32 MFMA
            return ("mfma_bf16" if mse_split_route(spec) else "mfma_f32"), 2 * (2 * m * n * n), "flop"
        return "mfma_bf16", 2 * (2 * N * n * m), "flop"     # 2 N n m each, bf16 MFMA
    if name == "rtn_quantize":
        return "hbm", m * n * wb + m * n // 2 + pg * m * ng, "byte"
    if name == "dequant":
        return "hbm", m * n // 2 + pg * m * ng + 2 * m * n, "byte"
    return "hbm", 0, "byte"


def traffic_of(workload, layer, call):
    """HBM bytes per call from the committed counter summary, if it was taken on the kernel
    sources as they are now (else None)."""
    try:
        from post_weight_quantization_27_amd import profile_summary
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            data = json.load(f)
        e = data.get(f"{workload}/{layer}")
        if not e or e.get("source_hash") != profile_summary.source_hash():
            return None
        c = e["per_call"].get(call)
        return None if c is None else c["hbm_bytes"]
    except (OSError, ValueError, KeyError):
        return None


def time_quantized_matmul(layers, pwq, torch, tokens, iters=20):
    """Y = X What^T on each layer's packed GPTQ result (float16 X: the layer's first tokens),
    timed with HIP events on the current stream.  Algorithmic bytes: the nibbles, the scales
    (and zeros), X and Y, each once."""
    out = {}
    for L in layers:
        s = L.spec
        m, n = s.d_out, s.d_in
        if n % 32 or (s.group_size and s.group_size % 128):
            continue
        ng = 1 if s.group_size == 0 else -(-n // s.group_size)
        res = {}
        for T in tokens:
            X = L.X[:T].to(torch.float16).contiguous()
            Y = torch.empty((T, m), dtype=torch.float16, device=X.device)
            nb = pwq.lib().pwq_quantized_matmul_workspace_size(T, n, m)
            ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=X.device)
            zeros = L.gq.get("zeros")
            for _ in range(3):
                pwq.quantized_matmul(X, L.gq["packed"], L.gq["scales"], s.group_size, zeros=zeros, out=Y, ws=ws)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(iters):
                pwq.quantized_matmul(X, L.gq["packed"], L.gq["scales"], s.group_size, zeros=zeros, out=Y, ws=ws)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / iters * 1e3
            byt = m * n // 2 + m * ng * (4 if zeros is not None else 2) + T * n * 2 + T * m * 2
            gbs = byt / (us * 1e-6) / 1e9
            res[f"T{T}"] = {"us": round(us, 2), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / 8000.0, 4)}
        out[s.name] = res
    return out


def time_awq(layers, pwq, torch, K):
    """Activation-aware scaling per layer: channel means of |X| and the K-candidate search
    (undamped H formed first, outside the timed span).  Algorithmic work of the scoring
    products: 2 m n^2 flop per candidate on the float32 MFMA engine."""
    out = {}
    for L in layers:
        s = L.spec
        L.H.zero_()
        pwq.hessian_accumulate(L.X, L.H)
        pwq.awq_search(L.W, L.H, s.n_tok, pwq.channel_abs_mean(L.X), s.bits, s.group_size, K, zero_point=L.zp)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        a = pwq.channel_abs_mean(L.X)
        r = pwq.awq_search(L.W, L.H, s.n_tok, a, s.bits, s.group_size, K, zero_point=L.zp)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        mse = r["mse"].cpu().tolist()
        best = int(r["best"].item())
        flop = 2.0 * s.d_out * s.d_in * s.d_in * K
        out[s.name] = {"ms": round(ms, 3), "alpha": round(best / (K - 1), 3) if K > 1 else 0.0,
                       "mse_rtn": mse[0], "mse_awq": mse[best],
                       "score_tflops": round(flop / (ms * 1e-3) / 1e12, 2)}
        # the scores' product: the split bfloat16 route on large layers, else float32 MFMA
        pk = "mfma_bf16" if mse_split_route(s) else "mfma_f32"
        out[s.name]["score_peak"] = pk
        out[s.name]["score_frac"] = round(flop / (ms * 1e-3) / 1e12 / PEAK[pk], 4)
    return out


def time_tensor_scales(layers, pwq, torch, iters=20):
    """The per-tensor quantizer's pass over each layer's W (algorithmic bytes: W once)."""
    out = {}
    for L in layers:
        s = L.spec
        for _ in range(3):
            pwq.tensor_scales(L.W, s.bits, zero_point=L.zp)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            pwq.tensor_scales(L.W, s.bits, zero_point=L.zp)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / iters * 1e3
        byt = s.d_out * s.d_in * L.W.element_size()
        out[s.name] = {"us": round(us, 2), "GB/s": round(byt / (us * 1e-6) / 1e9, 1)}
    return out


def _cpu_info():
    """(threads the BLAS uses, CPU model name)."""
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return int(threads), model


def cpu_baseline(specs, synth, layer_name="", rows=256, zero_point=False):
    """The oracle as it stands, timed on a bounded sample of one layer of the workload: the
    Hessian over the first 8192-token tile, damping and the factor of that H (full size),
    GPTQ on ``rows`` seeded rows of W, RTN on every row, dequant of the sampled rows and both
    reconstruction errors of the sampled rows over the tile.  Steps that grow with the tokens
    (Hessian, errors) or the rows (GPTQ, dequant, errors) are scaled linearly to the whole
    layer; damping, the factor and RTN ran whole.  value = the layer's weights / that time."""
    import numpy as np
    import oracle as O
    if layer_name:
        s = next(x for x in specs if x.name == layer_name)
    else:
        s = min(specs, key=lambda x: (x.d_in, x.n_weights))
    sym = not zero_point
    W = synth.weight(s)
    X64 = synth.as_f64(synth.x_tile(s, 0), s.x_dtype)
    ntile = X64.shape[0]
    r = min(rows, s.d_out)
    sel = np.sort(np.random.default_rng([27, s.d_out, s.d_in]).choice(s.d_out, r, replace=False))
    t = {}

    def tick(name, f):
        t0 = time.perf_counter()
        out = f()
        t[name] = time.perf_counter() - t0
        return out

    H = tick("hessian", lambda: O.hessian([X64]))
    Hd, _ = tick("damp", lambda: O.damp_hessian(H, s.damp))
    U = tick("factor", lambda: O.chol_inverse_upper(Hd))
    g = tick("gptq", lambda: O.gptq(W[sel], U, s.bits, s.group_size, s.block_size, sym=sym))
    rt = tick("rtn", lambda: O.rtn(W, s.bits, s.group_size, sym=sym))
    tick("dequant", lambda: O.dequant(g["codes"], g["scales"], s.group_size, out_dtype=np.float16, zeros=g["zeros"]))
    tick("mse", lambda: (O.recon_mse([X64], W[sel], g["What"]), O.recon_mse([X64], W[sel], rt["What"][sel])))
    f_tok, f_row = s.n_tok / ntile, s.d_out / r
    scale = {"hessian": f_tok, "damp": 1.0, "factor": 1.0, "gptq": f_row, "rtn": 1.0, "dequant": f_row,
             "mse": f_tok * f_row}
    layer_s = {k: t[k] * scale[k] for k in t}
    total = sum(layer_s.values())
    threads, model = _cpu_info()
    return {"value": round(s.n_weights / total, 1), "unit": "weights/s", "cores": threads, "kind": "oracle",
            "sample": (f"layer {s.name} ({s.d_in}->{s.d_out}), act-order off: float64 numpy oracle on "
                       f"{ntile} of {s.n_tok} tokens and {r} of {s.d_out} rows (GPTQ, dequant, errors), factor "
                       f"and RTN whole; token- and row-proportional steps scaled to the layer; "
                       f"{sum(t.values()):.1f} s of CPU work"),
            "cpu_model": model, "blas_threads": threads,
            "sample_s": {k: round(v, 3) for k, v in t.items()},
            "layer_s": {k: round(v, 2) for k, v in layer_s.items()},
            "scale": {k: round(v, 3) for k, v in scale.items()}}


def copy_calibration(torch):
    """A plain copy of 1 GiB, three times: each dispatch reads and writes exactly 1 GiB, so a
    traffic counter's reading for it gives the factor between counter units and bytes."""
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 3
    print(json.dumps({"copy_bytes_each_way": 4 * n, "ms_per_copy": round(ms, 4),
                      "read_plus_write_GBps": round(2 * 4 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


def kernel_traffic(workload, layer, cls):
    """HBM bytes per launch of a kernel class from the committed counter summary, if it was
    taken on the kernel sources as they are now (else None)."""
    try:
        from post_weight_quantization_27_amd import profile_summary
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            data = json.load(f)
        e = data.get(f"{workload}/{layer}")
        if not e or e.get("source_hash") != profile_summary.source_hash():
            return None
        pk = e.get("per_kernel", {})
        k = pk.get(cls)
        if not k or not k.get("launches"):
            return None
        # the split route's bytes include its splitting kernels, per product launch
        extra = pk.get("update_split_pieces", {}).get("hbm_bytes", 0.0) if cls == "update_split" else 0.0
        return (k["hbm_bytes"] + extra) / k["launches"]
    except (OSError, ValueError, KeyError):
        return None


def measure(a, layers, streams, main_stream, pwq, torch, act):
    """Timed steps, per-call events and the per-kernel pass for one act-order setting."""
    for L in layers:
        L.act = act
    order = sorted(range(len(layers)), key=lambda i: -layers[i].spec.d_in)
    # The step is as long as its longest chain (the factor of the widest layer is a serial
    # sequence of small launches).  With staggering, that layer's Hessian runs alone, and
    # the other layers start once it is formed, so their large contractions overlap the
    # widest layer's latency-bound factor instead of its Hessian.
    stagger = bool(a.stagger) and bool(a.streams) and len(layers) > 1
    first_done = torch.cuda.Event()
    # The widest layer's round-to-nearest and its error need only W and X: they go to the
    # front of the second layer's stream, off the widest layer's chain.
    side = bool(a.streams) and len(layers) > 1

    def step(timers=None):
        for pos, i in enumerate(order):
            L, st = layers[i], streams[i]
            st.wait_stream(main_stream)
            if stagger and pos > 0:
                st.wait_event(first_done)
            with torch.cuda.stream(st):
                if side and pos == 1:
                    lead = order[0]
                    run_step(layers[lead], pwq, None if timers is None else timers[lead], parts="rtn")
                hook = (lambda: first_done.record()) if (stagger and pos == 0) else None
                run_step(L, pwq, None if timers is None else timers[i], after_hessian=hook,
                         parts="gptq" if (side and pos == 0) else "all")
        for st in streams:
            main_stream.wait_stream(st)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    # host time to submit one step (no synchronisation inside), to see whether launches keep up
    t_sub = time.perf_counter()
    step()
    submit_ms = (time.perf_counter() - t_sub) * 1e3
    torch.cuda.synchronize()

    # timed region: K steps, no per-call events (they would add records between launches)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / a.steps

    # per-call durations: the same K steps again, on the same streams, with HIP events around
    # every call on the stream it runs on; a name's time per step is the sum over its calls in
    # the step (recon_mse: the GPTQ and the RTN error)
    timers = [dict() for _ in layers]
    for _ in range(a.steps):
        step(timers)
    torch.cuda.synchronize()
    per = {}
    for L, T in zip(layers, timers):
        for name, ev in T.items():
            per[(L.spec.name, name)] = sum(x[0].elapsed_time(x[1]) for x in ev) / a.steps

    # per-kernel durations: each layer alone on its stream, the library's events around its
    # large kernels (the Hessian's contraction, the trailing updates, the column blocks)
    # large kernels, with per-call events as well (each call's duration uncontended)
    kern, alone = {}, {}
    for i, L in enumerate(layers):
        T = {}
        with torch.cuda.stream(streams[i]):
            pwq.profile_enable(True)
            for _ in range(a.prof_reps):
                run_step(L, pwq, T)
            torch.cuda.synchronize()
            got = pwq.profile_read()
            pwq.profile_enable(False)
        kern[L.spec.name] = {c: {"ms_per_step": v[0] / a.prof_reps, "work_per_step": v[1] / a.prof_reps,
                                 "launches_per_step": v[2] / a.prof_reps} for c, v in got.items()}
        for name, ev in T.items():
            alone[(L.spec.name, name)] = sum(x[0].elapsed_time(x[1]) for x in ev) / a.prof_reps
    return {"ms": ms, "wall": wall, "submit_ms": submit_ms, "per": per, "kern": kern, "alone": alone,
            "stagger": stagger, "side": side}


def report(a, layers, m, zero_point):
    """The measured figures of one act-order setting as JSON-ready objects."""
    per, kern = m["per"], m["kern"]
    specs = [L.spec for L in layers]
    weights = sum(s.n_weights for s in specs)
    breakdown = {}
    for (lname, name), d in per.items():
        breakdown[name] = breakdown.get(name, 0.0) + d
    out = {"value": round(weights / (m["ms"] * 1e-3), 1), "ms_per_step": round(m["ms"], 4),
           "wall_s_timed": round(m["wall"], 3), "host_submit_ms_per_step": round(m["submit_ms"], 3)}

    # candidate kernels for the roofline: the profiled kernel classes per layer, and the calls
    # that are a single kernel (RTN, dequant) with their HBM bytes
    cands = []
    for s in specs:
        k = kern[s.name]
        x = k["xtx"]
        if x["launches_per_step"]:
            pk = "mfma_bf16" if work_of("hessian_accumulate", s)[0] == "mfma_bf16" else "mfma_f32"
            cands.append(("xtx", s, x["ms_per_step"], x["work_per_step"], x["launches_per_step"], pk, "flop"))
        u = k["update"]
        if u["launches_per_step"]:
            cands.append(("update", s, u["ms_per_step"], u["work_per_step"], u["launches_per_step"], "mfma_f32",
                          "flop"))
        u = k["update_split"]
        if u["launches_per_step"]:
            cands.append(("update_split", s, u["ms_per_step"], u["work_per_step"], u["launches_per_step"], "mfma_bf16",
                          "flop"))
        for cls, call in (("rtn", "rtn_quantize"), ("dequant", "dequant")):
            k = kern[s.name][cls]
            if k["launches_per_step"]:
                cands.append((call, s, k["ms_per_step"], k["work_per_step"], k["launches_per_step"], "hbm", "byte"))
    dom = max(cands, key=lambda c: c[2])
    cls, s, dms, amt, nl, pk, unit = dom
    achieved = amt / (dms * 1e-3) / (1e9 if unit == "byte" else 1e12)
    names = {"xtx": "gemm_rs_kernel<2, DlTiled1, DlTiled1, UpperMap, EpiHess> (pwq_hessian_accumulate's contraction)",
             "update": "gemm_fdl_kernel<..., EpiSub> (pwq_gptq_quantize_layer's trailing updates)",
             "update_split": "gemm_rs_kernel<2, DlTiled6, DlTiled6, XcdRectMap, EpiSub> with its split kernels "
                             "(pwq_gptq_quantize_layer's deep trailing updates on six bf16 products)",
             "rtn_quantize": "pwq_rtn_quantize", "dequant": "pwq_dequant"}
    traffic = None
    if not zero_point and cls in ("xtx", "update", "update_split"):
        tb = kernel_traffic(a.workload, s.name, cls)
        traffic = None if tb is None else tb * nl
    elif not zero_point:
        traffic = traffic_of(a.workload, s.name, cls)
    out["roofline"] = {"bound": "hbm" if pk == "hbm" else "mfma", "kernel": names[cls], "layer": s.name,
                       "achieved": round(achieved, 3), "peak": PEAK[pk],
                       "unit": "GB/s" if unit == "byte" else "TFLOP/s", "frac": round(achieved / PEAK[pk], 5),
                       "traffic": traffic, "launch_ms": round(dms / nl, 4), "launches_per_step": nl,
                       "algorithmic": amt / nl, "peak_kind": pk}
    # the metric's MFMA utilisations: X^T X (the kernel, and the whole call with its
    # transposed copy) and the trailing update, per layer
    xtx, xtx_call, upd, upd_detail, cols = {}, {}, {}, {}, {}
    for s in specs:
        k = kern[s.name]
        pk = work_of("hessian_accumulate", s)[0]
        if k["xtx"]["ms_per_step"]:
            xtx[s.name] = round(k["xtx"]["work_per_step"] / (k["xtx"]["ms_per_step"] * 1e-3) / 1e12 / PEAK[pk], 4)
        d = per.get((s.name, "hessian_accumulate"))
        if d:
            xtx_call[s.name] = round(work_of("hessian_accumulate", s)[1] / (d * 1e-3) / 1e12 / PEAK[pk], 4)
        u, us = k["update"], k["update_split"]
        ms_u = u["ms_per_step"] + us["ms_per_step"]
        if ms_u:
            # the MFMA utilisation of the update's time: each route's executed work against the
            # peak of the pipe it runs on (float32 products; bf16 products of the split route)
            busy_s = u["work_per_step"] / (PEAK["mfma_f32"] * 1e12) + us["work_per_step"] / (PEAK["mfma_bf16"] * 1e12)
            upd[s.name] = round(busy_s / (ms_u * 1e-3), 4)
            alg = s.d_out * s.d_in * (s.d_in - s.block_size)
            # float32 work done: the split route executes six bf16 products per float32 one
            # (its depth, 1024 error columns, is a whole multiple of 64)
            f32_work = u["work_per_step"] + us["work_per_step"] / 6.0
            routes = {}
            if u["ms_per_step"]:
                tf = u["work_per_step"] / (u["ms_per_step"] * 1e-3) / 1e12
                routes["f32"] = {"ms": round(u["ms_per_step"], 3), "launches": u["launches_per_step"],
                                 "flops": u["work_per_step"], "TFLOP/s": round(tf, 2),
                                 "frac_peak": round(tf / PEAK["mfma_f32"], 4)}
            if us["ms_per_step"]:
                tf = us["work_per_step"] / (us["ms_per_step"] * 1e-3) / 1e12
                routes["bf16_split"] = {"ms": round(us["ms_per_step"], 3), "launches": us["launches_per_step"],
                                        "bf16_flops": us["work_per_step"], "TFLOP/s": round(tf, 2),
                                        "frac_peak": round(tf / PEAK["mfma_bf16"], 4)}
            upd_detail[s.name] = {"ms": round(ms_u, 3), "launches": u["launches_per_step"] + us["launches_per_step"],
                                  "algorithmic_flops": alg, "f32_flops_done": f32_work,
                                  "f32_equivalent_TFLOP/s": round(f32_work / (ms_u * 1e-3) / 1e12, 2), "routes": routes}
            tb = None if zero_point else kernel_traffic(a.workload, s.name, "update")
            tbs = None if zero_point or not us["launches_per_step"] else kernel_traffic(a.workload, s.name,
                                                                                        "update_split")
            if tb is not None and (tbs is not None or not us["launches_per_step"]):
                hb = tb * u["launches_per_step"] + (tbs * us["launches_per_step"] if tbs else 0.0)
                # without lazy batching every column's error would be applied to all later
                # columns of the float32 working copy at once: a read and a write of each
                # (d_out x (d_in - j - 1)) slab, 8 d_out (d_in - j - 1) bytes for column j
                per_col = 8.0 * s.d_out * s.d_in * (s.d_in - 1) / 2
                upd_detail[s.name].update({"hbm_bytes": hb, "per_column_update_bytes": per_col,
                                           "traffic_reduction": round(per_col / hb, 1)})
        c = k["columns"]
        if c["ms_per_step"]:
            cols[s.name] = {"ms": round(c["ms_per_step"], 3), "launches": c["launches_per_step"]}
    out["xtx_mfma_util"] = xtx
    out["xtx_call_mfma_util"] = xtx_call
    out["update_mfma_util"] = upd
    out["update"] = upd_detail
    out["column_blocks"] = cols
    alone = m["alone"]
    codec = {}
    for s in specs:
        for cls, call in (("rtn", "rtn_quantize"), ("dequant", "dequant")):
            k = kern[s.name][cls]
            if k["launches_per_step"]:
                ms_k = k["ms_per_step"] / k["launches_per_step"]
                gbs = k["work_per_step"] / k["launches_per_step"] / (ms_k * 1e-3) / 1e9
                codec[f"{s.name}/{call}"] = {"us": round(ms_k * 1e3, 1), "GB/s": round(gbs, 1),
                                             "frac_hbm": round(gbs / PEAK["hbm"], 4),
                                             "call_us": round(alone.get((s.name, call), 0.0) * 1e3, 1)}
    out["codec_hbm"] = codec
    out["breakdown_ms"] = {k: round(v, 4) for k, v in sorted(breakdown.items(), key=lambda kv: -kv[1])}
    out["breakdown_ms_by_layer"] = {f"{ln}/{nm}": round(v, 4) for (ln, nm), v in sorted(per.items(), key=lambda kv: -kv[1])}
    # each layer alone on the GPU (the per-kernel pass): what the layer costs without the others
    out["layer_ms_alone"] = {s.name: round(sum(v for (ln, _), v in alone.items() if ln == s.name), 3) for s in specs}
    out["breakdown_ms_alone_by_layer"] = {f"{ln}/{nm}": round(v, 4)
                                          for (ln, nm), v in sorted(alone.items(), key=lambda kv: -kv[1])}
    out["mse_gptq_rtn"] = {L.spec.name: [float(x) for x in L.mse.cpu().tolist()] for L in layers}
    return out


def main():
    a = parse()
    if a.gpus != 1:
        print("bench.py measures one GPU; runs on several GPUs are not supported (use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    if a.copy_calibration:
        copy_calibration(torch)
        return
    from post_weight_quantization_27_amd import pwq, synth
    pwq.lib()
    specs = synth.workload(a.workload)
    if a.layers:
        keep = set(a.layers.split(","))
        specs = [s for s in specs if s.name in keep]
    settings = {"off": [False], "on": [True], "both": [False, True]}[a.act_order]
    if a.streams < 0:
        a.streams = 1 if max(s.d_in for s in specs) < 4096 else 0
    t_in = time.perf_counter()
    layers = [Layer(s, torch, pwq, synth, settings[0], a.zero_point) for s in specs]
    torch.cuda.synchronize()
    print(f"inputs resident after {time.perf_counter() - t_in:.1f} s", file=sys.stderr, flush=True)

    # layers are independent: each runs on its own stream (default priority), so the
    # single-workgroup and few-workgroup kernels of one layer overlap with the others
    main_stream = torch.cuda.current_stream()
    streams = [torch.cuda.Stream() for _ in layers] if a.streams else [main_stream for _ in layers]

    results = []
    for act in settings:
        m = measure(a, layers, streams, main_stream, pwq, torch, act)
        results.append((act, m, report(a, layers, m, a.zero_point)))
        print(f"act-order {'on' if act else 'off'}: {m['ms']:.3f} ms per step", file=sys.stderr, flush=True)
    act0, m0, r0 = results[0]
    toks = [int(x) for x in a.matmul_tokens.split(",") if x.strip()]
    qmm = time_quantized_matmul(layers, pwq, torch, toks) if toks else {}
    pts = time_tensor_scales(layers, pwq, torch) if toks else {}
    awq = time_awq(layers, pwq, torch, a.awq_alphas) if a.awq_alphas > 0 else {}

    bf = specs[0].x_dtype == "bf16"
    out = {
        "metric": METRIC, "value": r0["value"], "unit": "weights/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": r0["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16 X: bf16 MFMA with f32 accumulation (X^T X); f32 factor and GPTQ loop, their deep "
                  "products on 256-tile grids as six bf16 MFMA products of three-piece bf16 splits (f32-level "
                  "terms, f32 accumulation)" if bf else
                  "f32 X as bf16 hi/lo pairs on bf16 MFMA, f32 accumulation (X^T X); f32 factor and GPTQ loop, their "
                  "deep products on 256-tile grids as six bf16 MFMA products of three-piece bf16 splits"),
        "data": "synthetic",
        "config": {"workload": a.workload, "layers": [f"{s.name}:{s.d_in}->{s.d_out}" for s in specs],
                   "n_tok": specs[0].n_tok, "bits": specs[0].bits, "group_size": specs[0].group_size,
                   "block_size": specs[0].block_size, "damp": specs[0].damp, "act_order": act0,
                   "zero_point": bool(a.zero_point), "layer_streams": bool(a.streams), "stagger": m0["stagger"],
                   "mse_route": {L.spec.name: ("hessian" if L.mse_h else "tokens") for L in layers},
                   "rtn_off_chain": m0["side"]},
    }
    for k, v in r0.items():
        if k not in ("value", "ms_per_step"):
            out[k] = v
    for act, m, r in results[1:]:
        out["act_order_on" if act else "act_order_off"] = r
    out["quantized_matmul"] = qmm
    out["tensor_scales"] = pts
    out["awq"] = awq
    # steps of the path each layer ran (for counter summaries): per setting, warm-up, one
    # submit-timed step, K timed, K with per-call events, and the per-kernel pass
    out["path_steps_run"] = len(settings) * (a.warmup + 1 + 2 * a.steps + a.prof_reps)
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(specs, synth, a.cpu_layer, a.cpu_rows, a.zero_point)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
