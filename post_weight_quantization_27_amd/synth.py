"""Seeded synthetic inputs for layer-wise weight quantization.

This module only draws inputs: weight matrices W (d_out x d_in) and calibration
activations X (tokens x d_in) with the shapes, dtypes and value distributions of
the layer sets the method is applied to.  It holds none of the quantization
arithmetic, so the CPU oracle and the GPU path can both take their inputs from
here without sharing any part of the method.

Recipe (every draw is float64, then rounded once, round-to-nearest-even, to the
stored dtype):

* one numpy ``default_rng([27, workload_id, layer, tensor, tile])`` stream per
  tensor; tensor ids are W=0, X=1, outlier-channel choice=2, W-outlier
  positions=3, per-row std jitter=4;
* X is drawn per tile of 8192 tokens (tile index in the seed), in row chunks,
  so no caller ever needs two copies of a large X;
* "1% outlier channels x f": k = round(0.01 * d_in) column indices chosen
  without replacement; those columns of X are multiplied by f for every token;
* "0.1% outlier weights x10": round(0.001 * d_out * d_in) flat positions of W
  chosen without replacement, multiplied by 10;
* row jitter: row r of W has std 0.02 * u_r with u_r ~ U(0.5, 2);
* heavy-tailed rows: w = 0.015 * t / sqrt(2), t ~ Student-t(4) (unit variance).

The calibration sets of the pages (ag_news samples, 128 C4 samples of 2048
tokens) are not available; these synthetic X stand in for them with the same
token counts.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import List, Optional

import numpy as np

SEED_ROOT = 27
TILE_TOKENS = 8192
T_W, T_X, T_OUTCH, T_WOUT, T_JITTER = 0, 1, 2, 3, 4

F32, F16, BF16 = "f32", "f16", "bf16"


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    """One linear layer y = x W^T with W of shape d_out x d_in."""

    workload_id: int
    layer: int
    name: str
    d_in: int
    d_out: int
    n_tok: int
    w_dtype: str          # "f32" | "f16"
    x_dtype: str          # "f32" | "bf16"
    w_kind: str           # "normal" | "normal_jitter" | "normal_wout" | "student_t"
    x_outlier_factor: float
    group_size: int       # 0 = one scale per output row
    act_order: bool = False
    bits: int = 4
    block_size: int = 128
    damp: float = 0.01

    @property
    def n_weights(self) -> int:
        return self.d_in * self.d_out

    def with_(self, **kw) -> "LayerSpec":
        return dataclasses.replace(self, **kw)


def _gpt2_block_layers(wid: int, first: int, block: int, n_tok: int, jitter: bool) -> List[LayerSpec]:
    kind = "normal_jitter" if jitter else "normal"
    shapes = [("c_attn", 768, 2304), ("attn_c_proj", 768, 768), ("c_fc", 768, 3072), ("mlp_c_proj", 3072, 768)]
    out = []
    for i, (nm, din, dout) in enumerate(shapes):
        out.append(LayerSpec(wid, first + i, f"h{block}.{nm}", din, dout, n_tok, F32, F32, kind, 20.0, 128))
    return out


def workload(name: str) -> List[LayerSpec]:
    """Layer list of a named workload."""
    if name == "single_768":
        # one 768 -> 768 layer, 20 sequences x 64 tokens, one scale per row
        return [LayerSpec(1, 0, "linear_768", 768, 768, 1280, F32, F32, "normal", 20.0, 0)]
    if name == "gpt2_block":
        # one GPT-2-small-shaped block: four independent fp32 layers, 8192 tokens
        return _gpt2_block_layers(2, 0, 0, 8192, True)
    if name == "gpt2_stack":
        layers = []
        for b in range(12):
            layers += _gpt2_block_layers(3, 4 * b, b, 8192, True)
        layers.append(LayerSpec(3, 48, "lm_head", 768, 50257, 8192, F32, F32, "normal", 20.0, 128))
        return layers
    if name == "gpt2_1p3b":
        layers = []
        shapes = [("qkv", 2048, 6144), ("o", 2048, 2048), ("fc1", 2048, 8192), ("fc2", 8192, 2048)]
        for b in range(24):
            for i, (nm, din, dout) in enumerate(shapes):
                layers.append(LayerSpec(4, 4 * b + i, f"h{b}.{nm}", din, dout, 262144, F16, BF16,
                                        "normal_wout", 20.0, 128))
        return layers
    if name == "llama70b":
        shapes = [("q_proj", 8192, 8192), ("gate_up_proj", 8192, 28672), ("down_proj", 28672, 8192)]
        return [LayerSpec(5, i, nm, din, dout, 262144, F16, BF16, "student_t", 50.0, 128)
                for i, (nm, din, dout) in enumerate(shapes)]
    raise KeyError(name)


WORKLOADS = ("single_768", "gpt2_block", "gpt2_stack", "gpt2_1p3b", "llama70b")


def layer(name: str, layer_name: str) -> LayerSpec:
    for s in workload(name):
        if s.name == layer_name:
            return s
    raise KeyError(layer_name)


def _rng(spec: LayerSpec, tensor: int, tile: int = 0) -> np.random.Generator:
    return np.random.default_rng([SEED_ROOT, spec.workload_id, spec.layer, tensor, tile])


# ---------------------------------------------------------------- rounding of draws

def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values once (nearest, ties to even) to bfloat16; return the raw uint16 bits.

    bfloat16 keeps float32's exponent range, so rounding the 52-bit significand to 7
    stored bits in float64 and then narrowing to float32 is exact; no double rounding.
    Inputs here are finite and far from the subnormal range.
    """
    b = np.ascontiguousarray(x, dtype=np.float64).view(np.uint64)
    lsb = (b >> np.uint64(45)) & np.uint64(1)
    r = (b + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    f = r.view(np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == F32:
        return x64.astype(np.float32)
    if dtype == F16:
        return x64.astype(np.float16)     # numpy narrows float64 -> float16 with one RNE rounding
    if dtype == BF16:
        return f64_to_bf16_bits(x64)
    raise ValueError(dtype)


def as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Promote stored values (float32, float16 or bf16 bits) to float64, exactly."""
    if dtype == BF16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a).astype(np.float64)


# ---------------------------------------------------------------- weights

def weight(spec: LayerSpec) -> np.ndarray:
    """W, d_out x d_in, in spec.w_dtype (float32 or float16)."""
    m, n = spec.d_out, spec.d_in
    rng = _rng(spec, T_W)
    if spec.w_kind == "normal":
        w = rng.standard_normal((m, n)) * 0.02
    elif spec.w_kind == "normal_jitter":
        u = _rng(spec, T_JITTER).uniform(0.5, 2.0, size=m)
        w = rng.standard_normal((m, n)) * (0.02 * u)[:, None]
    elif spec.w_kind == "normal_wout":
        w = rng.standard_normal((m, n)) * 0.02
        k = int(round(0.001 * m * n))
        pos = _rng(spec, T_WOUT).choice(m * n, size=k, replace=False)
        w.reshape(-1)[pos] *= 10.0
    elif spec.w_kind == "student_t":
        w = rng.standard_t(4.0, size=(m, n)) * (0.015 / np.sqrt(2.0))
    else:
        raise ValueError(spec.w_kind)
    return _store(w, spec.w_dtype)


# ---------------------------------------------------------------- activations

def outlier_channels(spec: LayerSpec) -> np.ndarray:
    k = int(round(0.01 * spec.d_in))
    return np.sort(_rng(spec, T_OUTCH).choice(spec.d_in, size=k, replace=False))


def n_tiles(spec: LayerSpec) -> int:
    return (spec.n_tok + TILE_TOKENS - 1) // TILE_TOKENS


def x_tile(spec: LayerSpec, tile: int, rows: Optional[slice] = None) -> np.ndarray:
    """Tokens [8192*tile, 8192*tile + 8192) of X (fewer in a last short tile), stored dtype.

    bf16 is returned as raw uint16 bits.  ``rows`` selects a sub-range of the tile's rows
    (the stream is drawn in order, so the values do not depend on how it is cut).
    """
    t0 = tile * TILE_TOKENS
    nrow = min(TILE_TOKENS, spec.n_tok - t0)
    if nrow <= 0:
        raise IndexError(tile)
    r0, r1 = (0, nrow) if rows is None else (rows.start or 0, min(rows.stop, nrow))
    rng = _rng(spec, T_X, tile)
    n = spec.d_in
    out_dt = np.uint16 if spec.x_dtype == BF16 else np.float32
    out = np.empty((r1 - r0, n), dtype=out_dt)
    ch = outlier_channels(spec)
    chunk = max(1, (1 << 22) // n)
    pos = 0
    while pos < r1:
        c = min(chunk, r1 - pos)
        blk = rng.standard_normal((c, n))
        lo, hi = max(pos, r0), min(pos + c, r1)
        if hi > lo:
            part = blk[lo - pos:hi - pos]
            part[:, ch] *= spec.x_outlier_factor
            out[lo - r0:hi - r0] = _store(part, spec.x_dtype)
        pos += c
    return out


def x_full(spec: LayerSpec, threads: int = 8) -> np.ndarray:
    """All of X (n_tok x d_in), stored dtype, tiles drawn in parallel (values are thread-count independent)."""
    nt = n_tiles(spec)
    out_dt = np.uint16 if spec.x_dtype == BF16 else np.float32
    out = np.empty((spec.n_tok, spec.d_in), dtype=out_dt)

    def one(t):
        out[t * TILE_TOKENS: t * TILE_TOKENS + min(TILE_TOKENS, spec.n_tok - t * TILE_TOKENS)] = x_tile(spec, t)

    if nt == 1 or threads <= 1:
        for t in range(nt):
            one(t)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(nt)))
    return out


def x_rows(spec: LayerSpec, token_idx: np.ndarray) -> np.ndarray:
    """Selected token rows of X (stored dtype), drawing only the tiles that hold them."""
    token_idx = np.asarray(token_idx, dtype=np.int64)
    out_dt = np.uint16 if spec.x_dtype == BF16 else np.float32
    out = np.empty((token_idx.size, spec.d_in), dtype=out_dt)
    tiles = token_idx // TILE_TOKENS
    for t in np.unique(tiles):
        sel = np.nonzero(tiles == t)[0]
        local = token_idx[sel] - t * TILE_TOKENS
        hi = int(local.max()) + 1
        blk = x_tile(spec, int(t), slice(0, hi))
        out[sel] = blk[local]
    return out
