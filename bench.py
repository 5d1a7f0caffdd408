"""Throughput of the layer-wise quantization path on one MI355X.

One step = every step of the path for every layer of the workload, on inputs already
resident in HBM: Hessian from X, damping, [act-order], H^-1 factor, GPTQ (INT4 packed +
fp16 scales), RTN, dequant of the GPTQ result, and the reconstruction MSE of both (through
the tokens, or through H when n_tok >= 10 d_in, where that product is the cheaper one).
The value is weights quantized per second (sum of d_out * d_in over the layers / step).

Prints ONE JSON line.  The value comes from K timed steps with no events between the
launches; per-call durations come from K more steps with HIP events recorded around every
call on the stream it runs on (each layer has its own stream, which the binding passes to
libpwq).  The roofline object describes the longest (layer, call) launch.
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
    ap.add_argument("--workload", default="gpt2_block")
    ap.add_argument("--layers", default="", help="comma-separated layer names (default: all)")
    ap.add_argument("--act-order", action="store_true")
    ap.add_argument("--zero-point", action="store_true", help="the asymmetric form (a scale and a zero per group)")
    ap.add_argument("--streams", type=int, default=1, help="1: one stream per layer (default), 0: all on one stream")
    ap.add_argument("--stagger", type=int, default=1,
                    help="1: the layer with the longest chain starts alone and the others once its Hessian is "
                         "formed (default), 0: all layers start together")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--awq-alphas", type=int, default=21,
                    help="grid size of the activation-aware scaling search timed per layer (0 to skip)")
    ap.add_argument("--matmul-tokens", default="1,16",
                    help="token counts at which Y = X What^T is timed on each layer's GPTQ output ('' to skip)")
    ap.add_argument("--cpu-layers", default="", help="layers the oracle baseline runs (default: all)")
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


# kernels one call launches, for the roofline's description (chol and gptq per 128 columns)
def launches_of(name, spec):
    nb = -(-spec.d_in // 128)
    if name == "chol_inverse_upper":            # below 4096 the next diagonal factor joins the update launch
        return 2 + (2 if spec.d_in < 4096 else 3) * nb
    if name == "gptq_quantize_layer":
        return 1 + 2 * nb
    if name == "recon_mse":                     # decode, (split H,) product, final sum; two calls
        return 8 if mse_through_hessian(spec) and mse_split_route(spec) else 6
    return None


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


def cpu_baseline(specs, synth, budget_layers, zero_point=False):
    """The oracle, as it stands, on one full step of the selected layers."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    t0 = time.perf_counter()
    weights = 0
    for s in specs:
        if budget_layers and s.name not in budget_layers:
            continue
        W = synth.weight(s)
        X = synth.x_full(s)
        X64 = synth.as_f64(X, s.x_dtype)
        r = O.quantize_layer(W, [X64], s.bits, s.group_size, s.block_size, s.damp, False, sym=not zero_point)
        O.dequant(r["codes"], r["scales"], s.group_size, g_idx=r["g_idx"], out_dtype=np.float16, zeros=r["zeros"])
        weights += s.n_weights
    dt = time.perf_counter() - t0
    names = [s.name for s in specs if not budget_layers or s.name in budget_layers]
    return {"value": weights / dt, "unit": "weights/s", "cores": int(cores), "kind": "oracle",
            "sample": f"one full step of layers {','.join(names)} in float64 numpy ({dt:.1f} s)"}


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
    layers = [Layer(s, torch, pwq, synth, a.act_order, a.zero_point) for s in specs]
    torch.cuda.synchronize()

    # layers are independent: each runs on its own stream (default priority), so the
    # single-workgroup and few-workgroup kernels of one layer overlap with the others
    main = torch.cuda.current_stream()
    streams = [torch.cuda.Stream() for _ in layers] if a.streams else [main for _ in layers]
    # the layer with the longest serial chain (largest d_in: most factor blocks) goes first
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
            st.wait_stream(main)
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
            main.wait_stream(st)

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
    # every call on the stream it runs on (kept out of the first timed region, which gives the
    # value, so the event records do not sit between its launches); a name's time per step is
    # the sum over its calls in the step (recon_mse: the GPTQ and the RTN error)
    timers = [dict() for _ in layers]
    for _ in range(a.steps):
        step(timers)
    torch.cuda.synchronize()
    per = {}
    for L, T in zip(layers, timers):
        for name, ev in T.items():
            d = sum(x[0].elapsed_time(x[1]) for x in ev) / a.steps
            per[(L.spec.name, name)] = d
    breakdown = {}
    for (lname, name), d in per.items():
        breakdown[name] = breakdown.get(name, 0.0) + d
    # roofline of the dominant launch: the (layer, call) with the longest duration
    (dl, dn), dms = max(per.items(), key=lambda kv: kv[1])
    dspec = next(L.spec for L in layers if L.spec.name == dl)
    bound, amount, unit = work_of(dn, dspec, a.zero_point)
    achieved = amount / (dms * 1e-3) / (1e9 if unit == "byte" else 1e12)
    peak = PEAK[bound]
    roof = {"bound": "hbm" if bound == "hbm" else "mfma", "kernel": f"pwq_{dn}", "layer": dl,
            "kernels_per_call": launches_of(dn, dspec),
            "achieved": round(achieved, 3), "peak": peak, "unit": "GB/s" if unit == "byte" else "TFLOP/s",
            "frac": round(achieved / peak, 5), "traffic": None if a.zero_point else traffic_of(a.workload, dl, dn), "launch_ms": round(dms, 4),
            "algorithmic": amount, "peak_kind": bound}
    # the metric's X^T X MFMA utilisation, per layer
    xtx = {}
    for L in layers:
        bnd, amt, _ = work_of("hessian_accumulate", L.spec)
        d = per.get((L.spec.name, "hessian_accumulate"))
        if d:
            xtx[L.spec.name] = round(amt / (d * 1e-3) / 1e12 / PEAK[bnd], 4)
    mses = {L.spec.name: [float(x) for x in L.mse.cpu().tolist()] for L in layers}
    toks = [int(x) for x in a.matmul_tokens.split(",") if x.strip()]
    qmm = time_quantized_matmul(layers, pwq, torch, toks) if toks else {}
    pts = time_tensor_scales(layers, pwq, torch) if toks else {}
    awq = time_awq(layers, pwq, torch, a.awq_alphas) if a.awq_alphas > 0 else {}

    weights = sum(s.n_weights for s in specs)
    value = weights / (ms * 1e-3)
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "weights/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32" if specs[0].x_dtype == "f32" else "bf16-in/f32-acc",
        "data": "synthetic",
        "config": {"workload": a.workload, "layers": [f"{s.name}:{s.d_in}->{s.d_out}" for s in specs],
                   "n_tok": specs[0].n_tok, "bits": specs[0].bits, "group_size": specs[0].group_size,
                   "block_size": specs[0].block_size, "damp": specs[0].damp, "act_order": bool(a.act_order),
                   "zero_point": bool(a.zero_point), "layer_streams": bool(a.streams), "stagger": stagger,
                   "mse_route": {L.spec.name: ("hessian" if L.mse_h else "tokens") for L in layers},
                   "rtn_off_chain": side},
        "roofline": roof,
        "xtx_mfma_util": xtx,
        "breakdown_ms": {k: round(v, 4) for k, v in sorted(breakdown.items(), key=lambda kv: -kv[1])},
        "breakdown_ms_by_layer": {f"{ln}/{nm}": round(v, 4) for (ln, nm), v in sorted(per.items(), key=lambda kv: -kv[1])},
        "mse_gptq_rtn": mses,
        "quantized_matmul": qmm,
        "tensor_scales": pts,
        "awq": awq,
        "wall_s_timed": round(wall, 3),
        "host_submit_ms_per_step": round(submit_ms, 3),
    }
    if not a.no_cpu_baseline:
        cl = set(a.cpu_layers.split(",")) if a.cpu_layers else set()
        out["cpu_baseline"] = cpu_baseline(specs, synth, cl, a.zero_point)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
