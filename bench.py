"""Benchmark of the ternary-weight FP16 GEMM on one MI355X.

One step = one pass of the hot path over the K = 8192 workloads:
  * TQ2, M in {1, 2, 4, 8, 16, 32, 64, 128} on (K, N) = (8192, 8192) and (8192, 28672)
    (i.i.d. trits with P(0) = 0.31, fp16 block scales ~ U(0.01, 0.03));
  * TQ1, M in {1, 4, 16, 64} on the same two shapes (P(0) = 0.3).
Weights, scales and activations are resident in HBM before timing starts; every
call reads its own copy from a ring of buffer sets (>= 1 GiB per shape and
format) so that nothing is served from the 256 MB Infinity Cache.

Printed: one JSON line.  ``value`` is the step's fraction of the roofline,
sum over calls of max(bytes / 8 TB/s, flops / 2.5 PFLOP/s) divided by the
measured step time.  Per-call TB/s, TFLOP/s and fractions are in ``calls``.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
MFMA_F16_PEAK = 2.5e15     # dense FP16 MFMA flop/s
K_MAIN = 8192
SHAPES = [(8192, 8192), (8192, 28672)]  # (K, N)
TQ2_MS = [1, 2, 4, 8, 16, 32, 64, 128]
TQ1_MS = [1, 4, 16, 64]
RING_BYTES = 1 << 30
# TQ1 batch calls take the workspace product from its switch point on
# (--no-workspace: every TQ1 call through tq_gemm_tq1, which needs none)
USE_WORKSPACE = True


def tq1_ldq(K):
    return (-(-K // 5) + 15) // 16 * 16


def alg_bytes(fmt, M, N, K):
    """Bytes the method must move: packed weights, scales, X, Y (for "bwd":
    dY [M][N] in, dX [M][K] out, the same sizes; for "ste", the latent-weight
    gradient: dY [M][N] and X [M][K] in, dW [N][K] fp32 out)."""
    if fmt == "ste":
        return 2 * M * N + 2 * M * K + 4 * N * K
    w = N * K // 4 if fmt in ("tq2", "bwd") else N * tq1_ldq(K)
    return w + 2 * N * (K // 256) + 2 * M * K + 2 * M * N


def alg_flops(M, N, K):
    return 2 * M * N * K


def t_roof(fmt, M, N, K):
    return max(alg_bytes(fmt, M, N, K) / HBM_PEAK, alg_flops(M, N, K) / MFMA_F16_PEAK)


def workload_calls():
    calls = []
    for K, N in SHAPES:
        for M in TQ2_MS:
            calls.append(("tq2", M, N, K))
    for K, N in SHAPES:
        for M in TQ1_MS:
            calls.append(("tq1", M, N, K))
    return calls


PREFILL_MS = [256, 1024, 4096]

# QAT backward: dX = dY (s . T) for the three weight shapes of a 70B layer
# ((N, K) = (8192, 8192) for q / o, (28672, 8192) for gate / up, (8192,
# 28672) for down) at 4096 tokens.
BWD_CALLS = [("bwd", 4096, 8192, 8192), ("bwd", 4096, 28672, 8192), ("bwd", 4096, 8192, 28672)]
# ... and the gradient reaching the latent weights, dW = dY^T X (fp32), same shapes
BWD_CALLS += [("ste", M, N, K) for _, M, N, K in BWD_CALLS]


def prefill_calls():
    """Prompt-sized products on the same two shapes (both formats)."""
    return [(fmt, M, N, K) for fmt in ("tq2", "tq1") for K, N in SHAPES for M in PREFILL_MS]


def tq1_uses_workspace(tq, M, N, K):
    return USE_WORKSPACE and M >= tq.tq_tq1_transcode_min_m(N, K)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- GPU

def build_inputs(torch, tq, calls):
    from synth import activations_fp16, block_scales_fp16, seed_for, ternary_iid
    rings = {}
    for fmt, M, N, K in calls:
        key = (fmt, N, K)
        if key in rings or fmt == "ste":  # dense operands only: nothing packed
            continue
        rng = seed_for(500, N, K, 1 if fmt == "tq2" else 2)
        T = ternary_iid(rng, N, K, 0.31 if fmt == "tq2" else 0.3)
        s = block_scales_fp16(rng, N, K)
        qs = tq.tq_pack_tq1(T)[0] if fmt == "tq1" else tq.tq_pack_tq2(T)[0]
        del T
        per_set = qs.nbytes + s.nbytes
        R = max(2, -(-RING_BYTES // per_set))
        q0 = torch.from_numpy(qs).cuda()
        s0 = torch.from_numpy(s).cuda()
        ring = [(q0, s0)] + [(q0.clone(), s0.clone()) for _ in range(R - 1)]
        rings[key] = {"sets": ring, "next": 0}
        log(f"[bench] {fmt} N={N} K={K}: {R} buffer sets of {per_set / 1e6:.1f} MB")
    xs, ys = {}, {}
    for fmt, M, N, K in calls:
        if fmt == "ste":
            for shape in ((M, N), (M, K)):
                if shape not in xs:
                    xs[shape] = torch.from_numpy(activations_fp16(seed_for(501, *shape),
                                                                  *shape)).cuda()
            if ("w", N, K) not in ys:
                ys[("w", N, K)] = torch.empty((N, K), dtype=torch.float32, device="cuda")
            continue
        xin, yout = ((M, N), (M, K)) if fmt == "bwd" else ((M, K), (M, N))
        if xin not in xs:
            xs[xin] = torch.from_numpy(activations_fp16(seed_for(501, *xin), *xin)).cuda()
        if yout not in ys:
            ys[yout] = torch.empty(yout, dtype=torch.float16, device="cuda")
        if fmt == "tq1" and tq1_uses_workspace(tq, M, N, K) and ("ws", N, K) not in xs:
            xs[("ws", N, K)] = torch.empty(N * K // 4, dtype=torch.uint8, device="cuda")
    return rings, xs, ys


def run_call(tq, fmt, M, N, K, rings, xs, ys, stream):
    if fmt == "ste":
        dY, X, dW = xs[(M, N)], xs[(M, K)], ys[("w", N, K)]
        st = tq.lib.tq_ste_grad_w(dY.data_ptr(), X.data_ptr(), dW.data_ptr(), M, N, K, 0, stream)
        if st != 0:
            raise RuntimeError(f"tq_ste_grad_w failed: {tq.tq_status_string(st)}")
        return
    r = rings[(fmt, N, K)]
    q, s = r["sets"][r["next"]]
    r["next"] = (r["next"] + 1) % len(r["sets"])
    if fmt == "bwd":
        dY, dX = xs[(M, N)], ys[(M, K)]
        st = tq.lib.tq_gemm_tq2_bwd_x(dY.data_ptr(), q.data_ptr(), s.data_ptr(), dX.data_ptr(),
                                      M, N, K, stream)
        if st != 0:
            raise RuntimeError(f"tq_gemm_tq2_bwd_x failed: {tq.tq_status_string(st)}")
        return
    X, Y = xs[(M, K)], ys[(M, N)]
    if fmt == "tq2":
        st = tq.lib.tq_gemm_tq2(X.data_ptr(), q.data_ptr(), s.data_ptr(), Y.data_ptr(), M, N, K,
                                stream)
    elif tq1_uses_workspace(tq, M, N, K):
        # batch and prefill sizes: transcode once per call into the workspace,
        # then the TQ2 kernels (both inside the timed call)
        ws = xs[("ws", N, K)]
        st = tq.lib.tq_gemm_tq1_ws(X.data_ptr(), q.data_ptr(), q.shape[1], s.data_ptr(),
                                   Y.data_ptr(), M, N, K, ws.data_ptr(), ws.numel(), stream)
    else:
        st = tq.lib.tq_gemm_tq1(X.data_ptr(), q.data_ptr(), q.shape[1], s.data_ptr(),
                                Y.data_ptr(), M, N, K, stream)
    if st != 0:
        raise RuntimeError(f"tq_gemm_{fmt} failed: {tq.tq_status_string(st)}")


def kernel_label(tq, fmt, M, N, K):
    """The kernel(s) a call runs, as profilers name them."""
    if fmt == "bwd":
        return "tq2_bwd_x_kernel"
    if fmt == "ste":
        return "tq_ste_grad_w_kernel"
    if fmt == "tq1" and tq1_uses_workspace(tq, M, N, K):
        return "tq1_to_tq2_kernel + " + tq.tq_kernel_name(2, M, N, K)
    return tq.tq_kernel_name(2 if fmt == "tq2" else 1, M, N, K)


def gpu_bench(args, calls):
    """Time the step through HIP graphs (one captured graph per timed step, the
    calls inside rotate through the buffer rings), so host launch overhead is
    not in the measurement.  Per-call averages come from one graph per call
    holding `reps` back-to-back launches of that call."""
    import torch
    import bit_mixed_precision_amd.binding as tq

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    torch.cuda.set_device(0)
    rings, xs, ys = build_inputs(torch, tq, calls)
    torch.cuda.synchronize()

    # one eager pass: kernel attributes are set outside any capture
    for c in calls:
        run_call(tq, *c, rings, xs, ys, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()

    cap = torch.cuda.Stream()

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                fn(cap.cuda_stream)
        return g

    def one_step(sp):
        for c in calls:
            run_call(tq, *c, rings, xs, ys, sp)

    n_graphs = args.warmup + args.steps
    graphs = [capture(one_step) for _ in range(n_graphs)]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    for g in graphs[:args.warmup]:
        g.replay()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")

    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for g in graphs[args.warmup:]:
        g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / args.steps
    log(f"[bench] timed {args.steps} steps: {ms_step:.4f} ms/step (wall {wall:.3f} s)")
    del graphs

    per_call = []
    for fmt, M, N, K in calls:
        reps = args.reps
        g = capture(lambda sp: [run_call(tq, fmt, M, N, K, rings, xs, ys, sp) for _ in range(reps)])
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        del g
        b, f = alg_bytes(fmt, M, N, K), alg_flops(M, N, K)
        tr = t_roof(fmt, M, N, K)
        per_call.append({
            "fmt": fmt, "M": M, "N": N, "K": K,
            "kernel": kernel_label(tq, fmt, M, N, K),
            "us": round(us, 3), "TBps": round(b / us / 1e6, 3), "TFLOPps": round(f / us / 1e6, 2),
            "bound": "hbm" if b / HBM_PEAK >= f / MFMA_F16_PEAK else "mfma",
            "hbm_frac": round(b / HBM_PEAK / (us * 1e-6), 4),
            "mfma_frac": round(f / MFMA_F16_PEAK / (us * 1e-6), 4),
            "roof_frac": round(tr / (us * 1e-6), 4),
        })
    return calls, per_call, ms_step


def context_bench(calls, per_call):
    """Context beside the metric (not part of `value`): the practical read
    ceiling -- one plain streaming-read launch of the bytes an M = 1 TQ2 call
    streams, timed like the calls (a graph of back-to-back launches over
    rotating buffers of at least 1 GiB) -- and torch's FP16 matmul on the TQ2
    sweep shapes, with FP16 weights rotating the same way, for the speedup of
    the packed kernels over plain FP16 weights."""
    import torch
    import bit_mixed_precision_amd.binding as tq

    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    shapes = sorted({(N, K) for fmt, M, N, K in calls if fmt == "tq2"})
    out = {"read_ceiling": [], "fp16_matmul": []}
    ceiling = {}
    reps = 60
    for N, K in shapes:
        nbytes = alg_bytes("tq2", 1, N, K) // 16 * 16
        R = max(2, -(-RING_BYTES // nbytes))
        bufs = [torch.zeros(nbytes, dtype=torch.uint8, device="cuda") for _ in range(R)]
        cap = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for i in range(reps):
                    st = tq.lib.tq_stream_read(bufs[i % R].data_ptr(), nbytes, sink.data_ptr(),
                                               cap.cuda_stream)
                    if st != 0:
                        raise RuntimeError(f"tq_stream_read failed: {tq.tq_status_string(st)}")
        g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        ceiling[(N, K)] = us
        out["read_ceiling"].append({"N": N, "K": K, "bytes": nbytes, "us": round(us, 3),
                                    "TBps": round(nbytes / us / 1e6, 3),
                                    "hbm_frac": round(nbytes / HBM_PEAK / (us * 1e-6), 4)})
        del g, bufs
    for c in per_call:
        if c["fmt"] == "tq2" and c["M"] == 1 and (c["N"], c["K"]) in ceiling:
            c["of_read_ceiling"] = round(ceiling[(c["N"], c["K"])] / c["us"], 4)
    tq2_us = {(c["M"], c["N"], c["K"]): c["us"] for c in per_call if c["fmt"] == "tq2"}
    for N, K in shapes:
        R = max(2, -(-RING_BYTES // (K * N * 2)))
        gen = torch.Generator(device="cuda").manual_seed(502)
        w = [torch.randn(K, N, device="cuda", dtype=torch.float16, generator=gen) * 0.02
             for _ in range(R)]
        for M in sorted({M for fmt, M, n, k in calls if fmt == "tq2" and (n, k) == (N, K)}):
            X = torch.randn(M, K, device="cuda", dtype=torch.float16, generator=gen)
            Y = torch.empty(M, N, device="cuda", dtype=torch.float16)
            for i in range(R):
                torch.mm(X, w[i], out=Y)
            torch.cuda.synchronize()
            n_mm = 30
            e0.record(stream)
            for i in range(n_mm):
                torch.mm(X, w[i % R], out=Y)
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / n_mm * 1e3
            t2 = tq2_us[(M, N, K)]
            out["fp16_matmul"].append({"M": M, "N": N, "K": K, "us": round(us, 3),
                                       "TFLOPps": round(alg_flops(M, N, K) / us / 1e6, 2),
                                       "tq2_us": t2, "tq2_speedup": round(us / t2, 2)})
        del w
    return out


def bwd_context(per_call, reps=3):
    """Context beside the backward metric (not part of `value`): torch's dense
    FP16 products (hipBLASLt) on the same shapes -- dX = dY W with an FP16
    weight matrix, and dW = dY^T X with FP32 output (torch.mm out_dtype) --
    timed with HIP events around `reps` back-to-back calls after two warm-up
    calls, next to the library's kernels' own per-call times."""
    import torch
    out = []
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    for c in per_call:
        M, N, K = c["M"], c["N"], c["K"]
        dY = torch.randn(M, N, dtype=torch.float16, device="cuda")
        if c["fmt"] == "bwd":
            W = torch.randn(N, K, dtype=torch.float16, device="cuda")
            fn = lambda: torch.mm(dY, W)  # noqa: E731
            what = "dX = dY W, FP16 W"
        else:
            X = torch.randn(M, K, dtype=torch.float16, device="cuda")
            try:
                torch.mm(dY.t(), X, out_dtype=torch.float32)
                fn = lambda: torch.mm(dY.t(), X, out_dtype=torch.float32)  # noqa: E731
                what = "dW = dY^T X, FP32 out"
            except (RuntimeError, TypeError):
                fn = lambda: torch.mm(dY.t(), X)  # noqa: E731
                what = "dW = dY^T X, FP16 out"
        for _ in range(2):
            fn()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        out.append({"fmt": c["fmt"], "M": M, "N": N, "K": K, "torch": what, "us": round(us, 1),
                    "TFLOPps": round(alg_flops(M, N, K) / us / 1e6, 1),
                    "ours_us": c["us"], "ours_over_torch_time": round(c["us"] / us, 3)})
        del dY
        torch.cuda.empty_cache()
    return out


def _time_graph(torch, launch, reps):
    """Average µs of one launch: a captured graph of ``reps`` calls of
    ``launch(i, stream)``, replayed once to warm up and once timed."""
    stream = torch.cuda.current_stream()
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for i in range(reps):
                launch(i, cap.cuda_stream)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / reps * 1e3


def _ring(torch, arrays, per_set):
    """Device copies of ``arrays`` (numpy), enough sets for >= 1 GiB in all."""
    R = max(2, -(-RING_BYTES // per_set))
    first = [torch.from_numpy(a).cuda() for a in arrays]
    return [first] + [[t.clone() for t in first] for _ in range(R - 1)]


def _call_record(fmt, M, N, K, us, kernel):
    b, f = alg_bytes(fmt, M, N, K), alg_flops(M, N, K)
    return {"fmt": fmt, "M": M, "N": N, "K": K, "kernel": kernel, "us": round(us, 3),
            "TBps": round(b / us / 1e6, 3), "TFLOPps": round(f / us / 1e6, 2),
            "bound": "hbm" if b / HBM_PEAK >= f / MFMA_F16_PEAK else "mfma",
            "roof_frac": round(t_roof(fmt, M, N, K) / (us * 1e-6), 4)}


def _gemm_launcher(tq, fmt, M, N, K, X, Y, ring, ws=None):
    def launch(i, sp):
        q, sc = ring[i % len(ring)]
        if fmt == "tq2":
            st = tq.lib.tq_gemm_tq2(X.data_ptr(), q.data_ptr(), sc.data_ptr(), Y.data_ptr(), M, N,
                                    K, sp)
        elif ws is not None and M >= tq.tq_tq1_transcode_min_m(N, K):
            st = tq.lib.tq_gemm_tq1_ws(X.data_ptr(), q.data_ptr(), q.shape[1], sc.data_ptr(),
                                       Y.data_ptr(), M, N, K, ws.data_ptr(), ws.numel(), sp)
        else:
            st = tq.lib.tq_gemm_tq1(X.data_ptr(), q.data_ptr(), q.shape[1], sc.data_ptr(),
                                    Y.data_ptr(), M, N, K, sp)
        if st != 0:
            raise RuntimeError(f"tq_gemm_{fmt} failed: {tq.tq_status_string(st)}")
    return launch


# The decode linears of a 3B-class layer at M = 1 (name, K, N), and the
# 1024 x 1024 GEMV; weights ternarized from N(0, 0.02) latents (eps = 1e-5)
# by the host packer, scales fp16(gamma).
SMALL_LAYER = [("q", 3072, 3072), ("k", 3072, 3072), ("v", 3072, 3072), ("o", 3072, 3072),
               ("gate", 3072, 8192), ("up", 3072, 8192), ("down", 8192, 3072)]


def other_configs_bench(reps=30):
    """µs per call of the 1024 x 1024 GEMV (M = 1) and of the seven decode
    linears of a 3B-class layer (M = 1), both formats, latent-ternarized
    weights rotating through >= 1 GiB like the sweep.  These calls are a few
    µs or less, so launch cost dominates: reported as latency beside their
    HBM fractions, not part of ``value``."""
    import torch
    import bit_mixed_precision_amd.binding as tq
    from synth import activations_fp16, latent_weights_f32, seed_for
    out = {"gemv_1024": [], "layer_3b_m1": []}
    shapes = [("gemv_1024", "w", 1024, 1024)] + [("layer_3b_m1", n, K, N) for n, K, N in SMALL_LAYER]
    for group, name, K, N in shapes:
        W = latent_weights_f32(seed_for(900, K, N, len(name)), N, K, 0.02)
        X = torch.from_numpy(activations_fp16(seed_for(901, 1, K), 1, K)).cuda()
        Y = torch.empty((1, N), dtype=torch.float16, device="cuda")
        for fmt in ("tq2", "tq1"):
            qs, sc, _ = (tq.tq_pack_tq2 if fmt == "tq2" else tq.tq_pack_tq1)(W, eps=1e-5)
            ring = _ring(torch, [qs, sc], qs.nbytes + sc.nbytes)
            us = _time_graph(torch, _gemm_launcher(tq, fmt, 1, N, K, X, Y, ring), reps)
            rec = _call_record(fmt, 1, N, K, us, tq.tq_kernel_name(2 if fmt == "tq2" else 1, 1, N, K))
            rec["linear"] = name
            out[group].append(rec)
            del ring
    for fmt in ("tq2", "tq1"):
        rows = [r for r in out["layer_3b_m1"] if r["fmt"] == fmt]
        t = sum(r["us"] for r in rows)
        b = sum(alg_bytes(fmt, 1, r["N"], r["K"]) for r in rows)
        out[f"layer_3b_m1_{fmt}_total"] = {"us": round(t, 3), "TBps": round(b / t / 1e6, 3),
                                           "hbm_frac": round(b / HBM_PEAK / (t * 1e-6), 4)}
    return out


TQ1_PS = [0.3, 0.5, 0.9]


def tq1_vs_tq2_bench(reps=30):
    """TQ1 against TQ2 on the same weights: for each zero fraction p, one i.i.d.
    trit matrix and one scale table per shape, packed both ways, timed at
    M in {1, 4, 16, 64} exactly as the step times its calls (TQ1 through the
    workspace product from its switch point on)."""
    import torch
    import bit_mixed_precision_amd.binding as tq
    from synth import activations_fp16, block_scales_fp16, seed_for, ternary_iid
    rows = []
    for K, N in SHAPES:
        xs = {M: torch.from_numpy(activations_fp16(seed_for(902, M, K), M, K)).cuda()
              for M in TQ1_MS}
        ys = {M: torch.empty((M, N), dtype=torch.float16, device="cuda") for M in TQ1_MS}
        ws = torch.empty(N * K // 4, dtype=torch.uint8, device="cuda")
        for p in TQ1_PS:
            rng = seed_for(903, N, K, int(p * 100))
            T = ternary_iid(rng, N, K, p)
            s = block_scales_fp16(rng, N, K)
            packed = {"tq2": tq.tq_pack_tq2(T)[0], "tq1": tq.tq_pack_tq1(T)[0]}
            del T
            us = {}
            for fmt, qs in packed.items():
                ring = _ring(torch, [qs, s], qs.nbytes + s.nbytes)
                for M in TQ1_MS:
                    us[(fmt, M)] = _time_graph(
                        torch, _gemm_launcher(tq, fmt, M, N, K, xs[M], ys[M], ring, ws), reps)
                del ring
            for M in TQ1_MS:
                r1, r2 = (_call_record(f, M, N, K, us[(f, M)], kernel_label(tq, f, M, N, K))
                          for f in ("tq1", "tq2"))
                rows.append({"p": p, "M": M, "N": N, "K": K, "tq1": r1, "tq2": r2,
                             "tq1_over_tq2_time": round(r1["us"] / r2["us"], 3)})
            log(f"[bench] tq1 vs tq2 N={N} p={p} done")
    return rows


def kernel_source_sha():
    """sha256 (first 16 hex) over the kernel sources, as recorded with the counters."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "bit_mixed_precision_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy of known size),
    or None when there is none or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha") != kernel_source_sha():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("traffic_bytes_per_launch")


def roofline_of(per_call):
    """Roofline object for the kernel that takes the most time in the step."""
    by_kernel = {}
    for c in per_call:
        by_kernel.setdefault(c["kernel"], []).append(c)
    dom = max(by_kernel, key=lambda k: sum(c["us"] for c in by_kernel[k]))
    cs = by_kernel[dom]
    t = sum(c["us"] for c in cs) * 1e-6
    nbytes = sum(alg_bytes(c["fmt"], c["M"], c["N"], c["K"]) for c in cs)
    flops = sum(alg_flops(c["M"], c["N"], c["K"]) for c in cs)
    hbm_bound = nbytes / HBM_PEAK >= flops / MFMA_F16_PEAK
    if hbm_bound:
        achieved, peak, unit = nbytes / t / 1e9, HBM_PEAK / 1e9, "GB/s"
    else:
        achieved, peak, unit = flops / t / 1e12, MFMA_F16_PEAK / 1e12, "TFLOP/s"
    traffic = recorded_traffic(dom)
    return {"kernel": dom, "bound": "hbm" if hbm_bound else "mfma",
            "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic,
            "algorithmic_bytes_per_launch": round(nbytes / len(cs)),
            "launches_per_step": len(cs),
            "avg_launch_us": round(t / len(cs) * 1e6, 3)}


# ----------------------------------------------------------------------------- CPU baseline

def cpu_model():
    """The host CPU's model name (lscpu, else /proc/cpuinfo), or None."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(calls, cols=1024, single_thread_cols=128):
    """The fp64 oracle on the host: each call of the step on ``cols`` sampled
    output columns, time scaled by N / cols, with every BLAS thread; then the
    same on ``single_thread_cols`` columns with BLAS limited to one thread."""
    res = _cpu_baseline_run(calls, cols)
    single_thread_cols = min(cols, single_thread_cols)
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            one = _cpu_baseline_run(calls, single_thread_cols)
        res["single_thread"] = {"value": one["value"], "cores": 1, "s_per_step": one["s_per_step"],
                                "sample": f"every call on {single_thread_cols} sampled output "
                                          f"columns, BLAS limited to one thread, time scaled "
                                          f"by N/{single_thread_cols}"}
    except ImportError:  # pragma: no cover
        res["single_thread"] = None
    res["cpu_model"] = cpu_model()
    res["host_cpus"] = os.cpu_count()
    return res


def _cpu_baseline_run(calls, cols):
    from oracle import gemm_bwd_x_ref, gemm_ref, ste_grad_w_ref
    from synth import activations_fp16, block_scales_fp16, seed_for, ternary_iid
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    weights = {}
    total_t = total_roof = total_bytes = total_flops = 0.0
    for fmt, M, N, K in calls:
        if fmt == "ste":  # dW on `cols` sampled rows n
            dY = activations_fp16(seed_for(604, M, cols), M, cols)
            X = activations_fp16(seed_for(605, M, K), M, K)
            t = time.perf_counter()
            ste_grad_w_ref(dY, X)
            dt = (time.perf_counter() - t) * (N / cols)
        elif fmt == "bwd":  # dX on `cols` sampled columns k: the full N x cols weight slice
            rng = seed_for(602, N, K)
            T = ternary_iid(rng, N, 256, 0.31)
            s = block_scales_fp16(rng, N, 256)
            dY = activations_fp16(seed_for(603, M, N), M, N)
            t = time.perf_counter()
            gemm_bwd_x_ref(dY, T, s)
            dt = (time.perf_counter() - t) * (K / 256)
        else:
            key = (fmt, K)
            if key not in weights:
                rng = seed_for(600, K, 1 if fmt == "tq2" else 2)
                weights[key] = (ternary_iid(rng, cols, K, 0.31), block_scales_fp16(rng, cols, K))
            T, s = weights[key]
            X = activations_fp16(seed_for(601, M, K), M, K)
            t = time.perf_counter()
            gemm_ref(X, T, s)
            dt = (time.perf_counter() - t) * (N / cols)
        total_t += dt
        total_roof += t_roof(fmt, M, N, K)
        total_bytes += alg_bytes(fmt, M, N, K)
        total_flops += alg_flops(M, N, K)
    return {"value": round(total_roof / total_t, 8), "unit": "fraction of MI355X roofline",
            "cores": threads, "kind": "oracle",
            "sample": f"every call of one step on {cols} sampled output columns (fp64 dequantize + "
                      f"numpy matmul), time scaled by N/{cols}",
            "s_per_step": round(total_t, 3),
            "TBps": round(total_bytes / total_t / 1e12, 6),
            "TFLOPps": round(total_flops / total_t / 1e12, 6)}


# ----------------------------------------------------------------------------- device pack

PACK_SHAPE = (28672, 8192)  # (N, K): the largest linear of the sweep, 940 MB of fp32 latents


def pack_bytes(fmt, N, K):
    """The method's traffic: gamma needs all of |W| before any trit is known, so
    W is read twice (4 B per weight each), then qs and the scales are written."""
    q = N * K // 4 if fmt == 2 else N * tq1_ldq(K)
    return 2 * 4 * N * K + q + 2 * N * (K // 256)


def pack_bench(args):
    import torch
    import bit_mixed_precision_amd.binding as tq
    from synth import latent_weights_f32, seed_for

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    torch.cuda.set_device(0)
    N, K = PACK_SHAPE
    W = torch.from_numpy(latent_weights_f32(seed_for(700, N, K), N, K)).cuda()
    stream = torch.cuda.current_stream()
    out = []
    for fmt in (2, 1):
        tq.tq_pack_dev(fmt, W)  # warm
        torch.cuda.synchronize()
        reps = max(1, args.steps // 4)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            _, _, _, st = tq.tq_pack_dev(fmt, W)
        e1.record(stream)
        torch.cuda.synchronize()
        assert int(st.item()) == tq.TQ_OK
        us = e0.elapsed_time(e1) / reps * 1e3
        b = pack_bytes(fmt, N, K)
        out.append({"fmt": "tq%d" % fmt, "N": N, "K": K, "us": round(us, 1),
                    "TBps": round(b / us / 1e6, 3), "hbm_frac": round(b / HBM_PEAK / (us * 1e-6), 4)})
        log(f"[bench] pack tq{fmt}: {us:.1f} us, {b / us / 1e6:.2f} TB/s")
    return out


def pack_cpu_baseline(rows=64):
    """The oracle's ternarize + pack on ``rows`` rows of the same latents
    (gamma over those rows), time scaled by N / rows."""
    from oracle import pack_tq1_ref, pack_tq2_ref, ternarize_ref
    from synth import latent_weights_f32, seed_for
    N, K = PACK_SHAPE
    W = latent_weights_f32(seed_for(701, rows, K), rows, K)
    res = {}
    for fmt in (2, 1):
        t = time.perf_counter()
        T, _ = ternarize_ref(W, 1e-5)
        pack_tq2_ref(T) if fmt == 2 else pack_tq1_ref(T)
        res["tq%d" % fmt] = (time.perf_counter() - t) * (N / rows)
    tot_b = sum(pack_bytes(f, N, K) for f in (2, 1))
    tot_t = sum(res.values())
    return {"value": round(tot_b / tot_t / 1e12 / (HBM_PEAK / 1e12), 8),
            "unit": "fraction of HBM roofline", "cores": 1, "kind": "oracle",
            "sample": f"ternarize + pack of {rows} rows of the {N} x {K} latents, time scaled "
                      f"by N/{rows}", "s_tq2": round(res["tq2"], 3), "s_tq1": round(res["tq1"], 3)}


# ----------------------------------------------------------------------------- layer stack

# One decoder layer of the 80-layer stack, (name, K, N): 68.45 B weights, 17.65 GB TQ2.
STACK_LAYER = [("q", 8192, 8192), ("k", 8192, 1024), ("v", 8192, 1024), ("o", 8192, 8192),
               ("gate", 8192, 28672), ("up", 8192, 28672), ("down", 28672, 8192)]
STACK_LAYERS = 80
STACK_MS = [1, 16]


def stack_bench(args):
    """All 560 TQ2 linears of the stack, each with its own weights in HBM, back to
    back in one HIP graph per M (activations random per linear shape), run two
    ways over the same buffers: seven products per layer, and the fused decode
    step of four launches per layer (q, k, v as one product over the
    row-concatenated matrices; o; gate / up with SwiGLU in one launch; down)."""
    import torch
    import bit_mixed_precision_amd.binding as tq
    from synth import activations_fp16, block_scales_fp16, seed_for, ternary_iid

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    torch.cuda.set_device(0)
    base = {}
    for name, K, N in STACK_LAYER:
        rng = seed_for(800, K, N, len(name))
        T = ternary_iid(rng, N, K, 0.31)
        s = block_scales_fp16(rng, N, K)
        base[name] = (tq.tq_pack_tq2(T)[0], s)
        del T
    qkv_q = np.concatenate([base[n][0] for n in ("q", "k", "v")])
    qkv_s = np.concatenate([base[n][1] for n in ("q", "k", "v")])
    dev = lambda a: torch.from_numpy(a).cuda()
    layers = []  # every linear of every layer in its own buffers
    for _ in range(STACK_LAYERS):
        L = {"qkv": (dev(qkv_q), dev(qkv_s))}
        r0 = 0
        for n in ("q", "k", "v"):
            rows = base[n][0].shape[0]
            L[n] = (L["qkv"][0][r0:r0 + rows], L["qkv"][1][r0:r0 + rows])  # views, same memory
            r0 += rows
        for n in ("o", "gate", "up", "down"):
            L[n] = (dev(base[n][0]), dev(base[n][1]))
        layers.append(L)
    torch.cuda.synchronize()
    log(f"[bench] stack: {STACK_LAYERS} layers x {len(STACK_LAYER)} linears in HBM")
    dims = {name: (K, N) for name, K, N in STACK_LAYER}
    results = []
    stream = torch.cuda.current_stream()
    for M in STACK_MS:
        xs = {K: torch.from_numpy(activations_fp16(seed_for(801, M, K), M, K)).cuda()
              for K in (8192, 28672)}
        ys = {N: torch.empty((M, N), dtype=torch.float16, device="cuda")
              for N in (1024, 8192, 10240, 28672)}

        def gemm(q, sc, K, N, sp):
            st = tq.lib.tq_gemm_tq2(xs[K].data_ptr(), q.data_ptr(), sc.data_ptr(),
                                    ys[N].data_ptr(), M, N, K, sp)
            if st != 0:
                raise RuntimeError(tq.tq_status_string(st))

        def step_separate(sp):
            for L in layers:
                for name, K, N in STACK_LAYER:
                    gemm(*L[name], K, N, sp)

        def step_fused(sp):
            for L in layers:
                gemm(*L["qkv"], 8192, 10240, sp)
                gemm(*L["o"], 8192, 8192, sp)
                st = tq.lib.tq_gemm_tq2_swiglu(xs[8192].data_ptr(), L["gate"][0].data_ptr(),
                                               L["gate"][1].data_ptr(), L["up"][0].data_ptr(),
                                               L["up"][1].data_ptr(), ys[28672].data_ptr(), M,
                                               28672, 8192, sp)
                if st != 0:
                    raise RuntimeError(tq.tq_status_string(st))
                gemm(*L["down"], 28672, 8192, sp)

        row = {"M": M}
        for label, step in (("separate", step_separate), ("fused", step_fused)):
            step(stream.cuda_stream)  # eager pass: kernel attributes outside capture
            torch.cuda.synchronize()
            cap = torch.cuda.Stream()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(cap):
                with torch.cuda.graph(g, stream=cap):
                    step(cap.cuda_stream)
            for _ in range(2):
                g.replay()
            torch.cuda.synchronize()
            reps = max(1, args.steps // 4)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            row[label + "_ms"] = round(e0.elapsed_time(e1) / reps, 4)
            del g
        ms = min(row["separate_ms"], row["fused_ms"])
        nbytes = STACK_LAYERS * sum(alg_bytes("tq2", M, N, K) for _, K, N in STACK_LAYER)
        flops = STACK_LAYERS * sum(alg_flops(M, N, K) for _, K, N in STACK_LAYER)
        roof = max(nbytes / HBM_PEAK, flops / MFMA_F16_PEAK)
        row.update({"ms_per_step": row["fused_ms"], "TBps": round(nbytes / row["fused_ms"] / 1e9, 3),
                    "roofline_ms": round(roof * 1e3, 4),
                    "roof_frac": round(roof * 1e3 / row["fused_ms"], 4),
                    "launches_per_step": {"separate": STACK_LAYERS * len(STACK_LAYER),
                                          "fused": STACK_LAYERS * 4}})
        results.append(row)
        log(f"[bench] stack M={M}: separate {row['separate_ms']:.3f} ms, fused {row['fused_ms']:.3f} ms "
            f"per step ({nbytes / ms / 1e9:.2f} TB/s at the better)")
    return results


def stack_cpu_baseline(cols=256):
    """The oracle on one layer (every linear on ``cols`` sampled output columns,
    time scaled by N / cols), times 80 layers, at M = 1."""
    from oracle import gemm_ref
    from synth import activations_fp16, block_scales_fp16, seed_for, ternary_iid
    t_total = 0.0
    for name, K, N in STACK_LAYER:
        rng = seed_for(802, K)
        T, s = ternary_iid(rng, cols, K, 0.31), block_scales_fp16(rng, cols, K)
        X = activations_fp16(seed_for(803, 1, K), 1, K)
        t = time.perf_counter()
        gemm_ref(X, T, s)
        t_total += (time.perf_counter() - t) * (N / cols)
    t_step = t_total * STACK_LAYERS
    nbytes = STACK_LAYERS * sum(alg_bytes("tq2", 1, N, K) for _, K, N in STACK_LAYER)
    return {"value": round(nbytes / HBM_PEAK / t_step, 8), "unit": "fraction of HBM roofline",
            "cores": os.cpu_count() or 1, "kind": "oracle",
            "sample": f"one layer at M = 1, every linear on {cols} sampled output columns, time "
                      f"scaled by N/{cols} and by {STACK_LAYERS} layers", "s_per_step": round(t_step, 3)}


# ----------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--reps", type=int, default=30, help="launches per call when timing each call")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the read-ceiling and FP16-matmul context of the sweep")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the timing of the 1024 x 1024 GEMV, the 3B-class layer and the "
                         "TQ1-vs-TQ2 zero-fraction sweep")
    ap.add_argument("--calls-out", default=None, help="also write the per-call table here (JSON)")
    ap.add_argument("--bwd", action="store_true",
                    help="QAT backward dX = dY (s.T) at the 70B layer shapes, 4096 tokens")
    ap.add_argument("--stack", action="store_true",
                    help="the 560 linears of an 80-layer stack, back to back in one HIP graph")
    ap.add_argument("--pack", action="store_true",
                    help="on-device ternarize + pack of a 28672 x 8192 latent matrix")
    ap.add_argument("--prefill", action="store_true",
                    help="prompt-sized products (M = 256 .. 4096) instead of the M <= 128 step")
    ap.add_argument("--no-workspace", action="store_true",
                    help="every TQ1 call through tq_gemm_tq1 (no workspace: the table-decode "
                         "tiled kernel above 16 rows) instead of the workspace product from "
                         "its switch point on")
    args = ap.parse_args()
    global USE_WORKSPACE
    USE_WORKSPACE = not args.no_workspace
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the product has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.stack:
        rows = stack_bench(args)
        m1 = rows[0]
        out = {
            "metric": "80-layer ternary stack: 560 TQ2 linears per step (fused: 320 launches) vs HBM roofline (M = 1, 16)",
            "value": m1["roof_frac"],
            "unit": "fraction of roofline at M = 1 (HBM 8 TB/s)",
            "n_gpus": 1, "steps": args.steps, "warmup": 2, "ms_per_step": m1["ms_per_step"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f16", "data": "synthetic",
            "config": {"workload": "80 x {q 8192->8192, k/v 8192->1024, o 8192->8192, gate/up "
                                   "8192->28672, down 28672->8192}, 17.65 GB TQ2, one HIP graph; "
                                   "fused step: qkv as one product, gate/up + SwiGLU in one launch",
                       "global_batch": None, "seq_len": None, "parallelism": "none"},
            "per_M": rows,
        }
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = stack_cpu_baseline()
        print(json.dumps(out), flush=True)
        return
    if args.pack:
        rows = pack_bench(args)
        t_roof_sum = sum(pack_bytes(2 if r["fmt"] == "tq2" else 1, r["N"], r["K"]) for r in rows)
        t_sum = sum(r["us"] for r in rows) * 1e-6
        best = max(rows, key=lambda r: r["us"])
        out = {
            "metric": "on-device ternarize + pack throughput vs HBM roofline (TQ2, TQ1)",
            "value": round(t_roof_sum / HBM_PEAK / t_sum, 4),
            "unit": "fraction of HBM roofline (8 TB/s); W is read twice, qs and scales written",
            "n_gpus": 1, "steps": args.steps, "warmup": 1, "ms_per_step": round(t_sum * 1e3, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f32", "data": "synthetic",
            "config": {"workload": "latents N(0, 0.02) fp32, N x K = %d x %d, eps = 1e-5"
                                   % PACK_SHAPE, "global_batch": None, "seq_len": None,
                       "parallelism": "none"},
            "roofline": {"kernel": "tq_pack_tq%s_dev (3 kernels)" % best["fmt"][-1],
                         "bound": "hbm", "achieved": round(best["TBps"] * 1e3, 1),
                         "peak": HBM_PEAK / 1e9, "unit": "GB/s", "frac": best["hbm_frac"],
                         "traffic": None},
            "calls": rows,
        }
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = pack_cpu_baseline()
        print(json.dumps(out), flush=True)
        return
    calls = BWD_CALLS if args.bwd else prefill_calls() if args.prefill else workload_calls()
    if args.prefill or args.bwd:
        args.reps = min(args.reps, 3)
    calls, per_call, ms_step = gpu_bench(args, calls)
    roof_sum = sum(t_roof(*c) for c in calls)
    value = roof_sum / (ms_step * 1e-3)
    if args.bwd:
        out = {
            "metric": "QAT backward dX = dY (s.T) and straight-through dW = dY^T X TFLOP/s vs "
                      "FP16 MFMA peak, 70B layer shapes at 4096 tokens",
            "value": round(value, 4),
            "unit": "fraction of roofline (FP16 MFMA 2.5 PFLOP/s; every call is MFMA-bound)",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms_step, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f16", "data": "synthetic",
            "config": {"workload": "dX and dW for (N,K) in {(8192,8192),(28672,8192),"
                                   "(8192,28672)}, M=4096 tokens; i.i.d. trits, fp16 block "
                                   "scales; dW fp32",
                       "global_batch": None, "seq_len": None, "parallelism": "none"},
            "roofline": roofline_of(per_call),
            "tflops_total": round(sum(alg_flops(*c[1:]) for c in calls) / (ms_step * 1e-3) / 1e12,
                                  1),
        }
        if not args.no_context:
            log("[bench] context: torch dense FP16 products ...")
            out["context"] = {"torch_dense_fp16": bwd_context(per_call)}
        if not args.no_cpu_baseline:
            log("[bench] CPU baseline (oracle) ...")
            cb = cpu_baseline(calls)
            cb["sample"] = "dX: every call on 256 sampled columns k (the full N x 256 weight " \
                           "slice, fp64 dequantize + numpy matmul), time scaled by K/256; dW: " \
                           "1024 sampled rows n, time scaled by N/1024"
            out["cpu_baseline"] = cb
        out["calls"] = per_call
        print(json.dumps(out), flush=True)
        return
    if args.prefill:
        out = {
            "metric": "ternary GEMM TFLOP/s vs FP16 MFMA peak at prefill sizes M=256..4096, K=8192 "
                      "(TQ2, TQ1)",
            "value": round(value, 4),
            "unit": "fraction of roofline (FP16 MFMA 2.5 PFLOP/s; every call is MFMA-bound)",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms_step, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f16", "data": "synthetic",
            "config": {"workload": "TQ2 and TQ1, M in {256, 1024, 4096} on (K,N)=(8192,8192),"
                                   "(8192,28672); i.i.d. trits, fp16 block scales",
                       "tq1_batch": "workspace product from its switch point" if USE_WORKSPACE
                                    else "no workspace (tq_gemm_tq1)",
                       "global_batch": None, "seq_len": None, "parallelism": "none"},
            "roofline": roofline_of(per_call),
            "tflops_total": round(sum(alg_flops(*c[1:]) for c in calls) / (ms_step * 1e-3) / 1e12,
                                  1),
        }
        if not args.no_cpu_baseline:
            log("[bench] CPU baseline (oracle) ...")
            out["cpu_baseline"] = cpu_baseline(calls, cols=64)
        out["calls"] = per_call
        print(json.dumps(out), flush=True)
        return
    out = {
        "metric": "ternary GEMM TB/s + TFLOP/s vs roofline at M=1..128, K=8192 (TQ2, TQ1)",
        "value": round(value, 4),
        "unit": "fraction of roofline (HBM 8 TB/s, FP16 MFMA 2.5 PFLOP/s)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": "TQ2 batch sweep M=1..128 and TQ1 M in {1,4,16,64} on "
                               "(K,N)=(8192,8192),(8192,28672); i.i.d. trits, fp16 block scales",
                   "tq1_batch": "workspace product from its switch point" if USE_WORKSPACE
                                else "no workspace (tq_gemm_tq1)",
                   "global_batch": None, "seq_len": None, "parallelism": "none"},
        "roofline": roofline_of(per_call),
    }
    hbm = [c for c in per_call if c["bound"] == "hbm"]
    mf = [c for c in per_call if c["bound"] == "mfma"]
    out["hbm_bound_calls"] = {"n": len(hbm), "mean_hbm_frac": round(float(np.mean([c["hbm_frac"] for c in hbm])), 4) if hbm else None}
    out["mfma_bound_calls"] = {"n": len(mf), "mean_mfma_frac": round(float(np.mean([c["mfma_frac"] for c in mf])), 4) if mf else None}
    if not args.no_context:
        log("[bench] context: read ceiling and FP16 matmul ...")
        out["context"] = context_bench(calls, per_call)
    if not args.no_configs:
        log("[bench] other workloads: 1024 x 1024 GEMV, 3B-class layer, TQ1 vs TQ2 ...")
        out["other_configs"] = other_configs_bench()
        out["tq1_vs_tq2_same_weights"] = tq1_vs_tq2_bench()
    if not args.no_cpu_baseline:
        log("[bench] CPU baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(calls)
    out["calls"] = per_call
    if args.calls_out:
        with open(args.calls_out, "w") as f:
            json.dump(per_call, f, indent=1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
