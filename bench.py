"""Benchmark of the CPR Gated DeltaNet library on one MI355X.

Main line: prefill throughput (tokens/s) on B=4, T=2048, 16 q/k heads, 32 v
heads, d=128, C=64, bf16 inputs, fp32 state and arithmetic, h0 ~ N(0, 0.02).
A "step" is one gdn_prefill call over that batch, inputs already in HBM.
Also reported: the same batch through the native-mixed baseline
(gdn_prefill_chunked), decode us/step for 64 sequences after a 4096-token
prefill (256 steps, resync steps included), trainer fwd+bwd on B=8, T=4096,
a packed varlen prefill (32 sequences, lengths uniform in [128, 8192]), and
the fp64 oracle's CPU throughput on a bounded sample of the prefill workload.

Timing: the main line's K steps carry HIP events around every launch (the
kernel durations behind its roofline come from those same steps); the other
legs take their wall clock with no per-launch events and their per-kernel
breakdown from a separate, profiled pass of the same work.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-decode]
                       [--no-train] [--no-varlen]
"""

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks
PEAK_HBM_GBS = 8000.0
PEAK_FP32_VECTOR_TFLOPS = 157.3

# HBM bytes per launch of the roofline kernels, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE readings scaled by what the same counters read for a 1 GiB device
# copy (x2.000 and x1.000).  Each entry holds only for the kernel source it was
# taken on (sha256 prefix of gdn_kernels.hip); for any other source the
# traffic field is reported as null.
MEASURED_TRAFFIC = {
    "f56816315c954ec0": {"k_rec": 612.7e6 + 134.2e6, "k_decode": 135.9e6 + 136.4e6},
}
KERNEL_SRC = os.path.join(ROOT, "linear_attention_rnn_gated_amd", "csrc", "gdn_kernels.hip")


def measured_traffic(kernel):
    import hashlib
    with open(KERNEL_SRC, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()[:16]
    return MEASURED_TRAFFIC.get(sha, {}).get(kernel)


PREFILL = dict(N=4, T=2048, H_qk=16, H_v=32, d=128, C=64)
DECODE = dict(N=64, P=4096, S=256, H_qk=16, H_v=32, d=128, C=64)
TRAIN = dict(N=8, T=4096, H_qk=16, H_v=32, d=128, C=64)
VARLEN = dict(N=32, lo=128, hi=8192, seed=4, H_qk=16, H_v=32, d=128, C=64)


def r_flops_per_token_head(d):
    # token step per state element: alpha*s (1), fma delta*k (2), o-dot (2), next k-dot (2)
    return 7 * d * d


# Algorithmic work of the chunk form per chunk-head (flops, an FMA counted as
# 2, lower-triangular products as half): the chunk factors (Gram matrix C^2 d,
# the two solves 2 C^2 d, the triangular inverse C^3 / 3) and the state scan
# (Delta = U - W S^T and S' = gam S + Delta^T K: 4 C d^2).
def wy_flops_per_chunk_head(d, C):
    return 3 * C * C * d + C ** 3 / 3


def scan_flops_per_chunk_head(d, C):
    return 4 * C * d * d


def prefill_flops(full_chunks, T, H_v, d, C):
    """The whole CPR prefill call: the chunk form over the full chunks, the
    token step over every token."""
    return (full_chunks * H_v * (wy_flops_per_chunk_head(d, C) + scan_flops_per_chunk_head(d, C))
            + T * H_v * r_flops_per_token_head(d))


def fwd_bwd_flops(T, H_v, d, C):
    """The whole trainer call per token-head: the CPR forward (chunk form
    amortised over C tokens plus the token step) and the backward, i.e. the
    chunk form recomputed and twice the chunk form with outputs
    (6 C^2 d + 6 C d^2 + C^3 / 3 per chunk-head)."""
    b = (wy_flops_per_chunk_head(d, C) + scan_flops_per_chunk_head(d, C)) / C
    chunk_out = (6 * C * C * d + 6 * C * d * d + C ** 3 / 3) / C
    return T * H_v * (b + r_flops_per_token_head(d) + b + 2 * chunk_out)


def call_roofline(flop, ms):
    achieved = flop / (ms * 1e-3) / 1e12
    return dict(bound="alu+mfma", flop_per_call=float(f"{flop:.5e}"),
                achieved=round(achieved, 2), peak=PEAK_FP32_VECTOR_TFLOPS, unit="TFLOP/s",
                frac=round(achieved / PEAK_FP32_VECTOR_TFLOPS, 4))


def decode_bytes_per_seq_head(d, C, G, resync=True):
    """Algorithmic HBM bytes of one decode step per (sequence, value head), as
    the method needs them (not as this library moves them): the fp32 state
    read and written; the token's q and k (bf16, shared by the G value heads
    of a group), v (bf16), beta and g (fp32) in, o (fp32) out; the token
    appended to the chunk buffer (raw k shared per group, v, beta, g); and,
    amortised over the C steps of a chunk, the resync's state read and
    written plus its reading of the buffered chunk."""
    state = 2 * d * d * 4
    token_io = (2 * d * 2) / G + d * 2 + 8 + d * 4
    append = (d * 2) / G + d * 2 + 8
    total = state + token_io + append
    if resync:
        total += (2 * d * d * 4 + C * append) / C
    return total


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--decode-reps", type=int, default=3)
    ap.add_argument("--no-train", action="store_true")
    ap.add_argument("--no-varlen", action="store_true")
    ap.add_argument("--train-steps", type=int, default=5)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 5 plain device copies of 1 GiB (the reference kernel for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings)")
    return ap.parse_args()


def wall_then_profile(step, n_wall, n_prof, names, B, torch):
    """Wall-clock milliseconds per step over n_wall steps with no per-launch
    events, then each named kernel's (total ms, launches) over a separate pass
    of n_prof steps with events around every launch."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n_wall):
        step()
    torch.cuda.synchronize()
    ms_step = 1e3 * (time.perf_counter() - t0) / n_wall if n_wall else 0.0
    B.profile_read("")  # drop anything recorded so far
    B.profile_enable(True)
    for _ in range(n_prof):
        step()
    torch.cuda.synchronize()
    B.profile_enable(False)
    return ms_step, {name: B.profile_read(name) for name in names}


def bench_prefill(args, B, torch, make_inputs):
    c = PREFILL
    dev = "cuda"
    inp = make_inputs([c["T"]] * c["N"], c["H_qk"], c["H_v"], c["d"], "bf16", seed=1,
                      h0="normal", device=dev)
    shape = B.make_shape(c["H_qk"], c["H_v"], c["d"], c["C"], torch.bfloat16)
    T = inp["T"]
    ws = torch.empty(B.workspace_bytes(shape, c["N"], T, B.OP_PREFILL), dtype=torch.uint8,
                     device=dev)
    o = torch.empty(T, c["H_v"], c["d"], dtype=torch.float32, device=dev)
    cu = inp["cu_seqlens"].to(dev)
    cu_h = inp["cu_seqlens"].to("cpu", torch.int32)  # host copy: no device sync per call

    def step():
        B.gdn_prefill(shape, inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], cu,
                      h0=inp["h0"], ws=ws, out=o, cu_seqlens_host=cu_h)

    for _ in range(args.warmup):
        step()
    # the timed steps carry events around the roofline kernel's launches only
    # (events around all four launches of a step add about 3% to it), so its
    # duration is that of the timed steps; the other kernels' split comes from
    # a separate pass with events around every launch
    torch.cuda.synchronize()
    B.profile_read("")  # drop anything recorded so far
    B.profile_filter("k_rec")
    B.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    B.profile_enable(False)
    B.profile_filter("")
    rec_ms, rec_n = B.profile_read("k_rec")
    _, prof = wall_then_profile(step, 0, min(args.steps, 10),
                                ["k_plan", "k_prep", "k_wy", "k_scan"], B, torch)
    per_kernel = {name: dict(avg_us=1e3 * ms / max(n, 1), launches=n) for name, (ms, n) in prof.items()}
    per_kernel["k_rec"] = dict(avg_us=1e3 * rec_ms / max(rec_n, 1), launches=rec_n)
    ms_step = 1e3 * (t1 - t0) / args.steps
    tokens = T
    rec_us = per_kernel["k_rec"]["avg_us"]
    rec_flops = r_flops_per_token_head(c["d"]) * T * c["H_v"]
    achieved = rec_flops / (rec_us * 1e-6) / 1e12
    full = c["N"] * (c["T"] // c["C"])
    kernel_tflops = {
        "k_wy": full * c["H_v"] * wy_flops_per_chunk_head(c["d"], c["C"]),
        "k_scan": full * c["H_v"] * scan_flops_per_chunk_head(c["d"], c["C"]),
        "k_rec": rec_flops}
    kernel_tflops = {k: round(f / (per_kernel[k]["avg_us"] * 1e-6) / 1e12, 2)
                     for k, f in kernel_tflops.items()}
    return dict(ms_per_step=ms_step, value=tokens / (ms_step * 1e-3), tokens=tokens,
                per_kernel=per_kernel, kernel_tflops=kernel_tflops,
                call_roofline=call_roofline(prefill_flops(full, T, c["H_v"], c["d"], c["C"]),
                                            ms_step),
                roofline=dict(kernel="k_rec", bound="alu", achieved=round(achieved, 3),
                              peak=PEAK_FP32_VECTOR_TFLOPS, unit="TFLOP/s",
                              frac=round(achieved / PEAK_FP32_VECTOR_TFLOPS, 4),
                              traffic=measured_traffic("k_rec"), traffic_unit="B per launch",
                              algorithmic_per_launch=f"{rec_flops:.4e} flop"),
                inputs=inp, shape=shape)


def bench_native_mixed(args, B, torch, pf):
    """The same prefill workload through gdn_prefill_chunked: chunk-form outputs
    (what a chunked prefill paired with a recurrent decode computes), i.e. the
    native-mixed baseline without the bitwise prefill/decode guarantee."""
    c = PREFILL
    dev = "cuda"
    inp, shape = pf["inputs"], pf["shape"]
    T = inp["T"]
    ws = torch.empty(B.workspace_bytes(shape, c["N"], T, B.OP_PREFILL_CHUNKED),
                     dtype=torch.uint8, device=dev)
    o = torch.empty(T, c["H_v"], c["d"], dtype=torch.float32, device=dev)
    cu = inp["cu_seqlens"].to(dev)
    cu_h = inp["cu_seqlens"].to("cpu", torch.int32)  # host copy: no device sync per call

    def step():
        B.gdn_prefill_chunked(shape, inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], cu,
                              h0=inp["h0"], ws=ws, out=o, cu_seqlens_host=cu_h)

    for _ in range(args.warmup):
        step()
    ms_step, prof = wall_then_profile(step, args.steps, min(args.steps, 10),
                                      ["k_plan", "k_prep", "k_wy", "k_scan", "k_chunk_o"], B, torch)
    per_kernel = {name: round(1e3 * ms / max(n, 1), 2) for name, (ms, n) in prof.items()}
    return dict(ms_per_step=round(ms_step, 4), tokens_per_s=round(T / (ms_step * 1e-3), 1),
                cpr_over_native=round(pf["ms_per_step"] / ms_step, 3),
                per_kernel_us=per_kernel)


def bench_varlen(args, B, torch, make_inputs):
    """One packed gdn_prefill over 32 sequences of lengths uniform in
    [128, 8192] (about 148k tokens at seed 4)."""
    c = VARLEN
    dev = "cuda"
    inp = make_inputs(("uniform", c["N"], c["lo"], c["hi"]), c["H_qk"], c["H_v"], c["d"], "bf16",
                      seed=c["seed"], h0="zero", device=dev)
    shape = B.make_shape(c["H_qk"], c["H_v"], c["d"], c["C"], torch.bfloat16)
    T = inp["T"]
    ws = torch.empty(B.workspace_bytes(shape, c["N"], T, B.OP_PREFILL), dtype=torch.uint8,
                     device=dev)
    o = torch.empty(T, c["H_v"], c["d"], dtype=torch.float32, device=dev)
    cu = inp["cu_seqlens"].to(dev)
    cu_h = inp["cu_seqlens"].to("cpu", torch.int32)  # host copy: no device sync per call

    def step():
        B.gdn_prefill(shape, inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], cu,
                      h0=None, ws=ws, out=o, cu_seqlens_host=cu_h)

    step()
    ms_step, prof = wall_then_profile(step, 5, 2, ["k_plan", "k_prep", "k_wy", "k_scan", "k_rec"],
                                      B, torch)
    per = {name: round(1e3 * ms / max(n, 1), 1) for name, (ms, n) in prof.items()}
    rec_flops = r_flops_per_token_head(c["d"]) * T * c["H_v"]
    full = sum(L // c["C"] for L in inp["lens"])
    return dict(ms_per_step=round(ms_step, 3), tokens=T,
                tokens_per_s=round(T / (ms_step * 1e-3), 1),
                k_rec_tflops=round(rec_flops / (per["k_rec"] * 1e-6) / 1e12, 2),
                call_roofline=call_roofline(prefill_flops(full, T, c["H_v"], c["d"], c["C"]),
                                            ms_step),
                per_kernel_us=per,
                workload="varlen prefill, 32 seqs, lengths U[128, 8192] (seed 4), 16 q/k / 32 v "
                         "heads, d128 C64 bf16, h0 = 0")


def bench_decode(args, B, torch, make_inputs):
    c = DECODE
    dev = "cuda"
    N, P, S = c["N"], c["P"], c["S"]
    shape = B.make_shape(c["H_qk"], c["H_v"], c["d"], c["C"], torch.bfloat16)
    pre = make_inputs([P] * N, c["H_qk"], c["H_v"], c["d"], "bf16", seed=2, h0="zero",
                      device=dev)
    cache = B.Cache(shape, N, dev, torch.bfloat16)
    B.gdn_prefill(shape, pre["q"], pre["k"], pre["v"], pre["beta"], pre["g"],
                  pre["cu_seqlens"].to(dev), cache=cache, want_hT=False)
    del pre
    tok = make_inputs([N] * S, c["H_qk"], c["H_v"], c["d"], "bf16", seed=3, device=dev)
    q = tok["q"].view(S, N, c["H_qk"], c["d"])
    k = tok["k"].view(S, N, c["H_qk"], c["d"])
    v = tok["v"].view(S, N, c["H_v"], c["d"])
    be = tok["beta"].view(S, N, c["H_v"])
    g = tok["g"].view(S, N, c["H_v"])
    o = torch.empty(N, c["H_v"], c["d"], dtype=torch.float32, device=dev)
    ws = torch.empty(B.workspace_bytes(shape, N, 0, B.OP_DECODE), dtype=torch.uint8,
                     device=dev)
    snap = cache.clone()
    torch.cuda.synchronize()
    L = B.lib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cs = cache.struct()
    pos0 = cache.pos.cpu()
    pos_bufs = [((pos0 + s) % c["C"]).to(torch.int32).contiguous() for s in range(S)]
    args_s = [(ctypes.c_void_p(q[s].data_ptr()), ctypes.c_void_p(k[s].data_ptr()),
               ctypes.c_void_p(v[s].data_ptr()), ctypes.c_void_p(be[s].data_ptr()),
               ctypes.c_void_p(g[s].data_ptr()), ctypes.c_void_p(pos_bufs[s].data_ptr()))
              for s in range(S)]
    shp, csp = ctypes.byref(shape), ctypes.byref(cs)
    op, wsp, wsn = ctypes.c_void_p(o.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ws.numel()

    def run_steps():
        for s in range(S):
            a = args_s[s]
            rc = L.gdn_decode_step(shp, N, a[0], a[1], a[2], a[3], a[4], csp, a[5], op, wsp,
                                   wsn, st)
            if rc != 0:
                raise RuntimeError(f"gdn_decode_step: {rc}")

    def restore():
        for dst, src in zip(cache.tensors(), snap.tensors()):
            dst.copy_(src)
        torch.cuda.synchronize()

    run_steps()  # warm-up pass
    # wall clock without the timing events, then one pass with them for the
    # per-kernel split
    times = []
    for rep in range(args.decode_reps):
        restore()
        t0 = time.perf_counter()
        run_steps()
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
    per = {"k_decode": [0.0, 0], "k_wy_resync": [0.0, 0], "k_scan_resync": [0.0, 0]}
    restore()
    B.profile_read("")
    B.profile_enable(True)
    run_steps()
    torch.cuda.synchronize()
    B.profile_enable(False)
    for name in per:
        ms, n = B.profile_read(name)
        per[name][0] += ms
        per[name][1] += n
    # the same 256 calls captured once in a HIP graph and replayed (the serving
    # form: the host mirror of pos records the resync launches where they fall)
    graph = torch.cuda.CUDAGraph()
    restore()
    with torch.cuda.graph(graph):
        stc = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for s in range(S):
            a = args_s[s]
            rc = L.gdn_decode_step(shp, N, a[0], a[1], a[2], a[3], a[4], csp, a[5], op, wsp,
                                   wsn, stc)
            if rc != 0:
                raise RuntimeError(f"gdn_decode_step (capture): {rc}")
    gtimes = []
    for rep in range(args.decode_reps):
        restore()
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        gtimes.append(time.perf_counter() - t0)
    us_step = 1e6 * min(times) / S
    us_graph = 1e6 * min(gtimes) / S
    # native-mixed baseline: the plain recurrent step on the same post-prefill
    # state and the same 256 tokens, no chunk buffers and no resync
    Sn = snap.S_run.clone()
    nat_times = []
    for rep in range(args.decode_reps):
        Sn.copy_(snap.S_run)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(S):
            a = args_s[s]
            rc = L.gdn_decode_step_native(shp, N, a[0], a[1], a[2], a[3], a[4],
                                          ctypes.c_void_p(Sn.data_ptr()), op, st)
            if rc != 0:
                raise RuntimeError(f"gdn_decode_step_native: {rc}")
        torch.cuda.synchronize()
        nat_times.append(time.perf_counter() - t0)
    us_native = 1e6 * min(nat_times) / S
    # k_decode's own duration: the first C - 1 steps (no resync falls there,
    # every sequence starts at a chunk edge) between two events on the launch
    # stream; events around every launch would add their own cost to a 40 us
    # kernel
    assert int(pos0.max()) == 0
    nwin = c["C"] - 1
    dwin = []
    for rep in range(args.decode_reps):
        restore()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for s in range(nwin):
            a = args_s[s]
            L.gdn_decode_step(shp, N, a[0], a[1], a[2], a[3], a[4], csp, a[5], op, wsp, wsn, st)
        e1.record()
        torch.cuda.synchronize()
        dwin.append(e0.elapsed_time(e1) * 1e3 / nwin)
    dec_us = min(dwin)
    G = c["H_v"] // c["H_qk"]
    step_bytes_alg = decode_bytes_per_seq_head(c["d"], c["C"], G) * N * c["H_v"]
    dec_kernel_bytes = decode_bytes_per_seq_head(c["d"], c["C"], G, resync=False) * N * c["H_v"]
    achieved = dec_kernel_bytes / (dec_us * 1e-6) / 1e9
    big = decode_window_large(args, B, torch, make_inputs, shape, c)
    return dict(us_per_step=round(us_step, 2),
                step_hbm_frac=round(step_bytes_alg / (us_step * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                us_per_step_graph=round(us_graph, 2),
                step_hbm_frac_graph=round(step_bytes_alg / (us_graph * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                per_kernel={k: dict(avg_us=1e3 * v[0] / max(v[1], 1), launches=v[1])
                            for k, v in per.items()},
                k_decode_window_us=round(dec_us, 2),
                native_mixed=dict(us_per_step=round(us_native, 2),
                                  cpr_over_native=round(us_step / us_native, 3)),
                step_bytes_algorithmic=step_bytes_alg,
                k_decode_256seq=big,
                roofline=dict(kernel="k_decode", bound="hbm", achieved=round(achieved, 1),
                              peak=PEAK_HBM_GBS, unit="GB/s",
                              frac=round(achieved / PEAK_HBM_GBS, 4),
                              traffic=measured_traffic("k_decode"), traffic_unit="B per launch"),
                workload="decode 64 seqs x (4096 prefill + 256 steps), 16 q/k / 32 v heads, "
                         "d128 C64 bf16")


def decode_window_large(args, B, torch, make_inputs, shape, c):
    """k_decode over C - 1 resync-free steps of 256 sequences: 1 GiB of
    running state, four times the 256 MB Infinity Cache, so the state streams
    from DRAM on every step (the 64-sequence state, 256 MiB, could partly stay
    in that cache).  Same per-(sequence, head) bytes as the main decode leg."""
    N, dev = 256, "cuda"
    gen = torch.Generator(device=dev).manual_seed(5)
    h0 = 0.02 * torch.randn(N, c["H_v"], c["d"], c["d"], generator=gen, device=dev)
    cache = B.gdn_cache_init(shape, N, dev, torch.bfloat16, h0=h0)
    del h0
    nwin = c["C"] - 1
    tok = make_inputs([N] * nwin, c["H_qk"], c["H_v"], c["d"], "bf16", seed=6, device=dev)
    q = tok["q"].view(nwin, N, c["H_qk"], c["d"])
    k = tok["k"].view(nwin, N, c["H_qk"], c["d"])
    v = tok["v"].view(nwin, N, c["H_v"], c["d"])
    be = tok["beta"].view(nwin, N, c["H_v"])
    g = tok["g"].view(nwin, N, c["H_v"])
    o = torch.empty(N, c["H_v"], c["d"], dtype=torch.float32, device=dev)
    ws = torch.empty(B.workspace_bytes(shape, N, 0, B.OP_DECODE), dtype=torch.uint8, device=dev)
    snap = cache.clone()
    pos = [torch.full((N, c["H_v"]), s, dtype=torch.int32) for s in range(nwin)]
    best = None
    for rep in range(args.decode_reps):
        for dst, src in zip(cache.tensors(), snap.tensors()):
            dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for s in range(nwin):
            B.gdn_decode_step(shape, q[s], k[s], v[s], be[s], g[s], cache, pos_host=pos[s],
                              ws=ws, out=o)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / nwin
        best = us if best is None else min(best, us)
    G = c["H_v"] // c["H_qk"]
    kb = decode_bytes_per_seq_head(c["d"], c["C"], G, resync=False) * N * c["H_v"]
    gbs = kb / (best * 1e-6) / 1e9
    return dict(window_us=round(best, 2), achieved_gbs=round(gbs, 1),
                frac=round(gbs / PEAK_HBM_GBS, 4),
                workload="256 seqs, 63 resync-free steps, 16 q/k / 32 v heads, d128 C64 bf16")


def bench_fwd_bwd(args, B, torch, make_inputs):
    c = TRAIN
    dev = "cuda"
    inp = make_inputs([c["T"]] * c["N"], c["H_qk"], c["H_v"], c["d"], "bf16", seed=3,
                      h0="normal", with_do=True, device=dev)
    shape = B.make_shape(c["H_qk"], c["H_v"], c["d"], c["C"], torch.bfloat16)
    T = inp["T"]
    ws = torch.empty(B.workspace_bytes(shape, c["N"], T, B.OP_FWD_BWD), dtype=torch.uint8,
                     device=dev)
    cu = inp["cu_seqlens"].to(dev)
    cu_h = inp["cu_seqlens"].to("cpu", torch.int32)  # host copy: no device sync per call

    def step():
        B.gdn_fwd_bwd(shape, inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], cu, inp["do"],
                      h0=inp["h0"], ws=ws, cu_seqlens_host=cu_h)

    step()
    ms_step, prof = wall_then_profile(
        step, args.train_steps, 1,
        ["k_prep", "k_wy", "k_scan", "k_rec", "k_bwd_prep", "k_bwd_scan", "k_bwd_chunk", "k_bwd_qk"],
        B, torch)
    per = {name: round(1e3 * ms / max(n, 1), 1) for name, (ms, n) in prof.items()}

    def native_step():  # native-mixed baseline: chunk-form forward outputs
        B.gdn_fwd_bwd_chunked(shape, inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], cu,
                              inp["do"], h0=inp["h0"], ws=ws, cu_seqlens_host=cu_h)

    native_step()
    ms_native, nprof = wall_then_profile(native_step, args.train_steps, 1, ["k_chunk_o"], B, torch)
    return dict(ms_per_step=round(ms_step, 3), tokens_per_s=round(T / (ms_step * 1e-3), 1),
                call_roofline=call_roofline(fwd_bwd_flops(T, c["H_v"], c["d"], c["C"]), ms_step),
                native_mixed=dict(ms_per_step=round(ms_native, 3),
                                  cpr_over_native=round(ms_step / ms_native, 3),
                                  k_chunk_o_us=round(1e3 * nprof["k_chunk_o"][0] /
                                                     max(nprof["k_chunk_o"][1], 1), 1)),
                per_kernel_us=per,
                workload="fwd+bwd B8 T4096, 16 q/k / 32 v heads, d128 C64 bf16, dO ~ N(0,1)")


# CPU baseline workers: the oracle's inputs are memory-mapped .npy files (no
# copy per worker), and each worker runs the oracle with BLAS on one thread.
_CPU = {}
HEADS_PER_CPU_TASK = 1


def _cpu_init(paths):
    import numpy as np
    try:
        from threadpoolctl import threadpool_limits
        _CPU["limits"] = threadpool_limits(1)
    except ImportError:  # pragma: no cover
        pass
    _CPU["arr"] = {key: np.load(path, mmap_mode="r") for key, path in paths.items()}


def _cpu_ready(_):
    return os.getpid()


def _cpu_task(task):
    """The oracle forward of q/k heads h0q .. h1q - 1 (and their value heads)
    of one sequence (tokens t0 .. t1 - 1); returns the token-heads done."""
    import numpy as np
    from oracle import recurrent_fwd
    n, h0q, h1q, t0, t1, G = task
    a = _CPU["arr"]
    hv = slice(h0q * G, h1q * G)
    h0 = a["h0"][n:n + 1, hv] if "h0" in a else None
    recurrent_fwd(a["q"][t0:t1, h0q:h1q], a["k"][t0:t1, h0q:h1q], a["v"][t0:t1, hv],
                  a["beta"][t0:t1, hv], a["g"][t0:t1, hv], np.array([0, t1 - t0]), h0=h0)
    return (t1 - t0) * (h1q - h0q)


def cpu_baseline(inp, passes=3):
    """The fp64 oracle on the whole prefill batch over a pool of worker
    processes, one per host core this process may run on (at most 16), each
    with BLAS on one thread: the heads are independent, so every sequence is
    split into blocks of q/k heads (and their value heads), about one task per
    worker in all; the median of `passes` passes."""
    import multiprocessing as mp
    import shutil
    from concurrent.futures import ProcessPoolExecutor
    import tempfile
    import numpy as np
    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    cu = [int(x) for x in inp["cu_seqlens"].cpu()]
    H_qk, H_v = int(inp["H_qk"]), int(inp["H_v"])
    G = H_v // H_qk
    tmp = tempfile.mkdtemp(prefix="gdn_cpu_baseline_")
    try:
        paths = {}
        for key in ["q", "k", "v", "beta", "g", "h0"]:
            if inp.get(key) is None:
                continue
            # bf16 values are exact in fp32; the oracle widens to fp64 itself
            arr = inp[key].detach().to("cpu", dtype=inp[key].dtype).float().numpy()
            paths[key] = os.path.join(tmp, key + ".npy")
            np.save(paths[key], arr)
        N = len(cu) - 1
        hb = HEADS_PER_CPU_TASK if H_qk % HEADS_PER_CPU_TASK == 0 else 1
        nb = H_qk // hb
        tasks = [(n, b * hb, (b + 1) * hb, cu[n], cu[n + 1], G) for n in range(N)
                 for b in range(nb)]
        # fresh interpreters (spawn): the workers never touch the GPU; a worker
        # that fails breaks the pool and raises instead of being restarted
        ctx = mp.get_context("spawn")
        times = []
        with ProcessPoolExecutor(cores, mp_context=ctx, initializer=_cpu_init,
                                 initargs=(paths,)) as pool:
            list(pool.map(_cpu_ready, range(4 * cores)))  # workers up and importing
            list(pool.map(_cpu_task, tasks[:cores]))      # warm the page cache
            for _ in range(passes):
                t0 = time.perf_counter()
                ntok = sum(pool.map(_cpu_task, tasks)) // H_qk  # token-heads / heads
                times.append(time.perf_counter() - t0)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    dt = sorted(times)[len(times) // 2]
    return dict(value=round(ntok / dt, 2), unit="tokens/s", cores=cores, kind="oracle",
                sample=f"the whole prefill batch ({ntok} tokens, all {H_v} v heads) as "
                       f"{len(tasks)} (sequence, block of {hb} q/k heads) tasks on {cores} "
                       f"worker processes "
                       f"(BLAS 1 thread each), fp64 numpy token recurrence, median of "
                       f"{passes} passes ({dt:.2f} s each, about {sum(times) * cores:.0f} "
                       f"core-seconds in all)")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only (asked for --gpus {args.gpus}); "
              "the layer shards by sequence/head without communication, see the design notes",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": a.numel() * 4, "copies": 5}), flush=True)
        return
    from linear_attention_rnn_gated_amd import binding as B
    from linear_attention_rnn_gated_amd.inputs import make_inputs
    assert torch.cuda.is_available(), "bench needs a GPU"
    B.lib()
    pf = bench_prefill(args, B, torch, make_inputs)
    line = {
        "metric": "GDN prefill tokens/s (CPR; B4 T2048, 16 q/k / 32 v heads, d128, C64)",
        "value": round(pf["value"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pf["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "prefill B4 T2048 H_qk16 H_v32 d128 C64 bf16-in fp32-state",
                   "global_batch": PREFILL["N"], "seq_len": PREFILL["T"],
                   "parallelism": "single-gpu"},
        "roofline": pf["roofline"],
        "call_roofline": pf["call_roofline"],
        "per_kernel_us": {k: round(v["avg_us"], 2) for k, v in pf["per_kernel"].items()},
        "kernel_tflops": pf["kernel_tflops"],
        "contract": B.contract_id(),
    }
    line["native_mixed_prefill"] = bench_native_mixed(args, B, torch, pf)
    if not args.no_decode:
        dc = bench_decode(args, B, torch, make_inputs)
        line["decode"] = dc
    if not args.no_train:
        line["fwd_bwd"] = bench_fwd_bwd(args, B, torch, make_inputs)
    if not args.no_varlen:
        line["varlen"] = bench_varlen(args, B, torch, make_inputs)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(pf["inputs"])
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
