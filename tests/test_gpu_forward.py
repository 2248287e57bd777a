"""GPU parity and bit-consistency of the forward paths (prefill, decode).

Parity bar: max-abs difference to the fp64 oracle <= 2e-3 for bf16 inputs and
<= 1e-5 for fp32 inputs, on o and on the final state.  Bit-consistency is
exact: compared as int32 bit patterns.
"""

import numpy as np
import pytest
import torch

from gdn_helpers import (bit_equal, decode_tokens, group_slice, make_inputs, maxabs,
                         oracle_fwd, rows_of, run_prefill, shape_for, sub_inputs, to_dev)
from linear_attention_rnn_gated_amd import binding as B

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "f32": 1e-5}


def say(*a):
    print(*a, flush=True)


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def check_parity(inp, o, hT, tol, seqs=None, scale=1.0, qk_l2norm=True):
    ro, rh = oracle_fwd(inp, seqs=seqs, scale=scale, qk_l2norm=qk_l2norm)
    if seqs is None:
        e_o, e_h = maxabs(o, ro), maxabs(hT, rh)
    else:
        rows = rows_of(inp, seqs)
        e_o = maxabs(o.cpu()[rows], ro[rows])
        e_h = maxabs(hT.cpu()[seqs], rh[seqs])
    say(f"  parity: max|o-oracle|={e_o:.3e} max|hT-oracle|={e_h:.3e} (tol {tol})")
    assert np.isfinite(e_o) and np.isfinite(e_h)
    assert e_o <= tol and e_h <= tol


# ------------------------------------------------------------------ tiny fp32

def test_tiny_fp32_prefill_parity_and_64_decode_steps_bit_identical():
    """B=1, H=2, T=64, d=16, C=16, fp32, zero initial state."""
    say("case: tiny fp32 d16 C16 T64")
    inp = make_inputs([64], 2, 2, 16, "f32", seed=0, h0="zero")
    o, hT, _ = run_prefill(inp)
    check_parity(inp, o, hT, TOL["f32"])
    shape = shape_for(inp)
    cache = B.gdn_cache_init(shape, 1, "cuda", torch.float32)
    od = decode_tokens(inp, cache, shape, 0, 64)
    assert bit_equal(od[:, 0], o), "decode o != prefill o"
    assert bit_equal(cache.S_run, hT), "decode state != prefill state"
    assert bit_equal(cache.S_chunk, hT)


# ------------------------------------------------------------------ d=128 parity

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_ragged_parity(dtype):
    lens = [200, 64, 1, 130, 0, 129]
    say(f"case: ragged prefill {dtype} lens={lens}")
    inp = make_inputs(lens, 2, 4, 128, dtype, seed=11, h0="normal")
    o, hT, _ = run_prefill(inp)
    check_parity(inp, o, hT, TOL[dtype])


def test_prefill_scale_without_norm():
    say("case: scale 0.5, qk_l2norm off")
    inp = make_inputs([150, 70], 1, 2, 128, "bf16", seed=12, h0="normal")
    o, hT, _ = run_prefill(inp, scale=0.5, qk_l2norm=False)
    check_parity(inp, o, hT, TOL["bf16"], scale=0.5, qk_l2norm=False)


def test_degenerate_inputs():
    say("case: beta = 0 with zero state gives o == 0")
    inp = make_inputs([100, 64], 1, 2, 128, "bf16", seed=13, h0="zero")
    inp["beta"] = torch.zeros_like(inp["beta"])
    o, hT, _ = run_prefill(inp)
    assert torch.count_nonzero(o) == 0 and torch.count_nonzero(hT) == 0
    say("case: near-reset gates (g = -30 on every 7th token)")
    inp = make_inputs([150, 64], 1, 2, 128, "bf16", seed=14, h0="normal")
    inp["g"][::7] = -30.0
    o, hT, _ = run_prefill(inp)
    check_parity(inp, o, hT, TOL["bf16"])
    say("case: all sequences empty")
    inp = make_inputs([0, 0], 1, 2, 128, "bf16", seed=15, h0="normal")
    o, hT, _ = run_prefill(inp)
    assert bit_equal(hT, inp["h0"].cuda())
    say("case: growing state (g = +0.4 on every token, decay factor 1.49)")
    inp = make_inputs([100, 64], 1, 2, 128, "bf16", seed=16, h0="normal")
    inp["g"][:] = 0.4
    o, hT, _ = run_prefill(inp)
    ro, rh = oracle_fwd(inp)
    # The state grows 1.49x per token (~1e16 after 100 tokens), and a rounding
    # error made at token t grows with it, so the bar is relative: 1e-4 of the
    # largest value (~100 tokens x fp32 rounding of O(d)-term dot products).
    for name, got, want in [("o", o, ro), ("hT", hT, rh)]:
        err, top = maxabs(got, want), float(np.max(np.abs(want)))
        say(f"  {name}: max err {err:.3e}, max |oracle| {top:.3e}, relative {err / top:.2e}")
        assert np.isfinite(err) and err <= 1e-4 * top, name


@pytest.mark.parametrize("gval", [0.4, -30.0])
def test_extreme_gates_decode_equals_prefill(gval):
    """Decode across tokens with a growing (g > 0) or near-reset (g = -30)
    decay gives the prefill's o and state bit for bit."""
    say(f"case: g = {gval} on every 3rd token, prefill 40 + decode 60")
    total, pre = 100, 40
    inp = make_inputs([total] * 2, 1, 2, 128, "bf16", seed=17, h0="normal")
    inp["g"][::3] = gval
    o_full, h_full, _ = run_prefill(inp, cache=True)
    shape = shape_for(inp)
    first = dict(inp)
    idx = torch.cat([torch.arange(n * total, n * total + pre) for n in range(2)])
    for key in ["q", "k", "v", "beta", "g"]:
        first[key] = inp[key][idx].contiguous()
    first["cu_seqlens"] = torch.tensor([0, pre, 2 * pre], dtype=torch.int32)
    _, _, cache = run_prefill(first, cache=True)
    od = decode_tokens(inp, cache, shape, pre, total - pre)
    for n in range(2):
        assert bit_equal(od[:, n], o_full[n * total + pre:(n + 1) * total]), f"o seq {n}"
    assert bit_equal(cache.S_run, h_full)


# ------------------------------------------------------------------ bit consistency

@pytest.mark.parametrize("pre,use_pos_host", [(70, True), (64, False), (0, True)])
def test_decode_continues_prefill_bit_exactly(pre, use_pos_host):
    """Prefill `pre` tokens, decode the rest one by one; o and final states equal
    one prefill of the whole sequence, bit for bit."""
    total = 148
    say(f"case: prefill {pre} + decode {total - pre}, pos_host={use_pos_host}")
    inp = make_inputs([total] * 3, 2, 4, 128, "bf16", seed=21, h0="normal")
    o_full, h_full, c_full = run_prefill(inp, cache=True)
    shape = shape_for(inp)
    if pre > 0:
        first = dict(inp)
        idx = torch.cat([torch.arange(n * total, n * total + pre) for n in range(3)])
        for key in ["q", "k", "v", "beta", "g"]:
            first[key] = inp[key][idx].contiguous()
        first["cu_seqlens"] = torch.tensor([0, pre, 2 * pre, 3 * pre], dtype=torch.int32)
        _, _, cache = run_prefill(first, cache=True)
    else:
        cache = B.gdn_cache_init(shape, 3, "cuda", torch.bfloat16, h0=inp["h0"].cuda())
    od = decode_tokens(inp, cache, shape, pre, total - pre, use_pos_host=use_pos_host)
    for n in range(3):
        assert bit_equal(od[:, n], o_full[n * total + pre:(n + 1) * total]), f"o seq {n}"
    assert bit_equal(cache.S_run, h_full)
    # the full prefill's cache equals the decoded cache's current chunk state
    assert bit_equal(cache.S_chunk, c_full.S_chunk)
    assert torch.equal(cache.pos.cpu(), c_full.pos.cpu())


@pytest.mark.parametrize("Hq,Hv", [(1, 1), (1, 3), (2, 8), (1, 8)])
def test_head_group_ratios_prefill_parity_and_decode(Hq, Hv):
    """Value heads per q/k head of 1, 3, 4 and 8 (the largest group the library
    accepts): prefill parity with the oracle,
    and a prefix prefill plus decode across a chunk edge equals one prefill."""
    total, pre = 100, 30
    say(f"case: head groups H_qk={Hq} H_v={Hv}, 2 x {total} tokens, decode from {pre}")
    inp = make_inputs([total] * 2, Hq, Hv, 128, "bf16", seed=41, h0="normal")
    o_full, h_full, _ = run_prefill(inp, cache=True)
    check_parity(inp, o_full, h_full, TOL["bf16"])
    first = dict(inp)
    idx = torch.cat([torch.arange(n * total, n * total + pre) for n in range(2)])
    for key in ["q", "k", "v", "beta", "g"]:
        first[key] = inp[key][idx].contiguous()
    first["cu_seqlens"] = torch.tensor([0, pre, 2 * pre], dtype=torch.int32)
    _, _, cache = run_prefill(first, cache=True)
    od = decode_tokens(inp, cache, shape_for(inp), pre, total - pre)
    for n in range(2):
        assert bit_equal(od[:, n], o_full[n * total + pre:(n + 1) * total]), f"o seq {n}"
    assert bit_equal(cache.S_run, h_full)


def test_long_sequence_parity():
    """One 32768-token sequence (512 chunks in one serial scan, token offsets
    past 2^15 per head): o and the final state against the oracle."""
    lens = [32768]
    say(f"case: long sequence {lens[0]} tokens, H_qk=1 H_v=2, d128 bf16")
    inp = make_inputs(lens, 1, 2, 128, "bf16", seed=43, h0="normal")
    o, hT, _ = run_prefill(inp)
    check_parity(inp, o, hT, TOL["bf16"])


def test_mixed_position_decode_equals_prefill():
    """Sequences sitting at different offsets inside their chunks decode together
    (one call per step, each sequence resyncing on its own step); every output
    and final state equals a prefill of the whole sequence, bit for bit."""
    pre = [70, 64, 1, 130, 0, 129]
    steps = 80
    say(f"case: mixed-position decode, prefixes {pre} + {steps} steps")
    inp = make_inputs([p + steps for p in pre], 2, 4, 128, "bf16", seed=31, h0="normal")
    o_full, h_full, _ = run_prefill(inp)
    cu = inp["cu_seqlens"].tolist()
    n_seq = len(pre)
    first = dict(inp)
    idx = torch.cat([torch.arange(cu[n], cu[n] + pre[n]) for n in range(n_seq)])
    for key in ["q", "k", "v", "beta", "g"]:
        first[key] = inp[key][idx].contiguous()
    first["cu_seqlens"] = torch.tensor([0] + list(np.cumsum(pre)), dtype=torch.int32)
    _, _, cache = run_prefill(first, cache=True)
    shape = shape_for(inp)
    pos = cache.pos.cpu()
    assert sorted(set(pos[:, 0].tolist())) == sorted({p % 64 for p in pre})
    for s in range(steps):
        rows = torch.tensor([cu[n] + pre[n] + s for n in range(n_seq)])
        o = B.gdn_decode_step(shape, *[inp[k_][rows].cuda().contiguous()
                                       for k_ in ["q", "k", "v", "beta", "g"]],
                              cache, pos_host=pos)
        pos = (pos + 1) % shape.C
        assert bit_equal(o, o_full[rows.cuda()]), f"step {s}"
    assert bit_equal(cache.S_run, h_full)


def test_decode_step_in_hip_graph_replays_bit_exactly():
    """One decode step (device-side resync decision, no host pos mirror)
    captured in a HIP graph and replayed token after token, with eager work and
    synchronisations between replays, equals eager decode on every replay,
    including the replays that resync."""
    n_seq, pre, steps = 3, 60, 10
    say(f"case: decode step captured in a graph, {n_seq} seqs, prefill {pre}, {steps} replays")
    inp = make_inputs([pre + steps] * n_seq, 2, 4, 128, "bf16", seed=32, h0="normal")
    cu = inp["cu_seqlens"].tolist()
    first = dict(inp)
    idx = torch.cat([torch.arange(cu[n], cu[n] + pre) for n in range(n_seq)])
    for key in ["q", "k", "v", "beta", "g"]:
        first[key] = inp[key][idx].contiguous()
    first["cu_seqlens"] = torch.tensor([0, pre, 2 * pre, 3 * pre], dtype=torch.int32)
    _, _, cache_e = run_prefill(first, cache=True)
    cache_g = cache_e.clone()
    shape = shape_for(inp)
    names = ["q", "k", "v", "beta", "g"]
    static = {k_: inp[k_][idx[:n_seq]].cuda().contiguous() for k_ in names}
    out = torch.empty(n_seq, 4, 128, dtype=torch.float32, device="cuda")
    ws = torch.empty(B.workspace_bytes(shape, n_seq, 0, B.OP_DECODE), dtype=torch.uint8,
                     device="cuda")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.gdn_decode_step(shape, *[static[k_] for k_ in names], cache_g, ws=ws, out=out)
    for s in range(steps):
        rows = torch.tensor([cu[n] + pre + s for n in range(n_seq)])
        for k_ in names:
            static[k_].copy_(inp[k_][rows])
        graph.replay()
        o_e = B.gdn_decode_step(shape, *[inp[k_][rows].cuda().contiguous() for k_ in names],
                                cache_e)
        torch.cuda.synchronize()
        assert bit_equal(out, o_e), f"replay {s}"
    assert bit_equal(cache_g.S_run, cache_e.S_run) and bit_equal(cache_g.S_chunk, cache_e.S_chunk)
    assert torch.equal(cache_g.pos, cache_e.pos)


def test_split_at_chunk_boundary_equals_one_prefill():
    say("case: two prefills split at a chunk edge == one prefill")
    inp = make_inputs([192, 256], 2, 4, 128, "bf16", seed=22, h0="normal")
    o, hT, _ = run_prefill(inp)
    cu = inp["cu_seqlens"].tolist()
    a = dict(inp)
    b = dict(inp)
    cut = [128, 64]
    ia = torch.cat([torch.arange(cu[n], cu[n] + cut[n]) for n in range(2)])
    ib = torch.cat([torch.arange(cu[n] + cut[n], cu[n + 1]) for n in range(2)])
    for key in ["q", "k", "v", "beta", "g"]:
        a[key] = inp[key][ia].contiguous()
        b[key] = inp[key][ib].contiguous()
    a["cu_seqlens"] = torch.tensor([0, 128, 192], dtype=torch.int32)
    b["cu_seqlens"] = torch.tensor([0, 64, 256], dtype=torch.int32)
    oa, ha, _ = run_prefill(a)
    b["h0"] = ha.cpu()
    ob, hb, _ = run_prefill(b)
    o_re = torch.cat([oa[:128], ob[:64], oa[128:], ob[64:]])
    assert bit_equal(o_re, o) and bit_equal(hb, hT)


def test_batch_composition_invariance():
    lens = [300, 17, 64, 129, 0, 65]
    say(f"case: packed vs alone vs reshuffled, lens={lens}")
    inp = make_inputs(lens, 2, 4, 128, "bf16", seed=23, h0="normal")
    o, hT, _ = run_prefill(inp)
    cu = inp["cu_seqlens"].tolist()
    for n in range(len(lens)):
        on, hn, _ = run_prefill(sub_inputs(inp, [n]))
        assert bit_equal(on, o[cu[n]:cu[n + 1]]), f"alone {n}"
        assert bit_equal(hn[0], hT[n])
    perm = [3, 5, 1, 0, 4, 2]
    sp = sub_inputs(inp, perm)
    op, hp, _ = run_prefill(sp)
    cp = sp["cu_seqlens"].tolist()
    for i, n in enumerate(perm):
        assert bit_equal(op[cp[i]:cp[i + 1]], o[cu[n]:cu[n + 1]]), f"reshuffled {n}"
        assert bit_equal(hp[i], hT[n])


def test_run_to_run_bit_identical():
    say("case: run to run")
    inp = make_inputs([333, 64, 1000], 2, 4, 128, "bf16", seed=24, h0="normal")
    o1, h1, _ = run_prefill(inp)
    o2, h2, _ = run_prefill(inp)
    assert bit_equal(o1, o2) and bit_equal(h1, h2)


def test_cache_checkpoint_resume():
    say("case: decode cache saved to host and restored mid-chunk")
    total, pre, mid = 200, 50, 40
    inp = make_inputs([total] * 2, 1, 2, 128, "bf16", seed=25, h0="normal")
    shape = shape_for(inp)
    first = dict(inp)
    idx = torch.cat([torch.arange(n * total, n * total + pre) for n in range(2)])
    for key in ["q", "k", "v", "beta", "g"]:
        first[key] = inp[key][idx].contiguous()
    first["cu_seqlens"] = torch.tensor([0, pre, 2 * pre], dtype=torch.int32)
    _, _, cache = run_prefill(first, cache=True)
    decode_tokens(inp, cache, shape, pre, mid)
    saved = [t.cpu() for t in cache.tensors()]
    rest = total - pre - mid
    o_a = decode_tokens(inp, cache, shape, pre + mid, rest)
    restored = B.Cache(shape, 2, "cuda", torch.bfloat16)
    for dst, src in zip(restored.tensors(), saved):
        dst.copy_(src.cuda())
    o_b = decode_tokens(inp, restored, shape, pre + mid, rest)
    assert bit_equal(o_a, o_b) and bit_equal(cache.S_run, restored.S_run)


# ------------------------------------------------------------------ full-size shapes

def test_prefill_b4_t2048_full_size():
    """B=4, T=2048, 16 q/k heads, 32 v heads, d=128, C=64, bf16, h0 ~ N(0, 0.02):
    oracle on one q/k group of two sequences; all outputs finite."""
    say("case: prefill B4 T2048 H16/32 d128 (sampled oracle)")
    inp = make_inputs([2048] * 4, 16, 32, 128, "bf16", seed=1, h0="normal")
    o, hT, _ = run_prefill(inp)
    assert torch.isfinite(o).all() and torch.isfinite(hT).all()
    for hq in [0, 11]:
        gi, hv = group_slice(inp, hq)
        ro, rh = oracle_fwd(gi, seqs=[0, 3])
        rows = rows_of(inp, [0, 3])
        e_o = maxabs(o.cpu()[rows][:, hv], ro[rows])
        e_h = maxabs(hT.cpu()[[0, 3]][:, hv], rh[[0, 3]])
        say(f"  group {hq}: max|o-oracle|={e_o:.3e} max|hT-oracle|={e_h:.3e}")
        assert e_o <= TOL["bf16"] and e_h <= TOL["bf16"]
    o2, h2, _ = run_prefill(inp)
    assert bit_equal(o, o2) and bit_equal(hT, h2)


def test_decode_64_seqs_4096_plus_256_equals_single_prefill():
    """64 sequences prefilled with 4096 tokens, then 256 decode steps; outputs and
    states equal one 4352-token prefill bit for bit; one group checked against
    the oracle on one sequence's decoded tokens."""
    say("case: decode 64 x (4096 + 256) vs prefill 4352")
    N, P, S = 64, 4096, 256
    inp = make_inputs([P + S] * N, 16, 32, 128, "bf16", seed=2, h0="zero")
    o_full, h_full, _ = run_prefill(inp)
    first = dict(inp)
    idx = torch.cat([torch.arange(n * (P + S), n * (P + S) + P) for n in range(N)])
    for key in ["q", "k", "v", "beta", "g"]:
        first[key] = inp[key][idx].contiguous()
    first["cu_seqlens"] = torch.arange(0, (N + 1) * P, P, dtype=torch.int32)
    _, _, cache = run_prefill(first, cache=True)
    shape = shape_for(inp)
    od = decode_tokens(inp, cache, shape, P, S)
    for n in range(N):
        assert bit_equal(od[:, n], o_full[n * (P + S) + P:(n + 1) * (P + S)]), f"seq {n}"
    assert bit_equal(cache.S_run, h_full)
    gi, hv = group_slice(inp, 5)
    ro, rh = oracle_fwd(gi, seqs=[7])
    e = maxabs(od[:, 7, hv].cpu(), ro[7 * (P + S) + P:8 * (P + S)])
    eh = maxabs(h_full[7, hv].cpu(), rh[7])
    say(f"  seq 7 group 5: max|o-oracle|={e:.3e} max|hT-oracle|={eh:.3e}")
    assert e <= TOL["bf16"] and eh <= TOL["bf16"]


def test_varlen_32_seqs_packed_alone_reshuffled():
    """32 sequences, lengths uniform in [128, 8192], packed; each sequence's
    output equals running it alone and in a reshuffled batch, bit for bit."""
    inp = make_inputs(("uniform", 32, 128, 8192), 16, 32, 128, "bf16", seed=4, h0="zero")
    say(f"case: varlen 32 seqs, T={inp['T']}")
    o, hT, _ = run_prefill(inp)
    assert torch.isfinite(o).all()
    cu = inp["cu_seqlens"].tolist()
    for n in range(32):
        on, hn, _ = run_prefill(sub_inputs(inp, [n]))
        assert bit_equal(on, o[cu[n]:cu[n + 1]]) and bit_equal(hn[0], hT[n]), f"alone {n}"
    perm = list(np.random.default_rng(0).permutation(32))
    sp = sub_inputs(inp, perm)
    op, hp, _ = run_prefill(sp)
    cp = sp["cu_seqlens"].tolist()
    for i, n in enumerate(perm):
        assert bit_equal(op[cp[i]:cp[i + 1]], o[cu[n]:cu[n + 1]]), f"reshuffled {n}"
        assert bit_equal(hp[i], hT[n])
    short = int(np.argmin(inp["lens"]))
    gi, hv = group_slice(inp, 3)
    ro, rh = oracle_fwd(gi, seqs=[short])
    rows = rows_of(inp, [short])
    e = maxabs(o.cpu()[rows][:, hv], ro[rows])
    say(f"  shortest seq {short} (len {inp['lens'][short]}): max|o-oracle|={e:.3e}")
    assert e <= TOL["bf16"]


# ------------------------------------------------------------------ native-mixed baseline

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_chunked_baseline_prefill_parity(dtype):
    """gdn_prefill_chunked (chunk-form outputs, the native-mixed baseline)
    computes the same function: parity with the oracle on ragged lengths,
    including partial last chunks and an empty sequence."""
    lens = [200, 64, 1, 130, 0, 129]
    say(f"case: chunk-form baseline prefill {dtype} lens={lens}")
    inp = make_inputs(lens, 2, 4, 128, dtype, seed=41, h0="normal")
    shape = shape_for(inp)
    d = to_dev(inp)
    o, hT = B.gdn_prefill_chunked(shape, d["q"], d["k"], d["v"], d["beta"], d["g"],
                                  d["cu_seqlens"], h0=d["h0"])
    check_parity(inp, o, hT, TOL[dtype])
    # the CPR prefill agrees within the same bar (not bit for bit)
    o_c, h_c, _ = run_prefill(inp)
    assert maxabs(o, o_c) <= 2 * TOL[dtype] and maxabs(hT, h_c) <= 2 * TOL[dtype]


# ------------------------------------------------------------------ prefill continuation

def _token_range(inp, starts, lens):
    """Packed sub-batch holding tokens starts[n] .. starts[n] + lens[n] - 1 of
    each sequence n."""
    cu = inp["cu_seqlens"].tolist()
    idx = [torch.arange(cu[n] + s, cu[n] + s + m) for n, (s, m) in enumerate(zip(starts, lens))]
    idx = torch.cat(idx) if idx else torch.zeros(0, dtype=torch.int64)
    out = dict(inp)
    for key in ["q", "k", "v", "beta", "g"]:
        out[key] = inp[key][idx].contiguous()
    c = torch.zeros(len(lens) + 1, dtype=torch.int32)
    c[1:] = torch.cumsum(torch.tensor(lens, dtype=torch.int32), 0)
    out["cu_seqlens"] = c
    out["T"] = int(sum(lens))
    return out, idx


def _continue(inp_part, cache, shape, pos):
    d = to_dev(inp_part)
    return B.gdn_prefill_continue(shape, d["q"], d["k"], d["v"], d["beta"], d["g"],
                                  d["cu_seqlens"], cache, pos)


def _check_cache_equal(c, ref, C):
    assert bit_equal(c.S_run, ref.S_run) and bit_equal(c.S_chunk, ref.S_chunk)
    pos = c.pos.cpu()
    assert torch.equal(pos, ref.pos.cpu())
    for n in range(pos.shape[0]):  # buffered rows of the current chunk
        p = int(pos[n, 0])
        for name in ["kbuf", "vbuf", "bbuf", "gbuf"]:
            a, b = getattr(c, name)[n, :p], getattr(ref, name)[n, :p]
            assert torch.equal(a.cpu().view(torch.uint8), b.cpu().view(torch.uint8)), name


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (16, "f32")])
def test_prefill_continue_equals_one_prefill(d, dtype):
    """Prefill a first part that stops inside a chunk, then continue with the
    rest through gdn_prefill_continue (twice): outputs, final states and cache
    equal one prefill of the whole sequences, bit for bit."""
    a = [70, 64, 1, 130, 0, 129, 5]
    b = [50, 0, 100, 3, 64, 200, 0]
    c = [9, 77, 0, 61, 1, 2, 11]
    tot = [x + y + z for x, y, z in zip(a, b, c)]
    say(f"case: continuation d{d} {dtype} parts {a} + {b} + {c}")
    inp = make_inputs(tot, 2, 4, d, dtype, seed=43, h0="normal")
    shape = shape_for(inp)
    C = shape.C
    o_full, h_full, c_full = run_prefill(inp, cache=True)
    pa, _ = _token_range(inp, [0] * len(a), a)
    _, _, cache = run_prefill(pa, cache=True)
    starts = list(a)
    for part in (b, c):
        pb, idx = _token_range(inp, starts, part)
        pos = [s % C for s in starts]
        assert torch.equal(cache.pos.cpu()[:, 0], torch.tensor(pos, dtype=torch.int32))
        o, hT = _continue(pb, cache, shape, pos)
        assert bit_equal(o, o_full[idx.cuda()]), "o"
        starts = [s + m for s, m in zip(starts, part)]
    assert bit_equal(hT, h_full), "hT"
    _check_cache_equal(cache, c_full, C)


def test_decode_then_continue_equals_one_prefill():
    """Prefill, a few decode steps (positions spread over the chunk), then a
    continuation: equals one prefill, bit for bit; decoding afterwards still
    matches."""
    a = [70, 64, 1, 130, 0, 129]
    steps, b, tail = 7, [90, 1, 64, 0, 130, 57], 5
    tot = [x + steps + y + tail for x, y in zip(a, b)]
    say(f"case: prefill {a} + decode {steps} + continue {b} + decode {tail}")
    inp = make_inputs(tot, 2, 4, 128, "bf16", seed=44, h0="normal")
    shape = shape_for(inp)
    C = shape.C
    o_full, h_full, c_full = run_prefill(inp, cache=True)
    pa, _ = _token_range(inp, [0] * len(a), a)
    _, _, cache = run_prefill(pa, cache=True)
    cu = inp["cu_seqlens"].tolist()
    N = len(a)

    def step_tokens(starts):
        idx = torch.tensor([cu[n] + starts[n] for n in range(N)])
        d = {k: inp[k][idx].cuda().contiguous() for k in ["q", "k", "v", "beta", "g"]}
        o = B.gdn_decode_step(shape, d["q"], d["k"], d["v"], d["beta"], d["g"], cache)
        assert bit_equal(o, o_full[(idx).cuda()]), "decode o"

    starts = list(a)
    for _ in range(steps):
        step_tokens(starts)
        starts = [s + 1 for s in starts]
    pb, idx = _token_range(inp, starts, b)
    o, _ = _continue(pb, cache, shape, [s % C for s in starts])
    assert bit_equal(o, o_full[idx.cuda()]), "continue o"
    starts = [s + m for s, m in zip(starts, b)]
    for _ in range(tail):
        step_tokens(starts)
        starts = [s + 1 for s in starts]
    assert bit_equal(cache.S_run, h_full)
    _check_cache_equal(cache, c_full, C)


# ------------------------------------------------------------------ batch sizes

def test_prefill_b4_t2048_batch_sizes_1_2_4():
    """The B4 T2048 prefill (16 q/k / 32 v heads, d128) run as one batch of 4,
    two batches of 2 and four batches of 1: every sequence's outputs and final
    state are the same bits."""
    say("case: prefill B4 T2048 as batches of 4 / 2 / 1")
    inp = make_inputs([2048] * 4, 16, 32, 128, "bf16", seed=1, h0="normal")
    o4, h4, _ = run_prefill(inp)
    cu = inp["cu_seqlens"].tolist()
    for group in ([0, 1], [2, 3], [0], [1], [2], [3]):
        o, h, _ = run_prefill(sub_inputs(inp, group))
        off = 0
        for j, n in enumerate(group):
            L = cu[n + 1] - cu[n]
            assert bit_equal(o[off:off + L], o4[cu[n]:cu[n + 1]]), f"o seq {n} in {group}"
            assert bit_equal(h[j], h4[n]), f"hT seq {n} in {group}"
            off += L


def test_decode_batches_64_32_1():
    """Decode of 64 sequences (prefill 130 + 70 steps, crossing chunk edges),
    and of 32 of them and of one alone: per-sequence outputs and states equal
    bit for bit."""
    n_all, pre, steps = 64, 130, 70
    say(f"case: decode batches 64 / 32 / 1, prefill {pre} + {steps} steps")
    inp = make_inputs([pre + steps] * n_all, 2, 4, 128, "bf16", seed=45, h0="normal")
    shape = shape_for(inp)

    def run(seqs):
        sub = sub_inputs(inp, seqs)
        first, _ = _token_range(sub, [0] * len(seqs), [pre] * len(seqs))
        _, _, cache = run_prefill(first, cache=True)
        return decode_tokens(sub, cache, shape, pre, steps), cache

    o_all, c_all = run(list(range(n_all)))
    for seqs in (list(range(0, n_all, 2)), [37]):
        o, c = run(seqs)
        for j, n in enumerate(seqs):
            assert bit_equal(o[:, j], o_all[:, n]), f"o seq {n}"
            assert bit_equal(c.S_run[j], c_all.S_run[n]), f"S_run seq {n}"
            assert bit_equal(c.S_chunk[j], c_all.S_chunk[n]), f"S_chunk seq {n}"


# ------------------------------------------------------------------ host copy

def test_host_copy_of_cu_seqlens_same_bits():
    """Passing the host copy of cu_seqlens (no device-to-host copy per call)
    changes nothing: prefill and trainer outputs are the same bits."""
    say("case: cu_seqlens_host given / not given, ragged d128 bf16")
    inp = make_inputs([200, 64, 1, 130], 2, 4, 128, "bf16", seed=61, h0="normal")
    shape = shape_for(inp)
    d = to_dev(inp, "cuda")
    cu_h = inp["cu_seqlens"].to("cpu", torch.int32)
    o1, h1 = B.gdn_prefill(shape, d["q"], d["k"], d["v"], d["beta"], d["g"], d["cu_seqlens"],
                           h0=d["h0"])
    o2, h2 = B.gdn_prefill(shape, d["q"], d["k"], d["v"], d["beta"], d["g"], d["cu_seqlens"],
                           h0=d["h0"], cu_seqlens_host=cu_h)
    assert bit_equal(o1, o2) and bit_equal(h1, h2)
    dO = torch.randn(inp["T"], 4, 128, generator=torch.Generator().manual_seed(62)).cuda()
    r1 = B.gdn_fwd_bwd(shape, d["q"], d["k"], d["v"], d["beta"], d["g"], d["cu_seqlens"], dO,
                       h0=d["h0"])
    r2 = B.gdn_fwd_bwd(shape, d["q"], d["k"], d["v"], d["beta"], d["g"], d["cu_seqlens"], dO,
                       h0=d["h0"], cu_seqlens_host=cu_h)
    for key in r1:
        assert bit_equal(r1[key], r2[key]), key
    say("  cu_seqlens_host NULL: the library copies the device copy itself")
    o3, h3 = B.gdn_prefill(shape, d["q"], d["k"], d["v"], d["beta"], d["g"], d["cu_seqlens"],
                           h0=d["h0"], cu_seqlens_host=False)
    assert bit_equal(o1, o3) and bit_equal(h1, h3)
    r3 = B.gdn_fwd_bwd(shape, d["q"], d["k"], d["v"], d["beta"], d["g"], d["cu_seqlens"], dO,
                       h0=d["h0"], cu_seqlens_host=False)
    for key in r1:
        assert bit_equal(r1[key], r3[key]), key
    oc1, hc1 = B.gdn_prefill_chunked(shape, d["q"], d["k"], d["v"], d["beta"], d["g"],
                                     d["cu_seqlens"], h0=d["h0"])
    oc2, hc2 = B.gdn_prefill_chunked(shape, d["q"], d["k"], d["v"], d["beta"], d["g"],
                                     d["cu_seqlens"], h0=d["h0"], cu_seqlens_host=False)
    assert bit_equal(oc1, oc2) and bit_equal(hc1, hc2)
    c1 = B.Cache(shape, 4, "cuda", torch.bfloat16)
    B.gdn_prefill(shape, d["q"], d["k"], d["v"], d["beta"], d["g"], d["cu_seqlens"],
                  h0=d["h0"], cache=c1)
    c2 = c1.clone()
    nx = make_inputs([10, 70, 0, 5], 2, 4, 128, "bf16", seed=63)
    nd = to_dev(nx, "cuda")
    pos = [int(x) for x in c1.pos[:, 0].cpu()]
    x1 = B.gdn_prefill_continue(shape, nd["q"], nd["k"], nd["v"], nd["beta"], nd["g"],
                                nd["cu_seqlens"], c1, pos)
    x2 = B.gdn_prefill_continue(shape, nd["q"], nd["k"], nd["v"], nd["beta"], nd["g"],
                                nd["cu_seqlens"], c2, pos, cu_seqlens_host=False)
    assert bit_equal(x1[0], x2[0]) and bit_equal(x1[1], x2[1])


@pytest.mark.parametrize("dtype,d,Hq,Hv", [("bf16", 128, 2, 4), ("f32", 16, 2, 2)])
def test_native_mixed_decode_parity(dtype, d, Hq, Hv):
    """gdn_decode_step_native (the native-mixed baseline's plain recurrent
    decode, no resync) computes the same function: 100 tokens from a random
    initial state against the oracle, every output and the final state."""
    steps, N = 100, 3
    say(f"case: native-mixed decode {dtype} d{d}, {N} seqs x {steps} tokens")
    inp = make_inputs([steps] * N, Hq, Hv, d, dtype, seed=45, h0="normal")
    shape = shape_for(inp)
    S = inp["h0"].cuda().clone()
    outs = []
    for s in range(steps):
        idx = torch.tensor([n * steps + s for n in range(N)])
        t = {k: inp[k][idx].cuda().contiguous() for k in ["q", "k", "v", "beta", "g"]}
        outs.append(B.gdn_decode_step_native(shape, t["q"], t["k"], t["v"], t["beta"], t["g"], S))
    od = torch.stack(outs, 1).reshape(N * steps, Hv, d)  # [N, steps] -> packed rows
    ro, rh = oracle_fwd(inp)
    e_o, e_h = maxabs(od, ro), maxabs(S, rh)
    say(f"  max|o-oracle|={e_o:.2e} max|S-oracle|={e_h:.2e} (tol {TOL[dtype]})")
    assert e_o <= TOL[dtype] and e_h <= TOL[dtype]


def test_decode_3000_sequences_across_a_chunk_edge():
    """A large decode batch (3000 sequences, grid.x = 3000): prefill 60 tokens,
    decode 10 one at a time (every sequence resyncs after its 64th token),
    equal to one 70-token prefill bit for bit; the no-allocation entry point
    (twelve resync groups of the fixed scratch at this shape) gives the same
    bits as gdn_decode_step."""
    N, pre, total = 3000, 60, 70
    say(f"case: decode {N} sequences, prefill {pre} + decode {total - pre}")
    inp = make_inputs([total] * N, 1, 2, 128, "bf16", seed=81, h0="normal")
    o_full, h_full, _ = run_prefill(inp)
    shape = shape_for(inp)
    first = dict(inp)
    idx = torch.cat([torch.arange(n * total, n * total + pre) for n in range(N)])
    for key in ["q", "k", "v", "beta", "g"]:
        first[key] = inp[key][idx].contiguous()
    first["cu_seqlens"] = torch.arange(0, (N + 1) * pre, pre, dtype=torch.int32)
    _, _, cache = run_prefill(first, cache=True)
    c2 = cache.clone()
    od = decode_tokens(inp, cache, shape, pre, total - pre)
    rows = torch.cat([torch.arange(n * total + pre, (n + 1) * total) for n in range(N)])
    assert bit_equal(od.transpose(0, 1).reshape(-1, 2, 128), o_full[rows.cuda()])
    assert bit_equal(cache.S_run, h_full)
    cu = inp["cu_seqlens"].tolist()
    for s in range(total - pre):
        ix = torch.tensor([cu[n] + pre + s for n in range(N)])
        t = {k: inp[k][ix].cuda().contiguous() for k in ["q", "k", "v", "beta", "g"]}
        on = B.gdn_decode_step_noalloc(shape, t["q"], t["k"], t["v"], t["beta"], t["g"], c2)
        assert bit_equal(on, od[s]), f"no-alloc step {s}"
    assert bit_equal(c2.S_run, cache.S_run) and bit_equal(c2.S_chunk, cache.S_chunk)
