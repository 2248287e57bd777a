"""gdn_decode_step_noalloc (no workspace; the library's fixed device scratch)
against gdn_decode_step: the same o and the same cache, bit for bit, on two
calls in a row, the second with a smaller batch.

The first batch (20 sequences x 32 value heads at d = 128) needs two resync
groups of the fixed scratch; its sequences stand at different chunk offsets,
so the groups resync on different steps.  The second batch is smaller and
runs after it, so it starts from the scratch contents the first one left.
"""

import pytest
import torch

from gdn_helpers import bit_equal, make_inputs, shape_for
from linear_attention_rnn_gated_amd import binding as B

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def caches_equal(a, b):
    pos = a.pos.cpu()
    if not (bit_equal(a.S_run, b.S_run) and bit_equal(a.S_chunk, b.S_chunk)
            and torch.equal(a.pos, b.pos)):
        return False
    for n in range(a.n):
        p = int(pos[n, 0])
        for x, y in [(a.kbuf, b.kbuf), (a.bbuf, b.bbuf), (a.gbuf, b.gbuf)]:
            if not bit_equal(x[n, :p], y[n, :p]):
                return False
        if not torch.equal(a.vbuf[n, :p], b.vbuf[n, :p]):
            return False
    return True


def run_pair(lens, Hq, Hv, d, dtype, steps, seed, use_pos_host):
    """Prefills `lens`, then decodes `steps` tokens per sequence through both
    entry points from identical caches; checks every step's o and the final
    caches."""
    say(f"case: no-alloc decode N={len(lens)} H {Hq}/{Hv} d{d} {dtype}, {steps} steps, "
        f"pos_host={use_pos_host}")
    inp = make_inputs(lens, Hq, Hv, d, dtype, seed=seed, h0="normal")
    shape = shape_for(inp)
    N = inp["N"]
    cache = B.Cache(shape, N, "cuda", inp["q"].dtype)
    dd = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    B.gdn_prefill(shape, dd["q"], dd["k"], dd["v"], dd["beta"], dd["g"], dd["cu_seqlens"],
                  h0=dd["h0"], cache=cache)
    ca, cb = cache, cache.clone()
    dec = make_inputs([steps] * N, Hq, Hv, d, dtype, seed=seed + 1)
    ob = torch.empty(N, Hv, d, dtype=torch.float32, device="cuda")
    ws = torch.empty(B.workspace_bytes(shape, N, 0, B.OP_DECODE), dtype=torch.uint8,
                     device="cuda")
    resyncs = 0
    for s in range(steps):
        idx = torch.tensor([n * steps + s for n in range(N)])
        t = {k: dec[k][idx].cuda().contiguous() for k in ["q", "k", "v", "beta", "g"]}
        ph = cb.pos.cpu() if use_pos_host else None
        if ph is not None:
            resyncs += int((ph == shape.C - 1).any())
        oa = B.gdn_decode_step(shape, t["q"], t["k"], t["v"], t["beta"], t["g"], ca,
                               pos_host=ph, ws=ws)
        B.gdn_decode_step_noalloc(shape, t["q"], t["k"], t["v"], t["beta"], t["g"], cb,
                                  pos_host=ph, out=ob)
        assert bit_equal(oa, ob), f"o differs at step {s}"
    assert caches_equal(ca, cb), "caches differ"
    say(f"  {steps} steps bit-identical ({resyncs} with a resync seen on the host)")


def test_no_alloc_decode_equals_decode_step_two_calls():
    # first call: two resync groups (15 + 5 sequences), offsets spread over the chunk
    lens = [60 + (7 * n) % 64 for n in range(20)]
    run_pair(lens, 16, 32, 128, "bf16", 70, seed=71, use_pos_host=True)
    # second call: a smaller batch after the first, device-side resync decision
    run_pair([10, 63, 64], 2, 4, 128, "bf16", 70, seed=73, use_pos_host=False)
    # and the fp32 claim at d = 16
    run_pair([5, 16], 2, 2, 16, "f32", 20, seed=75, use_pos_host=False)
