"""Runs every entry point of the library once on fixed seeded inputs and
prints one JSON line mapping each output to the SHA-256 of its bytes.

Used by tests/test_gpu_isolation.py in a child process: the parent computes the
same digests in its own process (different allocations, a different warm-up
history, a fresh HIP context here) and requires them to be equal.
"""

import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)

import torch  # noqa: E402

from gdn_helpers import make_inputs, shape_for, to_dev  # noqa: E402
from linear_attention_rnn_gated_amd import binding as B  # noqa: E402

LENS = [300, 17, 64, 129, 0, 65]
NEW = [30, 100, 5, 0, 64, 1]
STEPS = 70


def digest(t):
    return hashlib.sha256(t.detach().contiguous().cpu().view(torch.uint8).numpy().tobytes()) \
        .hexdigest()


def run(dev="cuda"):
    """Digests of prefill (o, hT, cache), decode steps, a continuation and
    fwd_bwd (all outputs) on one batch at d = 128, bf16 inputs."""
    out = {}
    inp = make_inputs(LENS, 2, 4, 128, "bf16", seed=61, h0="normal", with_do=True)
    shape = shape_for(inp)
    d = to_dev(inp, dev)
    cache = B.Cache(shape, inp["N"], dev, torch.bfloat16)
    o, hT = B.gdn_prefill(shape, d["q"], d["k"], d["v"], d["beta"], d["g"], d["cu_seqlens"],
                          h0=d["h0"], cache=cache)
    out["prefill.o"], out["prefill.hT"] = digest(o), digest(hT)
    out["prefill.S_run"], out["prefill.S_chunk"] = digest(cache.S_run), digest(cache.S_chunk)
    out["prefill.pos"] = digest(cache.pos)
    # decode STEPS tokens of every sequence (each at its own chunk offset)
    dec = make_inputs([STEPS] * inp["N"], 2, 4, 128, "bf16", seed=62)
    dc = cache.clone()
    outs = []
    for s in range(STEPS):
        idx = torch.tensor([n * STEPS + s for n in range(inp["N"])])
        t = {k: dec[k][idx].to(dev).contiguous() for k in ["q", "k", "v", "beta", "g"]}
        outs.append(B.gdn_decode_step(shape, t["q"], t["k"], t["v"], t["beta"], t["g"], dc))
    out["decode.o"] = digest(torch.stack(outs))
    out["decode.S_run"], out["decode.S_chunk"] = digest(dc.S_run), digest(dc.S_chunk)
    # continuation of the prefilled cache by a ragged batch of new tokens
    nx = make_inputs(NEW, 2, 4, 128, "bf16", seed=63)
    nd = to_dev(nx, dev)
    cc = cache.clone()
    pos = [int(x) for x in cache.pos[:, 0].cpu()]
    oc, hc = B.gdn_prefill_continue(shape, nd["q"], nd["k"], nd["v"], nd["beta"], nd["g"],
                                    nd["cu_seqlens"], cc, pos)
    out["continue.o"], out["continue.hT"] = digest(oc), digest(hc)
    out["continue.S_run"] = digest(cc.S_run)
    r = B.gdn_fwd_bwd(shape, d["q"], d["k"], d["v"], d["beta"], d["g"], d["cu_seqlens"],
                      d["do"], h0=d["h0"])
    for k, v in r.items():
        out["fwd_bwd." + k] = digest(v)
    torch.cuda.synchronize()
    return out


if __name__ == "__main__":
    print("bits_child: running", flush=True, file=sys.stderr)
    print(json.dumps(run()), flush=True)
