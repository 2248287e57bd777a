"""Shared helpers: run the library and the oracle on the same seeded inputs."""

import numpy as np
import torch

from linear_attention_rnn_gated_amd import binding as B
from linear_attention_rnn_gated_amd.inputs import make_inputs, to_numpy_f64

CLAIM_C = {16: 16, 128: 64}


def shape_for(inp, scale=1.0, qk_l2norm=True):
    d = inp["d"]
    return B.make_shape(inp["H_qk"], inp["H_v"], d, CLAIM_C[d], inp["q"].dtype,
                        qk_l2norm=qk_l2norm, scale=scale)


def to_dev(inp, dev="cuda"):
    out = {}
    for k, v in inp.items():
        out[k] = v.to(dev) if isinstance(v, torch.Tensor) else v
    return out


def oracle_fwd(inp, seqs=None, scale=1.0, qk_l2norm=True):
    from oracle import recurrent_fwd
    f = to_numpy_f64
    return recurrent_fwd(f(inp["q"]), f(inp["k"]), f(inp["v"]), f(inp["beta"]), f(inp["g"]),
                         inp["cu_seqlens"].numpy(), h0=f(inp["h0"]), scale=scale,
                         qk_l2norm=qk_l2norm, seqs=seqs)


def oracle_bwd(inp, seqs=None, dhT=None, scale=1.0):
    from oracle import recurrent_bwd
    f = to_numpy_f64
    return recurrent_bwd(f(inp["q"]), f(inp["k"]), f(inp["v"]), f(inp["beta"]), f(inp["g"]),
                         inp["cu_seqlens"].numpy(), f(inp["do"]), h0=f(inp["h0"]),
                         dhT=f(dhT), scale=scale, seqs=seqs)


def rows_of(inp, seqs):
    cu = inp["cu_seqlens"].tolist()
    return np.concatenate([np.arange(cu[n], cu[n + 1]) for n in seqs]).astype(np.int64)


def maxabs(a, b):
    a = a.detach().double().cpu().numpy() if isinstance(a, torch.Tensor) else np.asarray(a)
    b = b.detach().double().cpu().numpy() if isinstance(b, torch.Tensor) else np.asarray(b)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def bits(t):
    """Bit pattern of a float32 tensor (so -0.0 != +0.0 and NaN == NaN)."""
    return t.detach().contiguous().view(torch.int32).cpu()


def bit_equal(a, b):
    return a.shape == b.shape and torch.equal(bits(a), bits(b))


def sub_inputs(inp, seqs):
    """The packed inputs of a subset of sequences, in the given order."""
    cu = inp["cu_seqlens"].tolist()
    idx = torch.cat([torch.arange(cu[n], cu[n + 1]) for n in seqs]) if seqs else \
        torch.zeros(0, dtype=torch.int64)
    lens = [cu[n + 1] - cu[n] for n in seqs]
    out = dict(inp)
    for key in ["q", "k", "v", "beta", "g", "do"]:
        if inp.get(key) is not None:
            out[key] = inp[key][idx].contiguous()
    if inp.get("h0") is not None:
        out["h0"] = inp["h0"][list(seqs)].contiguous()
    c = torch.zeros(len(seqs) + 1, dtype=torch.int32)
    if seqs:
        c[1:] = torch.cumsum(torch.tensor(lens), 0)
    out["cu_seqlens"] = c
    out["lens"] = lens
    out["N"] = len(seqs)
    out["T"] = int(sum(lens))
    return out


def run_prefill(inp, dev="cuda", cache=False, scale=1.0, qk_l2norm=True):
    shape = shape_for(inp, scale, qk_l2norm)
    d = to_dev(inp, dev)
    c = B.Cache(shape, inp["N"], dev, inp["q"].dtype) if cache else None
    o, hT = B.gdn_prefill(shape, d["q"], d["k"], d["v"], d["beta"], d["g"], d["cu_seqlens"],
                          h0=d["h0"], cache=c)
    return o, hT, c


def decode_tokens(inp, cache, shape, start, steps, dev="cuda", use_pos_host=True):
    """Feeds tokens start..start+steps-1 of every (equal-length) sequence one at a
    time.  Returns o [steps, N, H_v, d]."""
    cu = inp["cu_seqlens"].tolist()
    N = inp["N"]
    outs = []
    pos = cache.pos.cpu() if use_pos_host else None
    for s in range(steps):
        idx = torch.tensor([cu[n] + start + s for n in range(N)])
        q = inp["q"][idx].to(dev).contiguous()
        k = inp["k"][idx].to(dev).contiguous()
        v = inp["v"][idx].to(dev).contiguous()
        b = inp["beta"][idx].to(dev).contiguous()
        g = inp["g"][idx].to(dev).contiguous()
        outs.append(B.gdn_decode_step(shape, q, k, v, b, g, cache,
                                      pos_host=pos))
        if pos is not None:
            pos = (pos + 1) % shape.C
    return torch.stack(outs) if outs else None


__all__ = ["make_inputs", "shape_for", "to_dev", "oracle_fwd", "oracle_bwd", "rows_of",
           "maxabs", "bits", "bit_equal", "sub_inputs", "run_prefill", "decode_tokens",
           "group_slice"]


def group_slice(inp, hq):
    """Inputs restricted to query/key head hq and its value heads (heads are
    independent, so the oracle can check one group of a large problem)."""
    G = inp["H_v"] // inp["H_qk"]
    hv = slice(hq * G, (hq + 1) * G)
    out = dict(inp)
    out["q"] = inp["q"][:, hq:hq + 1].contiguous()
    out["k"] = inp["k"][:, hq:hq + 1].contiguous()
    for key in ["v", "beta", "g", "do"]:
        if inp.get(key) is not None:
            out[key] = inp[key][:, hv].contiguous()
    if inp.get("h0") is not None:
        out["h0"] = inp["h0"][:, hv].contiguous()
    out["H_qk"] = 1
    out["H_v"] = G
    return out, hv
