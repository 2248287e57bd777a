"""Seeded synthetic inputs for the gated delta-rule layer.

This module only draws random tensors; it holds none of the layer's arithmetic.
The tests feed the same tensors to the GPU library and to the CPU oracle.

Recipe (one torch CPU generator per call, seeded; draw order fixed):
  lengths (only for the uniform-length mix), q, k, v, beta logits, g logits,
  h0, dO.
  * q, k ~ N(0, 1), each token's vector scaled to unit length in fp32, then cast
    to the input dtype (the layer normalises again in-kernel);
  * v ~ N(0, 1), cast to the input dtype;
  * beta = sigmoid(N(0, 1)), fp32;
  * g = log(alpha) = -softplus(N(0, 1)), fp32;
  * h0: zero, or N(0, 0.02) fp32 in the stored layout [N, H_v, d_k, d_v];
  * dO ~ N(0, 1) fp32.
"""

import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def uniform_lengths(n, lo, hi, seed):
    """n integers uniform in [lo, hi], from the seed's generator (first draw)."""
    gen = torch.Generator().manual_seed(seed)
    return [int(x) for x in torch.randint(lo, hi + 1, (n,), generator=gen)]


def make_inputs(lens, H_qk, H_v, d, dtype="bf16", seed=0, h0="zero",
                with_do=False, d_v=None, device="cpu"):
    """Packed inputs for sequences of the given lengths.

    Returns a dict of CPU tensors: q, k [T, H_qk, d]; v [T, H_v, d_v];
    beta, g [T, H_v] fp32; h0 [N, H_v, d, d_v] fp32 or None; do [T, H_v, d_v]
    fp32 or None; cu_seqlens int32 [N + 1]; plus the shape fields.  With
    device="cuda" the tensors are drawn there by that device's generator (same
    recipe, different stream of numbers; used for large benchmark inputs); the
    lengths of the uniform mix are the CPU generator's first draw on every
    device, so a benchmark's batch has the tests' lengths.
    """
    d_v = d if d_v is None else d_v
    gen = torch.Generator(device=device).manual_seed(seed)
    if isinstance(lens, tuple) and lens and lens[0] == "uniform":
        _, n, lo, hi = lens
        if torch.device(device).type == "cpu":
            lens = [int(x) for x in torch.randint(lo, hi + 1, (n,), generator=gen)]
        else:
            lens = uniform_lengths(n, lo, hi, seed)
    lens = [int(x) for x in lens]
    T = sum(lens)
    N = len(lens)
    cu = torch.zeros(N + 1, dtype=torch.int32)
    if N:
        cu[1:] = torch.cumsum(torch.tensor(lens, dtype=torch.int64), 0).to(torch.int32)
    dt = DTYPES[dtype]

    def unit(x):
        return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)

    kw = dict(generator=gen, device=device)
    q = unit(torch.randn(T, H_qk, d, **kw)).to(dt)
    k = unit(torch.randn(T, H_qk, d, **kw)).to(dt)
    v = torch.randn(T, H_v, d_v, **kw).to(dt)
    beta = torch.sigmoid(torch.randn(T, H_v, **kw))
    g = -torch.nn.functional.softplus(torch.randn(T, H_v, **kw))
    if h0 == "normal":
        h0t = 0.02 * torch.randn(N, H_v, d, d_v, **kw)
    elif h0 == "zero":
        h0t = None
    else:
        raise ValueError(h0)
    do = torch.randn(T, H_v, d_v, **kw) if with_do else None
    return dict(q=q, k=k, v=v, beta=beta.contiguous(), g=g.contiguous(), h0=h0t,
                do=do, cu_seqlens=cu, lens=lens, T=T, N=N, H_qk=H_qk, H_v=H_v,
                d=d, d_v=d_v, dtype=dtype)


def to_numpy_f64(t):
    """Exact widening of a CPU tensor (bf16 values are exact in fp64)."""
    return None if t is None else t.to(torch.float64).numpy()
