"""Plain fp64 CPU oracle for the gated delta-rule layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg import this module.  The GPU library never calls it, shares no
code with it, and must fail loudly rather than fall back to it.

What is computed
----------------
The layer is Gated DeltaNet (GDN).  The IsoExec pages name it (agentlenshq.com
write-up "IsoExec: SkyRLにおけるトレーナーと推論のミスマッチを解消する",
section "Chunkwise-Parallel Recurrent (CPR) Gated DeltaNet") but do not write
its equations.  The definition used here is the gated delta rule in the form
in which the problem this library solves is stated: per value head, with the
state S a d_v x d_k matrix,

    S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
    o_t = S_t q_t,

with alpha_t = exp(g_t), q and k L2-normalised per token and head.  CPR (same
section of the write-up; daily.dev digest, Q&A "What is chunkwise-parallel
recurrent (CPR)") is a schedule for evaluating exactly this function, so the
oracle is the plain definition, evaluated token by token in fp64.

Readings taken where the pages are silent:
  * the state is stored [d_k][d_v] (d_v fastest), i.e. the transpose of S;
  * g is log(alpha); beta and g are per value head;
  * value head h reads query/key head h // (H_v / H_qk) (contiguous groups);
  * L2 norm: x / sqrt(sum x^2 + eps), eps = 1e-6; q is multiplied by `scale`
    after normalisation;
  * sequences are packed along the token axis and delimited by cu_seqlens.

Functions
---------
  l2norm_rows      the normalisation step
  recurrent_fwd    the recurrence, token by token (the parity reference)
  recurrent_bwd    reverse-mode gradient of recurrent_fwd, token by token
  chunk_fwd        a second, independent formula: the chunk (WY) algebra
                   derived from the recurrence; used to pin recurrent_fwd

Pins (tests/test_oracle.py): zero output for beta = 0 and zero state, the
beta = 0 closed form, the alpha = 0 reset, exact delta-rule recall for
alpha = beta = 1, orthonormal-key recall, linearity in (v, h0), the factored
matrix form, the d_k = 1 sum-of-products closed form, split and batch
invariance, chunk algebra == recurrence, and central finite differences for
every gradient.  No function here is "parity unpinned".
"""

import numpy as np

EPS = 1e-6


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def l2norm_rows(x, eps=EPS):
    """x / sqrt(sum(x^2) + eps) over the last axis, in fp64."""
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def _prep_qk(q, k, scale, qk_l2norm, eps):
    q = _f64(q)
    k = _f64(k)
    if qk_l2norm:
        q = l2norm_rows(q, eps)
        k = l2norm_rows(k, eps)
    return q * float(scale), k


def _head_map(H_qk, H_v):
    if H_v % H_qk:
        raise ValueError("H_v must be a multiple of H_qk")
    return np.arange(H_v) // (H_v // H_qk)


def _check_cu(cu_seqlens, T):
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0, end at T and be non-decreasing")
    return cu


def _state_in(h0, n, H_v, d_k, d_v):
    """Math-form state S[h] (d_v x d_k) of sequence n from the stored layout."""
    if h0 is None:
        return np.zeros((H_v, d_v, d_k))
    return _f64(h0[n]).transpose(0, 2, 1).copy()


def _step(S, qt, kt, vt, bt, gt):
    """One token of the recurrence for every value head at once.

    S [H, d_v, d_k]; qt, kt [H, d_k]; vt [H, d_v]; bt, gt [H].
    Returns (S_t, o_t, P, u, delta); P, u, delta are kept for the gradient.
    """
    a = np.exp(gt)
    P = a[:, None, None] * S                       # alpha * S_{t-1}
    u = np.matmul(P, kt[:, :, None])[:, :, 0]       # P k
    delta = bt[:, None] * (vt - u)                  # beta (v - P k)
    S_new = P + delta[:, :, None] * kt[:, None, :]  # P + delta k^T
    o = np.matmul(S_new, qt[:, :, None])[:, :, 0]   # S_t q
    return S_new, o, P, u, delta


def recurrent_fwd(q, k, v, beta, g, cu_seqlens, h0=None, scale=1.0,
                  qk_l2norm=True, eps=EPS, seqs=None):
    """Token-by-token fp64 recurrence.

    q, k : [T, H_qk, d_k]      v : [T, H_v, d_v]      beta, g : [T, H_v]
    cu_seqlens : [N+1]         h0 : [N, H_v, d_k, d_v] or None (zero state)
    seqs : optional iterable of sequence indices to evaluate (others stay 0).
    Returns o [T, H_v, d_v] and h_T [N, H_v, d_k, d_v] (stored layout).
    """
    T, H_qk, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    cu = _check_cu(cu_seqlens, T)
    N = len(cu) - 1
    hm = _head_map(H_qk, H_v)
    qh, kh = _prep_qk(q, k, scale, qk_l2norm, eps)
    v = _f64(v)
    beta = _f64(beta)
    g = _f64(g)
    o = np.zeros((T, H_v, d_v))
    hT = np.zeros((N, H_v, d_k, d_v))
    for n in (range(N) if seqs is None else seqs):
        S = _state_in(h0, n, H_v, d_k, d_v)
        for t in range(cu[n], cu[n + 1]):
            S, o[t], _, _, _ = _step(S, qh[t][hm], kh[t][hm], v[t], beta[t], g[t])
        hT[n] = S.transpose(0, 2, 1)
    return o, hT


def _norm_bwd(x, dxh, scale, eps):
    """Gradient through xh = scale * x / sqrt(sum x^2 + eps)."""
    r = 1.0 / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)
    xn = x * r
    return scale * r * (dxh - xn * np.sum(xn * dxh, axis=-1, keepdims=True))


def recurrent_bwd(q, k, v, beta, g, cu_seqlens, do, h0=None, dhT=None,
                  scale=1.0, qk_l2norm=True, eps=EPS, ckpt=64, seqs=None):
    """Reverse-mode gradient of recurrent_fwd, token by token, in fp64.

    do : [T, H_v, d_v] upstream gradient of o;  dhT : [N, H_v, d_k, d_v] or
    None (zero) upstream gradient of h_T.  States are re-run from checkpoints
    every `ckpt` tokens so memory stays bounded.  Returns a dict with dq, dk
    [T, H_qk, d_k], dv [T, H_v, d_v], dbeta, dg [T, H_v], dh0 [N, H_v, d_k, d_v].
    Rows of sequences not in `seqs` stay zero.
    """
    T, H_qk, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    cu = _check_cu(cu_seqlens, T)
    N = len(cu) - 1
    hm = _head_map(H_qk, H_v)
    q64, k64 = _f64(q), _f64(k)
    qh, kh = _prep_qk(q64, k64, scale, qk_l2norm, eps)
    v = _f64(v)
    beta = _f64(beta)
    g = _f64(g)
    do = _f64(do)
    dqh_v = np.zeros((T, H_v, d_k))   # per value head, before the group sum
    dkh_v = np.zeros((T, H_v, d_k))
    dv = np.zeros((T, H_v, d_v))
    dbeta = np.zeros((T, H_v))
    dg = np.zeros((T, H_v))
    dh0 = np.zeros((N, H_v, d_k, d_v))
    for n in (range(N) if seqs is None else seqs):
        t0, t1 = int(cu[n]), int(cu[n + 1])
        # forward: keep the state at every checkpoint
        marks = list(range(t0, t1, ckpt)) + [t1]
        S = _state_in(h0, n, H_v, d_k, d_v)
        saved = {t0: S.copy()}
        for a_, b_ in zip(marks[:-1], marks[1:]):
            for t in range(a_, b_):
                S = _step(S, qh[t][hm], kh[t][hm], v[t], beta[t], g[t])[0]
            saved[b_] = S.copy()
        dS = np.zeros((H_v, d_v, d_k)) if dhT is None else _f64(dhT[n]).transpose(0, 2, 1).copy()
        # reverse, one checkpoint segment at a time
        for a_, b_ in reversed(list(zip(marks[:-1], marks[1:]))):
            S = saved[a_]
            seg = []
            for t in range(a_, b_):
                S_prev = S
                S, _, P, u, delta = _step(S, qh[t][hm], kh[t][hm], v[t], beta[t], g[t])
                seg.append((S_prev, S, P, u, delta))
            for t in range(b_ - 1, a_ - 1, -1):
                S_prev, S_t, P, u, delta = seg[t - a_]
                qt, kt = qh[t][hm], kh[t][hm]
                alpha = np.exp(g[t])
                # o_t = S_t q_t
                dS = dS + do[t][:, :, None] * qt[:, None, :]
                dqh_v[t] = np.matmul(S_t.transpose(0, 2, 1), do[t][:, :, None])[:, :, 0]
                # S_t = P + delta k^T
                dP = dS.copy()
                ddelta = np.matmul(dS, kt[:, :, None])[:, :, 0]
                dk_t = np.matmul(dS.transpose(0, 2, 1), delta[:, :, None])[:, :, 0]
                # delta = beta (v - u)
                dbeta[t] = np.sum(ddelta * (v[t] - u), axis=1)
                dv[t] = beta[t][:, None] * ddelta
                du = -beta[t][:, None] * ddelta
                # u = P k
                dP = dP + du[:, :, None] * kt[:, None, :]
                dk_t = dk_t + np.matmul(P.transpose(0, 2, 1), du[:, :, None])[:, :, 0]
                dkh_v[t] = dk_t
                # P = alpha S_{t-1},  alpha = exp(g)
                dg[t] = alpha * np.sum(dP * S_prev, axis=(1, 2))
                dS = alpha[:, None, None] * dP
        dh0[n] = dS.transpose(0, 2, 1)
    # sum over the value heads of each group, ascending value-head order
    dqh = np.zeros((T, H_qk, d_k))
    dkh = np.zeros((T, H_qk, d_k))
    for h in range(H_v):
        dqh[:, hm[h]] += dqh_v[:, h]
        dkh[:, hm[h]] += dkh_v[:, h]
    if qk_l2norm:
        dq = _norm_bwd(q64, dqh, scale, eps)
        dk = _norm_bwd(k64, dkh, 1.0, eps)
    else:
        dq = dqh * float(scale)
        dk = dkh
    return dict(dq=dq, dk=dk, dv=dv, dbeta=dbeta, dg=dg, dh0=dh0)


def chunk_fwd(q, k, v, beta, g, cu_seqlens, C, h0=None, scale=1.0,
              qk_l2norm=True, eps=EPS):
    """The chunk (WY/UT) algebra: a second formula for the same function.

    Derived from the recurrence by unrolling it over a chunk that starts from
    the state S0 (d_v x d_k).  With G_p the running sum of g inside the chunk
    and gam_p = exp(G_p):
        S_p      = gam_p S0 + sum_{r<=p} exp(G_p - G_r) delta_r k_r^T
        delta_p  = beta_p v_p - beta_p gam_p S0 k_p - sum_{r<p} A_pr delta_r,
        A_pr     = beta_p (k_p . k_r) exp(G_p - G_r)            (p > r)
    so (I + A) Delta = diag(beta) V - diag(beta gam) K S0^T.  Forward
    substitution gives W, U with Delta = U - W S0^T, and then
        o_p      = gam_p S0 q_p + sum_{r<=p} (q_p . k_r) exp(G_p - G_r) Delta_r
        S_next   = gam_C S0 + sum_p exp(G_C - G_p) Delta_p k_p^T.
    Chunks are counted from each sequence's first token; the last chunk may be
    shorter than C.  g must be finite here.  Returns o and h_T like
    recurrent_fwd.
    """
    T, H_qk, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    cu = _check_cu(cu_seqlens, T)
    N = len(cu) - 1
    hm = _head_map(H_qk, H_v)
    qh, kh = _prep_qk(q, k, scale, qk_l2norm, eps)
    v = _f64(v)
    beta = _f64(beta)
    g = _f64(g)
    o = np.zeros((T, H_v, d_v))
    hT = np.zeros((N, H_v, d_k, d_v))
    for n in range(N):
        S = _state_in(h0, n, H_v, d_k, d_v)
        for c0 in range(cu[n], cu[n + 1], C):
            c1 = min(c0 + C, cu[n + 1])
            L = c1 - c0
            Kc = kh[c0:c1][:, hm].transpose(1, 0, 2)   # [H, L, d_k]
            Qc = qh[c0:c1][:, hm].transpose(1, 0, 2)   # [H, L, d_k]
            Vc = v[c0:c1].transpose(1, 0, 2)           # [H, L, d_v]
            bc = beta[c0:c1].T                         # [H, L]
            G = np.cumsum(g[c0:c1].T, axis=1)          # [H, L]
            gam = np.exp(G)
            low = np.tril(np.ones((L, L), dtype=bool))     # r <= p
            diff = np.where(low[None], G[:, :, None] - G[:, None, :], 0.0)
            decay = np.where(low[None], np.exp(diff), 0.0)  # [H, p, r]
            KK = np.matmul(Kc, Kc.transpose(0, 2, 1))       # [H, p, r]
            A = bc[:, :, None] * KK * decay
            W = np.zeros((H_v, L, d_k))
            U = np.zeros((H_v, L, d_v))
            for p in range(L):
                W[:, p] = (bc[:, p] * gam[:, p])[:, None] * Kc[:, p]
                U[:, p] = bc[:, p][:, None] * Vc[:, p]
                for r in range(p):
                    W[:, p] -= A[:, p, r][:, None] * W[:, r]
                    U[:, p] -= A[:, p, r][:, None] * U[:, r]
            Delta = U - np.matmul(W, S.transpose(0, 2, 1))            # [H, L, d_v]
            QK = np.matmul(Qc, Kc.transpose(0, 2, 1)) * decay      # masked r <= p
            Oc = gam[:, :, None] * np.matmul(Qc, S.transpose(0, 2, 1)) + np.matmul(QK, Delta)
            o[c0:c1] = Oc.transpose(1, 0, 2)
            tail = np.exp(G[:, -1:] - G)                               # [H, L]
            S = gam[:, -1][:, None, None] * S + np.matmul(
                (tail[:, :, None] * Delta).transpose(0, 2, 1), Kc)
        hT[n] = S.transpose(0, 2, 1)
    return o, hT
