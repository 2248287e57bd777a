"""Pins of the fp64 oracle against facts fixed by the mathematics.

The pages print no worked example for the layer, so every pin here is a closed
form, an invariant, an independent second formula or a finite-difference
check.  Each is chosen so that a plausible slip in the oracle (a dropped alpha,
a wrong sign in delta, S used before instead of after the update, a transposed
state, a wrong head map, a lost norm term) makes at least one test fail.
"""

import numpy as np
import pytest

from oracle import chunk_fwd, l2norm_rows, recurrent_bwd, recurrent_fwd


def rand_case(rng, lens, H_qk, H_v, d_k, d_v, h0=True, unit=False):
    T = sum(lens)
    q = rng.standard_normal((T, H_qk, d_k))
    k = rng.standard_normal((T, H_qk, d_k))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H_v, d_v))
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, H_v))))
    g = -np.log1p(np.exp(rng.standard_normal((T, H_v))))
    hh = 0.3 * rng.standard_normal((len(lens), H_v, d_k, d_v)) if h0 else None
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return q, k, v, beta, g, hh, cu


# ---------------------------------------------------------------- forward pins

def test_beta_zero_zero_state_gives_zero_output():
    rng = np.random.default_rng(1)
    q, k, v, beta, g, _, cu = rand_case(rng, [7, 5], 2, 4, 8, 6)
    o, hT = recurrent_fwd(q, k, v, 0 * beta, g, cu, h0=None)
    assert np.all(o == 0.0) and np.all(hT == 0.0)


def test_beta_zero_closed_form_pins_state_layout_and_decay():
    # beta = 0: S_t = exp(G_t) S_0, so o_t[j] = exp(G_t) sum_i h0[i][j] qhat_t[i]
    # (h0 stored [d_k][d_v]); written with explicit indices, not matrix helpers.
    rng = np.random.default_rng(2)
    lens, H_qk, H_v, dk, dv = [9], 1, 2, 5, 3
    q, k, v, beta, g, h0, cu = rand_case(rng, lens, H_qk, H_v, dk, dv)
    scale = 0.7
    o, hT = recurrent_fwd(q, k, v, 0 * beta, g, cu, h0=h0, scale=scale)
    qn = q / np.sqrt((q ** 2).sum(-1, keepdims=True) + 1e-6)
    for h in range(H_v):
        G = 0.0
        for t in range(lens[0]):
            G += g[t, h]
            for j in range(dv):
                want = np.exp(G) * sum(h0[0, h, i, j] * scale * qn[t, 0, i] for i in range(dk))
                assert abs(o[t, h, j] - want) < 1e-12
        assert np.allclose(hT[0, h], np.exp(G) * h0[0, h], atol=1e-14, rtol=1e-12)


def test_alpha_zero_resets_state():
    # g = -inf (alpha = 0): S_t = beta_t v_t khat_t^T, o_t = beta_t v_t (khat_t . qhat_t)
    rng = np.random.default_rng(3)
    q, k, v, beta, g, h0, cu = rand_case(rng, [6], 2, 2, 4, 3)
    g[:] = -np.inf
    o, hT = recurrent_fwd(q, k, v, beta, g, cu, h0=h0)
    qn, kn = l2norm_rows(q), l2norm_rows(k)
    for t in range(6):
        for h in range(2):
            want = beta[t, h] * v[t, h] * np.dot(kn[t, h], qn[t, h])
            assert np.allclose(o[t, h], want, atol=1e-14)
    want_T = beta[5, :, None, None] * kn[5][:, :, None] * v[5][:, None, :]
    assert np.allclose(hT[0], want_T, atol=1e-14)


def test_delta_rule_recall_alpha_beta_one_unit_keys():
    # alpha = beta = 1 and q_t = k_t of unit norm: S_t k_t = v_t exactly, so
    # o_t = v_t for ANY unit keys and any initial state (l2norm off: keys exact).
    rng = np.random.default_rng(4)
    q, k, v, beta, g, h0, cu = rand_case(rng, [11, 4], 1, 2, 6, 5, unit=True)
    o, _ = recurrent_fwd(k, k, v, np.ones_like(beta), np.zeros_like(g), cu,
                         h0=h0, qk_l2norm=False)
    assert np.allclose(o, v, atol=1e-12)


def test_orthonormal_keys_recall_earlier_tokens():
    # With distinct basis-vector keys, alpha = beta = 1 and S_0 = 0,
    # S_t = sum_{j<=t} v_j k_j^T, so a query equal to an earlier key k_j reads v_j.
    rng = np.random.default_rng(5)
    d = 8
    T = d
    perm = rng.permutation(d)
    k = np.zeros((T, 1, d))
    k[np.arange(T), 0, perm] = 1.0
    v = rng.standard_normal((T, 1, 3))
    src = np.array([rng.integers(0, t + 1) for t in range(T)])  # earlier token to recall
    q = k[src].copy()
    o, _ = recurrent_fwd(q, k, v, np.ones((T, 1)), np.zeros((T, 1)), [0, T],
                         qk_l2norm=False)
    assert np.allclose(o[:, 0], v[src, 0], atol=1e-13)


def test_linear_in_v_and_h0_jointly():
    rng = np.random.default_rng(6)
    q, k, v, beta, g, h0, cu = rand_case(rng, [8, 3], 2, 4, 5, 4)
    v2 = rng.standard_normal(v.shape)
    h02 = rng.standard_normal(h0.shape)
    c = -1.7
    oa, ha = recurrent_fwd(q, k, v, beta, g, cu, h0=h0)
    ob, hb = recurrent_fwd(q, k, v2, beta, g, cu, h0=h02)
    oc, hc = recurrent_fwd(q, k, v + c * v2, beta, g, cu, h0=h0 + c * h02)
    assert np.allclose(oc, oa + c * ob, atol=1e-12)
    assert np.allclose(hc, ha + c * hb, atol=1e-12)


def test_factored_matrix_form():
    # The defining form S_t = alpha S_{t-1} (I - beta k k^T) + beta v k^T,
    # evaluated as explicit matrix products (the oracle uses the expanded form).
    rng = np.random.default_rng(7)
    q, k, v, beta, g, h0, cu = rand_case(rng, [10], 1, 1, 4, 3)
    o, hT = recurrent_fwd(q, k, v, beta, g, cu, h0=h0)
    qn, kn = l2norm_rows(q), l2norm_rows(k)
    S = h0[0, 0].T
    for t in range(10):
        kk = np.outer(kn[t, 0], kn[t, 0])
        S = np.exp(g[t, 0]) * S @ (np.eye(4) - beta[t, 0] * kk) + beta[t, 0] * np.outer(v[t, 0], kn[t, 0])
        assert np.allclose(o[t, 0], S @ qn[t, 0], atol=1e-13)
    assert np.allclose(hT[0, 0], S.T, atol=1e-13)


def test_dk_one_sum_of_products_closed_form():
    # d_k = 1, keys +-1 (l2norm off): S_t = a_t S_{t-1} + b_t with
    # a_t = alpha_t (1 - beta_t), b_t = beta_t v_t k_t, hence
    # S_T = (prod_t a_t) S_0 + sum_t (prod_{r>t} a_r) b_t.
    rng = np.random.default_rng(8)
    T = 12
    k = rng.choice([-1.0, 1.0], size=(T, 1, 1))
    q = rng.standard_normal((T, 1, 1))
    v = rng.standard_normal((T, 1, 2))
    beta = rng.uniform(0, 1, (T, 1))
    g = -rng.uniform(0, 2, (T, 1))
    h0 = rng.standard_normal((1, 1, 1, 2))
    o, hT = recurrent_fwd(q, k, v, beta, g, [0, T], h0=h0, qk_l2norm=False)
    a = np.exp(g[:, 0]) * (1 - beta[:, 0])
    b = beta[:, 0, None] * v[:, 0] * k[:, 0]
    for t in range(T):
        S = np.prod(a[:t + 1]) * h0[0, 0, 0] + sum(np.prod(a[r + 1:t + 1]) * b[r] for r in range(t + 1))
        assert np.allclose(o[t, 0], S * q[t, 0, 0], atol=1e-13)
    assert np.allclose(hT[0, 0, 0], S, atol=1e-13)


def test_split_invariance():
    rng = np.random.default_rng(9)
    q, k, v, beta, g, h0, cu = rand_case(rng, [13], 2, 4, 6, 5)
    o, hT = recurrent_fwd(q, k, v, beta, g, cu, h0=h0)
    a = 5
    o1, h1 = recurrent_fwd(q[:a], k[:a], v[:a], beta[:a], g[:a], [0, a], h0=h0)
    o2, h2 = recurrent_fwd(q[a:], k[a:], v[a:], beta[a:], g[a:], [0, 13 - a], h0=h1)
    assert np.array_equal(np.concatenate([o1, o2]), o) and np.array_equal(h2, hT)


def test_packed_batch_equals_each_sequence_alone():
    rng = np.random.default_rng(10)
    lens = [4, 0, 9, 2]
    q, k, v, beta, g, h0, cu = rand_case(rng, lens, 1, 2, 4, 4)
    o, hT = recurrent_fwd(q, k, v, beta, g, cu, h0=h0)
    for n in range(len(lens)):
        s, e = cu[n], cu[n + 1]
        on, hn = recurrent_fwd(q[s:e], k[s:e], v[s:e], beta[s:e], g[s:e], [0, e - s], h0=h0[n:n + 1])
        assert np.array_equal(on, o[s:e]) and np.array_equal(hn[0], hT[n])


def test_value_heads_read_their_group_query_key_head():
    # value head h reads q/k head h // (H_v / H_qk): run each value head alone
    # with its q/k head and compare.
    rng = np.random.default_rng(11)
    q, k, v, beta, g, h0, cu = rand_case(rng, [7], 2, 6, 4, 3)
    o, hT = recurrent_fwd(q, k, v, beta, g, cu, h0=h0)
    for h in range(6):
        hq = h // 3
        oh, hh = recurrent_fwd(q[:, hq:hq + 1], k[:, hq:hq + 1], v[:, h:h + 1], beta[:, h:h + 1],
                               g[:, h:h + 1], cu, h0=h0[:, h:h + 1])
        assert np.array_equal(oh[:, 0], o[:, h]) and np.array_equal(hh[:, 0], hT[:, h])


@pytest.mark.parametrize("C", [1, 2, 4, 16])
def test_chunk_algebra_equals_recurrence(C):
    rng = np.random.default_rng(12 + C)
    q, k, v, beta, g, h0, cu = rand_case(rng, [37, 16, 5], 2, 4, 8, 6)
    o, hT = recurrent_fwd(q, k, v, beta, g, cu, h0=h0, scale=0.9)
    oc, hc = chunk_fwd(q, k, v, beta, g, cu, C, h0=h0, scale=0.9)
    assert np.allclose(oc, o, atol=1e-12, rtol=1e-12)
    assert np.allclose(hc, hT, atol=1e-12, rtol=1e-12)


def test_chunk_algebra_c1_has_no_intra_chunk_terms():
    # With C = 1 every chunk is one token, so A is empty and W = beta gam k,
    # U = beta v: the chunk form collapses to one recurrence step per token.
    rng = np.random.default_rng(13)
    q, k, v, beta, g, h0, cu = rand_case(rng, [6], 1, 1, 3, 3)
    o, hT = recurrent_fwd(q, k, v, beta, g, cu, h0=h0)
    oc, hc = chunk_fwd(q, k, v, beta, g, cu, 1, h0=h0)
    assert np.allclose(oc, o, atol=1e-14) and np.allclose(hc, hT, atol=1e-14)


# ---------------------------------------------------------------- gradient pins

def _loss(args, do, dhT, scale):
    q, k, v, beta, g, h0, cu = args
    o, hT = recurrent_fwd(q, k, v, beta, g, cu, h0=h0, scale=scale)
    return np.sum(o * do) + np.sum(hT * dhT)


@pytest.mark.parametrize("l2", [True, False])
def test_gradient_matches_central_finite_differences(l2):
    rng = np.random.default_rng(20 + l2)
    lens = [5, 3]
    q, k, v, beta, g, h0, cu = rand_case(rng, lens, 1, 2, 3, 2)
    do = rng.standard_normal(v.shape)
    dhT = rng.standard_normal(h0.shape)
    scale = 0.8
    grads = recurrent_bwd(q, k, v, beta, g, cu, do, h0=h0, dhT=dhT, scale=scale,
                          qk_l2norm=l2, ckpt=2)
    names = ["q", "k", "v", "beta", "g", "h0"]
    args = [q, k, v, beta, g, h0]

    def loss(a):
        o, hT = recurrent_fwd(a[0], a[1], a[2], a[3], a[4], cu, h0=a[5], scale=scale, qk_l2norm=l2)
        return np.sum(o * do) + np.sum(hT * dhT)

    eps = 1e-6
    for i, name in enumerate(names):
        fd = np.zeros_like(args[i])
        it = np.nditer(args[i], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[i][idx] += eps
            minus[i][idx] -= eps
            fd[idx] = (loss(plus) - loss(minus)) / (2 * eps)
        got = grads["d" + name]
        assert np.allclose(got, fd, atol=1e-7, rtol=1e-6), (name, np.abs(got - fd).max())


def test_checkpoint_interval_does_not_change_gradient():
    rng = np.random.default_rng(30)
    q, k, v, beta, g, h0, cu = rand_case(rng, [9, 4], 1, 2, 3, 3)
    do = rng.standard_normal(v.shape)
    a = recurrent_bwd(q, k, v, beta, g, cu, do, h0=h0, ckpt=1)
    b = recurrent_bwd(q, k, v, beta, g, cu, do, h0=h0, ckpt=64)
    for key in a:
        assert np.allclose(a[key], b[key], atol=1e-13), key


def test_dv_exact_by_linearity_and_zero_for_beta_zero():
    # o is linear in v, so <dv, e> = <dO, o(v + e) - o(v)> exactly (up to rounding).
    rng = np.random.default_rng(31)
    q, k, v, beta, g, h0, cu = rand_case(rng, [6], 1, 2, 4, 3)
    do = rng.standard_normal(v.shape)
    e = rng.standard_normal(v.shape)
    dv = recurrent_bwd(q, k, v, beta, g, cu, do, h0=h0)["dv"]
    o0, _ = recurrent_fwd(q, k, v, beta, g, cu, h0=h0)
    o1, _ = recurrent_fwd(q, k, v + e, beta, g, cu, h0=h0)
    assert abs(np.sum(dv * e) - np.sum(do * (o1 - o0))) < 1e-10
    dv0 = recurrent_bwd(q, k, v, 0 * beta, g, cu, do, h0=h0)["dv"]
    assert np.all(dv0 == 0.0)


# ---------------------------------------------------------------- normalisation pins

def test_l2norm_unit_length_for_large_vectors_and_below_one_always():
    # |x|^2 >> eps: the result has length 1 up to eps / (2 |x|^2); eps > 0 added
    # inside the root makes every length strictly below 1.
    rng = np.random.default_rng(40)
    x = rng.standard_normal((50, 7)) * rng.uniform(0.5, 50.0, (50, 1))
    n = np.linalg.norm(l2norm_rows(x), axis=-1)
    sq = np.sum(x * x, axis=-1)
    assert np.all(n < 1.0)
    assert np.all(np.abs(1.0 - n) <= 1e-6 / (2 * sq) + 1e-15)


def test_l2norm_keeps_direction_and_is_scale_invariant_up_to_eps():
    # positive multiple of x; l2norm(c x) differs from l2norm(x) only through
    # eps, by at most |1/c^2 - 1| eps / (2 |x|^2) relative, and grows with c
    rng = np.random.default_rng(41)
    x = rng.standard_normal((20, 5))
    y = l2norm_rows(x)
    ratio = y / x
    assert np.all(ratio > 0) and np.allclose(ratio, ratio[:, :1], rtol=1e-14, atol=0)
    sq = np.sum(x * x, axis=-1, keepdims=True)
    for c in [0.5, 3.0, 1e3]:
        yc = l2norm_rows(c * x)
        bound = abs(1.0 / c ** 2 - 1.0) * 1e-6 / (2 * sq) + 1e-14
        assert np.all(np.abs(yc - y) <= bound * np.abs(y))
        if c > 1:
            assert np.all(np.linalg.norm(yc, axis=-1) > np.linalg.norm(y, axis=-1))


def test_l2norm_small_vectors_scale_by_inverse_root_eps():
    # |x|^2 << eps: the result is x / sqrt(eps) (1e3 x), not a unit vector
    x = np.array([[3e-9, -4e-9, 1e-9]])
    y = l2norm_rows(x)
    assert np.allclose(y, 1e3 * x, rtol=1e-10, atol=0)


def test_l2norm_exact_where_the_root_is_exact():
    # |x|^2 + eps = 1/4 exactly gives y = 2 x; rows are normalised separately
    a = np.sqrt(0.25 - 1e-6)
    x = np.array([[a, 0.0, 0.0], [0.0, 0.0, -a], [3.0, 4.0, 0.0]])
    y = l2norm_rows(x)
    assert np.allclose(y[0], [2 * a, 0, 0], rtol=1e-15, atol=0)
    assert np.allclose(y[1], [0, 0, -2 * a], rtol=1e-15, atol=0)
    assert abs(np.linalg.norm(y[2]) - 5.0 / np.sqrt(25.0 + 1e-6)) < 1e-15
