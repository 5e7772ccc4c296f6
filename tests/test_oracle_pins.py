"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Every test here checks the oracle against something other than its own code:
closed forms, textbook special cases, invariants, an optimisation identity
evaluated by finite differences, or a second algebraic form.  Each is chosen
so that a plausible slip in the oracle (a dropped term, a sign, the decay
applied after the write instead of before, a transposed state, a readout taken
before the update, a per-head / per-sequence indexing error) fails at least one.
"""
import math

import numpy as np
import pytest

from oracle import oracle
from tests.chunkwise_fp64 import chunkwise_fwd


def rnd(seed, B=1, T=24, H=2, DK=8, DV=6, g_lo=1e-3, g_hi=0.5, state=True, normalise=True):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, T, H, DK))
    k = r.standard_normal((B, T, H, DK))
    if normalise:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, T, H, DV))
    g = -np.exp(r.uniform(math.log(g_lo), math.log(g_hi), (B, T, H, DK)))
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal((B, T, H))))
    S0 = 0.3 * r.standard_normal((B, H, DK, DV)) if state else None
    return q, k, v, g, beta, S0


SCALE = 0.37


# --- closed forms ------------------------------------------------------------

def test_beta_zero_is_pure_per_channel_decay():
    """beta = 0: S_T = Diag(exp(sum g)) S0 and o_t = scale (Diag(exp(G_t)) S0)^T q_t
    (the write term vanishes; only the diagonal gate acts) [core.today ch.4 혁신 1/2]."""
    q, k, v, g, beta, S0 = rnd(1)
    beta[:] = 0.0
    o, S = oracle.fwd(q, k, v, g, beta, SCALE, S0)
    G = np.cumsum(g, axis=1)                                   # [B, T, H, DK]
    decayed = np.exp(G)[..., None] * S0[:, None]               # [B, T, H, DK, DV]
    o_ref = SCALE * np.einsum("bthij,bthi->bthj", decayed, q)
    S_ref = np.exp(G[:, -1])[..., None] * S0
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S, S_ref, rtol=1e-12, atol=1e-14)


def test_beta_zero_unit_gate_leaves_state_unchanged():
    """beta = 0, alpha = 1: S never changes and o_t = scale S0^T q_t, a plain GEMV."""
    q, k, v, g, beta, S0 = rnd(2)
    beta[:] = 0.0
    g[:] = 0.0
    o, S = oracle.fwd(q, k, v, g, beta, SCALE, S0)
    np.testing.assert_array_equal(S, S0)
    for h in range(q.shape[2]):
        o_ref = SCALE * (q[0, :, h, :] @ S0[0, h])
        np.testing.assert_allclose(o[0, :, h, :], o_ref, rtol=1e-13, atol=1e-15)


def test_single_token_from_zero_state():
    """T = 1, S0 = 0: S_1 = beta k v^T and o = scale beta (k.q) v."""
    q, k, v, g, beta, _ = rnd(3, T=1, H=3)
    o, S = oracle.fwd(q, k, v, g, beta, SCALE, None)
    for h in range(3):
        b, kk, vv, qq = beta[0, 0, h], k[0, 0, h], v[0, 0, h], q[0, 0, h]
        np.testing.assert_allclose(S[0, h], b * np.outer(kk, vv), rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(o[0, 0, h], SCALE * b * (kk @ qq) * vv, rtol=1e-13, atol=1e-15)


def test_single_token_rank_one_delta_step():
    """T = 1 with a state: S_1 - Diag(alpha) S0 is the rank-1 matrix beta k e^T,
    with e = v - (Diag(alpha) S0)^T k [core.today ch.3, delta rule; ch.4 혁신 2]."""
    q, k, v, g, beta, S0 = rnd(4, T=1, H=2)
    _, S = oracle.fwd(q, k, v, g, beta, SCALE, S0)
    for h in range(2):
        Sd = np.exp(g[0, 0, h])[:, None] * S0[0, h]
        D = S[0, h] - Sd
        assert np.linalg.matrix_rank(D, tol=1e-10) == 1
        kk = k[0, 0, h]
        # the column space is spanned by k, and k^T D / (k.k) = beta (v - Sd^T k)
        np.testing.assert_allclose(D, np.outer(kk, kk @ D) / (kk @ kk), atol=1e-13)
        np.testing.assert_allclose(kk @ D / (kk @ kk), beta[0, 0, h] * (v[0, 0, h] - Sd.T @ kk),
                                   rtol=1e-12, atol=1e-14)


# --- textbook special cases --------------------------------------------------

def test_one_hot_keys_reduce_to_gated_linear_attention():
    """Distinct one-hot keys never interfere, so the delta error is v itself and
    KDA becomes causal gated linear attention:
      o_t = scale * sum_{s<=t} beta_s (sum_c q_tc k_sc exp(G_tc - G_sc)) v_s.
    Pins the gate direction, its per-channel action, beta's placement and the
    readout after the update (s = t included)."""
    T, H, DK, DV = 10, 2, 12, 5
    q, _, v, g, beta, _ = rnd(5, T=T, H=H, DK=DK, DV=DV)
    r = np.random.default_rng(55)
    k = np.zeros((1, T, H, DK))
    for h in range(H):
        chans = r.permutation(DK)[:T]
        k[0, np.arange(T), h, chans] = 1.0
    o, S = oracle.fwd(q, k, v, g, beta, SCALE, None)
    G = np.cumsum(g[0], axis=0)                                 # [T, H, DK]
    for h in range(H):
        for t in range(T):
            acc = np.zeros(DV)
            for s in range(t + 1):
                w = np.sum(q[0, t, h] * k[0, s, h] * np.exp(G[t, h] - G[s, h]))
                acc += beta[0, s, h] * w * v[0, s, h]
            np.testing.assert_allclose(o[0, t, h], SCALE * acc, rtol=1e-12, atol=1e-14)
        S_ref = sum(beta[0, s, h] * np.outer(k[0, s, h] * np.exp(G[-1, h] - G[s, h]), v[0, s, h])
                    for s in range(T))
        np.testing.assert_allclose(S[0, h], S_ref, rtol=1e-12, atol=1e-14)


def test_scalar_gate_is_rescaled_deltanet():
    """A gate equal across channels (Gated DeltaNet's scalar decay
    [hnts03 "논문 리뷰: Kimi Delta Attention", section "Kimi Delta Attention"])
    factors out: with P_t = exp(sum_{s<=t} gamma_s),
      S_t = P_t * D_t,  o_t = P_t * o^D_t,
    where D is plain DeltaNet (alpha = 1) run on v_t / P_t from the same S0.
    This fails if the decay is applied after the delta error instead of before."""
    T, H, DK, DV = 20, 2, 8, 6
    q, k, v, _, beta, S0 = rnd(6, T=T, H=H, DK=DK, DV=DV)
    gamma = -np.random.default_rng(66).uniform(0.01, 0.2, (1, T, H))
    g = np.repeat(gamma[..., None], DK, axis=-1)
    o, S = oracle.fwd(q, k, v, g, beta, SCALE, S0)
    P = np.exp(np.cumsum(gamma, axis=1))                        # [1, T, H]
    oD, SD = oracle.fwd(q, k, v / P[..., None], np.zeros_like(g), beta, SCALE, S0)
    np.testing.assert_allclose(o, P[..., None] * oD, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(S, P[:, -1][..., None, None] * SD, rtol=1e-11, atol=1e-13)


def test_update_is_one_sgd_step_on_the_recall_loss():
    """Meta-learning view [core.today ch.9]: after the decay, each token takes one
    gradient step of size beta on L(S) = 0.5 ||S^T k - v||^2.  The gradient is
    taken here by central finite differences (brute force), independently of
    any closed form of the update."""
    T, H, DK, DV = 6, 1, 4, 3
    q, k, v, g, beta, S0 = rnd(7, T=T, H=H, DK=DK, DV=DV)
    S_prev = S0[0, 0]
    for t in range(T):
        _, S_t = oracle.fwd(q[:, :t + 1], k[:, :t + 1], v[:, :t + 1], g[:, :t + 1],
                            beta[:, :t + 1], SCALE, S0)
        Sd = np.exp(g[0, t, 0])[:, None] * S_prev
        kk, vv = k[0, t, 0], v[0, t, 0]

        def loss(S):
            r_ = S.T @ kk - vv
            return 0.5 * float(r_ @ r_)

        grad = np.zeros_like(Sd)
        h = 1e-6
        for i in range(DK):
            for j in range(DV):
                Sp, Sm = Sd.copy(), Sd.copy()
                Sp[i, j] += h
                Sm[i, j] -= h
                grad[i, j] = (loss(Sp) - loss(Sm)) / (2 * h)
        np.testing.assert_allclose(S_t[0, 0], Sd - beta[0, t, 0] * grad, rtol=1e-7, atol=1e-8)
        S_prev = S_t[0, 0]


def test_write_then_read_recovers_value():
    """beta = 1 with unit keys: right after writing (k_t, v_t), reading with k_t
    returns v_t exactly (the delta rule stores the error, not the value)."""
    T, H, DK, DV = 12, 2, 8, 5
    q, k, v, g, beta, S0 = rnd(8, T=T, H=H, DK=DK, DV=DV)
    beta[:] = 1.0
    for t in (0, 3, T - 1):
        _, S = oracle.fwd(q[:, :t + 1], k[:, :t + 1], v[:, :t + 1], g[:, :t + 1],
                          beta[:, :t + 1], SCALE, S0)
        for h in range(H):
            np.testing.assert_allclose(S[0, h].T @ k[0, t, h], v[0, t, h], rtol=1e-12, atol=1e-13)


def test_literal_transition_matrix_form_agrees():
    """The bracketed d_k x d_k transition of the update equation, formed
    explicitly, agrees with the decay-then-delta evaluation."""
    q, k, v, g, beta, S0 = rnd(9, B=2, T=16, H=2, DK=6, DV=4, normalise=False)
    o1, S1 = oracle.fwd(q, k, v, g, beta, SCALE, S0)
    o2, S2 = oracle.fwd(q, k, v, g, beta, SCALE, S0, literal=True)
    np.testing.assert_allclose(o1, o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S1, S2, rtol=1e-11, atol=1e-12)


# --- invariants ----------------------------------------------------------------

def test_linear_in_values_and_initial_state():
    q, k, v1, g, beta, S1 = rnd(10)
    _, _, v2, _, _, S2 = rnd(11)
    a, b = 0.7, -1.9
    o1, F1 = oracle.fwd(q, k, v1, g, beta, SCALE, S1)
    o2, F2 = oracle.fwd(q, k, v2, g, beta, SCALE, S2)
    o3, F3 = oracle.fwd(q, k, a * v1 + b * v2, g, beta, SCALE, a * S1 + b * S2)
    np.testing.assert_allclose(o3, a * o1 + b * o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(F3, a * F1 + b * F2, rtol=1e-11, atol=1e-12)


def test_value_columns_are_independent():
    """Permuting v's channels and S0's columns permutes o's and S_T's columns."""
    q, k, v, g, beta, S0 = rnd(12, DV=7)
    perm = np.random.default_rng(0).permutation(7)
    o, S = oracle.fwd(q, k, v, g, beta, SCALE, S0)
    op, Sp = oracle.fwd(q, k, v[..., perm], g, beta, SCALE, S0[..., perm])
    np.testing.assert_array_equal(op, o[..., perm])
    np.testing.assert_array_equal(Sp, S[..., perm])


def test_causal():
    q, k, v, g, beta, S0 = rnd(13, T=30)
    o, _ = oracle.fwd(q, k, v, g, beta, SCALE, S0)
    t = 17
    r = np.random.default_rng(1)
    q2, k2, v2, g2, b2 = q.copy(), k.copy(), v.copy(), g.copy(), beta.copy()
    for x in (q2, k2, v2, g2):
        x[:, t + 1:] += r.standard_normal(x[:, t + 1:].shape)
    b2[:, t + 1:] = r.uniform(0, 1, b2[:, t + 1:].shape)
    o2, _ = oracle.fwd(q2, k2, v2, g2, b2, SCALE, S0)
    np.testing.assert_array_equal(o2[:, :t + 1], o[:, :t + 1])
    assert np.abs(o2[:, t + 1:] - o[:, t + 1:]).max() > 1e-3


def test_state_handoff_equals_one_run():
    """Running the second half from the first half's final state reproduces the
    whole run (the pages' initial/final state arguments
    [trend.ondo.sh "MoonshotAI/FlashKDA", section "커널 API와 제약 조건"])."""
    q, k, v, g, beta, S0 = rnd(14, B=2, T=40)
    o, S = oracle.fwd(q, k, v, g, beta, SCALE, S0)
    for cut in (20, 13):
        oa, Sa = oracle.fwd(q[:, :cut], k[:, :cut], v[:, :cut], g[:, :cut], beta[:, :cut],
                            SCALE, S0)
        ob, Sb = oracle.fwd(q[:, cut:], k[:, cut:], v[:, cut:], g[:, cut:], beta[:, cut:],
                            SCALE, Sa)
        np.testing.assert_array_equal(np.concatenate([oa, ob], axis=1), o)
        np.testing.assert_array_equal(Sb, S)


def test_varlen_packing_equals_separate_runs():
    """Packed sequences with cu_seqlens (B = 1) equal separate runs, including a
    zero-length sequence (which returns its initial state)."""
    lengths = [7, 0, 19, 1, 13]
    T = sum(lengths)
    q, k, v, g, beta, _ = rnd(15, T=T)
    S0 = 0.3 * np.random.default_rng(3).standard_normal((len(lengths), 2, 8, 6))
    cu = np.concatenate([[0], np.cumsum(lengths)])
    o, S = oracle.fwd(q, k, v, g, beta, SCALE, S0, cu_seqlens=cu)
    for n, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        on, Sn = oracle.fwd(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b], SCALE,
                            S0[n:n + 1])
        np.testing.assert_array_equal(o[:, a:b], on)
        np.testing.assert_array_equal(S[n], Sn[0])
    np.testing.assert_array_equal(S[1], S0[1])


def test_head_subset_matches_full_run():
    q, k, v, g, beta, S0 = rnd(16, H=4)
    o, S = oracle.fwd(q, k, v, g, beta, SCALE, S0)
    o2, S2 = oracle.fwd(q, k, v, g, beta, SCALE, S0, heads=[3, 1])
    for h in (1, 3):
        np.testing.assert_array_equal(o2[:, :, h], o[:, :, h])
        np.testing.assert_array_equal(S2[:, h], S[:, h])
    assert not o2[:, :, 0].any() and not o2[:, :, 2].any()


def test_transition_is_non_expansive():
    """With unit keys, beta in [0, 1] and alpha in (0, 1], the transition
    (I - beta k k^T) Diag(alpha) has spectral norm <= 1, so
    ||S_t||_2 <= ||S_{t-1}||_2 + beta_t ||v_t||."""
    T, DK, DV = 25, 8, 6
    q, k, v, g, beta, S0 = rnd(17, T=T, H=1, DK=DK, DV=DV)
    prev = np.linalg.norm(S0[0, 0], 2)
    for t in range(T):
        _, S = oracle.fwd(q[:, :t + 1], k[:, :t + 1], v[:, :t + 1], g[:, :t + 1],
                          beta[:, :t + 1], SCALE, S0)
        cur = np.linalg.norm(S[0, 0], 2)
        assert cur <= prev + beta[0, t, 0] * np.linalg.norm(v[0, t, 0]) + 1e-12
        prev = cur


# --- the chunk algebra the kernels implement -----------------------------------

@pytest.mark.parametrize("C", [1, 16, 32, 64])
def test_chunkwise_algebra_matches_token_serial(C):
    """The WY/UT chunkwise evaluation at chunk size C (any C; the kernels use 64)
    equals the token-serial recurrence; T = 200 leaves a partial last chunk."""
    T, DK, DV = 200, 16, 8
    q, k, v, g, beta, S0 = rnd(18, T=T, H=1, DK=DK, DV=DV)
    o, S = oracle.fwd(q, k, v, g, beta, SCALE, S0)
    oc, Sc = chunkwise_fwd(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0], SCALE,
                           S0[0, 0], C)
    np.testing.assert_allclose(oc, o[0, :, 0], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(Sc, S[0, 0], rtol=1e-10, atol=1e-12)


def test_full_head_dim_chunkwise_on_tiny_workload():
    """d = 128, C = 64 on the tiny workload's distributions (T = 256, 4 chunks)."""
    from linear_attention_kda_amd.workloads import make_inputs
    x = make_inputs(0, "cpu")
    o, S = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"], None)
    f = lambda t: t[0, :, 0].double().numpy()  # noqa: E731
    oc, Sc = chunkwise_fwd(f(x["q"]), f(x["k"]), f(x["v"]), f(x["g"]),
                           x["beta"][0, :, 0].double().numpy(), x["scale"], None, 64)
    np.testing.assert_allclose(oc, o[0, :, 0], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(Sc, S[0, 0], rtol=1e-9, atol=1e-12)


def test_column_block_tasks_are_bitwise_identical():
    q, k, v, g, beta, S0 = rnd(19, B=2, T=33, H=3, DV=10)
    o, S = oracle.fwd(q, k, v, g, beta, SCALE, S0)
    for cb in (1, 3, 4):
        o2, S2 = oracle.fwd(q, k, v, g, beta, SCALE, S0, col_block=cb)
        np.testing.assert_array_equal(o2, o)
        np.testing.assert_array_equal(S2, S)


# --- scalar-gate (Gated DeltaNet) oracle ----------------------------------------

def rnd_scalar_gate(seed, B=1, T=24, H=2, DK=8, DV=6):
    q, k, v, _, beta, S0 = rnd(seed, B=B, T=T, H=H, DK=DK, DV=DV)
    gamma = -np.random.default_rng(seed + 1000).uniform(0.01, 0.4, (B, T, H))
    return q, k, v, gamma, beta, S0


def test_gdn_literal_scalar_transition():
    """Brute force in numpy: S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
    o_t = scale S_t^T q_t, with one scalar decay per token and head
    [core.today "Kimi Linear 특집", ch.4 혁신 1; hnts03 "논문 리뷰: Kimi Delta
    Attention", section "Kimi Delta Attention"]."""
    T, H, DK, DV = 15, 2, 5, 4
    q, k, v, gamma, beta, S0 = rnd_scalar_gate(31, T=T, H=H, DK=DK, DV=DV)
    o, S = oracle.gdn_fwd(q, k, v, gamma, beta, SCALE, S0)
    for h in range(H):
        St = S0[0, h].copy()
        for t in range(T):
            kk = k[0, t, h]
            A = math.exp(gamma[0, t, h]) * (np.eye(DK) - beta[0, t, h] * np.outer(kk, kk))
            St = A @ St + beta[0, t, h] * np.outer(kk, v[0, t, h])
            np.testing.assert_allclose(o[0, t, h], SCALE * St.T @ q[0, t, h], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(S[0, h], St, rtol=1e-12, atol=1e-13)


def test_gdn_is_kda_with_the_gate_repeated_over_channels():
    """The per-channel gate of KDA generalises the scalar one: the KDA oracle fed
    the same gate on every channel gives the scalar-gate result (the two oracle
    functions are separate loops)."""
    q, k, v, gamma, beta, S0 = rnd_scalar_gate(32, B=2, T=21, H=3, DK=8, DV=6)
    o1, S1 = oracle.gdn_fwd(q, k, v, gamma, beta, SCALE, S0)
    o2, S2 = oracle.fwd(q, k, v, np.repeat(gamma[..., None], 8, axis=-1), beta, SCALE, S0)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S1, S2, rtol=1e-12, atol=1e-14)


def test_gdn_beta_zero_is_pure_scalar_decay():
    """beta = 0: o_t = scale exp(sum_{s<=t} g_s) S0^T q_t and S_T = exp(sum g) S0."""
    T, H, DK, DV = 17, 2, 6, 5
    q, k, v, gamma, beta, S0 = rnd_scalar_gate(33, T=T, H=H, DK=DK, DV=DV)
    beta[:] = 0.0
    o, S = oracle.gdn_fwd(q, k, v, gamma, beta, SCALE, S0)
    P = np.exp(np.cumsum(gamma, axis=1))
    for h in range(H):
        for t in range(T):
            np.testing.assert_allclose(o[0, t, h], SCALE * P[0, t, h] * (S0[0, h].T @ q[0, t, h]),
                                       rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(S[0, h], P[0, -1, h] * S0[0, h], rtol=1e-12, atol=1e-14)


def test_gdn_varlen_packing_equals_separate_runs():
    lens = [5, 0, 9, 3]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q, k, v, gamma, beta, _ = rnd_scalar_gate(34, T=T, H=2)
    S0 = 0.2 * np.random.default_rng(35).standard_normal((len(lens), 2, 8, 6))
    o, S = oracle.gdn_fwd(q, k, v, gamma, beta, SCALE, S0, cu_seqlens=cu)
    for n in range(len(lens)):
        sl = slice(int(cu[n]), int(cu[n + 1]))
        on, Sn = oracle.gdn_fwd(q[:, sl], k[:, sl], v[:, sl], gamma[:, sl], beta[:, sl], SCALE,
                                S0[n:n + 1])
        np.testing.assert_allclose(o[:, sl], on, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(S[n], Sn[0], rtol=1e-13, atol=1e-15)


# --- backward oracle ---------------------------------------------------------------

def _loss(o, S, Wo, WS):
    return float((o * Wo).sum() + (S * WS).sum())


def _fd_grad(f, x, h=1e-6):
    """Central finite differences of scalar f over every entry of array x."""
    gr = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        old = x[idx]
        x[idx] = old + h
        fp = f()
        x[idx] = old - h
        fm = f()
        x[idx] = old
        gr[idx] = (fp - fm) / (2 * h)
    return gr


@pytest.mark.parametrize("varlen", [False, True])
def test_backward_matches_finite_differences(varlen):
    """Brute force: every gradient of L = <o, Wo> + <S_final, WS> against central
    finite differences of the forward oracle, on tiny shapes (an independent
    evaluation of the derivative of the printed recurrence)."""
    DK, DV, H = 4, 3, 2
    if varlen:
        lens = [3, 0, 4]
        cu = np.concatenate([[0], np.cumsum(lens)])
        B, T, N = 1, int(cu[-1]), len(lens)
    else:
        cu, B, T, N = None, 2, 4, 2
    q, k, v, g, beta, _ = rnd(40 + varlen, B=B, T=T, H=H, DK=DK, DV=DV, g_lo=0.05, g_hi=0.8)
    S0 = 0.3 * np.random.default_rng(41).standard_normal((N, H, DK, DV))
    r = np.random.default_rng(42)
    Wo = r.standard_normal(v.shape)
    WS = r.standard_normal(S0.shape)
    gr = oracle.bwd(q, k, v, g, beta, SCALE, Wo, S0, WS, cu_seqlens=cu)

    def L():
        o, S = oracle.fwd(q, k, v, g, beta, SCALE, S0, cu_seqlens=cu)
        return _loss(o, S, Wo, WS)

    for name, x in (("dq", q), ("dk", k), ("dv", v), ("dg", g), ("dbeta", beta), ("dS0", S0)):
        np.testing.assert_allclose(gr[name], _fd_grad(L, x), rtol=1e-6, atol=1e-8, err_msg=name)


def test_backward_without_final_state_gradient_and_state():
    """dS_final = None and S0 = None: the gradient of <o, Wo> alone from a zero
    state (checked by finite differences on the inputs that still matter)."""
    DK, DV, H, T = 3, 2, 1, 5
    q, k, v, g, beta, _ = rnd(43, T=T, H=H, DK=DK, DV=DV)
    Wo = np.random.default_rng(44).standard_normal(v.shape)
    gr = oracle.bwd(q, k, v, g, beta, SCALE, Wo)

    def L():
        o, _ = oracle.fwd(q, k, v, g, beta, SCALE, None)
        return float((o * Wo).sum())

    for name, x in (("dq", q), ("dk", k), ("dv", v), ("dg", g), ("dbeta", beta)):
        np.testing.assert_allclose(gr[name], _fd_grad(L, x), rtol=1e-6, atol=1e-8, err_msg=name)
