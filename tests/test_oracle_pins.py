"""Pins the fp64 oracle to facts the pages and the mathematics fix (CPU only).

Each test names the passage or the closed form it checks.  None of them
re-types the oracle's own formula: they use hand-derived closed forms, special
cases, invariants, finite differences and a worked example from the pages.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
RNG = np.random.default_rng(12345)


def _rand(*shape):
    return RNG.standard_normal(shape)


# ---------------------------------------------------------------------------
# Worked example: FlashAttention-2 review, 'core algorithm' answer, section 3.
# ---------------------------------------------------------------------------
def _example():
    with open(os.path.join(HERE, "golden", "worked_example.json")) as f:
        ex = json.load(f)
    return ex, np.array(ex["Q"], float), np.array(ex["K"], float), np.array(ex["V"], float)


def _example_closed_form(scale, causal, N=4):
    """q_i.k_j = 8ij + 6i + 6j + 4 and V_j = (j+1)(1,1): derived by hand from the page's inputs."""
    O, LSE = [], []
    for i in range(N):
        a = scale * (8 * i + 6)
        js = range(i + 1) if causal else range(N)
        top = max(a * j for j in js)
        w = [math.exp(a * j - top) for j in js]
        O.append(sum((j + 1) * wj for j, wj in zip(js, w)) / sum(w))
        LSE.append(scale * (6 * i + 4) + top + math.log(sum(w)))
    return np.array(O), np.array(LSE)


@pytest.mark.parametrize("scale", [1.0, 1.0 / math.sqrt(2.0)])
@pytest.mark.parametrize("causal", [False, True])
def test_worked_example_closed_form(scale, causal):
    ex, Q, K, V = _example()
    O, LSE = oracle.fwd(Q, K, V, scale=scale, causal=causal)
    O_ref, LSE_ref = _example_closed_form(scale, causal)
    np.testing.assert_allclose(O[:, 0], O_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(O[:, 1], O_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(LSE, LSE_ref, rtol=0, atol=1e-12)


def test_worked_example_block_scores():
    """S_11 = Q_1 K_1^T of the 2x2 blocking: recover S from P and LSE (S_ij = ln P_ij + LSE_i)."""
    ex, Q, K, V = _example()
    O, LSE, P = oracle.fwd_probs(Q, K, V, scale=ex["scale_on_page"], causal=False)
    S = np.log(P) + LSE[:, None]
    np.testing.assert_allclose(S[0, :2], ex["S11_row0_printed"], atol=1e-9)
    np.testing.assert_allclose(S[1, :2], ex["S11_row1_definition"], atol=1e-9)
    assert not np.allclose(S[1, :2], ex["S11_row1_printed"])


def test_default_scale_is_inverse_sqrt_d():
    """'IO-4 FlashAttention' problem setup: softmax(QK^T / sqrt(d_k)) V."""
    ex, Q, K, V = _example()
    O_def, L_def = oracle.fwd(Q, K, V)
    O_ref, L_ref = _example_closed_form(1 / math.sqrt(2), False)
    np.testing.assert_allclose(L_def, L_ref, atol=1e-12)
    np.testing.assert_allclose(O_def[:, 0], O_ref, atol=1e-12)


# ---------------------------------------------------------------------------
# Forward special cases and invariants.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_P_sum_to_one(causal):
    q, k, v = _rand(37, 8), _rand(37, 8), _rand(37, 8)
    O, LSE, P = oracle.fwd_probs(q, k, v, causal=causal)
    np.testing.assert_allclose(P.sum(1), 1.0, atol=1e-15 * 37)
    assert (P >= 0).all()
    if causal:
        assert (np.triu(P, 1) == 0).all()
    np.testing.assert_allclose(O, P @ v, atol=1e-13)     # O is a convex combination of V rows


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_average_values(causal):
    """Q = 0 gives uniform weights: O_i = mean of the allowed V_j, LSE_i = ln(#allowed)."""
    N, d = 23, 6
    q, k, v = np.zeros((N, d)), _rand(N, d), _rand(N, d)
    O, LSE = oracle.fwd(q, k, v, causal=causal)
    for i in range(N):
        n = i + 1 if causal else N
        np.testing.assert_allclose(O[i], v[:n].mean(0), atol=1e-14)
        assert abs(LSE[i] - math.log(n)) < 1e-14


def test_causal_first_row():
    """Row 0 under the causal mask sees only key 0: O_0 = V_0, LSE_0 = scale q_0.k_0."""
    N, d = 19, 7
    q, k, v = _rand(N, d), _rand(N, d), _rand(N, d)
    O, LSE = oracle.fwd(q, k, v, scale=0.3, causal=True)
    np.testing.assert_allclose(O[0], v[0], atol=1e-15)
    assert abs(LSE[0] - 0.3 * float(q[0] @ k[0])) < 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_single_key(causal):
    q, k, v = _rand(1, 5), _rand(1, 5), _rand(1, 5)
    O, LSE = oracle.fwd(q, k, v, scale=0.7, causal=causal)
    np.testing.assert_allclose(O, v, atol=1e-15)
    assert abs(LSE[0] - 0.7 * float(q[0] @ k[0])) < 1e-14


def test_constant_values():
    N, d = 17, 4
    q, k = _rand(N, d), _rand(N, d)
    v = np.full((N, d), -2.5)
    for causal in (False, True):
        O, _ = oracle.fwd(q, k, v, causal=causal)
        np.testing.assert_allclose(O, -2.5, atol=1e-14)


def test_two_keys_sigmoid():
    """N = 2, d = 1: the softmax over two scores is the logistic function of their difference."""
    q, k, v = np.array([[0.9], [-1.3]]), np.array([[0.4], [2.0]]), np.array([[3.0], [-1.0]])
    s = 0.8
    O, LSE = oracle.fwd(q, k, v, scale=s, causal=False)
    for i in range(2):
        s0, s1 = s * q[i, 0] * k[0, 0], s * q[i, 0] * k[1, 0]
        p0 = 1.0 / (1.0 + math.exp(s1 - s0))
        assert abs(O[i, 0] - (p0 * 3.0 + (1 - p0) * -1.0)) < 1e-15
        assert abs(LSE[i] - (max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))))) < 1e-14
    Oc, Lc = oracle.fwd(q, k, v, scale=s, causal=True)
    s10, s11 = s * q[1, 0] * k[0, 0], s * q[1, 0] * k[1, 0]
    p10 = 1.0 / (1.0 + math.exp(s11 - s10))
    assert abs(Oc[1, 0] - (p10 * 3.0 + (1 - p10) * -1.0)) < 1e-15
    assert abs(Oc[0, 0] - 3.0) < 1e-15


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    """K_j -> K_j + u shifts every score of row i by scale q_i.u: O unchanged, LSE_i + scale q_i.u."""
    N, d, s = 21, 5, 0.45
    q, k, v, u = _rand(N, d), _rand(N, d), _rand(N, d), _rand(d)
    O1, L1 = oracle.fwd(q, k, v, scale=s, causal=causal)
    O2, L2 = oracle.fwd(q, k + u, v, scale=s, causal=causal)
    np.testing.assert_allclose(O2, O1, atol=1e-12)
    np.testing.assert_allclose(L2, L1 + s * (q @ u), atol=1e-12)


def test_permutation_equivariance():
    N, d = 29, 6
    q, k, v = _rand(N, d), _rand(N, d), _rand(N, d)
    O, L = oracle.fwd(q, k, v, causal=False)
    pk = RNG.permutation(N)
    O2, L2 = oracle.fwd(q, k[pk], v[pk], causal=False)     # keys and values moved together
    np.testing.assert_allclose(O2, O, atol=1e-13)
    np.testing.assert_allclose(L2, L, atol=1e-13)
    pq = RNG.permutation(N)
    O3, L3 = oracle.fwd(q[pq], k, v, causal=False)          # queries permute the output rows
    np.testing.assert_allclose(O3, O[pq], atol=1e-13)
    np.testing.assert_allclose(L3, L[pq], atol=1e-13)


def test_dominant_key():
    """A score gap of 60 puts all but exp(-60) of the weight on one key."""
    N, d = 9, 3
    q = np.zeros((N, d)); q[:, 0] = 1.0
    k = np.zeros((N, d)); k[4, 0] = 60.0
    v = _rand(N, d)
    O, LSE = oracle.fwd(q, k, v, scale=1.0)
    np.testing.assert_allclose(O, np.repeat(v[4:5], N, 0), atol=1e-20)
    np.testing.assert_allclose(LSE, 60.0 + math.log1p((N - 1) * math.exp(-60)), atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("blocks", [(1, 1), (2, 2), (3, 5), (64, 64), (7, 1)])
def test_online_recurrence_matches_naive(causal, blocks):
    """FlashAttention-2 review, 'core algorithm' answer, section 2 (2) item 2; IO-4 note section 4:
    the tiled running-max / running-sum recurrence reaches the plain softmax result."""
    N, d = 41, 8
    q, k, v = _rand(2, N, d) * 2, _rand(2, N, d) * 2, _rand(2, N, d)
    O, L = oracle.fwd(q, k, v, causal=causal)
    Br, Bc = blocks
    O2, L2 = oracle.fwd_online(q, k, v, causal=causal, Br=Br, Bc=Bc)
    np.testing.assert_allclose(O2, O, atol=1e-13)
    np.testing.assert_allclose(L2, L, atol=1e-13)


def test_online_recurrence_large_scores():
    """Scores near 700 overflow exp() unless the running max is subtracted; both modes must survive."""
    N, d = 16, 2
    q = np.ones((N, d)) * 20.0
    k = _rand(N, d) * 20.0
    v = _rand(N, d)
    O, L = oracle.fwd(q, k, v, scale=1.0, causal=True)
    O2, L2 = oracle.fwd_online(q, k, v, scale=1.0, causal=True, Br=3, Bc=4)
    assert np.isfinite(O).all() and np.isfinite(L).all()
    np.testing.assert_allclose(O2, O, atol=1e-12)
    np.testing.assert_allclose(L2, L, rtol=1e-14, atol=1e-12)


# ---------------------------------------------------------------------------
# Backward: finite differences and identities.
# ---------------------------------------------------------------------------
def _loss(q, k, v, do, scale, causal):
    O, _ = oracle.fwd(q, k, v, scale=scale, causal=causal)
    return float((O * do).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_backward_finite_differences(causal):
    """Central differences of L = sum(dO o O) against the analytic dQ, dK, dV."""
    N, d, s, h = 6, 3, 0.7, 1e-5
    q, k, v, do = _rand(N, d), _rand(N, d), _rand(N, d), _rand(N, d)
    dQ, dK, dV = oracle.bwd(q, k, v, do, scale=s, causal=causal)
    for name, x, g in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], do, s, causal)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], do, s, causal)
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_identities(causal):
    N, d = 33, 7
    q, k, v, do = _rand(3, N, d), _rand(3, N, d), _rand(3, N, d), _rand(3, N, d)
    dQ, dK, dV, D, D2 = oracle.bwd(q, k, v, do, causal=causal, return_D=True)
    np.testing.assert_allclose(dK.sum(-2), 0.0, atol=1e-12)          # rows of dS sum to 0
    np.testing.assert_allclose(dV.sum(-2), do.sum(-2), atol=1e-12)   # rows of P sum to 1
    np.testing.assert_allclose(D, D2, atol=1e-12)                     # sum_j P dP = dO . O


def test_backward_zero_queries():
    """Q = 0 (non-causal): uniform P, so dK = scale dS^T Q = 0 and dV_j = mean_i dO_i."""
    N, d = 15, 4
    q, k, v, do = np.zeros((N, d)), _rand(N, d), _rand(N, d), _rand(N, d)
    dQ, dK, dV = oracle.bwd(q, k, v, do, causal=False)
    np.testing.assert_allclose(dK, 0.0, atol=1e-15)
    np.testing.assert_allclose(dV, np.repeat(do.mean(0, keepdims=True), N, 0), atol=1e-14)


def test_backward_causal_last_key():
    """Under the causal mask only the last query sees the last key: dV_{N-1} = P_{N-1,N-1} dO_{N-1}."""
    N, d = 12, 5
    q, k, v, do = _rand(N, d), _rand(N, d), _rand(N, d), _rand(N, d)
    _, _, P = oracle.fwd_probs(q, k, v, causal=True)
    dQ, dK, dV = oracle.bwd(q, k, v, do, causal=True)
    np.testing.assert_allclose(dV[-1], P[-1, -1] * do[-1], atol=1e-14)
    # and the first query sees only key 0, where the softmax is constant: dQ_0 = 0
    np.testing.assert_allclose(dQ[0], 0.0, atol=1e-14)


# ---------------------------------------------------------------------------
# Sampled-row / sampled-column forms used at full size.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_rows_and_cols_match_full(causal):
    N, d = 45, 8
    q, k, v, do = _rand(N, d), _rand(N, d), _rand(N, d), _rand(N, d)
    O, L = oracle.fwd(q, k, v, causal=causal)
    dQ, dK, dV = oracle.bwd(q, k, v, do, causal=causal)
    idx = [0, 1, 7, 44, 30]
    Or, Lr, dQr = oracle.rows(q, k, v, do, idx, causal=causal)
    np.testing.assert_allclose(Or, O[idx], atol=1e-13)
    np.testing.assert_allclose(Lr, L[idx], atol=1e-13)
    np.testing.assert_allclose(dQr, dQ[idx], atol=1e-13)
    dKc, dVc = oracle.cols(q, k, v, do, idx, causal=causal)
    np.testing.assert_allclose(dKc, dK[idx], atol=1e-13)
    np.testing.assert_allclose(dVc, dV[idx], atol=1e-13)


def test_bad_arguments_rejected():
    q = np.zeros((4, 2))
    with pytest.raises(RuntimeError):
        oracle.fwd(q, q, q, scale=float("nan"))
    with pytest.raises(RuntimeError):
        oracle.rows(q, q, q, None, [4])


# ---------------------------------------------------------------------------
# Block-sparse masks: FlashAttention-2 review, 'sparse/hybrid' answer,
# section 3 (1) -- only the kept blocks of the score matrix are computed.
# Special cases that reduce to dense attention on smaller problems, the
# online recurrence, and finite differences.
# ---------------------------------------------------------------------------
def _mask(T, density, seed, empty_rows=()):
    m = (np.random.default_rng(seed).random((T, T)) < density).astype(np.uint8)
    for a in empty_rows:
        m[a] = 0
    return m


@pytest.mark.parametrize("causal", [False, True])
def test_mask_all_kept_is_dense(causal):
    N, d, blk = 23, 5, 4
    q, k, v, do = _rand(2, N, d), _rand(2, N, d), _rand(2, N, d), _rand(2, N, d)
    T = (N + blk - 1) // blk
    ones = np.ones((T, T), np.uint8)
    np.testing.assert_array_equal(oracle.fwd(q, k, v, causal=causal, block_mask=ones, block=blk)[0],
                                  oracle.fwd(q, k, v, causal=causal)[0])
    for a, b in zip(oracle.bwd(q, k, v, do, causal=causal, block_mask=ones, block=blk),
                    oracle.bwd(q, k, v, do, causal=causal)):
        np.testing.assert_array_equal(a, b)


def test_mask_lower_triangle_with_causal_is_causal():
    """A block mask that keeps the blocks on and below the diagonal changes nothing under causal."""
    N, d, blk = 21, 4, 3
    q, k, v, do = _rand(N, d), _rand(N, d), _rand(N, d), _rand(N, d)
    T = (N + blk - 1) // blk
    tri = np.tril(np.ones((T, T), np.uint8))
    O1, L1 = oracle.fwd(q, k, v, causal=True, block_mask=tri, block=blk)
    O2, L2 = oracle.fwd(q, k, v, causal=True)
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(L1, L2)
    # without causal the same mask is a different (block-causal) problem
    O3, _ = oracle.fwd(q, k, v, causal=False, block_mask=tri, block=blk)
    assert np.abs(O3 - O2).max() > 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_mask_block_diagonal_is_independent_segments(causal):
    """A block-diagonal mask splits the sequence into independent attention problems."""
    N, d, blk = 26, 6, 5
    q, k, v, do = _rand(N, d), _rand(N, d), _rand(N, d), _rand(N, d)
    T = (N + blk - 1) // blk
    eye = np.eye(T, dtype=np.uint8)
    O, L = oracle.fwd(q, k, v, causal=causal, block_mask=eye, block=blk)
    dQ, dK, dV = oracle.bwd(q, k, v, do, causal=causal, block_mask=eye, block=blk)
    for a in range(T):
        r = slice(a * blk, min(N, (a + 1) * blk))
        Os, Ls = oracle.fwd(q[r], k[r], v[r], causal=causal)
        gs = oracle.bwd(q[r], k[r], v[r], do[r], causal=causal)
        np.testing.assert_allclose(O[r], Os, atol=1e-13)
        np.testing.assert_allclose(L[r], Ls, atol=1e-13)
        for full, seg in zip((dQ, dK, dV), gs):
            np.testing.assert_allclose(full[r], seg, atol=1e-13)


def test_mask_one_block_per_row_is_dense_on_that_block():
    """Query block a keeps only key block pi(a): dense attention of Q_a on K_pi(a), V_pi(a)."""
    N, d, blk = 24, 4, 6
    q, k, v = _rand(N, d), _rand(N, d), _rand(N, d)
    T = N // blk
    pi = [2, 0, 3, 1]
    m = np.zeros((T, T), np.uint8)
    for a in range(T):
        m[a, pi[a]] = 1
    O, L = oracle.fwd(q, k, v, block_mask=m, block=blk)
    for a in range(T):
        r, c = slice(a * blk, (a + 1) * blk), slice(pi[a] * blk, (pi[a] + 1) * blk)
        # P_a = softmax(scale q_a k_c^T): the dense oracle on a problem whose keys are block c
        Os, Ls = oracle.fwd(q[r], k[c], v[c])
        np.testing.assert_allclose(O[r], Os, atol=1e-13)
        np.testing.assert_allclose(L[r], Ls, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_mask_empty_rows(causal):
    """A query block that keeps no key: O = 0, LSE = -inf, dQ = 0, and it adds nothing to dK, dV."""
    N, d, blk = 20, 4, 4
    q, k, v, do = _rand(N, d), _rand(N, d), _rand(N, d), _rand(N, d)
    T = N // blk
    m = _mask(T, 0.6, 3, empty_rows=(2,))
    m[np.arange(T), np.arange(T)] = 1
    m[2] = 0
    O, L = oracle.fwd(q, k, v, causal=causal, block_mask=m, block=blk)
    r = slice(8, 12)
    assert np.all(O[r] == 0.0) and np.all(np.isneginf(L[r]))
    dQ, dK, dV = oracle.bwd(q, k, v, do, causal=causal, block_mask=m, block=blk)
    assert np.all(dQ[r] == 0.0)
    # the empty rows add nothing to dK, dV: zeroing their dO changes nothing
    do0 = do.copy()
    do0[r] = 0.0
    _, dK0, dV0 = oracle.bwd(q, k, v, do0, causal=causal, block_mask=m, block=blk)
    np.testing.assert_array_equal(dK, dK0)
    np.testing.assert_array_equal(dV, dV0)
    # the other rows are those of the same mask with the empty block row kept on its diagonal
    m2 = m.copy()
    m2[2, 2] = 1
    O2, L2 = oracle.fwd(q, k, v, causal=causal, block_mask=m2, block=blk)
    keep = np.r_[0:8, 12:N]
    np.testing.assert_array_equal(O2[keep], O[keep])
    np.testing.assert_array_equal(L2[keep], L[keep])
    assert np.isfinite(L2[r]).all()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("blocks", [(1, 1), (3, 2), (4, 4)])
def test_mask_online_recurrence_matches_naive(causal, blocks):
    """The tiled online recurrence under a mask (with an empty query block) equals the explicit softmax."""
    N, d, blk = 22, 5, 4
    q, k, v = _rand(N, d), _rand(N, d), _rand(N, d)
    T = (N + blk - 1) // blk
    m = _mask(T, 0.5, 11, empty_rows=(1,))
    O1, L1 = oracle.fwd(q, k, v, causal=causal, block_mask=m, block=blk)
    O2, L2 = oracle.fwd_online(q, k, v, causal=causal, Br=blocks[0], Bc=blocks[1], block_mask=m, block=blk)
    assert np.isfinite(O2).all()
    np.testing.assert_allclose(O2, O1, rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(np.isneginf(L2), np.isneginf(L1))
    fin = np.isfinite(L1)
    np.testing.assert_allclose(L2[fin], L1[fin], rtol=1e-14, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_mask_backward_finite_differences(causal):
    """Central differences of L = sum(dO o O) under a block mask with an empty block row."""
    N, d, s, h, blk = 8, 3, 0.9, 1e-5, 2
    q, k, v, do = _rand(N, d), _rand(N, d), _rand(N, d), _rand(N, d)
    m = np.array([[1, 0, 1, 0], [0, 0, 0, 0], [1, 1, 0, 1], [0, 1, 1, 1]], np.uint8)
    dQ, dK, dV = oracle.bwd(q, k, v, do, scale=s, causal=causal, block_mask=m, block=blk)

    def loss(qq, kk, vv):
        O, _ = oracle.fwd(qq, kk, vv, scale=s, causal=causal, block_mask=m, block=blk)
        return float((O * do).sum())

    for name, x, g in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            args = {"q": q, "k": k, "v": v}
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args[name] = xp
            lp = loss(args["q"], args["k"], args["v"])
            args[name] = xm
            lm = loss(args["q"], args["k"], args["v"])
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
def test_mask_rows_and_cols_match_full(causal):
    N, d, blk = 40, 6, 8
    q, k, v, do = _rand(N, d), _rand(N, d), _rand(N, d), _rand(N, d)
    T = N // blk
    m = _mask(T, 0.5, 5, empty_rows=(3,))
    O, L = oracle.fwd(q, k, v, causal=causal, block_mask=m, block=blk)
    dQ, dK, dV = oracle.bwd(q, k, v, do, causal=causal, block_mask=m, block=blk)
    idx = [0, 9, 25, 39, 17, 30]
    Or, Lr, dQr = oracle.rows(q, k, v, do, idx, causal=causal, block_mask=m, block=blk)
    np.testing.assert_allclose(Or, O[idx], atol=1e-13)
    np.testing.assert_array_equal(np.isneginf(Lr), np.isneginf(L[idx]))
    fin = np.isfinite(L[idx])
    np.testing.assert_allclose(Lr[fin], L[idx][fin], atol=1e-13)
    np.testing.assert_allclose(dQr, dQ[idx], atol=1e-13)
    dKc, dVc = oracle.cols(q, k, v, do, idx, causal=causal, block_mask=m, block=blk)
    np.testing.assert_allclose(dKc, dK[idx], atol=1e-13)
    np.testing.assert_allclose(dVc, dV[idx], atol=1e-13)


def test_mask_shape_checked():
    q = np.zeros((10, 2))
    with pytest.raises(ValueError):
        oracle.fwd(q, q, q, block_mask=np.ones((2, 2)), block=4)       # T = 3
