"""Pins of the fp64 oracle against what the page and the mathematics fix.

Each test checks the oracle against something other than itself: a library
routine (torch SDPA / softmax / elu in float64), exact rationals, brute force
on tiny inputs, the page's printed budget values, or an identity that holds
exactly (ideal factorisation, Eq. 5 bias identity, additivity).
Source: "Residual-Mass Accounting for Partial-KV Decoding" (paperpeel page).
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _sdpa(q, K, V):
    """Textbook softmax attention through torch's SDPA in float64 on the CPU."""
    qt = torch.from_numpy(np.asarray(q, np.float64)).view(1, 1, 1, -1)
    Kt = torch.from_numpy(np.asarray(K, np.float64)).view(1, 1, K.shape[0], -1)
    Vt = torch.from_numpy(np.asarray(V, np.float64)).view(1, 1, V.shape[0], -1)
    return torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt).view(-1).numpy()


def _softmax_over(q, K, V, support):
    s = torch.from_numpy(K[support] @ q / math.sqrt(q.shape[0]))
    p = torch.softmax(s, dim=0)
    return (p @ torch.from_numpy(V[support])).numpy()


def _unit(seed, L=96, d=8, m=6, n_gen=0, bf16=False):
    r = _rng(seed)
    T = L + n_gen
    K = r.standard_normal((T, d)).astype(np.float32)
    V = r.standard_normal((T, d)).astype(np.float32)
    if bf16:
        K = torch.from_numpy(K).bfloat16().float().numpy()
        V = torch.from_numpy(V).bfloat16().float().numpy()
    q = (1.5 * r.standard_normal(d)).astype(np.float32)
    W = (r.standard_normal((m, d)) / math.sqrt(d)).astype(np.float32)
    b = (r.standard_normal(m) / math.sqrt(d)).astype(np.float32)
    return q, K, V, W, b


# ------------------------------------------------------------------ phi
def test_phi_matches_torch_elu_plus_one():
    r = _rng(1)
    x = r.standard_normal((50, 16))
    W = r.standard_normal((12, 16))
    b = r.standard_normal(12)
    z = torch.from_numpy(x) @ torch.from_numpy(W).T + torch.from_numpy(b)
    ref = (torch.nn.functional.elu(z) + 1.0).numpy()
    got = O.phi_features(x, W, b)
    # torch forms elu(z)+1 as expm1(z)+1: equal up to one rounding of the +1
    np.testing.assert_allclose(got, ref, rtol=1e-15, atol=4e-16)
    assert got.shape == (50, 12)


def test_phi_branches_and_positivity():
    W = np.eye(3)
    b = np.zeros(3)
    got = O.phi_features(np.array([[0.0, 1.0, -1.0]]), W, b)[0]
    assert got[0] == 1.0 and got[1] == 2.0
    assert got[2] == pytest.approx(math.exp(-1.0), rel=1e-16)
    big = O.phi_features(np.array([[-30.0, 30.0, -700.0]]), W, b)[0]
    assert (big > 0).all()                      # strictly positive (App. C.1)


# ------------------------------------------------------------------ summaries
def test_summaries_bruteforce_loops():
    r = _rng(2)
    P = r.random((7, 5))          # 7 tokens, m=5 features
    V = r.standard_normal((7, 3))  # d_v = 3 (m != d_v catches a transposed operand)
    S, u = O.summaries(P, V)
    assert S.shape == (5, 3) and u.shape == (5,)
    for f in range(5):
        assert u[f] == pytest.approx(sum(P[i, f] for i in range(7)), rel=1e-15)
        for c in range(3):
            assert S[f, c] == pytest.approx(sum(P[i, f] * V[i, c] for i in range(7)),
                                            rel=1e-13, abs=1e-15)


def test_summaries_additive_over_chunks():
    q, K, V, W, b = _unit(3, L=300, d=16, m=12)
    P = O.phi_features(K, W, b)
    S, u = O.summaries(P, V)
    r = _rng(4)
    cuts = np.sort(r.choice(np.arange(1, 300), size=9, replace=False))
    edges = np.concatenate([[0], cuts, [300]])
    S2 = np.zeros_like(S)
    u2 = np.zeros_like(u)
    for a, c in zip(edges[:-1], edges[1:]):
        Sc, uc = O.summaries(P[a:c], V[a:c])
        S2 += Sc
        u2 += uc
    np.testing.assert_allclose(S2, S, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(u2, u, rtol=1e-13)


# ------------------------------------------------------------------ partition
def test_partition_sets():
    A, M, G = O.partition(20, 3, 4, n_gen=2)
    assert A.tolist() == [0, 1, 2, 16, 17, 18, 19]
    assert M.tolist() == list(range(3, 16))
    assert G.tolist() == [20, 21]
    with pytest.raises(ValueError):
        O.partition(5, 3, 3)


def test_budget_rule_matches_printed_values():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "budget_k.txt"))
            if l.strip() and not l.startswith("#")]
    assert len(rows) == 2
    for frac, L, na, K in rows:
        assert O.budget_K(float(frac), int(L), int(na)) == int(K)


# ------------------------------------------------------------------ top-k
def _bruteforce_topk(q, Kmid, K):
    keys = [(sum((Fraction(float(a)) * Fraction(float(c)) for a, c in zip(q, row)), Fraction(0)), -i)
            for i, row in enumerate(Kmid)]
    order = sorted(range(len(keys)), key=lambda i: keys[i], reverse=True)
    return sorted(order[:K])


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_exact_bruteforce(seed):
    r = _rng(10 + seed)
    n, d = 37, 8
    Kmid = torch.from_numpy(r.standard_normal((n, d)).astype(np.float32)).bfloat16().float().numpy()
    q = r.standard_normal(d).astype(np.float32)
    for K in (0, 1, 5, 18, 36, 37):
        got = O.topk_indices(q, Kmid, K)
        assert got.tolist() == _bruteforce_topk(q, Kmid, K)


def test_topk_planted_ties_go_to_lower_index():
    r = _rng(20)
    n, d = 50, 8
    Kmid = r.standard_normal((n, d)).astype(np.float32)
    q = r.standard_normal(d).astype(np.float32)
    planted = (4.0 * q / np.linalg.norm(q)).astype(np.float32)
    for p in (7, 23, 41):
        Kmid[p] = planted
    assert O.topk_indices(q, Kmid, 2).tolist() == [7, 23]
    assert O.topk_indices(q, Kmid, 3).tolist() == [7, 23, 41]
    assert O.topk_indices(q, Kmid, 2, first_index=4).tolist() == [11, 27]


def test_topk_all_equal_keys():
    Kmid = np.ones((40, 8), np.float32)
    q = np.arange(8, dtype=np.float32)
    assert O.topk_indices(q, Kmid, 6).tolist() == list(range(6))


def test_topk_separates_ties_below_float64_resolution():
    # two keys whose exact scores differ by 2^-120 * (bf16 ulp): float64 rounds
    # both scores to the same value; the exact rational decides.
    d = 8
    q = np.zeros(d, np.float32)
    q[0] = 1.0
    q[1] = np.float32(2.0 ** -120)
    base = np.zeros(d, np.float32)
    base[0] = 1.0
    Kmid = np.tile(base, (5, 1)) * np.float32(0.5)
    Kmid[3] = base
    Kmid[1] = base
    Kmid[1, 1] = np.float32(1.0)     # k1 = k3 + e_1  -> q.k1 = q.k3 + 2^-120
    assert float(Kmid[1] @ q.astype(np.float64)) == float(Kmid[3] @ q.astype(np.float64))
    assert O.topk_indices(q, Kmid, 1).tolist() == [1]
    assert O.topk_indices(q, Kmid, 2).tolist() == [1, 3]


# ------------------------------------------------------------------ decode invariants
def _prefill(K, V, W, b, L, ns, nt):
    _, M, _ = O.partition(L, ns, nt)
    P = O.phi_features(K[M], W, b)
    S, u = O.summaries(P, V[M])
    return P, S, u


@pytest.mark.parametrize("n_gen", [0, 3])
def test_full_retrieval_equals_full_attention(n_gen):
    L, ns, nt = 96, 3, 7
    q, K, V, W, b = _unit(30, L=L, n_gen=n_gen, bf16=True)
    P, S, u = _prefill(K, V, W, b, L, ns, nt)
    f = O.phi_features(q[None], W, b)[0]
    y, idx, _ = O.decode_query(q, f, K, V, P, S, u, L, ns, nt, n_gen, K=L - ns - nt)
    np.testing.assert_allclose(y, _sdpa(q, K[:L + n_gen], V[:L + n_gen]), rtol=0, atol=1e-13)


@pytest.mark.parametrize("Kret", [0, 1, 9, 40])
def test_zero_residual_equals_selection_only(Kret):
    L, ns, nt, n_gen = 96, 3, 7, 2
    q, K, V, W, b = _unit(31, L=L, n_gen=n_gen)
    P, S, u = _prefill(K, V, W, b, L, ns, nt)
    f = np.zeros(P.shape[1])
    y, idx, _ = O.decode_query(q, f, K, V, P, S, u, L, ns, nt, n_gen, K=Kret)
    # exact support from the definitions: sinks, tail, brute-force top-K of M, generated
    sel = [ns + i for i in _bruteforce_topk(q, K[ns:L - nt], Kret)]
    assert idx.tolist() == sel
    E = np.array(list(range(ns)) + sel + list(range(L - nt, L)) + list(range(L, L + n_gen)))
    np.testing.assert_allclose(y, _softmax_over(q.astype(np.float64), K.astype(np.float64),
                                                V.astype(np.float64), E), atol=1e-13)
    y2, _, _ = O.decode_query(q, f, K, V, P, S, u, L, ns, nt, n_gen, K=Kret, variant="topk")
    np.testing.assert_allclose(y2, y, atol=1e-15)


def _codebook_unit(seed, L=80, d=8, C=6, ns=2, nt=5, n_gen=2):
    r = _rng(seed)
    book = (0.7 * r.standard_normal((C, d))).astype(np.float32)
    codes = r.integers(0, C, size=L + n_gen)
    K = book[codes]
    V = r.standard_normal((L + n_gen, d)).astype(np.float32)
    q = r.standard_normal(d).astype(np.float32)
    # ideal factorisation (Eq. 7): phi_k(k) = onehot(code), phi_q(q)_c = e^{q.book_c/sqrt d}
    _, M, _ = O.partition(L, ns, nt)
    Pk = np.eye(C)[codes[M]]
    f = np.exp(book.astype(np.float64) @ q.astype(np.float64) / math.sqrt(d))
    S, u = O.summaries(Pk, V[M])
    return q, K, V, Pk, f, S, u


@pytest.mark.parametrize("Kret", [0, 1, 7, 30, 72, 73])
def test_ideal_factorisation_recovers_full_attention(Kret):
    L, ns, nt, n_gen = 80, 2, 5, 2
    q, K, V, Pk, f, S, u = _codebook_unit(40, L=L, ns=ns, nt=nt, n_gen=n_gen)
    y, _, _ = O.decode_query(q, f, K, V, Pk, S, u, L, ns, nt, n_gen, K=Kret)
    np.testing.assert_allclose(y, _sdpa(q, K, V), rtol=0, atol=1e-12)
    if 0 < Kret < 73:
        # NoSub double-counts the retrieved tokens (§5.2, §7.1) and misses
        y_ns, _, _ = O.decode_query(q, f, K, V, Pk, S, u, L, ns, nt, n_gen, K=Kret,
                                    variant="nosub")
        assert np.abs(y_ns - y).max() > 1e-6


def test_subset_renormalisation_bias_identity():
    # Eq. 5: y_full - y_TopK = Z_R / (Z_E + Z_R) * (y_R - y_TopK), unshifted sums
    L, ns, nt = 96, 3, 7
    q, K, V, W, b = _unit(50, L=L)
    A, M, _ = O.partition(L, ns, nt)
    idx = O.topk_indices(q, K[M], 12, first_index=ns)
    m_star, N_E, Z_E = O.exact_terms(q, K, V, np.concatenate([A, idx]))
    nu_R, Z_R = O.residual_true(q, K, V, L, ns, nt, idx)
    Z_Eu, N_Eu = Z_E * math.exp(m_star), N_E * math.exp(m_star)
    y_topk = N_Eu / Z_Eu
    lhs = _sdpa(q, K[:L], V[:L]) - y_topk
    rhs = Z_R / (Z_Eu + Z_R) * (nu_R / Z_R - y_topk)
    np.testing.assert_allclose(lhs, rhs, atol=1e-13)


def test_direct_residual_equals_summary_minus_retrieved():
    L, ns, nt = 96, 3, 7
    q, K, V, W, b = _unit(60, L=L)
    P, S, u = _prefill(K, V, W, b, L, ns, nt)
    f = O.phi_features(q[None], W, b)[0]
    _, M, _ = O.partition(L, ns, nt)
    idx = O.topk_indices(q, K[M], 11, first_index=ns)
    loc = idx - ns
    nu, z, zk = O.residual_terms(f, P, V[M], S, u, loc, whole_mid_retrieved=False)
    R = np.setdiff1d(np.arange(M.size), loc)
    w = P[R] @ f
    np.testing.assert_allclose(nu, w @ V[M][R].astype(np.float64), rtol=1e-12, atol=1e-12)
    assert z == pytest.approx(w.sum(), rel=1e-13)
    assert zk == pytest.approx((P[loc] @ f).sum(), rel=1e-13)


def test_generated_token_adds_its_exact_term():
    L, ns, nt = 96, 3, 7
    q, K, V, W, b = _unit(70, L=L, n_gen=4)
    A, M, _ = O.partition(L, ns, nt)
    idx = O.topk_indices(q, K[M], 9, first_index=ns)
    base = np.concatenate([A, idx, np.arange(L, L + 2)])
    m1, N1, Z1 = O.exact_terms(q, K, V, base)
    m2, N2, Z2 = O.exact_terms(q, K, V, np.concatenate([base, [L + 2]]))
    s_new = float(K[L + 2].astype(np.float64) @ q.astype(np.float64)) / math.sqrt(8)
    np.testing.assert_allclose(N2 * math.exp(m2), N1 * math.exp(m1) + math.exp(s_new) * V[L + 2].astype(np.float64),
                               rtol=1e-13)
    assert Z2 * math.exp(m2) == pytest.approx(Z1 * math.exp(m1) + math.exp(s_new), rel=1e-14)


def test_sink_and_tail_edges_are_anchors():
    # the last sink and the first tail token carry the two largest scores; with
    # K = 0 and no residual they must still be in the exact support
    L, ns, nt = 40, 3, 4
    q, K, V, W, b = _unit(80, L=L)
    K[ns - 1] = 3.0 * q / np.linalg.norm(q)
    K[L - nt] = 2.5 * q / np.linalg.norm(q)
    P, S, u = _prefill(K, V, W, b, L, ns, nt)
    y, idx, _ = O.decode_query(q, np.zeros(P.shape[1]), K, V, P, S, u, L, ns, nt, 0, K=0)
    E = np.array(list(range(ns)) + list(range(L - nt, L)))
    np.testing.assert_allclose(y, _softmax_over(q.astype(np.float64), K.astype(np.float64),
                                                V.astype(np.float64), E), atol=1e-14)


def test_diagnostics():
    L, ns, nt = 64, 2, 4
    q, K, V, Pk, f, S, u = _codebook_unit(90, L=L, ns=ns, nt=nt, n_gen=0)
    idx = O.topk_indices(q, K[ns:L - nt], 10, first_index=ns)
    _, zr, _ = O.residual_terms(f, Pk, V[ns:L - nt], S, u, idx - ns, whole_mid_retrieved=False)
    _, Z_R = O.residual_true(q, K, V, L, ns, nt, idx)
    assert abs(O.log_partition_error(zr, Z_R)) < 1e-12        # ideal phi: no calibration error
    y = _sdpa(q, K[:L], V[:L])
    assert O.rel_l1(y, y) == 0.0
    Kflat = np.ones((L, 8), np.float32)
    assert O.h_mid(q, Kflat, L, ns, nt) == pytest.approx(1.0, abs=1e-12)
    Kpeak = np.zeros((L, 8), np.float32)
    Kpeak[10] = 200.0 * q / np.linalg.norm(q)
    assert O.h_mid(q, Kpeak, L, ns, nt) < 1e-6


def test_log_partitions_uniform_scores_closed_form():
    # all-zero keys: every score is 0, so each partition sum is a token count
    L, ns, nt, n_gen, Kret = 50, 3, 6, 2, 7
    q = _rng(91).standard_normal(8)
    keys = np.zeros((L + n_gen, 8))
    idx = np.arange(ns + 5, ns + 5 + Kret)
    zf, zm, zr = O.log_partitions(q, keys, L, ns, nt, n_gen, idx)
    assert zf == pytest.approx(math.log(L + n_gen), abs=1e-14)
    assert zm == pytest.approx(math.log(L - ns - nt), abs=1e-14)
    assert zr == pytest.approx(math.log(L - ns - nt - Kret), abs=1e-14)
    assert O.log_partitions(q, keys, L, ns, nt, n_gen, np.arange(ns, L - nt))[2] == -math.inf
    assert O.log_partitions(q, keys, L, ns, nt, n_gen)[2] is None


def test_log_partitions_split_into_exact_support_and_true_residual():
    # Z_full = (exact-support mass over A, K(q), Gen) + (true residual mass over M minus K(q))
    L, ns, nt, n_gen = 96, 3, 7, 3
    q, K, V, W, b = _unit(92, L=L, n_gen=n_gen)
    A, M, G = O.partition(L, ns, nt, n_gen)
    idx = O.topk_indices(q, K[M], 13, first_index=ns)
    m_star, _, Z_E = O.exact_terms(q, K, V, np.concatenate([A, idx, G]))
    _, Z_R = O.residual_true(q, K, V, L, ns, nt, idx)
    zf, zm, zr = O.log_partitions(q, K, L, ns, nt, n_gen, idx)
    assert math.exp(zf) == pytest.approx(Z_E * math.exp(m_star) + Z_R, rel=1e-13)
    assert zr == pytest.approx(math.log(Z_R), abs=1e-13)
    s_mid = torch.from_numpy(K[M].astype(np.float64) @ q.astype(np.float64) / math.sqrt(8))
    assert zm == pytest.approx(float(torch.logsumexp(s_mid, 0)), abs=1e-13)


def test_log_partitions_shift_with_the_scores():
    # adding alpha*sqrt(d)*q/|q|^2 to every key adds alpha to every score
    L, ns, nt, n_gen, alpha = 80, 2, 5, 1, 1.75
    q, K, V, W, b = _unit(93, L=L, n_gen=n_gen)
    q = q.astype(np.float64)
    K = K.astype(np.float64)
    idx = O.topk_indices(q, K[ns:L - nt], 9, first_index=ns)
    base = O.log_partitions(q, K, L, ns, nt, n_gen, idx)
    shifted = O.log_partitions(q, K + alpha * math.sqrt(8) * q / (q @ q), L, ns, nt, n_gen, idx)
    for a, b_ in zip(base, shifted):
        assert b_ == pytest.approx(a + alpha, abs=1e-12)


# ------------------------------------------------------------------ f4: MLP feature map
def _mlp_params(rng, d, H, m, alpha=0.5):
    return dict(W_in=rng.standard_normal((H, d)) / math.sqrt(d), b_in=0.1 * rng.standard_normal(H),
                W_1=rng.standard_normal((H, H)) / math.sqrt(H), b_1=0.1 * rng.standard_normal(H),
                W_2=rng.standard_normal((H, H)) / math.sqrt(H), b_2=0.1 * rng.standard_normal(H),
                alpha=alpha, W_o=0.3 * rng.standard_normal((m, H)) / math.sqrt(H),
                b_o=0.1 * rng.standard_normal(m))


def test_phi_mlp_architecture_matches_the_pages_parameter_totals():
    """§8 ("Scope and runtime"): at d_phi = 64 the phi modules hold 378.5M
    parameters for the 1B backbone (16 layers, 32 query / 8 kv heads, d_h = 64)
    and 559.3M for the 3B backbone (28 layers, 24 / 8 heads, d_h = 128).  One
    phi_q per query head and one phi_k per kv head, each of the reading in
    phi_mlp (width 512, biases on all four layers, one ReZero scalar), give
    both totals; the nearby alternatives do not."""
    def total(count, layers, hq, hkv):
        return count * layers * (hq + hkv)
    one_b = total(O.phi_mlp_param_count(64), 16, 32, 8)
    three_b = total(O.phi_mlp_param_count(128), 28, 24, 8)
    assert round(one_b / 1e6, 1) == 378.5 and round(three_b / 1e6, 1) == 559.3
    # without biases, with a LayerNorm (2 x 512 more per map), or at width 256 / 1024: off
    no_bias = lambda d: d * 512 + 2 * 512 * 512 + 512 * 64
    assert round(total(no_bias(64), 16, 32, 8) / 1e6, 1) != 378.5
    assert round(total(O.phi_mlp_param_count(64) + 1024, 16, 32, 8) / 1e6, 1) != 378.5
    for w in (256, 1024):
        assert round(total(O.phi_mlp_param_count(64, width=w), 16, 32, 8) / 1e6, 1) != 378.5


def test_phi_mlp_without_the_block_is_one_affine_map():
    """alpha = 0: the ReZero block adds nothing, so phi(x) = exp(W_o W_in x +
    W_o b_in + b_o), one composed affine map (checked through torch float64)."""
    rng = _rng(41)
    p = _mlp_params(rng, 8, 16, 5, alpha=0.0)
    x = rng.standard_normal((7, 8))
    A = torch.from_numpy(p["W_o"]) @ torch.from_numpy(p["W_in"])
    c = torch.from_numpy(p["W_o"]) @ torch.from_numpy(p["b_in"]) + torch.from_numpy(p["b_o"])
    ref = torch.exp(torch.from_numpy(x) @ A.T + c).numpy()
    assert np.allclose(O.phi_mlp(x, p), ref, rtol=1e-13, atol=0)


def test_phi_mlp_dead_activation_leaves_the_block_bias():
    """All first-layer pre-activations negative: relu gives 0, so the block adds
    alpha * b_2 exactly: phi(x) = exp(W_o (W_in x + b_in + alpha b_2) + b_o)."""
    rng = _rng(42)
    p = _mlp_params(rng, 6, 12, 4, alpha=0.75)
    p["b_1"] = np.full(12, -1e6)
    x = rng.standard_normal((5, 6))
    h = torch.from_numpy(x) @ torch.from_numpy(p["W_in"]).T + torch.from_numpy(p["b_in"] + 0.75 * p["b_2"])
    ref = torch.exp(h @ torch.from_numpy(p["W_o"]).T + torch.from_numpy(p["b_o"])).numpy()
    assert np.allclose(O.phi_mlp(x, p), ref, rtol=1e-13, atol=0)


def test_phi_mlp_brute_force_tiny_network():
    """Scalar loops over a 3-wide network with 2 inputs and 2 outputs."""
    rng = _rng(43)
    d, H, m = 2, 3, 2
    p = _mlp_params(rng, d, H, m, alpha=0.3)
    x = rng.standard_normal((4, d))
    out = O.phi_mlp(x, p)
    for r in range(4):
        h0 = [sum(p["W_in"][j][i] * x[r][i] for i in range(d)) + p["b_in"][j] for j in range(H)]
        a = [max(sum(p["W_1"][j][i] * h0[i] for i in range(H)) + p["b_1"][j], 0.0) for j in range(H)]
        h1 = [h0[j] + 0.3 * (sum(p["W_2"][j][i] * a[i] for i in range(H)) + p["b_2"][j]) for j in range(H)]
        for k in range(m):
            z = sum(p["W_o"][k][i] * h1[i] for i in range(H)) + p["b_o"][k]
            assert math.isclose(out[r][k], math.exp(z), rel_tol=1e-13)


def test_phi_mlp_features_are_positive():
    """App. C.1 ("Why positivity matters"): exponentiated outputs are positive."""
    rng = _rng(44)
    p = _mlp_params(rng, 64, 512, 64)
    x = 3.0 * rng.standard_normal((50, 64))
    assert (O.phi_mlp(x, p) > 0).all() and (O.phi_mlp(x, p, bf16_operands=True) > 0).all()


def test_round_bf16_ties_to_even_and_exact_values():
    vals = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20,
                     -(1.0 + 2.0 ** -8), 2.0 - 2.0 ** -9, 0.0, -3.5, 2.0 ** -130])
    want = np.array([1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -1.0, 2.0, 0.0, -3.5, 2.0 ** -130])
    assert np.array_equal(O.round_bf16(vals), want)


def test_phi_mlp_rounding_mirror_is_exact_on_representable_values():
    """With weights, inputs, biases and every intermediate value exactly
    representable in bfloat16, rounding the operands changes nothing."""
    rng = _rng(45)
    d, H, m = 4, 8, 3
    p = dict(W_in=rng.integers(-1, 2, (H, d)).astype(float), b_in=rng.integers(-2, 3, H).astype(float),
             W_1=rng.integers(-1, 2, (H, H)).astype(float), b_1=rng.integers(-2, 3, H).astype(float),
             W_2=rng.integers(-1, 2, (H, H)).astype(float), b_2=rng.integers(-2, 3, H).astype(float),
             alpha=0.5, W_o=0.125 * rng.integers(-1, 2, (m, H)).astype(float), b_o=np.zeros(m))
    x = rng.integers(-3, 4, (6, d)).astype(float)
    assert np.array_equal(O.phi_mlp(x, p, bf16_operands=True), O.phi_mlp(x, p))
    # and a value that is not representable is rounded (the mirror is active)
    p["W_in"][0, 0] = 1.0 + 2.0 ** -12
    x[:, 0] = 1.0
    assert not np.array_equal(O.phi_mlp(x, p, bf16_operands=True), O.phi_mlp(x, p))


# ------------------------------------------------------------------ references and diagnostics
@pytest.mark.parametrize("n_gen", [0, 3])
def test_full_attention_matches_sdpa_over_exactly_n_tokens(n_gen):
    """Eq. 1 over [0, L + n_gen): against torch SDPA in float64.  A key planted
    just past the range would dominate the softmax if it were included, and the
    last in-range key dominates if it were dropped, so an off-by-one in the
    token count fails by far more than the tolerance."""
    L, d = 50, 8
    q, K, V, _, _ = _unit(91, L=L, n_gen=n_gen + 1, d=d)
    n = L + n_gen
    qh = q / np.linalg.norm(q)
    K[n] = 40.0 * qh               # outside: must not count
    K[n - 1] = 6.0 * qh            # inside: carries most of the weight
    got = O.full_attention(q, K, V, n)
    np.testing.assert_allclose(got, _sdpa(q, K[:n], V[:n]), rtol=0, atol=1e-13)
    assert np.abs(got - _sdpa(q, K[:n + 1], V[:n + 1])).max() > 1e-2
    assert np.abs(got - _sdpa(q, K[:n - 1], V[:n - 1])).max() > 1e-2


def test_kappa_max_matches_scalar_loops():
    """The largest key 2-norm, by plain Python loops over rows and components."""
    r = _rng(92)
    K = r.standard_normal((37, 8))
    K[36] *= 5.0                    # the maximum sits on the last row
    ref = max(math.sqrt(sum(float(x) * float(x) for x in row)) for row in K)
    assert O.kappa_max(K) == pytest.approx(ref, rel=1e-15)
    assert O.kappa_max(np.zeros((0, 8))) == 0.0
    assert O.kappa_max(np.array([[3.0, -4.0]])) == 5.0


def test_rel_l1_hand_computed_pair():
    """sum |y - y_ref| / sum |y_ref| (§7.1 Table 3 metric): |(1,-2,3) - (2,-2,1)|_1
    = 3 over |(2,-2,1)|_1 = 5.  Dividing by the other vector's norm would give
    3/6, by the 2-norm 3/3."""
    assert O.rel_l1([1.0, -2.0, 3.0], [2.0, -2.0, 1.0]) == pytest.approx(0.6, rel=1e-15)
    assert O.rel_l1([2.0, -2.0, 1.0], [1.0, -2.0, 3.0]) == pytest.approx(0.5, rel=1e-15)


def test_log_partition_error_sign():
    """log Z_R_hat - log Z_R (§7.1 Table 3, §7.2): negative for an
    under-estimate.  Z_R_hat = Z_R / e gives exactly -1, Z_R * e^2 gives +2."""
    Z = 123.25
    assert O.log_partition_error(Z / math.e, Z) == pytest.approx(-1.0, abs=1e-14)
    assert O.log_partition_error(Z * math.e ** 2, Z) == pytest.approx(2.0, abs=1e-14)


@pytest.mark.parametrize("Kret", [1, 7, 30, 72])
def test_nosub_under_ideal_features_double_counts_the_retrieved_tokens(Kret):
    """NoSub (§5.2 Table 1 caption: the variant leaves out the retrieved-token
    subtraction).  Under the codebook features of Eq. 7, S^T f and u^T f are
    the exact whole-mid sums, so NoSub gives (N_full + nu_K) / (Z_full + Z_K):
    softmax attention over the whole context with the retrieved keys counted a
    second time.  SDPA over that multiset pins it; a NoSub that still
    subtracted would equal full attention instead."""
    L, ns, nt, n_gen = 80, 2, 5, 2
    q, K, V, Pk, f, S, u = _codebook_unit(41, L=L, ns=ns, nt=nt, n_gen=n_gen)
    y_ns, idx, _ = O.decode_query(q, f, K, V, Pk, S, u, L, ns, nt, n_gen, K=Kret, variant="nosub")
    Kd = np.concatenate([K, K[idx]])
    Vd = np.concatenate([V, V[idx]])
    np.testing.assert_allclose(y_ns, _sdpa(q, Kd, Vd), rtol=0, atol=1e-12)
    assert np.abs(y_ns - _sdpa(q, K, V)).max() > 1e-4
