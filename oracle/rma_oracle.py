"""fp64 CPU oracle for Top-K+phi residual-mass-accounting decode.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the HIP
library and its binding) never calls it, and it shares no code with that path.

Source: "Residual-Mass Accounting for Partial-KV Decoding" (the paperpeel page
of arXiv 2604.05438).  The page's display equations did not survive text
extraction; only the surrounding prose does.  Each function below states the
equation it stands for and the reading used for it.

Notation (page §3): one (layer, kv head) unit with a prefill segment of length
L, keys k_i and values v_i (i = 0..L-1), head dim d_h (d_v = d_h), query q.

* Eq. 1  scores s_i = q.k_i / sqrt(d_h), full prefill-segment attention
         y_full = sum_i e^{s_i} v_i / sum_i e^{s_i}.
* Eq. 2  anchors A = [0, n_sink) u [L - n_tail, L); mid-region M between them.
* Eq. 3-4 retrieved set K(q) (subset of M, |K(q)| = K), exact support
         E = A u K(q); unnormalised numerator/denominator over E.
* Eq. 5  subset-renormalisation bias (checked as an identity in the tests).
* Eq. 6  summaries S = sum_{i in M} phi_k(k_i) v_i^T, u = sum_{i in M} phi_k(k_i).
* Eq. 7  ideal factorisation e^{q.k/sqrt(d)} = phi_q(q)^T phi_k(k).
* Eq. 9  retrieved-token subtraction: nu_R = S^T f - sum_{K(q)} (f.phi_k(k_i)) v_i,
         Z_R = u^T f - sum_{K(q)} f.phi_k(k_i), with f = phi_q(q).
* Eq. 10 single normalisation y = (nu_E + nu_R_hat) / (Z_E + Z_R_hat).
* Eq. 11 generated tokens stay exact and join the exact numerator/denominator.

All inputs (fp32 or bf16 values) convert to float64 exactly; every result here
is computed in float64.  Top-K ranks by the exact real value of q.k (products
of the stored binary values, summed exactly), ties going to the lower index;
near-ties that float64 cannot separate are resolved with exact rationals.

Every function here is pinned by a test in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

F64 = np.float64


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=F64)


# ---------------------------------------------------------------- partition
def partition(L: int, n_sink: int, n_tail: int, n_gen: int = 0):
    """Anchor, mid-region and generated index sets (page §3, Eq. 2 and Eq. 11).

    The anchor set holds the initial sink tokens and the recent tail tokens of
    the prefill segment; the mid-region M is the part between them.  Generated
    tokens (positions L .. L+n_gen-1) are kept apart: they are always exact and
    never part of the residual.
    """
    if n_sink < 0 or n_tail < 0 or n_sink + n_tail > L:
        raise ValueError("anchors exceed the prefill segment")
    anchors = np.concatenate([np.arange(0, n_sink), np.arange(L - n_tail, L)]).astype(np.int64)
    mid = np.arange(n_sink, L - n_tail, dtype=np.int64)
    gen = np.arange(L, L + n_gen, dtype=np.int64)
    return anchors, mid, gen


def budget_K(fraction: float, L: int, n_anchor: int) -> int:
    """Retrieved-token count for a total exact-support budget (page §5.2 Table 1
    caption: anchors count toward the percentage; §7.1: a 1 % budget with 20
    anchors gives K = 21 at 4k and K = 636 at 64k).  The reading consistent with
    both printed values is K = ceil(fraction * L) - n_anchor."""
    return int(math.ceil(fraction * L - 1e-12)) - n_anchor


# ---------------------------------------------------------------- features
def phi_features(x, W, b) -> np.ndarray:
    """Positive feature map phi(x) = elu(W x + b) + 1, row-wise over x.

    The page (App. C.1, "Why positivity matters") requires strictly positive
    feature outputs; the workloads fix the form elu(.) + 1.  elu(z) + 1 equals
    z + 1 for z > 0 and e^z for z <= 0.
    """
    x = _f64(x)
    z = x @ _f64(W).T + _f64(b)
    return np.where(z > 0.0, z + 1.0, np.exp(np.minimum(z, 0.0)))


def round_bf16(x) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even), through float32 first: the
    value an fp32 accumulator holds is what the GPU rounds to bfloat16.  The
    result is returned as float64 (every bfloat16 value is exact there)."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    r = ((bits + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32).astype(np.float64)
    return np.where(np.isnan(f), np.nan, out)


def phi_mlp(x, params, bf16_operands: bool = False, return_terms: bool = False, operand_round=None):
    """The pages' feature-map family (f4), row-wise over x.

    Page §4.4 ("Training phi"): phi_q and phi_k are head-specific one-block
    ReZero MLPs; App. C.1 ("Why positivity matters"): their outputs are
    exponentiated, so every feature is positive; §8 ("Scope and runtime"):
    d_phi = 64.  App. C.2, which would give the architecture, is empty on the
    page.  Reading (pinned by the parameter totals of §8, see the tests): an
    input layer to width H = 512 with bias, one ReZero block
    h1 = h0 + alpha * (W_2 act(W_1 h0 + b_1) + b_2) with two H x H layers, and
    an output layer to d_phi with bias, exponentiated:

        h0 = W_in x + b_in,  h1 = h0 + alpha (W_2 relu(W_1 h0 + b_1) + b_2),
        phi(x) = exp(W_o h1 + b_o).

    The block's activation is not given anywhere on the pages; ReLU is the
    reading taken (parity for that choice is unpinned by the pages).

    params: dict with W_in [H, d], b_in [H], W_1 [H, H], b_1 [H], W_2 [H, H],
    b_2 [H], alpha (scalar), W_o [m, H], b_o [m].  Sums are float64.  With
    bf16_operands, every operand of a matrix product (the weights, x, h0, the
    activation and h1) is first rounded to bfloat16, as the GPU kernel's
    matrix-core products take them; biases, alpha, the residual sum and the
    exponential stay exact.  With return_terms, also returns the intermediate
    values (x, h0, r = W_1 h0 + b_1, a = relu(r), t = W_2 a + b_2, h1, z =
    W_o h1 + b_o) and the matrices used, for error analysis.  operand_round, a
    function applied at those same rounding points in place of the bfloat16
    rounding, serves the error model of the tests.
    """
    if operand_round is not None:
        rb = operand_round
    else:
        rb = round_bf16 if bf16_operands else (lambda a: _f64(a))
    W_in, W_1, W_2, W_o = (rb(params[k]) for k in ("W_in", "W_1", "W_2", "W_o"))
    b_in, b_1, b_2, b_o = (_f64(params[k]) for k in ("b_in", "b_1", "b_2", "b_o"))
    alpha = float(params["alpha"])
    x = rb(x)
    h0 = rb(x @ W_in.T + b_in)
    r = h0 @ W_1.T + b_1
    a = rb(np.maximum(r, 0.0))
    t = a @ W_2.T + b_2
    h1 = rb(h0 + alpha * t)
    z = h1 @ W_o.T + b_o
    phi = np.exp(z)
    if return_terms:
        return phi, dict(x=x, h0=h0, r=r, a=a, t=t, h1=h1, z=z, W_in=W_in, W_1=W_1, W_2=W_2,
                         W_o=W_o, alpha=alpha)
    return phi


def phi_mlp_param_count(d_h: int, width: int = 512, d_phi: int = 64) -> int:
    """Parameters of one map under the architecture reading of phi_mlp: the
    input, the two block and the output layers with their biases, and alpha."""
    return (d_h * width + width) + 2 * (width * width + width) + 1 + (width * d_phi + d_phi)


def summaries(phi_mid, v_mid):
    """Fixed-size summary states over the mid-region (page §1 and §4.1; Eq. 6):
    S = sum_i phi_k(k_i) v_i^T  (m x d_v),   u = sum_i phi_k(k_i)  (m)."""
    P = _f64(phi_mid)
    V = _f64(v_mid)
    return P.T @ V, P.sum(axis=0)


def kappa_max(k_mid) -> float:
    """Largest key 2-norm over the mid-region (used only by the GPU's error
    bound; the oracle reports it for comparison)."""
    k = _f64(k_mid)
    if k.shape[0] == 0:
        return 0.0
    return float(np.sqrt((k * k).sum(axis=1)).max())


# ---------------------------------------------------------------- selection
def raw_scores(q, keys) -> np.ndarray:
    """Unscaled scores r_i = q.k_i (page §3, Eq. 1 before the 1/sqrt(d_h) scale)."""
    return _f64(keys) @ _f64(q)


def _exact_dot(q, k) -> Fraction:
    return sum((Fraction(float(a)) * Fraction(float(c)) for a, c in zip(q, k)), Fraction(0))


def topk_indices(q, keys_mid, K: int, first_index: int = 0) -> np.ndarray:
    """Exhaustive Top-K over the mid-region (page §1: exhaustive Top-K is the
    control selector; §3 Eq. 3: K(q) is a subset of M of size K).

    Ranks every mid token by the exact real value of q.k_i, ties to the lower
    index, and returns the K winners as absolute positions (first_index + i) in
    ascending order.  Brute force: a float64 sort, then every token whose
    float64 score cannot be certified against the K-th boundary is rescored
    with exact rationals.
    """
    q = _f64(q)
    kk = _f64(keys_mid)
    n, d = kk.shape
    if K < 0 or K > n:
        raise ValueError("K out of range")
    if K == 0:
        return np.zeros(0, dtype=np.int64)
    if K == n:
        return np.arange(n, dtype=np.int64) + first_index
    r = kk @ q
    # |fl(sum) - exact| <= gamma_d * sum|q_j k_ij| for any summation order (the
    # products are exact in float64); doubled for the rounding of the bound.
    u = 2.0 ** -53
    gam = (d + 2) * u / (1.0 - (d + 2) * u)
    bnd = 2.0 * gam * (np.abs(kk) @ np.abs(q)) + 1e-300
    lo, hi = r - bnd, r + bnd
    t_lo = np.partition(lo, n - K)[n - K]     # K-th largest lower bound
    t_hi = np.partition(hi, n - K)[n - K]     # K-th largest upper bound
    sure_in = np.nonzero(lo > t_hi)[0]
    ambiguous = np.nonzero((lo <= t_hi) & (hi >= t_lo))[0]
    need = K - sure_in.size
    exact = [(_exact_dot(q, kk[i]), -int(i)) for i in ambiguous]
    order = sorted(range(len(ambiguous)), key=lambda j: exact[j], reverse=True)
    chosen = ambiguous[np.array(order[:need], dtype=np.int64)] if need > 0 else np.zeros(0, np.int64)
    sel = np.sort(np.concatenate([sure_in, chosen]).astype(np.int64))
    assert sel.size == K
    return sel + first_index


# ---------------------------------------------------------------- exact branch
def exact_terms(q, keys, values, support):
    """Exact unnormalised terms over the exact support (page §3 Eq. 3-4, with
    generated tokens added as in Eq. 11).  Returned with a running max m* so
    that no exponential overflows: N_E = sum e^{s_i - m*} v_i,
    Z_E = sum e^{s_i - m*}, s_i = q.k_i / sqrt(d_h)."""
    q = _f64(q)
    d = q.shape[0]
    support = np.asarray(support, dtype=np.int64)
    if support.size == 0:
        raise ValueError("empty exact support")
    s = (_f64(keys)[support] @ q) / math.sqrt(d)
    m_star = float(s.max())
    w = np.exp(s - m_star)
    return m_star, w @ _f64(values)[support], float(w.sum())


def residual_terms(f, phi_mid, v_mid, S, u, retrieved_local, whole_mid_retrieved: bool,
                   subtract: bool = True):
    """Residual estimate for the unretrieved mid-region (page §4.2, Eq. 9).

    nu_R_hat = S^T f - sum_{i in K(q)} (f.phi_k(k_i)) v_i,
    Z_R_hat  = max(u^T f - sum_{i in K(q)} f.phi_k(k_i), 0).
    The clamp guards only the finite-precision subtraction (page App. C.1:
    numerical clamps are used only against subtraction artifacts).  When the
    whole mid-region is retrieved the residual set is empty and both terms are
    exactly zero.  `subtract=False` gives the NoSub variant of §5.2 Table 1,
    which adds the whole-mid estimate and double-counts K(q).  Also returns the
    retrieved feature mass sum_{K(q)} f.phi_k(k_i).
    """
    f = _f64(f)
    Sm = _f64(S)
    um = _f64(u)
    if whole_mid_retrieved and subtract:
        return np.zeros(Sm.shape[1]), 0.0, float("nan")
    loc = np.asarray(retrieved_local, dtype=np.int64)
    P = _f64(phi_mid)[loc]
    w = P @ f
    zk = float(w.sum())
    if not subtract:
        return Sm.T @ f, max(float(um @ f), 0.0), zk
    nu = Sm.T @ f - w @ _f64(v_mid)[loc]
    z = float(um @ f) - zk
    return nu, max(z, 0.0), zk


def merge(m_star, N_E, Z_E, nu_R, Z_R):
    """Residual-mass accounting rule (page §4.3, Eq. 10): exact and estimated
    terms are added on the same unnormalised scale and normalised once.  The
    exact terms carry the factor e^{-m*}, so the residual terms are scaled by
    e^{-m*} too."""
    sc = math.exp(-m_star)
    return (_f64(N_E) + sc * _f64(nu_R)) / (Z_E + sc * Z_R)


# ---------------------------------------------------------------- decode
def decode_query(q, f, keys, values, phi_mid, S, u, L, n_sink, n_tail, n_gen, K,
                 variant: str = "sub"):
    """One decode query of Top-K+phi (page §1 summary of the method; §3-§4).

    keys/values: the unit's cache rows [0, L + n_gen).  phi_mid: phi_k rows of
    the mid-region (row i <-> position n_sink + i).  f = phi_q(q).
    variant: "sub" (Top-K+phi), "topk" (selection-only: residual dropped, the
    renormalisation over the exact support of §1), "nosub" (whole-mid estimate
    without subtraction, §5.2).
    Returns (y, idx, stats) with stats = (m*, Z_E, Z_R_hat, retrieved phi mass).
    """
    anchors, mid, gen = partition(L, n_sink, n_tail, n_gen)
    keys = _f64(keys)
    values = _f64(values)
    idx = topk_indices(q, keys[mid], K, first_index=n_sink)
    support = np.concatenate([anchors, idx, gen])
    m_star, N_E, Z_E = exact_terms(q, keys, values, support)
    if variant == "topk":
        return N_E / Z_E, idx, (m_star, Z_E, 0.0, float("nan"))
    nu, zr, zk = residual_terms(f, phi_mid, values[mid], S, u, idx - n_sink,
                                whole_mid_retrieved=(K == mid.size),
                                subtract=(variant == "sub"))
    return merge(m_star, N_E, Z_E, nu, zr), idx, (m_star, Z_E, zr, zk)


def prefill_unit(k_mid, v_mid, W, b):
    """Prefill for one unit: phi_k rows of the mid-region and the summaries."""
    P = phi_features(k_mid, W, b)
    S, u = summaries(P, v_mid)
    return P, S, u


# ---------------------------------------------------------------- references
def full_attention(q, keys, values, n_tokens):
    """Full attention over positions [0, n_tokens) (page §3, Eq. 1), computed
    with a max shift."""
    q = _f64(q)
    s = (_f64(keys)[:n_tokens] @ q) / math.sqrt(q.shape[0])
    w = np.exp(s - s.max())
    return (w @ _f64(values)[:n_tokens]) / w.sum()


def residual_true(q, keys, values, L, n_sink, n_tail, idx):
    """True residual terms nu_R, Z_R over R(q) = M minus K(q) (page §3, the
    definitions before Eq. 5), unshifted."""
    _, mid, _ = partition(L, n_sink, n_tail)
    R = np.setdiff1d(mid, np.asarray(idx, dtype=np.int64))
    q = _f64(q)
    s = (_f64(keys)[R] @ q) / math.sqrt(q.shape[0])
    w = np.exp(s)
    return w @ _f64(values)[R], float(w.sum())


def log_partitions(q, keys, L, n_sink, n_tail, n_gen=0, idx=None):
    """Natural logarithms of the unshifted partition sums of the exponential
    kernel (page §3: Eq. 1 for the whole context, the residual definitions
    before Eq. 5 for R(q); §7.1 Table 3 compares log Z_R_hat with log Z_R):
        log Z_full = log sum_{i < L + n_gen} e^{s_i},
        log Z_mid  = log sum_{i in M} e^{s_i},
        log Z_R    = log sum_{i in M minus K(q)} e^{s_i}
    with s_i = q.k_i / sqrt(d_h).  log Z_R is -inf when the whole mid-region
    is retrieved and None when idx is None.  float64 with a max shift."""
    _, mid, _ = partition(L, n_sink, n_tail, n_gen)
    q = _f64(q)
    s = (_f64(keys)[:L + n_gen] @ q) / math.sqrt(q.shape[0])

    def lse(x):
        if x.size == 0:
            return -math.inf
        mx = float(x.max())
        return mx + math.log(float(np.exp(x - mx).sum()))

    z_r = None
    if idx is not None:
        R = np.setdiff1d(mid, np.asarray(idx, dtype=np.int64))
        z_r = lse(s[R])
    return lse(s), lse(s[mid]), z_r


# ---------------------------------------------------------------- diagnostics
def rel_l1(y, y_ref) -> float:
    """Relative l1 attention-output error (page §7.1 Table 3 metric, per query)."""
    y, y_ref = _f64(y), _f64(y_ref)
    return float(np.abs(y - y_ref).sum() / np.abs(y_ref).sum())


def log_partition_error(Z_R_hat, Z_R) -> float:
    """Residual log-partition error log Z_R_hat - log Z_R (page §7.1 Table 3,
    §7.2); negative means under-estimation."""
    return math.log(Z_R_hat) - math.log(Z_R)


def h_mid(q, keys, L, n_sink, n_tail) -> float:
    """Entropy of the full attention restricted to the mid-region and
    renormalised there, divided by log|M| (page §6; the normalisation is the
    reading that makes "H_mid <~ 0.3" meaningful)."""
    _, mid, _ = partition(L, n_sink, n_tail)
    q = _f64(q)
    s = (_f64(keys)[mid] @ q) / math.sqrt(q.shape[0])
    p = np.exp(s - s.max())
    p /= p.sum()
    nz = p[p > 0]
    return float(-(nz * np.log(nz)).sum() / math.log(mid.size))
