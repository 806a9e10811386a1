"""GPU checks of the summaries over given phi_k rows (rma_build_summaries with
Wk == NULL: the rows are an input, page §4.1 Eq. 6 sums them with the values).
With bf16 K/V and bf16 rows this runs the matrix-core builder reading the rows
beside K and V.  The rows here are arbitrary positive bf16 values, so the
oracle's sums are exact float64 sums of the same binary values: S and u within
fp32 summation error (|dS| <= 2^-14 |Phi|^T |V| + 1e-5: a few thousand
fp32 additions; a wrong row or offset is off by O(1)), kappa as the oracle's
largest key norm rounded up, and pieces appended with RMA_BUILD_ACCUMULATE
equal to the whole range up to summation order.
"""
import numpy as np
import pytest
import torch

import oracle as O
from parity_util import R, log

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(d, m, U, L, n_sink, n_tail, seed):
    g = torch.Generator().manual_seed(seed)
    k = torch.randn(U, L, d, generator=g).to(torch.bfloat16)
    v = torch.randn(U, L, d, generator=g).to(torch.bfloat16)
    Lm = L - n_sink - n_tail
    phi = torch.exp(0.7 * torch.randn(U, Lm, m, generator=g)).to(torch.bfloat16)   # positive features
    return k, v, phi, R.Span(L, n_sink, n_tail, 0)


def _check(k, v, phi, S, u, kappa, n_sink, what):
    U, Lm = phi.shape[0], phi.shape[1]
    worst = 0.0
    for uu in range(U):
        P = phi[uu].double().numpy()
        V = v[uu, n_sink:n_sink + Lm].double().numpy()
        Sr, ur = O.summaries(P, V)
        bound = 2.0 ** -14 * (np.abs(P).T @ np.abs(V)) + 1e-5
        dS = np.abs(S[uu].double().cpu().numpy() - Sr)
        assert (dS <= bound).all(), f"{what} unit {uu}: S off by {float((dS / bound).max()):.2f} x bound"
        du = np.abs(u[uu].double().cpu().numpy() - ur)
        assert (du <= 2.0 ** -14 * ur + 1e-5).all(), f"{what} unit {uu}: u"
        kap = O.kappa_max(k[uu, n_sink:n_sink + Lm].double().numpy())
        kg = float(kappa[uu])
        assert kap <= kg <= kap * (1 + 2e-5) + 1e-30, f"{what} unit {uu}: kappa {kg} vs {kap}"
        worst = max(worst, float((dS / bound).max()))
    return worst


@pytest.mark.parametrize("d,m", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_summaries_over_given_rows_match_oracle(d, m):
    k, v, phi, sp = _case(d, m, U=3, L=2500 + 19, n_sink=4, n_tail=64, seed=d + m)
    _, S, u, kappa = R.rma_build_summaries(k.to(DEV), v.to(DEV), sp, None, None, m=m, phi_k=phi.to(DEV))
    torch.cuda.synchronize()
    worst = _check(k, v, phi, S.cpu(), u.cpu(), kappa.cpu(), 4, f"d{d} m{m}")
    log(f"given rows d{d} m{m}: worst |dS| / bound {worst:.3f}")


def test_given_rows_appended_in_pieces():
    d, m = 64, 128
    k, v, phi, sp = _case(d, m, U=2, L=3000 + 5, n_sink=4, n_tail=64, seed=3)
    kd, vd, pd = k.to(DEV), v.to(DEV), phi.to(DEV)
    Lm = phi.shape[1]
    S = torch.empty(2, m, d, device=DEV)
    u = torch.empty(2, m, device=DEV)
    kappa = torch.empty(2, device=DEV)
    cuts = [0, 1, Lm // 3 + 7, Lm - 1, Lm]
    for i, (a, b) in enumerate(zip(cuts, cuts[1:])):
        R.rma_build_summaries_range(kd, vd, sp, a, b, None, None, pd, S, u, kappa, accumulate=i > 0)
    torch.cuda.synchronize()
    _check(k, v, phi, S.cpu(), u.cpu(), kappa.cpu(), 4, "appended")
