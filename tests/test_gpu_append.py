"""GPU checks of summaries built in pieces (rma_build_summaries_range): the
summaries are sums over tokens (page §4.1, Eq. 6), so pieces appended with
RMA_BUILD_ACCUMULATE must give the whole-range result.

  * phi_k rows and kappa: identical bits (each row is computed from its own key
    with the same instruction sequence; kappa is a maximum);
  * S, u: equal up to fp32 summation order, |dS| <= 2^-18 (|Phi|^T |V|) + 1e-6
    (a few roundings of partial sums of at most L_mid positive-weighted terms);
  * the decode on appended summaries meets the oracle bar (bit-exact Top-K,
    2e-3 abs / 1e-2 rel).
"""
import numpy as np
import pytest
import torch

import oracle as O
from parity_util import (R, W, check_y, hip_decode, hip_prefill, host_unit, log, oracle_decode,
                         oracle_prefill, prefill_span)

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = {
    "c0": W.CONFIGS["c0"],
    "c1_small": W.CONFIGS["c1"].with_(L=4096 + 37, K=(41,)),
    "c2_small": W.CONFIGS["c2"].with_(L=6000 + 3, K=(118,)),
}


def _gen(cfg):
    torch.manual_seed(0)
    return W.generate(cfg, device=DEV)


def _pieces(Lm):
    # ragged cuts: not multiples of any tile or chunk
    a, b = Lm // 5 + 3, (2 * Lm) // 3 + 17
    return [(0, a), (a, b), (b, Lm)]


def _appended(inp, store_phi=True, pieces=None):
    cfg = inp.cfg
    sp = prefill_span(cfg)
    U, m, d = cfg.U, cfg.m, cfg.d
    phi_k = torch.empty(U, cfg.L_mid, m, dtype=cfg.torch_phi_dtype(), device=DEV) if store_phi else None
    S = torch.empty(U, m, d, dtype=torch.float32, device=DEV)
    u = torch.empty(U, m, dtype=torch.float32, device=DEV)
    kappa = torch.empty(U, dtype=torch.float32, device=DEV)
    for i, (a, b) in enumerate(pieces or _pieces(cfg.L_mid)):
        R.rma_build_summaries_range(inp.k, inp.v, sp, a, b, inp.W, inp.b, phi_k, S, u, kappa,
                                    accumulate=i > 0, phi_dtype=cfg.torch_phi_dtype())
    return phi_k, S, u, kappa


@pytest.mark.parametrize("name", list(CASES))
def test_appended_pieces_equal_whole_build(name):
    cfg = CASES[name]
    inp = _gen(cfg)
    whole = hip_prefill(inp)
    app = _appended(inp)
    torch.cuda.synchronize()
    assert torch.equal(whole[0], app[0]), "phi_k rows differ"
    assert torch.equal(whole[3], app[3]), "kappa differs"
    _, M, _ = O.partition(cfg.L, cfg.n_sink, cfg.n_tail)
    worst = 0.0
    for uu in range(cfg.U):
        P = whole[0][uu].double().cpu()
        V = inp.v[uu, cfg.n_sink:cfg.n_sink + cfg.L_mid].double().cpu()
        bound = 2.0 ** -18 * (P.abs().T @ V.abs()) + 1e-6
        dS = (whole[1][uu].double().cpu() - app[1][uu].double().cpu()).abs()
        assert bool((dS <= bound).all()), f"unit {uu}: S differs beyond reordering ({float((dS / bound).max()):.2f})"
        du = (whole[2][uu].double().cpu() - app[2][uu].double().cpu()).abs()
        assert bool((du <= 2.0 ** -18 * P.sum(0) + 1e-6).all()), f"unit {uu}: u differs"
        worst = max(worst, float((dS / bound).max()))
    log(f"{name}: appended vs whole, worst |dS| / bound {worst:.3f}")


@pytest.mark.parametrize("name", list(CASES))
def test_decode_on_appended_summaries_matches_oracle(name):
    cfg = CASES[name]
    inp = _gen(cfg)
    pre = _appended(inp)
    K = cfg.K[0]
    out = hip_decode(inp, pre, K, 0, fused_phi=True)
    torch.cuda.synchronize()
    for uu in range(cfg.U):
        hu = host_unit(inp, uu)
        ref_pre = oracle_prefill(cfg, hu)
        for g in range(cfg.G):
            y_ref, idx_ref, _ = oracle_decode(cfg, hu, ref_pre, K, 0, g)
            assert np.array_equal(out["idx"][uu, g].cpu().numpy().astype(np.int64), idx_ref)
            check_y(out["y"][uu, g].cpu().numpy(), y_ref, f"{name} u{uu} g{g}")


def test_appended_pieces_without_stored_rows():
    """Rows not stored (bf16 keys): the appended summaries equal the whole build's
    to reordering, and decode (recomputing the retrieved rows) meets the bar."""
    cfg = CASES["c1_small"]
    inp = _gen(cfg)
    whole = hip_prefill(inp, store_phi=False)
    app = _appended(inp, store_phi=False)
    torch.cuda.synchronize()
    assert app[0] is None and torch.equal(whole[3], app[3])
    rel = float(((whole[1] - app[1]).norm() / whole[1].norm()).item())
    assert rel <= 1e-6, rel
    out = hip_decode(inp, app, cfg.K[0], 0)
    ref = hip_decode(inp, whole, cfg.K[0], 0)
    assert torch.equal(out["idx"], ref["idx"])
    yr, yo = ref["y"].double(), out["y"].double()
    assert float(((yr - yo).norm(dim=-1) / yr.norm(dim=-1)).max()) <= 1e-5


def test_empty_and_single_piece_ranges():
    cfg = CASES["c1_small"]
    inp = _gen(cfg)
    whole = hip_prefill(inp)
    S, u, kappa = whole[1].clone(), whole[2].clone(), whole[3].clone()
    sp = prefill_span(cfg)
    # an empty range with accumulate leaves the summaries as they are
    R.rma_build_summaries_range(inp.k, inp.v, sp, 100, 100, inp.W, inp.b, whole[0], S, u, kappa, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(S, whole[1]) and torch.equal(u, whole[2]) and torch.equal(kappa, whole[3])
    # an empty range without accumulate gives empty sums
    R.rma_build_summaries_range(inp.k, inp.v, sp, 7, 7, inp.W, inp.b, whole[0], S, u, kappa)
    torch.cuda.synchronize()
    assert not S.any() and not u.any() and not kappa.any()
    # the full range in one piece is the whole build, bit for bit
    phi = torch.empty_like(whole[0])
    R.rma_build_summaries_range(inp.k, inp.v, sp, 0, cfg.L_mid, inp.W, inp.b, phi, S, u, kappa)
    torch.cuda.synchronize()
    for a, b in zip((phi, S, u, kappa), whole):
        assert torch.equal(a, b)
    # single-token pieces at both ends of the mid-region
    pieces = [(0, 1), (1, cfg.L_mid - 1), (cfg.L_mid - 1, cfg.L_mid)]
    app = _appended(inp, pieces=pieces)
    torch.cuda.synchronize()
    assert torch.equal(app[0], whole[0]) and torch.equal(app[3], whole[3])
    rel = float(((whole[1] - app[1]).norm() / whole[1].norm()).item())
    assert rel <= 1e-6, rel
