"""GPU parity of the full-attention reference and its diagnostics
(rma_decode_full, through the C ABI) against the fp64 oracle.

Tolerances (fp32 arithmetic over bf16/fp32 K and V):
  * y_full: the output bar of the method, max abs <= 2e-3 and per query
    ||dy||_2 / ||y||_2 <= 1e-2; the measured error is logged (~1e-6).
  * log Z (whole context, mid-region, residual set) and the max score: each sum
    is a sum of positive fp32 terms (relative error <~ 1e-5 over 131K terms,
    plus ~2e-6 from the exponential), so its log is within 1e-4 absolute.
  * H_mid = log Z_mid - T_mid / Z_mid over log|M|: T_mid / Z_mid averages
    score gaps of at most ~40 with ~1e-5 relative error, so 2e-4 absolute.
  * rel_l1 compares the same y_cmp with y_full on both sides; the difference is
    bounded by y_full's relative l1 error, so 1e-4 absolute.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from parity_util import R, W, check_y, decode_span, hip_decode, hip_prefill, host_unit, log

pytestmark = pytest.mark.gpu
DEV = "cuda"
LOGZ_TOL, H_TOL, L1_TOL = 1e-4, 2e-4, 1e-4

SMALL = {
    "c0": W.CONFIGS["c0"],
    "c1_small": W.CONFIGS["c1"].with_(L=4096 + 37, K=(41,)),
    "c2_small": W.CONFIGS["c2"].with_(L=6000 + 3, K=(118,)),
    "c3_small": W.CONFIGS["c3"].with_(batch=2, layers=2, L=3000, K=(29,), steps=3),
    "c4_small": W.CONFIGS["c4"].with_(batch=1, layers=2, L=5003, K=(50,), steps=2),
}


def _gen(cfg):
    torch.manual_seed(0)
    return W.generate(cfg, device=DEV)


def _oracle_full(cfg, hu, step, g, idx):
    """y_full and diag from the oracle for one query head (idx: positions or None)."""
    q = hu["q"][step, g]
    n_gen = cfg.n_gen(step)
    n_tok = cfg.L + n_gen
    y = O.full_attention(q, hu["k"], hu["v"], n_tok)
    lz, lzm, lzr = O.log_partitions(q, hu["k"], cfg.L, cfg.n_sink, cfg.n_tail, n_gen, idx)
    h = O.h_mid(q, hu["k"], cfg.L, cfg.n_sink, cfg.n_tail)
    smax = float(np.max(hu["k"][:n_tok] @ np.asarray(q, np.float64)) / math.sqrt(q.shape[0]))
    return y, (lz, lzm, lzr, h, smax)


def _check_diag(dg, ref, what):
    lz, lzm, lzr, h, smax = ref
    assert abs(dg[0] - lz) <= LOGZ_TOL, f"{what}: log Z_full {dg[0]} vs {lz}"
    assert abs(dg[1] - lzm) <= LOGZ_TOL, f"{what}: log Z_mid {dg[1]} vs {lzm}"
    if lzr is None:
        assert math.isnan(dg[2]), f"{what}: log Z_R should be NaN"
    elif lzr == -math.inf:
        assert dg[2] == -math.inf, f"{what}: log Z_R {dg[2]} should be -inf"
    else:
        assert abs(dg[2] - lzr) <= LOGZ_TOL, f"{what}: log Z_R {dg[2]} vs {lzr}"
    assert abs(dg[3] - h) <= H_TOL, f"{what}: H_mid {dg[3]} vs {h}"
    assert abs(dg[5] - smax) <= LOGZ_TOL, f"{what}: max score {dg[5]} vs {smax}"


def _run(cfg, units=None, steps=None, store_phi=True):
    inp = _gen(cfg)
    pre = hip_prefill(inp, store_phi=store_phi)
    K = cfg.K[0]
    units = range(cfg.U) if units is None else units
    steps = range(cfg.steps) if steps is None else steps
    worst = 0.0
    for s in steps:
        dec = hip_decode(inp, pre, K, s)
        q = inp.q[s].contiguous()
        yf, dg = R.rma_decode_full(q, inp.k, inp.v, decode_span(cfg, s), dec["idx"], K,
                                   y_cmp=dec["y"], want_diag=True)
        torch.cuda.synchronize()
        yf, dg = yf.cpu().numpy(), dg.cpu().numpy().astype(np.float64)
        idx, y = dec["idx"].cpu().numpy(), dec["y"].cpu().numpy()
        for u in units:
            hu = host_unit(inp, u)
            for g in range(cfg.G):
                what = f"{cfg.name} step {s} unit {u} head {g}"
                y_ref, ref = _oracle_full(cfg, hu, s, g, idx[u, g])
                a, _ = check_y(yf[u, g], y_ref, what)
                worst = max(worst, a)
                _check_diag(dg[u, g], ref, what)
                rl1 = O.rel_l1(y[u, g], y_ref)
                assert abs(dg[u, g, 4] - rl1) <= L1_TOL, f"{what}: rel_l1 {dg[u, g, 4]} vs {rl1}"
                assert dg[u, g, 6] == 0.0 and dg[u, g, 7] == 0.0
    log(f"{cfg.name}: worst |y_full - oracle| {worst:.2e}")


@pytest.mark.parametrize("name", list(SMALL))
def test_full_small_configs(name):
    cfg = SMALL[name]
    units = None if cfg.U <= 8 else [0, 5, cfg.U - 1]
    _run(cfg, units=units)


def test_full_c1_full_size():
    _run(W.CONFIGS["c1"])


def test_full_c2_full_size_sampled_heads():
    _run(W.CONFIGS["c2"], units=[0, 3, 7])


def test_full_edge_cases():
    """K = 0, no index list, the whole mid-region retrieved, no comparison output."""
    cfg = SMALL["c1_small"]
    inp = _gen(cfg)
    sp = decode_span(cfg, 0)
    q = inp.q[0].contiguous()
    Lm = cfg.L_mid
    hu = host_unit(inp, 2)
    # K = 0: the residual set is the whole mid-region
    _, dg = R.rma_decode_full(q, inp.k, inp.v, sp, None, 0, want_diag=True)
    dg = dg.cpu().numpy().astype(np.float64)
    assert np.array_equal(dg[..., 2], dg[..., 1]) and np.all(np.isnan(dg[..., 4]))
    # an index list is required for log Z_R when K > 0
    _, dg = R.rma_decode_full(q, inp.k, inp.v, sp, None, 7, want_diag=True)
    assert torch.isnan(dg[..., 2]).all()
    # every mid position retrieved: the residual set is empty, and the method's
    # output is full attention
    pre = hip_prefill(inp)
    dec = hip_decode(inp, pre, Lm, 0)
    yf, dg = R.rma_decode_full(q, inp.k, inp.v, sp, dec["idx"], Lm, y_cmp=dec["y"], want_diag=True)
    torch.cuda.synchronize()
    assert torch.all(dg[..., 2] == -math.inf)
    for g in range(cfg.G):
        y_ref, ref = _oracle_full(cfg, hu, 0, g, np.arange(cfg.n_sink, cfg.n_sink + Lm))
        check_y(yf[2, g].cpu().numpy(), y_ref, f"head {g}")
        check_y(dec["y"][2, g].cpu().numpy(), y_ref, f"merge, head {g}")
        _check_diag(dg[2, g].cpu().numpy().astype(np.float64), ref, f"all retrieved, head {g}")
    assert float(dg[..., 4].max()) < 1e-4
    # y_full alone (no diagnostics) equals the diagnostic run bit for bit
    y2 = R.rma_decode_full(q, inp.k, inp.v, sp)
    assert torch.equal(y2, yf)


def test_full_generated_tokens_only_context_edge():
    """Anchors only (L_mid = 0) with generated tokens: full attention still covers
    every position, the mid-region sums are empty."""
    cfg = SMALL["c1_small"]
    inp = _gen(cfg)
    L = 68
    sp = R.Span(L, 4, 64, 5)
    q = inp.q[0].contiguous()
    yf, dg = R.rma_decode_full(q, inp.k, inp.v, sp, None, 0, want_diag=True)
    torch.cuda.synchronize()
    hu = host_unit(inp, 1)
    for g in range(cfg.G):
        y_ref = O.full_attention(hu["q"][0, g], hu["k"], hu["v"], L + 5)
        check_y(yf[1, g].cpu().numpy(), y_ref, f"head {g}")
    d = dg.cpu().numpy()
    assert np.all(d[..., 1] == -np.inf) and np.all(d[..., 2] == -np.inf) and np.all(np.isnan(d[..., 3]))
