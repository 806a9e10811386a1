"""GPU parity of the pages' MLP feature map (one-block ReZero MLP, exponentiated
output; page §4.4, App. C.1, §8) and of the decode path built on it, against
the plain fp64 definition (oracle.phi_mlp without any rounding).

Feature rows: the kernel multiplies bf16 operands (x, the weights, h0, the
activation, h1, each rounded to nearest even) with fp32 sums, so its features
differ from the definition by the propagated rounding.  The per-feature
tolerance comes from the rounding model of tests/mlp_bound.py: 8 standard
deviations of the exponent's change when every rounding point gets an
independent relative error uniform in [-2^-8, 2^-8], plus fp32 summation and
the storage rounding of bf16 rows.  A systematic mistake (a dropped bias or
term, a wrong scale) moves the exponents by far more.  How often the kernel's
rows equal the oracle's rounding mirror (oracle.phi_mlp with bf16_operands)
is logged as a statistic, not asserted.

Path: phi_k rows from the kernel feed the summary build (rows injected), f =
phi_q(q) from the kernel feeds the merge.  The oracle computes its own rows,
summaries and features from the plain definition; the decode output meets the
usual bar (bit-exact Top-K, 2e-3 abs / 1e-2 rel).
"""
import numpy as np
import pytest
import torch

import oracle as O
from mlp_bound import check_rows
from parity_util import R, W, check_y, decode_span, log, prefill_span

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _host_params(params, p):
    return {k: v[p].double().cpu().numpy() if v.dim() > 1 else float(v[p]) for k, v in params.items()}


def _check_rows(got, x, params, bf16, what):
    """got: the kernel's rows for inputs x (float64 [rows, d]); the plain
    definition with the rounding-model tolerance, and the mirror statistic."""
    got = got.double().cpu().numpy()
    try:
        ratio, med = check_rows(got, x, params, bf16)
    except AssertionError as e:
        raise AssertionError(f"{what}: {e}") from None
    mirror = O.phi_mlp(x, params, bf16_operands=True)
    if bf16:
        same = float((got == O.round_bf16(mirror)).mean())
        log(f"{what}: worst {ratio:.2f} of the tolerance, median rel {med:.2e} vs the definition; "
            f"{same:.3f} of the rows bit-identical to the rounding mirror")
    else:
        same = float(np.median(np.abs(got - mirror) / mirror))
        log(f"{what}: worst {ratio:.2f} of the tolerance, median rel {med:.2e} vs the definition; "
            f"median rel {same:.2e} vs the rounding mirror")
    return ratio


# (d, m, x dtype, phi dtype, units, rows, param sets)
SHAPES = [
    (64, 64, torch.bfloat16, torch.bfloat16, 3, 300 + 5, 2),
    (128, 64, torch.bfloat16, torch.bfloat16, 2, 129, 2),
    (64, 128, torch.bfloat16, torch.float32, 2, 64, 1),
    (64, 64, torch.float32, torch.float32, 40, 1, 8),       # decode queries: one row per unit
    (128, 64, torch.float32, torch.bfloat16, 9, 3, 9),
    (128, 128, torch.float32, torch.float32, 5, 77, 5),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"d{s[0]}m{s[1]}{str(s[2])[-4:]}{str(s[3])[-4:]}U{s[4]}r{s[5]}")
def test_phi_mlp_rows_match_oracle(shape):
    d, m, xdt, pdt, U, rows, P = shape
    cfg = W.CONFIGS["c1"].with_(d=d, h_kv=P, h_q=P, layers=1, seed=11)
    params = W.generate_phi_mlp(cfg, "k", m=m)
    w = R.PhiMlpWeights(params)
    g = torch.Generator().manual_seed(5)
    x = (1.5 * torch.randn(U, rows + 7, d, generator=g))[:, 3:3 + rows]   # unit stride > rows * d
    xg = x.to(xdt).to(DEV)
    xs = torch.empty(U, rows + 8, d, dtype=xdt, device=DEV)
    xs[:, :rows] = xg
    phi = R.rma_phi_mlp_features(xs[:, :rows], w, phi_dtype=pdt)
    torch.cuda.synchronize()
    for u in range(U):
        _check_rows(phi[u], xg[u].double().cpu().numpy(), _host_params(params, u % P), pdt == torch.bfloat16,
                    f"phi_mlp d{d} m{m} unit {u} of {U}, {rows} rows")


def _sample_rows(n, seed, k=384):
    """Seeded sample of row indices (the rounding model's trials cost a few
    forward passes per row), always with the first and last row."""
    rng = np.random.default_rng(seed)
    pick = rng.choice(n, size=min(k, n), replace=False)
    return np.unique(np.concatenate([pick, [0, n - 1]]))


def _mlp_path(cfg, K, steps):
    torch.manual_seed(0)
    inp = W.generate(cfg, device=DEV)
    pk = W.generate_phi_mlp(cfg, "k", m=cfg.m, device=DEV)
    pq = W.generate_phi_mlp(cfg, "q", m=cfg.m, device=DEV)
    wk, wq = R.PhiMlpWeights(pk), R.PhiMlpWeights(pq)
    sp = prefill_span(cfg)
    kmid = inp.k[:, cfg.n_sink:cfg.n_sink + cfg.L_mid]
    phi_k = R.rma_phi_mlp_features(kmid, wk, phi_dtype=torch.bfloat16)
    _, S, u, kappa = R.rma_build_summaries(inp.k, inp.v, sp, None, None, phi_k=phi_k, m=cfg.m)
    outs = []
    for s in steps:
        q = inp.q[s].contiguous()
        f = R.rma_phi_mlp_features(q.view(cfg.U * cfg.G, 1, cfg.d), wq).view(cfg.U, cfg.G, cfg.m)
        dsp = decode_span(cfg, s)
        idx, sel = R.rma_decode_topk(q, inp.k, dsp, kappa, K)
        y, _ = R.rma_decode_merge(q, f, inp.k, inp.v, dsp, idx, sel, K, phi_k, S, u, m=cfg.m, want_stats=True)
        outs.append((s, idx.cpu(), y.cpu()))
    torch.cuda.synchronize()
    return inp, pk, pq, phi_k, outs


PATHS = {
    "d64": (W.CONFIGS["c1"].with_(L=4096 + 37, m=64), 41),
    "d128": (W.CONFIGS["c2"].with_(L=3000 + 11, m=64), 60),
    "d64_gen": (W.CONFIGS["c3"].with_(batch=1, layers=2, L=2000 + 3, K=(25,), m=64, steps=2), 25),
}


@pytest.mark.parametrize("name", list(PATHS))
def test_decode_with_mlp_features_matches_oracle(name):
    cfg, K = PATHS[name]
    steps = list(range(cfg.steps))
    inp, pk, pq, phi_k, outs = _mlp_path(cfg, K, steps)
    worst = 0.0
    units = sorted({0, cfg.U // 2, cfg.U - 1})
    for uu in units:
        k = inp.k[uu].float().cpu().numpy().astype(np.float64)
        v = inp.v[uu].float().cpu().numpy().astype(np.float64)
        mid = slice(cfg.n_sink, cfg.n_sink + cfg.L_mid)
        hk = _host_params(pk, uu % cfg.P)
        phi_ref = O.phi_mlp(k[mid], hk)                                     # the plain definition
        rows = _sample_rows(cfg.L_mid, uu)
        _check_rows(phi_k[uu][torch.from_numpy(rows).to(phi_k.device)], k[mid][rows], hk, True, f"{name} phi_k unit {uu} ({rows.size} rows)")
        S, u_ = O.summaries(phi_ref, v[mid])
        for s, idx, y in outs:
            for g in range(cfg.G):
                q = inp.q[s, uu, g].double().cpu().numpy()
                hq = _host_params(pq, (uu % cfg.P) * cfg.G + g)
                f = O.phi_mlp(q[None], hq)[0]
                y_ref, idx_ref, _ = O.decode_query(q, f, k, v, phi_ref, S, u_, cfg.L, cfg.n_sink, cfg.n_tail,
                                                   cfg.n_gen(s), K)
                assert np.array_equal(idx[uu, g].numpy().astype(np.int64), idx_ref)
                a, _ = check_y(y[uu, g].numpy(), y_ref, f"{name} u{uu} g{g} s{s}")
                worst = max(worst, a)
    log(f"{name}: MLP-feature decode, worst |y - oracle| {worst:.2e}")


def test_full_c1_with_mlp_features_sampled_units():
    """The full c1 workload (32K context, K = 328) on the MLP features, in the
    configuration bench.py --phi mlp times; the oracle checks two units (every
    query head) end to end: phi_k rows, top-K and outputs."""
    cfg = W.CONFIGS["c1"].with_(m=64)
    K = cfg.K[0]
    inp, pk, pq, phi_k, outs = _mlp_path(cfg, K, [0])
    for uu in (1, cfg.U - 2):
        k = inp.k[uu].float().cpu().numpy().astype(np.float64)
        v = inp.v[uu].float().cpu().numpy().astype(np.float64)
        mid = slice(cfg.n_sink, cfg.n_sink + cfg.L_mid)
        hk = _host_params(pk, uu % cfg.P)
        phi_ref = O.phi_mlp(k[mid], hk)                                     # the plain definition
        rows = _sample_rows(cfg.L_mid, uu)
        _check_rows(phi_k[uu][torch.from_numpy(rows).to(phi_k.device)], k[mid][rows], hk, True, f"c1 phi_k unit {uu} ({rows.size} rows)")
        S, u_ = O.summaries(phi_ref, v[mid])
        _, idx, y = outs[0]
        for g in range(cfg.G):
            q = inp.q[0, uu, g].double().cpu().numpy()
            f = O.phi_mlp(q[None], _host_params(pq, (uu % cfg.P) * cfg.G + g))[0]
            y_ref, idx_ref, _ = O.decode_query(q, f, k, v, phi_ref, S, u_, cfg.L, cfg.n_sink, cfg.n_tail, 0, K)
            assert np.array_equal(idx[uu, g].numpy().astype(np.int64), idx_ref)
            check_y(y[uu, g].numpy(), y_ref, f"c1 mlp u{uu} g{g}")
    log("c1 with MLP features: sampled units match the oracle")
