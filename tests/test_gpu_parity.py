"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Top-K indices must match bit for bit; outputs within 2e-3 abs / 1e-2 rel.
Inputs are seeded synthetic workloads (kv_cache_reads_amd.workload).
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from parity_util import (R, W, check_prefill, check_scan_error, check_summaries, check_y, hip_decode, hip_prefill,
                         host_unit, log, oracle_decode, oracle_prefill, prefill_span, decode_span)

pytestmark = pytest.mark.gpu
DEV = "cuda"

SMALL = {
    "c0": W.CONFIGS["c0"],
    # ragged mid-regions (not a multiple of any tile), several units and heads
    "c1_small": W.CONFIGS["c1"].with_(L=4096 + 37, K=(41,)),
    "c2_small": W.CONFIGS["c2"].with_(L=6000 + 3, K=(29, 59, 118, 236)),
    "c3_small": W.CONFIGS["c3"].with_(batch=2, layers=2, L=3000, K=(29,), steps=3),
    "c4_small": W.CONFIGS["c4"].with_(batch=1, layers=2, L=5003, K=(50,), steps=2),
}


def _gen(cfg):
    torch.manual_seed(0)
    return W.generate(cfg, device=DEV)


def _run_case(cfg, units, Ks=None, steps=None, check_pre=True, store_phi=True, fused_phi=False):
    inp = _gen(cfg)
    pre = hip_prefill(inp, store_phi=store_phi)
    torch.cuda.synchronize()
    steps = range(cfg.steps) if steps is None else steps
    Ks = cfg.K if Ks is None else Ks
    gpu = {}
    for K in Ks:
        for st in steps:
            out = hip_decode(inp, pre, K, st, fused_phi=fused_phi)
            gpu[(K, st)] = {k: v.cpu() for k, v in out.items() if v is not None}
    torch.cuda.synchronize()
    worst = (0.0, 0.0)
    for u in units:
        hu = host_unit(inp, u)
        ref_pre = oracle_prefill(cfg, hu)
        if check_pre:
            if pre[0] is not None:
                check_prefill(cfg, pre, u, ref_pre)
            _, M, _ = O.partition(cfg.L, cfg.n_sink, cfg.n_tail)
            check_summaries(cfg, pre, u, ref_pre, hu["v"][M])
        for (K, st), out in gpu.items():
            for g in range(cfg.G):
                y_ref, idx_ref, _ = oracle_decode(cfg, hu, ref_pre, K, st, g)
                idx = out["idx"][u, g].numpy().astype(np.int64)
                assert np.array_equal(idx, idx_ref), f"{cfg.name} unit {u} head {g} K={K} step {st}: top-K differs"
                a, r = check_y(out["y"][u, g].numpy(), y_ref, f"{cfg.name} u{u} g{g} K{K} s{st}")
                worst = (max(worst[0], a), max(worst[1], r))
    log(f"{cfg.name}: units {len(list(units))} worst abs {worst[0]:.2e} rel {worst[1]:.2e}")
    return inp, pre


@pytest.mark.parametrize("name", list(SMALL))
def test_small_configs_match_oracle(name):
    cfg = SMALL[name]
    log(f"case {name}: {cfg}")
    _run_case(cfg, range(cfg.U))


@pytest.mark.parametrize("name", [n for n in SMALL if SMALL[n].kv_dtype == "bf16"])
def test_small_configs_recomputed_phi_rows(name):
    """phi_k rows not stored: the merge recomputes the retrieved ones."""
    cfg = SMALL[name]
    log(f"case {name} (recomputed phi_k rows)")
    _run_case(cfg, range(cfg.U), store_phi=False)


@pytest.mark.parametrize("name", list(SMALL))
def test_small_configs_phi_q_inside_merge(name):
    """f = phi_q(q) computed inside the merge (no rma_phi_features launch)."""
    cfg = SMALL[name]
    log(f"case {name} (phi_q inside the merge)")
    _run_case(cfg, range(cfg.U), fused_phi=True)
    if cfg.kv_dtype == "bf16":
        _run_case(cfg, range(cfg.U), store_phi=False, fused_phi=True)


def test_phi_q_inside_merge_matches_separate_features():
    """Both ways compute f = elu(W q + b) + 1 in fp32 (different sum orders):
    the outputs agree to fp32 rounding of f."""
    cfg = SMALL["c1_small"]
    inp = _gen(cfg)
    pre = hip_prefill(inp)
    for flags in (R.RMA_MERGE_SUB, R.RMA_MERGE_NO_SUBTRACT, R.RMA_MERGE_NO_RESIDUAL):
        a = hip_decode(inp, pre, cfg.K[0], 0, flags=flags)
        b = hip_decode(inp, pre, cfg.K[0], 0, flags=flags, fused_phi=True)
        ya, yb = a["y"].double(), b["y"].double()
        rel = float(((ya - yb).norm(dim=-1) / ya.norm(dim=-1)).max())
        log(f"flags {flags}: separate vs fused phi_q max rel {rel:.2e}")
        assert rel <= 1e-5


def test_recomputed_phi_rows_match_stored_rows():
    """The recompute uses the builder's projection, rounding and MFMA order, so
    the rows subtracted equal the rows summed: y agrees with the stored-row path
    to fp32 rounding of the weights (a one-ulp bf16 difference in a row would
    show up at ~1e-3)."""
    cfg = SMALL["c1_small"]
    inp = _gen(cfg)
    K = cfg.K[0]
    a = hip_decode(inp, hip_prefill(inp, store_phi=True), K, 0)
    b = hip_decode(inp, hip_prefill(inp, store_phi=False), K, 0)
    assert torch.equal(a["idx"], b["idx"])
    ya, yb = a["y"].double(), b["y"].double()
    rel = float(((ya - yb).norm(dim=-1) / ya.norm(dim=-1)).max())
    log(f"stored vs recomputed rows: max rel {rel:.2e}")
    assert rel <= 1e-5
    sa, sb = a["stats"].double(), b["stats"].double()
    assert float(((sa[..., 3] - sb[..., 3]).abs() / sa[..., 3].abs()).max()) <= 1e-5


def test_c0_exact_ties_and_outputs():
    cfg = W.CONFIGS["c0"]
    inp, pre = _run_case(cfg, [0])
    # the three planted keys (identical vectors) are all retrieved by head 0
    out = hip_decode(inp, pre, cfg.K[0], 0)
    sel = set(out["idx"][0, 0].cpu().tolist())
    assert set(inp.needle_pos[0]) <= sel


@pytest.mark.parametrize("store_phi", [True, False])
@pytest.mark.parametrize("fused_phi", [False, True])
def test_c1_full(store_phi, fused_phi):
    cfg = W.CONFIGS["c1"]
    _run_case(cfg, range(cfg.U), store_phi=store_phi, fused_phi=fused_phi)


@pytest.mark.parametrize("store_phi", [True, False])
def test_c2_full_budget_sweep(store_phi):
    cfg = W.CONFIGS["c2"]
    _run_case(cfg, range(cfg.U), store_phi=store_phi)


@pytest.mark.parametrize("store_phi,fused_phi", [(True, False), (False, False), (True, True)])
def test_c3_full_sampled_units(store_phi, fused_phi):
    cfg = W.CONFIGS["c3"]
    # units spread over requests, layers and kv heads
    units = [0, 7, 129, 517, 1030, 1555, 2047]
    _run_case(cfg, units, check_pre=True, store_phi=store_phi, fused_phi=fused_phi)


def test_merge_variants_with_many_heads():
    """>= 2048 query heads at d=64 use the 256-thread merge: all three variants,
    both phi_q paths, against the oracle on sampled units."""
    cfg = W.CONFIGS["c3"].with_(batch=4, layers=16, L=700, K=(12,), steps=2)
    inp = _gen(cfg)
    pre = hip_prefill(inp)
    units = [0, 101, cfg.U - 1]
    variants = {R.RMA_MERGE_SUB: "sub", R.RMA_MERGE_NO_RESIDUAL: "topk", R.RMA_MERGE_NO_SUBTRACT: "nosub"}
    for flags, name in variants.items():
        for fused in (False, True):
            for st in range(cfg.steps):
                out = hip_decode(inp, pre, cfg.K[0], st, flags=flags, fused_phi=fused)
                y = out["y"].cpu()
                for u in units:
                    hu = host_unit(inp, u)
                    ref_pre = oracle_prefill(cfg, hu)
                    for g in range(cfg.G):
                        y_ref, _, _ = oracle_decode(cfg, hu, ref_pre, cfg.K[0], st, g, variant=name)
                        check_y(y[u, g].numpy(), y_ref, f"{name} fused={fused} u{u} g{g} s{st}")


@pytest.mark.slow
@pytest.mark.parametrize("store_phi", [True, False])
def test_c4_full_sampled_units(store_phi):
    cfg = W.CONFIGS["c4"]
    units = [0, 9, 230, 455, 895]   # both entropy regimes (even / odd layers)
    _run_case(cfg, units, steps=[0, 7], check_pre=True, store_phi=store_phi)


# ------------------------------------------------------------------ invariants on the GPU
def _manual_unit(L=2048, ns=4, nt=32, d=64, G=2, seed=0, ngen=0, kv_dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    T = L + ngen
    k = torch.randn(1, T, d, generator=g).to(kv_dtype)
    v = torch.randn(1, T, d, generator=g).to(kv_dtype)
    q = (1.5 * torch.randn(1, G, d, generator=g)).float()
    return k, v, q


def test_ideal_factorisation_recovers_full_attention():
    # keys from a 64-word codebook, phi_k = onehot(code), phi_q_c = e^{q.c/sqrt d}
    L, ns, nt, d, m, G = 3000, 4, 32, 64, 64, 2
    gen = torch.Generator().manual_seed(5)
    book = (0.5 * torch.randn(m, d, generator=gen)).bfloat16().float()
    codes = torch.randint(0, m, (L,), generator=gen)
    k = book[codes][None].bfloat16()
    v = torch.randn(1, L, d, generator=gen).bfloat16()
    q = torch.randn(1, G, d, generator=gen).float()
    M = torch.arange(ns, L - nt)
    phi_k = torch.nn.functional.one_hot(codes[M], m).bfloat16()[None]
    f = torch.exp(q.double() @ book.double().T / math.sqrt(d)).float()          # [1, G, m]
    span = R.Span(L, ns, nt, 0)
    kd, vd = k.to(DEV), v.to(DEV)
    phi_d, S, u, kappa = R.rma_build_summaries(kd, vd, span, None, None, m=m, phi_k=phi_k.to(DEV))
    kf, vf = k[0].double().numpy(), v[0].double().numpy()
    for K in (0, 1, 77, 1500, L - ns - nt - 1, L - ns - nt):
        idx, sel = (R.rma_decode_topk(q.to(DEV), kd, span, kappa, K) if K > 0 else (None, None))
        y = R.rma_decode_merge(q.to(DEV), f.to(DEV), kd, vd, span, idx, sel, K, phi_d, S, u).cpu()
        for g in range(G):
            y_full = O.full_attention(q[0, g].numpy(), kf, vf, L)
            check_y(y[0, g].numpy(), y_full, f"codebook K={K} g={g}")


@pytest.mark.parametrize("kv_dtype", [torch.bfloat16, torch.float32])
def test_whole_mid_retrieved_needs_no_phi_rows(kv_dtype):
    """K = |M| with the subtraction variant: the residual is exactly zero, so the
    merge reads no phi_k row and accepts neither rows nor Wk (a regression test:
    the rows used to be loaded through the NULL pointer).  y equals full
    attention over the prefill segment and the generated tokens (Eq. 1)."""
    L, ns, nt, G, ngen = 700, 4, 32, 3, 2
    k, v, q = _manual_unit(L=L, G=G, ngen=ngen, kv_dtype=kv_dtype)
    K = L - ns - nt
    kd, vd, qd = k.to(DEV), v.to(DEV), q.to(DEV)
    sp = R.Span(L, ns, nt, ngen)
    kappa = torch.full((1,), float(k[0].float().norm(dim=-1).max()) * 1.001, device=DEV)
    idx, sel = R.rma_decode_topk(qd, kd, sp, kappa, K)
    f = torch.ones(1, G, 128, device=DEV)
    S = torch.zeros(1, 128, 64, device=DEV)
    u = torch.zeros(1, 128, device=DEV)
    y, stats = R.rma_decode_merge(qd, f, kd, vd, sp, idx, sel, K, None, S, u, want_stats=True)
    y = y.cpu()
    kf, vf = k[0].double().numpy(), v[0].double().numpy()
    for g in range(G):
        y_full = O.full_attention(q[0, g].numpy(), kf, vf, L + ngen)
        check_y(y[0, g].numpy(), y_full, f"K = |M| without phi rows, g={g}")
    assert torch.all(stats[..., 2] == 0) and torch.all(stats[..., 3] == 0)


def test_zero_features_give_selection_only_topk():
    k, v, q = _manual_unit(L=4000, G=3, ngen=2)
    cfgW = torch.randn(1, 128, 64) / 8
    cfgb = torch.randn(1, 128) / 8
    L, ns, nt, K = 4000, 4, 32, 40
    kd, vd = k.to(DEV), v.to(DEV)
    pre = R.rma_build_summaries(kd, vd, R.Span(L, ns, nt, 0), cfgW.to(DEV), cfgb.to(DEV))
    sp = R.Span(L, ns, nt, 2)
    idx, sel = R.rma_decode_topk(q.to(DEV), kd, sp, pre[3], K)
    zero = torch.zeros(1, 3, 128, device=DEV)
    y0 = R.rma_decode_merge(q.to(DEV), zero, kd, vd, sp, idx, sel, K, pre[0], pre[1], pre[2]).cpu()
    y1 = R.rma_decode_merge(q.to(DEV), None, kd, vd, sp, idx, sel, K, None, None, None,
                            flags=R.RMA_MERGE_NO_RESIDUAL, m=128).cpu()
    kf, vf = k[0].double().numpy(), v[0].double().numpy()
    for g in range(3):
        sel_ref = O.topk_indices(q[0, g].numpy(), kf[ns:L - nt], K, first_index=ns)
        assert np.array_equal(idx[0, g].cpu().numpy(), sel_ref)
        E = np.concatenate([np.arange(ns), sel_ref, np.arange(L - nt, L), [L, L + 1]])
        s = kf[E] @ q[0, g].double().numpy() / 8.0
        p = np.exp(s - s.max())
        y_ref = (p @ vf[E]) / p.sum()
        check_y(y0[0, g].numpy(), y_ref, "f=0")
        check_y(y1[0, g].numpy(), y_ref, "NO_RESIDUAL")


def test_merge_variants_match_oracle():
    cfg = SMALL["c1_small"]
    inp = _gen(cfg)
    pre = hip_prefill(inp)
    K = cfg.K[0]
    for flags, variant in ((R.RMA_MERGE_NO_RESIDUAL, "topk"), (R.RMA_MERGE_NO_SUBTRACT, "nosub")):
        out = hip_decode(inp, pre, K, 0, flags=flags)
        for u in (0, cfg.U - 1):
            hu = host_unit(inp, u)
            rp = oracle_prefill(cfg, hu)
            for g in range(cfg.G):
                y_ref, _, _ = oracle_decode(cfg, hu, rp, K, 0, g, variant=variant)
                check_y(out["y"][u, g].cpu().numpy(), y_ref, f"{variant} u{u} g{g}")


def test_determinism_and_gqa_equivalence():
    cfg = SMALL["c1_small"]
    inp = _gen(cfg)
    pre = hip_prefill(inp)
    pre2 = hip_prefill(inp)
    for a, b in zip(pre, pre2):
        assert torch.equal(a, b)
    K = cfg.K[0]
    o1 = hip_decode(inp, pre, K, 0)
    o2 = hip_decode(inp, pre, K, 0)
    for key in ("idx", "sel", "y"):
        assert torch.equal(o1[key], o2[key]), key
    # each query head alone (G = 1, the kv head replicated per query head)
    U, G = cfg.U, cfg.G
    q = inp.q[0]                                      # [U, G, d]
    k1 = inp.k.repeat_interleave(G, dim=0)
    v1 = inp.v.repeat_interleave(G, dim=0)
    sp = R.Span(cfg.L, cfg.n_sink, cfg.n_tail, 0)
    kap1 = pre[3].repeat_interleave(G)
    idx1, sel1 = R.rma_decode_topk(q.reshape(U * G, 1, -1).contiguous(), k1, sp, kap1, K)
    assert torch.equal(idx1.view(U, G, K), o1["idx"])


def test_workspace_reuse_across_unit_counts():
    # the workspace holds scratch only: garbage left in it (here every byte
    # 0xff, over > 1024 units) must not change any result
    cfg = W.CONFIGS["c3"].with_(batch=9, layers=16, L=600, K=(6,), steps=1)   # 1152 units
    inp = _gen(cfg)
    ws = R.Workspace()
    buf = ws.get(64 << 20)
    buf[:] = 255
    pre = hip_prefill(inp, ws=ws)
    out = hip_decode(inp, pre, cfg.K[0], 0, ws=ws)
    for u in (0, 1030, cfg.U - 1):
        hu = host_unit(inp, u)
        rp = oracle_prefill(cfg, hu)
        for g in range(cfg.G):
            y_ref, idx_ref, _ = oracle_decode(cfg, hu, rp, cfg.K[0], 0, g)
            assert np.array_equal(out["idx"][u, g].cpu().numpy(), idx_ref)
            check_y(out["y"][u, g].cpu().numpy(), y_ref, f"ws reuse u{u} g{g}")


# ------------------------------------------------------------------ adversarial selection
# Every adversarial case runs for both head dims and both key dtypes: the scan,
# the select's band rescoring and the exact fallback are instantiated per
# (key dtype, d).
KEY_KINDS = [(64, torch.bfloat16), (128, torch.bfloat16), (64, torch.float32), (128, torch.float32)]
KEY_IDS = [f"d{d}-{str(t).split('.')[-1]}" for d, t in KEY_KINDS]


def _topk_case(k, q, L, ns, nt, K, units=(0,)):
    d = k.shape[2]
    kd = k.to(DEV)
    v = torch.zeros_like(k)
    pre = R.rma_build_summaries(kd, v.to(DEV), R.Span(L, ns, nt, 0), torch.randn(1, 64, d, device=DEV) / 8,
                                torch.zeros(1, 64, device=DEV))
    idx, sel = R.rma_decode_topk(q.to(DEV), kd, R.Span(L, ns, nt, 0), pre[3], K)
    for u in units:
        kf = k[u].double().numpy()
        for g in range(q.shape[1]):
            ref = O.topk_indices(q[u, g].numpy(), kf[ns:L - nt], K, first_index=ns)
            got = idx[u, g].cpu().numpy()
            assert np.array_equal(got, ref), \
                f"d={d} {k.dtype} K={K} unit {u} head {g}: {np.setdiff1d(got, ref)[:8]} vs {np.setdiff1d(ref, got)[:8]}"
            # selected scores are the fp32 scores of the selected tokens
            s_ref = kf[got] @ q[u, g].double().numpy() / math.sqrt(d)
            assert np.allclose(sel[u, g].cpu().numpy(), s_ref, rtol=1e-5, atol=1e-5 * np.abs(s_ref).max())
            check_scan_error(sel[u, g].cpu().numpy(), s_ref, q[u, g], kf, d, f"d={d} {k.dtype} K={K} u{u} g{g}")
    return idx


def _one_ulp_apart(base, i, dtype):
    """A copy of `base` (already in `dtype`) with component i % d moved by -1, 0
    or +1 unit in the last place of that dtype."""
    kk = base.clone()
    if dtype == torch.bfloat16:
        kk.view(torch.int16)[i % kk.numel()] += (i % 3) - 1
    else:
        kk.view(torch.int32)[i % kk.numel()] += (i % 3) - 1
    return kk.float()


@pytest.mark.parametrize("d,dtype", KEY_KINDS, ids=KEY_IDS)
@pytest.mark.parametrize("K", [1, 7, 300, 1999, 2000 - 36 - 1, 2000 - 36])
def test_topk_all_equal_keys(K, d, dtype):
    L, ns, nt = 2000, 4, 32
    k = torch.ones(1, L, d).to(dtype)
    q = torch.randn(1, 2, d)
    if K <= L - ns - nt:
        _topk_case(k, q, L, ns, nt, K)


@pytest.mark.parametrize("d,dtype", KEY_KINDS, ids=KEY_IDS)
def test_topk_planted_ties_and_near_ties_at_the_boundary(d, dtype):
    L, ns, nt, K = 6000, 4, 64, 50
    g = torch.Generator().manual_seed(3)
    k = torch.randn(1, L, d, generator=g)
    q = torch.randn(1, 4, d, generator=g)
    qh = q[0, 0] / q[0, 0].norm()
    # 60 copies of one key straddle the K-th boundary (exact ties -> lower index)
    pos = torch.randperm(L - ns - nt, generator=g)[:60] + ns
    k[0, pos] = (3.0 * qh).to(dtype).float()
    # near-ties: keys one ulp (of the key dtype) apart in one component
    base = (2.5 * qh).to(dtype)
    pos2 = torch.randperm(L - ns - nt, generator=g)[:40] + ns
    for i, p in enumerate(pos2.tolist()):
        k[0, p] = _one_ulp_apart(base, i, dtype)
    _topk_case(k.to(dtype), q, L, ns, nt, K)
    _topk_case(k.to(dtype), q, L, ns, nt, 75)


@pytest.mark.parametrize("d,dtype", KEY_KINDS, ids=KEY_IDS)
def test_topk_sorted_keys_force_fallback(d, dtype):
    # scores increase with position: every chunk holds only top tokens at its end;
    # the per-chunk reports cannot certify completeness and the exact path runs
    L, ns, nt = 3000, 4, 32
    q = torch.zeros(1, 1, d)
    q[0, 0, 0] = 1.0
    k = torch.zeros(1, L, d)
    k[0, :, 0] = torch.linspace(-2, 2, L)
    _topk_case(k.to(dtype), q, L, ns, nt, 500)
    _topk_case(k.to(dtype), q, L, ns, nt, 5)


@pytest.mark.parametrize("d,dtype", KEY_KINDS, ids=KEY_IDS)
def test_topk_many_units_use_small_select_blocks(d, dtype):
    """U*G >= 1024 (query heads) selects with 256-thread blocks: the tie and
    near-tie case and the forced exact fallback on that path."""
    L, ns, nt, U, G = 3000, 4, 32, 256, 4
    g = torch.Generator().manual_seed(5)
    k = torch.randn(U, L, d, generator=g)
    q = torch.randn(U, G, d, generator=g)
    qh = q[0, 0] / q[0, 0].norm()
    pos = torch.randperm(L - ns - nt, generator=g)[:40] + ns
    k[0, pos] = (3.0 * qh).to(dtype).float()            # exact ties at the boundary in unit 0
    k[U - 1, :, 0] = torch.linspace(-2, 2, L)            # unit U-1: sorted scores for head 0 ...
    k[U - 1, :, 1:] = 0.0
    q[U - 1, 0] = 0.0
    q[U - 1, 0, 0] = 1.0                                  # ... which forces the exact fallback
    _topk_case(k.to(dtype), q, L, ns, nt, 30, units=(0, 17, U - 1))
    _topk_case(k.to(dtype), q, L, ns, nt, 500, units=(0, U - 1))


def _select_layout(L, ns, nt, U, G, K, d=64):
    """The plan's chunking of the mid-region and the select's slot layout (the
    rule the library applies): (chunks, report capacity, grouped).  With a
    1024-thread select block each chunk's report slots belong to a group of
    1024 / 2^ceil(log2(chunks)) threads; when the capacity exceeds eight slots
    per thread of that group the wide-union path runs instead."""
    Lm = L - ns - nt
    tile = 64 if d == 64 else 32
    # tokens per chunk whose fp32 scores fit the scan block's LDS budget (54272
    # bytes: G score rows of ch + 8 words beside G 512-bin histograms and queries)
    ch_max = max(tile, ((54272 - G * (512 * 4 + d * 4) - 64) // (4 * G) - 8) // tile * tile)
    lo, hi = -(-Lm // ch_max), min(256, -(-Lm // tile))
    nc = max(lo, min(-(-512 // U), hi))
    ch = -(-(-(-Lm // nc)) // tile) * tile
    chunks = -(-Lm // ch)
    if K >= Lm:
        r_cap = ch
    else:
        mu = K / chunks
        rmin = max(16, (math.ceil(mu + 4 * math.sqrt(mu) + 4) + 7) // 8 * 8)
        r_cap = min(ch, 2 * min(ch, rmin) + 32)
    tpc = 1024 >> ((chunks - 1).bit_length() if chunks > 1 else 0)
    return chunks, r_cap, r_cap <= 8 * tpc


# (L, U, G, K, chunks, grouped): one chunk; chunk counts that are not powers of
# two on both report layouts (the wide one when the budget is large); a chunk
# count whose groups are four threads wide
SELECT_LAYOUTS = [
    (100, 1, 2, 10, 1, True),
    (5000, 1, 3, 50, 78, True),
    (3000, 2, 4, 300, 47, True),
    (12000, 8, 1, 2000, 63, False),
    (20000, 1, 3, 200, 156, False),
]


@pytest.mark.parametrize("case", SELECT_LAYOUTS, ids=lambda c: f"L{c[0]}U{c[1]}G{c[2]}K{c[3]}")
def test_topk_report_layouts(case):
    L, U, G, K, chunks, grouped = case
    ns, nt = 4, 32
    assert _select_layout(L, ns, nt, U, G, K)[0::2] == (chunks, grouped), _select_layout(L, ns, nt, U, G, K)
    g = torch.Generator().manual_seed(L + K)
    k = torch.randn(U, L, 64, generator=g)
    q = torch.randn(U, G, 64, generator=g)
    _topk_case(k.bfloat16(), q, L, ns, nt, K, units=tuple(range(U)))
