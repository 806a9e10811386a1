"""GPU parity of rma_decode (Top-K and merge in one call, through the C ABI).

* Against the two separate calls (rma_decode_topk, rma_decode_merge) on the
  same inputs: identical indices and selected scores; y equal up to fp32
  summation order (the fused kernel spreads a head's entries over more lane
  groups), relative difference <= 1e-5.
* Against the fp64 oracle: bit-exact Top-K, y within 2e-3 abs / 1e-2 rel, on
  every workload (small shapes with ragged tails; c1 and the c2 budget sweep in
  full; sampled units of c3 and c4 in the launch configuration bench.py times),
  all three merge variants, both phi_q sources.
* The kernels that run: the fused select-and-merge kernel where the plan
  allows it (with the slice combine when a head's list is split over several
  blocks), the separate select and merge kernels otherwise (recomputed phi_k
  rows, K = 0), checked through the kernel trace.
"""
import numpy as np
import pytest
import torch

import oracle as O
from parity_util import (R, W, check_prefill, check_summaries, check_y, hip_decode,
                         hip_decode_one_call, hip_prefill, host_unit, log, oracle_decode,
                         oracle_prefill)

pytestmark = pytest.mark.gpu
DEV = "cuda"

SMALL = {
    "c0": W.CONFIGS["c0"],
    "c1_small": W.CONFIGS["c1"].with_(L=4096 + 37, K=(41,)),
    "c2_small": W.CONFIGS["c2"].with_(L=6000 + 3, K=(29, 59, 118, 236)),
    "c3_small": W.CONFIGS["c3"].with_(batch=2, layers=2, L=3000, K=(29,), steps=3),
    "c4_small": W.CONFIGS["c4"].with_(batch=1, layers=2, L=5003, K=(50,), steps=2),
}
VARIANTS = {R.RMA_MERGE_SUB: "sub", R.RMA_MERGE_NO_RESIDUAL: "topk", R.RMA_MERGE_NO_SUBTRACT: "nosub"}


def _gen(cfg):
    torch.manual_seed(0)
    return W.generate(cfg, device=DEV)


def _kernels(fn):
    """Names of the kernels one call enqueues (the library's kernel trace)."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
    R.rma_trace_arm(evs)
    fn()
    torch.cuda.synchronize()
    return R.rma_trace_kernels()


def _rel(a, b):
    a, b = a.double(), b.double()
    return float(((a - b).norm(dim=-1) / b.norm(dim=-1).clamp_min(1e-300)).max())


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("flags", list(VARIANTS), ids=list(VARIANTS.values()))
def test_one_call_matches_two_calls(name, flags):
    cfg = SMALL[name]
    inp = _gen(cfg)
    pre = hip_prefill(inp)
    for K in cfg.K:
        for st in range(cfg.steps):
            for fused_phi in (False, True):
                a = hip_decode(inp, pre, K, st, flags=flags, fused_phi=fused_phi)
                b = hip_decode_one_call(inp, pre, K, st, flags=flags, fused_phi=fused_phi)
                assert torch.equal(a["idx"], b["idx"]), f"{name} K={K} step {st}: indices differ"
                assert torch.equal(a["sel"], b["sel"]), f"{name} K={K} step {st}: scores differ"
                r = _rel(b["y"], a["y"])
                assert r <= 1e-5, f"{name} K={K} step {st} fused_phi={fused_phi}: y rel {r:.2e}"
                sa, sb = a["stats"].double(), b["stats"].double()
                assert torch.equal(sa[..., 0], sb[..., 0])                    # m*: a maximum
                assert float(((sa[..., 1:] - sb[..., 1:]).abs() / sa[..., 1:].abs().clamp_min(1e-30)).max()) <= 1e-5


def _oracle_case(cfg, units, Ks=None, steps=None, store_phi=True, fused_phi=False, flags=R.RMA_MERGE_SUB):
    inp = _gen(cfg)
    pre = hip_prefill(inp, store_phi=store_phi)
    torch.cuda.synchronize()
    steps = range(cfg.steps) if steps is None else steps
    Ks = cfg.K if Ks is None else Ks
    gpu = {}
    for K in Ks:
        for st in steps:
            out = hip_decode_one_call(inp, pre, K, st, flags=flags, fused_phi=fused_phi)
            gpu[(K, st)] = {k: v.cpu() for k, v in out.items() if v is not None}
    worst = (0.0, 0.0)
    for u in units:
        hu = host_unit(inp, u)
        ref_pre = oracle_prefill(cfg, hu)
        for (K, st), out in gpu.items():
            for g in range(cfg.G):
                y_ref, idx_ref, _ = oracle_decode(cfg, hu, ref_pre, K, st, g, variant=VARIANTS[flags])
                idx = out["idx"][u, g].numpy().astype(np.int64)
                assert np.array_equal(idx, idx_ref), f"{cfg.name} unit {u} head {g} K={K} step {st}: top-K differs"
                a, r = check_y(out["y"][u, g].numpy(), y_ref, f"{cfg.name} u{u} g{g} K{K} s{st}")
                worst = (max(worst[0], a), max(worst[1], r))
    log(f"{cfg.name} one call: units {len(list(units))} worst abs {worst[0]:.2e} rel {worst[1]:.2e}")
    return inp, pre


@pytest.mark.parametrize("name", list(SMALL))
def test_one_call_matches_oracle(name):
    cfg = SMALL[name]
    _oracle_case(cfg, range(cfg.U))
    _oracle_case(cfg, range(cfg.U), fused_phi=True)


@pytest.mark.parametrize("flags", [R.RMA_MERGE_NO_RESIDUAL, R.RMA_MERGE_NO_SUBTRACT], ids=["topk", "nosub"])
def test_one_call_variants_match_oracle(flags):
    cfg = SMALL["c1_small"]
    _oracle_case(cfg, (0, cfg.U - 1), flags=flags)


def test_one_call_c1_full():
    cfg = W.CONFIGS["c1"]
    _oracle_case(cfg, range(cfg.U), fused_phi=True)


def test_one_call_c2_full_budget_sweep():
    cfg = W.CONFIGS["c2"]
    _oracle_case(cfg, range(cfg.U), fused_phi=True)


def test_one_call_c3_sampled_units():
    cfg = W.CONFIGS["c3"]
    _oracle_case(cfg, [0, 7, 129, 517, 1030, 1555, 2047], steps=[0, 7], fused_phi=True)


def test_one_call_c4_sampled_units():
    cfg = W.CONFIGS["c4"]
    _oracle_case(cfg, [0, 9, 230, 455, 895], steps=[0, 7], fused_phi=True)


def test_kernels_that_run():
    """c1 and the c2 budget sweep: scan + fused kernel; recomputed phi_k rows
    and K = 0: the separate kernels."""
    cfg = W.CONFIGS["c1"]
    inp = _gen(cfg)
    pre = hip_prefill(inp)
    pre_nophi = hip_prefill(inp, store_phi=False)
    K = cfg.K[0]
    names = _kernels(lambda: hip_decode_one_call(inp, pre, K, 0, fused_phi=True))
    log(f"c1 K={K}: {names}")
    assert names == ["topk_scan_kernel", "decode_fused_kernel"], names
    names = _kernels(lambda: hip_decode_one_call(inp, pre_nophi, K, 0, fused_phi=True))
    assert names == ["topk_scan_kernel", "topk_select_kernel", "merge_kernel"], names
    names = _kernels(lambda: hip_decode_one_call(inp, pre, 0, 0, fused_phi=True, want_idx=False))
    assert names == ["merge_kernel"], names
    cfg2 = W.CONFIGS["c2"]
    inp2 = _gen(cfg2)
    pre2 = hip_prefill(inp2)
    # the fused kernel's LDS (report slots + list + its own) fits the whole
    # c2 budget sweep; from four gather rounds on (K = 1310 with 256 entries per
    # round) each head's list is split over several blocks and the slices are
    # combined by a second kernel
    for K2 in cfg2.K:
        names = _kernels(lambda: hip_decode_one_call(inp2, pre2, K2, 0, fused_phi=True))
        log(f"c2 K={K2}: {names}")
        if K2 < 1310:
            assert names == ["topk_scan_kernel", "decode_fused_kernel"], names
        else:
            assert names == ["topk_scan_kernel", "decode_fused_kernel", "merge_combine_kernel"], names


def test_one_call_without_index_outputs_and_recomputed_rows():
    """idx / sel not requested gives the same y; recomputed phi_k rows (separate
    kernels) agree with stored rows."""
    cfg = SMALL["c1_small"]
    inp = _gen(cfg)
    pre = hip_prefill(inp)
    K = cfg.K[0]
    a = hip_decode_one_call(inp, pre, K, 0, fused_phi=True)
    b = hip_decode_one_call(inp, pre, K, 0, fused_phi=True, want_idx=False)
    assert torch.equal(a["y"], b["y"])
    c = hip_decode_one_call(inp, hip_prefill(inp, store_phi=False), K, 0, fused_phi=True)
    assert torch.equal(a["idx"], c["idx"])
    assert _rel(c["y"], a["y"]) <= 1e-5


def test_one_call_whole_mid_region_and_deterministic():
    cfg = SMALL["c0"]
    inp = _gen(cfg)
    pre = hip_prefill(inp)
    K = cfg.L_mid
    a = hip_decode_one_call(inp, pre, K, 0)
    b = hip_decode_one_call(inp, pre, K, 0)
    assert torch.equal(a["y"], b["y"]) and torch.equal(a["idx"], b["idx"])
    kf = inp.k[0].double().cpu().numpy()
    vf = inp.v[0].double().cpu().numpy()
    for g in range(cfg.G):
        y_full = O.full_attention(inp.q[0, 0, g].cpu().numpy(), kf, vf, cfg.L)
        check_y(a["y"][0, g].cpu().numpy(), y_full, f"K = |M| one call, g={g}")
