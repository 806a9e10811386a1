"""The fused select-and-merge kernel on adversarial selections (through rma_decode).

The cases of the Top-K tests in test_gpu_parity.py, run through the one-call
decode for both head dims and both key dtypes: all-equal keys (K up to the whole
mid-region), exact ties and near-ties at the K-th boundary (the band split by
double-double scores from lane groups), keys sorted by score (the certificate
fails and the block runs the exact fallback), many heads (256- and 512-thread
blocks), and report layouts whose chunk counts are not powers of two or whose
reports need several placement rounds.  In every case:
* the indices equal the oracle's exact Top-K (bit for bit) and the kept scores
  the fp32 scores of the selected tokens;
* y, the indices and the kept scores equal those of the two separate calls
  (rma_decode_topk + rma_decode_merge).  y may differ in fp32 summation order
  only: within 1e-5 of |y| plus 1e-6 sqrt(d) rms(v), the floor for sums that
  cancel (all-equal keys average thousands of random values into a y about
  sqrt(n) times smaller than they are);
* the fused kernel is the one that ran (with the slice combine when the plan
  splits a head's list over several blocks: few heads, four or more rounds).
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from kv_cache_reads_amd import rma as R
from parity_util import check_scan_error

pytestmark = pytest.mark.gpu
DEV = "cuda"

KEY_KINDS = [(64, torch.bfloat16), (128, torch.bfloat16), (64, torch.float32), (128, torch.float32)]
KEY_IDS = [f"d{d}-{str(t).split('.')[-1]}" for d, t in KEY_KINDS]


def _kernels(fn):
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
    R.rma_trace_arm(evs)
    fn()
    torch.cuda.synchronize()
    return R.rma_trace_kernels()


def _decode_case(k, q, L, ns, nt, K, units=(0,), m=64, seed=0):
    U, G, d = q.shape
    g = torch.Generator().manual_seed(seed)
    kd = k.to(DEV)
    v = torch.randn(k.shape, generator=g).to(k.dtype).to(DEV)
    W = (torch.randn(1, m, d, generator=g) / (2 * math.sqrt(d))).to(DEV)
    b = (torch.randn(1, m, generator=g) / 4).to(DEV)
    sp = R.Span(L, ns, nt, 0)
    phi_k, S, u, kappa = R.rma_build_summaries(kd, v, sp, W, b)
    qd = q.to(DEV)
    fused = {}

    def one_call():
        fused["y"], fused["idx"], fused["sel"], fused["st"] = R.rma_decode(
            qd, None, kd, v, sp, kappa, K, phi_k, S, u, m=m, want_idx=True, want_stats=True, Wq=W, bq=b)

    names = _kernels(one_call)
    assert names[:2] == ["topk_scan_kernel", "decode_fused_kernel"], names
    assert names[2:] in ([], ["merge_combine_kernel"]), names   # a split list's slice combine
    idx2, sel2 = R.rma_decode_topk(qd, kd, sp, kappa, K)
    y2, st2 = R.rma_decode_merge(qd, None, kd, v, sp, idx2, sel2, K, phi_k, S, u, m=m, want_stats=True,
                                 Wq=W, bq=b)
    torch.cuda.synchronize()
    assert torch.equal(fused["idx"], idx2), f"d={d} {k.dtype} K={K}: indices differ from the two calls"
    assert torch.equal(fused["sel"], sel2), f"d={d} {k.dtype} K={K}: kept scores differ from the two calls"
    yf, ys = fused["y"].double(), y2.double()
    bound = 1e-5 * ys.norm(dim=-1) + 1e-6 * math.sqrt(d) * float(v.double().pow(2).mean().sqrt())
    excess = float(((yf - ys).norm(dim=-1) / bound).max())
    assert excess <= 1.0, f"d={d} {k.dtype} K={K}: y differs from the two calls by {excess:.2f}x the bound"
    assert torch.equal(fused["st"][..., 0], st2[..., 0])   # m*: a maximum over the same scores
    idx = fused["idx"].cpu()
    sel = fused["sel"].cpu()
    for uu in units:
        kf = k[uu].double().numpy()
        for gg in range(G):
            ref = O.topk_indices(q[uu, gg].numpy(), kf[ns:L - nt], K, first_index=ns)
            got = idx[uu, gg].numpy()
            assert np.array_equal(got, ref), \
                f"d={d} {k.dtype} K={K} unit {uu} head {gg}: {np.setdiff1d(got, ref)[:8]} vs {np.setdiff1d(ref, got)[:8]}"
            s_ref = kf[got] @ q[uu, gg].double().numpy() / math.sqrt(d)
            assert np.allclose(sel[uu, gg].numpy(), s_ref, rtol=1e-5, atol=1e-5 * np.abs(s_ref).max())
            check_scan_error(sel[uu, gg].numpy(), s_ref, q[uu, gg], kf, d, f"d={d} {k.dtype} K={K} u{uu} g{gg}")
    return fused


def _one_ulp_apart(base, i, dtype):
    kk = base.clone()
    if dtype == torch.bfloat16:
        kk.view(torch.int16)[i % kk.numel()] += (i % 3) - 1
    else:
        kk.view(torch.int32)[i % kk.numel()] += (i % 3) - 1
    return kk.float()


@pytest.mark.parametrize("d,dtype", KEY_KINDS, ids=KEY_IDS)
@pytest.mark.parametrize("K", [1, 7, 300, 1963, 1964])
def test_decode_all_equal_keys(K, d, dtype):
    L, ns, nt = 2000, 4, 32          # the mid-region holds 1964 tokens
    k = torch.ones(1, L, d).to(dtype)
    q = torch.randn(1, 2, d, generator=torch.Generator().manual_seed(K))
    _decode_case(k, q, L, ns, nt, K)


@pytest.mark.parametrize("d,dtype", KEY_KINDS, ids=KEY_IDS)
def test_decode_planted_ties_and_near_ties_at_the_boundary(d, dtype):
    L, ns, nt, K = 6000, 4, 64, 50
    g = torch.Generator().manual_seed(3)
    k = torch.randn(1, L, d, generator=g)
    q = torch.randn(1, 4, d, generator=g)
    qh = q[0, 0] / q[0, 0].norm()
    pos = torch.randperm(L - ns - nt, generator=g)[:60] + ns
    k[0, pos] = (3.0 * qh).to(dtype).float()
    base = (2.5 * qh).to(dtype)
    pos2 = torch.randperm(L - ns - nt, generator=g)[:40] + ns
    for i, p in enumerate(pos2.tolist()):
        k[0, p] = _one_ulp_apart(base, i, dtype)
    _decode_case(k.to(dtype), q, L, ns, nt, K)
    _decode_case(k.to(dtype), q, L, ns, nt, 75)


@pytest.mark.parametrize("d,dtype", KEY_KINDS, ids=KEY_IDS)
def test_decode_sorted_keys_force_fallback(d, dtype):
    L, ns, nt = 3000, 4, 32
    q = torch.zeros(1, 1, d)
    q[0, 0, 0] = 1.0
    k = torch.zeros(1, L, d)
    k[0, :, 0] = torch.linspace(-2, 2, L)
    _decode_case(k.to(dtype), q, L, ns, nt, 500)
    _decode_case(k.to(dtype), q, L, ns, nt, 5)


@pytest.mark.parametrize("d,dtype", KEY_KINDS, ids=KEY_IDS)
def test_decode_many_heads_use_smaller_blocks(d, dtype):
    """U*G >= 1024 query heads: 256-thread fused blocks at d = 64, 512 at d = 128;
    ties at the boundary in unit 0, the exact fallback for head 0 of the last unit."""
    L, ns, nt, U, G = 3000, 4, 32, 256, 4
    g = torch.Generator().manual_seed(5)
    k = torch.randn(U, L, d, generator=g)
    q = torch.randn(U, G, d, generator=g)
    qh = q[0, 0] / q[0, 0].norm()
    pos = torch.randperm(L - ns - nt, generator=g)[:40] + ns
    k[0, pos] = (3.0 * qh).to(dtype).float()
    k[U - 1, :, 0] = torch.linspace(-2, 2, L)
    k[U - 1, :, 1:] = 0.0
    q[U - 1, 0] = 0.0
    q[U - 1, 0, 0] = 1.0
    _decode_case(k.to(dtype), q, L, ns, nt, 30, units=(0, 17, U - 1))
    _decode_case(k.to(dtype), q, L, ns, nt, 500, units=(0, U - 1))


# (L, U, G, K): one chunk; chunk counts that are not powers of two; reports wider
# than one placement round of the fused kernel's threads (several rounds)
LAYOUTS = [(100, 1, 2, 10), (5000, 1, 3, 50), (3000, 2, 4, 300), (12000, 8, 1, 2000), (20000, 1, 3, 200)]


@pytest.mark.parametrize("case", LAYOUTS, ids=lambda c: f"L{c[0]}U{c[1]}G{c[2]}K{c[3]}")
def test_decode_report_layouts(case):
    L, U, G, K = case
    ns, nt, d = 4, 32, 64
    g = torch.Generator().manual_seed(L + K)
    k = torch.randn(U, L, d, generator=g).to(torch.bfloat16)
    q = torch.randn(U, G, d, generator=g)
    _decode_case(k, q, L, ns, nt, K, units=range(U))
