"""rma_decode_topk_static (the Top-K call that allocates nothing: its scratch is
the library's static device array) against rma_decode_topk with a workspace,
through the C ABI: two calls in a row, the second on a smaller input with
another head dim, each bit-exact in indices and scores; an oversized call is
refused with RMA_ERR_WORKSPACE and leaves its outputs untouched."""
import ctypes

import pytest
import torch

from kv_cache_reads_amd import rma as R
from kv_cache_reads_amd import workload as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _static_call(q, k, span, kappa, K, idx, sel):
    kv, sp = R._kv(k, None), span._c()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return R.lib().rma_decode_topk_static(R._p(q), q.shape[1], ctypes.byref(kv), ctypes.byref(sp),
                                          R._p(kappa), K, R._p(idx), R._p(sel), st)


def _kappa(k, span):
    mid = k[:, span.n_sink:span.L - span.n_tail].float()
    return (mid.norm(dim=-1).amax(dim=1) * (1 + 1e-5)).contiguous()


def _case(cfg, K):
    torch.manual_seed(0)
    inp = W.generate(cfg, device=DEV)
    span = R.Span(cfg.L, cfg.n_sink, cfg.n_tail, 0)
    q = inp.q[0].contiguous()
    return q, inp.k, span, _kappa(inp.k, span), K


def _check(case):
    q, k, span, kappa, K = case
    U, G, _ = q.shape
    idx_ref, sel_ref = R.rma_decode_topk(q, k, span, kappa, K)
    idx = torch.full((U, G, K), -7, dtype=torch.int32, device=DEV)
    sel = torch.full((U, G, K), -7.0, dtype=torch.float32, device=DEV)
    assert _static_call(q, k, span, kappa, K, idx, sel) == R.RMA_OK, R.lib().rma_last_error()
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_ref), "indices differ from rma_decode_topk"
    assert torch.equal(sel, sel_ref), "scores differ from rma_decode_topk"


def test_static_scratch_topk_matches_workspace_topk():
    big = _case(W.CONFIGS["c1"], 328)                                   # 8 units x 4 heads, 32K
    small = _case(W.CONFIGS["c2"].with_(L=5003, K=(50,)), 50)          # 8 units x 3 heads, d = 128
    print(f"scratch needed: c1 {R.rma_workspace_bytes(R.RMA_OP_DECODE_TOPK, big[1], big[2], 4, 328)} B, "
          f"small {R.rma_workspace_bytes(R.RMA_OP_DECODE_TOPK, small[1], small[2], 3, 50)} B", flush=True)
    _check(big)
    _check(small)      # second call, smaller: the array keeps the first call's bytes


def test_static_scratch_refuses_oversized_calls():
    cfg = W.CONFIGS["c3"].with_(L=4096)                                 # 2048 units x 4 heads: 19 MB
    q, k, span, kappa, K = _case(cfg, 40)
    need = R.rma_workspace_bytes(R.RMA_OP_DECODE_TOPK, k, span, 4, K)
    assert need > R.RMA_STATIC_SCRATCH_BYTES, need
    idx = torch.full((cfg.U, 4, K), -7, dtype=torch.int32, device=DEV)
    sel = torch.zeros(cfg.U, 4, K, device=DEV)
    assert _static_call(q, k, span, kappa, K, idx, sel) == R.RMA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((idx == -7).all())
    _check(_case(W.CONFIGS["c1"].with_(L=3000, K=(30,)), 30))          # and the next call still works
