"""C-ABI library checks that need no GPU: it loads, exports every function that
include/rma.h declares, and rejects bad arguments on the host before any HIP
call (so these calls never touch a device)."""
import ctypes

import pytest

from kv_cache_reads_amd import rma as R

pytestmark = pytest.mark.skipif(not __import__("os").path.exists(R.LIB_PATH),
                                reason="librma.so not built")


def test_exports_every_declared_symbol():
    names = R.header_functions()
    assert set(names) >= {"rma_phi_features", "rma_phi_mlp_features", "rma_build_summaries", "rma_decode_topk",
                          "rma_decode_merge", "rma_decode_full", "rma_build_summaries_range",
                          "rma_workspace_bytes", "rma_status_string",
                          "rma_last_error", "rma_abi_version"}
    L = R.lib()
    for n in names:
        assert hasattr(L, n), n
    assert L.rma_abi_version() == 9
    assert L.rma_status_string(-3) == b"RMA_ERR_WORKSPACE"
    assert L.rma_status_string(7) == b"RMA_ERR_UNKNOWN"


def _kv(d=64, U=2, T=1024, dtype=R.RMA_BF16, ptr=0x10000):
    return R._KV(ptr, ptr + 0x100000, dtype, U, T, T * d, d, 0)


def _sp(L=1024, ns=4, nt=32, ng=0):
    return R._Span(L, ns, nt, ng)


def _topk(kv, sp, G=2, K=10, q=0x2000, kappa=0x3000, idx=0x4000, sel=0x5000, ws=0x6000, wsb=1 << 30):
    return R.lib().rma_decode_topk(q, G, ctypes.byref(kv), ctypes.byref(sp), kappa, K, idx, sel, ws, wsb, None)


def test_topk_validation_errors():
    L = R.lib()
    assert _topk(_kv(), _sp(), K=2000) == R.RMA_ERR_INVALID_ARG            # K > L_mid
    assert b"K 2000" in L.rma_last_error()
    assert _topk(_kv(), _sp(ns=600, nt=600)) == R.RMA_ERR_INVALID_ARG      # anchors exceed L
    assert _topk(_kv(d=96), _sp()) == R.RMA_ERR_UNSUPPORTED                # head dim
    assert _topk(_kv(), _sp(), G=9) == R.RMA_ERR_UNSUPPORTED               # group size
    assert _topk(_kv(dtype=5), _sp()) == R.RMA_ERR_UNSUPPORTED             # dtype
    assert _topk(_kv(), _sp(), q=0) == R.RMA_ERR_INVALID_ARG               # null q
    assert _topk(_kv(), _sp(), idx=0x4004) == R.RMA_ERR_INVALID_ARG        # misaligned
    assert _topk(_kv(ptr=0x10008), _sp()) == R.RMA_ERR_INVALID_ARG         # misaligned K
    assert _topk(_kv(T=1000), _sp(L=1024)) == R.RMA_ERR_INVALID_ARG        # t_cap < L
    assert _topk(_kv(), _sp(ng=5)) == R.RMA_ERR_INVALID_ARG                # t_cap < L + n_gen
    assert _topk(_kv(), _sp(), ws=0) == R.RMA_ERR_WORKSPACE
    assert _topk(_kv(), _sp(), wsb=16) == R.RMA_ERR_WORKSPACE
    assert _topk(_kv(), _sp(), K=0) == R.RMA_OK                            # nothing to do, nothing launched


def test_build_and_merge_validation_errors():
    L = R.lib()
    kv, sp = _kv(), _sp()
    P = ctypes.c_void_p
    st = L.rma_build_summaries(ctypes.byref(kv), ctypes.byref(sp), 0x1000, 0x1100, 96, 1, 0x2000,
                               R.RMA_BF16, 0x3000, 0x4000, 0x5000, 0x6000, 1 << 30, None)
    assert st == R.RMA_ERR_UNSUPPORTED                                     # m
    st = L.rma_build_summaries(ctypes.byref(kv), ctypes.byref(sp), 0x1000, 0, 128, 1, 0x2000,
                               R.RMA_BF16, 0x3000, 0x4000, 0x5000, 0x6000, 1 << 30, None)
    assert st == R.RMA_ERR_INVALID_ARG                                     # bk NULL
    st = L.rma_build_summaries(ctypes.byref(kv), ctypes.byref(sp), 0x1000, 0x1100, 128, 1, 0x2000,
                               R.RMA_BF16, 0x3000, 0x4000, 0x5000, 0x6000, 8, None)
    assert st == R.RMA_ERR_WORKSPACE
    # merge: empty exact support, unknown flags, NULL phi_q with residual
    sp0 = _sp(L=1024, ns=0, nt=0)
    st = L.rma_decode_merge(0x1000, 0x1100, None, None, 2, ctypes.byref(kv), ctypes.byref(sp0), 0x2000, 0x2100, 0,
                            0x3000, R.RMA_BF16, None, None, 1, 128, 0x4000, 0x5000, 0, 0x6000, None, 0x7000, 1 << 30, None)
    assert st == R.RMA_ERR_INVALID_ARG
    st = L.rma_decode_merge(0x1000, 0x1100, None, None, 2, ctypes.byref(kv), ctypes.byref(sp), 0x2000, 0x2100, 10,
                            0x3000, R.RMA_BF16, None, None, 1, 128, 0x4000, 0x5000, 7, 0x6000, None, 0x7000, 1 << 30, None)
    assert st == R.RMA_ERR_INVALID_ARG
    st = L.rma_decode_merge(0x1000, None, None, None, 2, ctypes.byref(kv), ctypes.byref(sp), 0x2000, 0x2100, 10,
                            0x3000, R.RMA_BF16, None, None, 1, 128, 0x4000, 0x5000, 0, 0x6000, None, 0x7000, 1 << 30, None)
    assert st == R.RMA_ERR_INVALID_ARG
    # phi_q computed in the call needs both Wq and bq, 16-byte aligned
    st = L.rma_decode_merge(0x1000, None, 0x8000, None, 2, ctypes.byref(kv), ctypes.byref(sp), 0x2000, 0x2100, 10,
                            0x3000, R.RMA_BF16, None, None, 1, 128, 0x4000, 0x5000, 0, 0x6000, None, 0x7000, 1 << 30, None)
    assert st == R.RMA_ERR_INVALID_ARG
    st = L.rma_decode_merge(0x1000, None, 0x8004, 0x9000, 2, ctypes.byref(kv), ctypes.byref(sp), 0x2000, 0x2100, 10,
                            0x3000, R.RMA_BF16, None, None, 1, 128, 0x4000, 0x5000, 0, 0x6000, None, 0x7000, 1 << 30, None)
    assert st == R.RMA_ERR_INVALID_ARG
    st = L.rma_phi_features(0x1000, R.RMA_F32, 1, 4, 4 * 64, 64, 0x2000, 0x3000, 100, 1, 0x4000,
                            R.RMA_F32, None)
    assert st == R.RMA_ERR_UNSUPPORTED
    # subtraction without phi_k rows needs Wk/bk to recompute them ...
    st = L.rma_decode_merge(0x1000, 0x1100, None, None, 2, ctypes.byref(kv), ctypes.byref(sp), 0x2000, 0x2100, 10,
                            None, R.RMA_BF16, None, None, 1, 128, 0x4000, 0x5000, 0, 0x6000, None, 0x7000,
                            1 << 30, None)
    assert st == R.RMA_ERR_INVALID_ARG
    # ... and bf16 keys (the builder's rounding)
    kvf = _kv(dtype=R.RMA_F32)
    st = L.rma_decode_merge(0x1000, 0x1100, None, None, 2, ctypes.byref(kvf), ctypes.byref(sp), 0x2000, 0x2100, 10,
                            None, R.RMA_BF16, 0x8000, 0x9000, 1, 128, 0x4000, 0x5000, 0, 0x6000, None, 0x7000,
                            1 << 30, None)
    assert st == R.RMA_ERR_UNSUPPORTED
    # the builder may skip the rows only when it computes bf16 features itself
    st = L.rma_build_summaries(ctypes.byref(kvf), ctypes.byref(sp), 0x1000, 0x1100, 128, 1, None,
                               R.RMA_BF16, 0x3000, 0x4000, 0x5000, 0x6000, 1 << 30, None)
    assert st == R.RMA_ERR_INVALID_ARG
    st = L.rma_build_summaries(ctypes.byref(kv), ctypes.byref(sp), None, None, 128, 1, None,
                               R.RMA_BF16, 0x3000, 0x4000, 0x5000, 0x6000, 1 << 30, None)
    assert st == R.RMA_ERR_INVALID_ARG


def test_build_range_validation_errors():
    L = R.lib()
    kv, sp = _kv(), _sp()          # L_mid = 1024 - 36 = 988

    def rng(a, b, flags=0, ws=0x6000):
        return L.rma_build_summaries_range(ctypes.byref(kv), ctypes.byref(sp), a, b, flags, 0x1000, 0x1100,
                                           128, 1, 0x2000, R.RMA_BF16, 0x3000, 0x4000, 0x5000, ws, 1 << 30,
                                           None)
    assert rng(-1, 10) == R.RMA_ERR_INVALID_ARG
    assert rng(20, 10) == R.RMA_ERR_INVALID_ARG
    assert rng(0, 989) == R.RMA_ERR_INVALID_ARG
    assert b"outside the mid-region" in L.rma_last_error()
    assert rng(0, 10, flags=2) == R.RMA_ERR_INVALID_ARG
    assert rng(0, 10, ws=0) == R.RMA_ERR_WORKSPACE
    assert L.rma_build_summaries(None, ctypes.byref(sp), 0x1000, 0x1100, 128, 1, 0x2000, R.RMA_BF16,
                                 0x3000, 0x4000, 0x5000, 0x6000, 1 << 30, None) == R.RMA_ERR_INVALID_ARG


def test_workspace_sizes_are_monotone_in_K_and_units():
    L = R.lib()
    sp = _sp(L=32768, ns=4, nt=64)
    sizes = []
    for U in (1, 8, 64):
        kv = _kv(U=U, T=32768)
        s = [L.rma_workspace_bytes(R.RMA_OP_DECODE_TOPK, ctypes.byref(kv), ctypes.byref(sp), 4, K, 0)
             for K in (1, 328, 3000)]
        assert all(x > 0 for x in s) and s == sorted(s)
        sizes.append(s[1])
        assert L.rma_workspace_bytes(R.RMA_OP_BUILD_SUMMARIES, ctypes.byref(kv), ctypes.byref(sp), 1, 0, 128) > 0
        assert L.rma_workspace_bytes(R.RMA_OP_DECODE_MERGE, ctypes.byref(kv), ctypes.byref(sp), 4, 328, 128) > 0
    assert sizes == sorted(sizes)
    kv = _kv()
    assert L.rma_workspace_bytes(R.RMA_OP_DECODE_TOPK, ctypes.byref(kv), ctypes.byref(_sp()), 2, 5000, 0) == 0
    assert L.rma_workspace_bytes(99, ctypes.byref(kv), ctypes.byref(_sp()), 2, 10, 128) == 0


def _full(kv, sp, G=2, K=0, q=0x2000, idx=None, ycmp=None, y=0x7000, diag=None, ws=0x6000, wsb=1 << 30):
    return R.lib().rma_decode_full(q, G, ctypes.byref(kv), ctypes.byref(sp), idx, K, ycmp, y, diag, ws, wsb, None)


def test_full_validation_errors():
    L = R.lib()
    kv, sp = _kv(), _sp()
    assert _full(kv, sp, q=0) == R.RMA_ERR_INVALID_ARG                     # null q
    assert _full(kv, sp, y=0) == R.RMA_ERR_INVALID_ARG                     # null y_full
    assert _full(kv, sp, G=9) == R.RMA_ERR_UNSUPPORTED
    assert _full(_kv(d=96), sp) == R.RMA_ERR_UNSUPPORTED
    assert _full(kv, sp, K=2000, idx=0x4000) == R.RMA_ERR_INVALID_ARG      # K > L_mid
    assert _full(kv, sp, diag=0x8004) == R.RMA_ERR_INVALID_ARG             # misaligned diag
    assert _full(kv, _sp(L=0, ns=0, nt=0)) == R.RMA_ERR_INVALID_ARG         # empty context
    assert _full(kv, sp, ws=0) == R.RMA_ERR_WORKSPACE
    assert _full(kv, sp, wsb=16) == R.RMA_ERR_WORKSPACE
    assert _full(_kv(T=1000), sp) == R.RMA_ERR_INVALID_ARG                 # t_cap < L
    n = L.rma_workspace_bytes(R.RMA_OP_DECODE_FULL, ctypes.byref(kv), ctypes.byref(sp), 2, 0, 0)
    assert n > 0
    assert L.rma_workspace_bytes(R.RMA_OP_DECODE_FULL, ctypes.byref(kv), ctypes.byref(sp), 4, 0, 0) > n
    assert _full(kv, sp, wsb=n - 1) == R.RMA_ERR_WORKSPACE


def test_trace_arm_validation():
    """Kernel-timing hook: argument checks only (arming stores handles; no HIP call)."""
    L = R.lib()
    VP = ctypes.c_void_p
    two = (VP * 2)(0x1000, 0x2000)
    assert L.rma_trace_arm(two, 1) == R.RMA_ERR_INVALID_ARG              # one event times nothing
    three = (VP * 3)(0x1000, 0x2000, 0x3000)
    assert L.rma_trace_arm(three, 3) == R.RMA_ERR_INVALID_ARG            # events come in pairs
    assert L.rma_trace_arm(two, 17) == R.RMA_ERR_INVALID_ARG             # more than RMA_TRACE_MAX_EVENTS
    assert L.rma_trace_arm((VP * 2)(0x1000, None), 2) == R.RMA_ERR_INVALID_ARG
    assert L.rma_trace_arm(None, 2) == R.RMA_ERR_INVALID_ARG
    assert L.rma_trace_arm(two, 2) == R.RMA_OK
    assert L.rma_trace_arm(None, 0) == R.RMA_OK                          # disarm
    assert L.rma_trace_count() == 0 and L.rma_trace_name(0) is None


def test_phi_mlp_validation():
    """MLP feature map: argument checks only (no HIP call is reached)."""
    L = R.lib()
    ptr = 0x100000
    w = R._PhiMlp(*([ptr] * 9))
    wb = ctypes.byref(w)
    ok = dict(x=ptr, xd=R.RMA_BF16, U=2, rows=100, st=100 * 64, d=64, m=64, P=1, phi=ptr, pd=R.RMA_BF16)

    def call(**kw):
        a = dict(ok, **kw)
        return L.rma_phi_mlp_features(a["x"], a["xd"], a["U"], a["rows"], a["st"], a["d"],
                                      kw.get("weights", wb), a["m"], a["P"], a["phi"], a["pd"], None)
    assert call(x=None) == R.RMA_ERR_INVALID_ARG
    assert call(phi=None) == R.RMA_ERR_INVALID_ARG
    assert call(weights=None) == R.RMA_ERR_INVALID_ARG
    bad = R._PhiMlp(*([ptr] * 8 + [0]))                        # b_o missing
    assert call(weights=ctypes.byref(bad)) == R.RMA_ERR_INVALID_ARG
    assert call(d=96) == R.RMA_ERR_UNSUPPORTED
    assert call(m=32) == R.RMA_ERR_UNSUPPORTED
    assert call(xd=7) == R.RMA_ERR_UNSUPPORTED
    assert call(U=0) == R.RMA_ERR_INVALID_ARG
    assert call(P=0) == R.RMA_ERR_INVALID_ARG
    assert call(st=99 * 64) == R.RMA_ERR_INVALID_ARG           # unit stride < rows * d
    assert call(x=ptr + 2) == R.RMA_ERR_INVALID_ARG            # misaligned
    odd = R._PhiMlp(*([ptr] * 2 + [ptr + 4] + [ptr] * 6))      # W_1 misaligned
    assert call(weights=ctypes.byref(odd)) == R.RMA_ERR_INVALID_ARG
    assert call(rows=0) == R.RMA_OK                            # nothing to do



def test_mlp_tile_order_matches_the_header_formula():
    """PhiMlpWeights' layout helper against the element formula in rma.h."""
    import torch
    P, N, K = 2, 64, 96
    W = torch.arange(P * N * K, dtype=torch.float32).reshape(P, N, K)
    T = R.mlp_tile_order(W).reshape(P, -1)
    for p in range(P):
        for n in (0, 5, 17, 63):
            for k in (0, 7, 8, 31, 32, 95):
                off = ((k // 32 * (N // 16) + n // 16) * 64 + (n % 16 + 16 * ((k % 32) // 8))) * 8 + k % 8
                assert T[p, off] == W[p, n, k]


def test_static_topk_refuses_oversized_calls_before_any_hip_call():
    """rma_decode_topk_static: a call whose scratch exceeds the static array is
    refused during validation (RMA_ERR_WORKSPACE), with no device touched."""
    L = R.lib()
    U, T, d = 2048, 4096, 64
    kv = _kv(U=U, T=T)
    sp = _sp(L=T, ns=4, nt=64)
    need = L.rma_workspace_bytes(R.RMA_OP_DECODE_TOPK, ctypes.byref(kv), ctypes.byref(sp), 4, 40, 0)
    assert need > R.RMA_STATIC_SCRATCH_BYTES
    r = L.rma_decode_topk_static(0x2000, 4, ctypes.byref(kv), ctypes.byref(sp), 0x3000, 40, 0x4000, 0x5000, None)
    assert r == R.RMA_ERR_WORKSPACE
    assert b"static" in L.rma_last_error()
    assert L.rma_decode_topk_static(0x2000, 4, ctypes.byref(kv), ctypes.byref(sp), 0x3000, 0, 0, 0, None) == R.RMA_OK


def _topk_plan_bytes(L, ns, nt, U, G, K, d):
    """The Top-K workspace by the planner's rule, written out: chunks of whole
    scan-block passes, as many as give ~512 blocks but no longer than the fp32
    scores a scan block keeps in its LDS budget (54272 bytes: G score rows of
    ch + 8 words beside G 512-bin histograms and the G queries), and per chunk
    room for 2 r_min + 32 reports, r_min = mu + 4 sqrt(mu) + 4 rounded up to 8
    (at least 16), mu = K / chunks."""
    import math

    Lm = L - ns - nt
    tile = 64 if d == 64 else 32
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
    up = lambda x: -(-x // 256) * 256
    return up(U * G * chunks * r_cap * 8) + up(U * G * chunks * 8) + up(U * G * 16), chunks, ch


@pytest.mark.parametrize("shape", [
    (1024, 4, 32, 1, 2, 10, 64),          # the tiny workload: 16 chunks
    (32768, 4, 64, 8, 4, 328, 64),        # 32K layer: 64 chunks of 512
    (65536, 4, 64, 8, 3, 2621, 128),      # 64K layer, 4 % budget
    (16384, 4, 64, 2048, 4, 163, 64),     # many units: chunks bounded by the LDS score store (2752)
    (131072, 4, 64, 896, 3, 1310, 128),   # 128K, d = 128: 35 chunks (at most 3840 tokens)
    (40000, 4, 64, 300, 8, 400, 64),      # eight heads per unit
])
def test_topk_workspace_follows_the_chunk_and_report_rule(shape):
    L_, ns, nt, U, G, K, d = shape
    kv = _kv(d=d, U=U, T=L_)
    got = R.lib().rma_workspace_bytes(R.RMA_OP_DECODE_TOPK, ctypes.byref(kv), ctypes.byref(_sp(L_, ns, nt)), G, K, 0)
    want, chunks, ch = _topk_plan_bytes(L_, ns, nt, U, G, K, d)
    assert got == want, (got, want, chunks, ch)
    if U == 2048:
        assert (chunks, ch) == (6, 2752)
    if U == 896:
        assert (chunks, ch) == (35, 3744)   # under the 3840-token bound


def test_stream_read_validation():
    L = R.lib()
    sink = 0x9000
    assert L.rma_stream_read(None, 1024, 4, sink, None) == R.RMA_ERR_INVALID_ARG
    assert L.rma_stream_read(0x10000, 1024, 4, None, None) == R.RMA_ERR_INVALID_ARG
    assert L.rma_stream_read(0x10008, 1024, 4, sink, None) == R.RMA_ERR_INVALID_ARG    # misaligned
    assert L.rma_stream_read(0x10000, 1000, 4, sink, None) == R.RMA_ERR_INVALID_ARG    # not 16-byte multiple
    assert L.rma_stream_read(0x10000, 0, 4, sink, None) == R.RMA_ERR_INVALID_ARG
    assert L.rma_stream_read(0x10000, 1024, 0, sink, None) == R.RMA_ERR_INVALID_ARG
    assert L.rma_stream_read(0x10000, 1024, (1 << 20) + 1, sink, None) == R.RMA_ERR_INVALID_ARG
