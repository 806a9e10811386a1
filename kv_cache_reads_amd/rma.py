"""ctypes binding of librma.so (include/rma.h).

Argument marshalling only: every step of the method runs in the library's HIP
kernels.  Tensors must live on the current HIP device; work is enqueued on
torch's current stream.  The functions keep the C names; output tensors are
allocated with torch when not supplied.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import re
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librma.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "rma.h")

RMA_OK, RMA_ERR_INVALID_ARG, RMA_ERR_UNSUPPORTED, RMA_ERR_WORKSPACE, RMA_ERR_HIP = 0, -1, -2, -3, -4
RMA_F32, RMA_BF16 = 0, 1
RMA_OP_BUILD_SUMMARIES, RMA_OP_DECODE_TOPK, RMA_OP_DECODE_MERGE, RMA_OP_DECODE_FULL, RMA_OP_DECODE = 1, 2, 3, 4, 5
RMA_MERGE_SUB, RMA_MERGE_NO_RESIDUAL, RMA_MERGE_NO_SUBTRACT = 0, 1, 2
RMA_BUILD_ACCUMULATE = 1


class RmaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class _KV(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("n_units", ctypes.c_int32), ("t_cap", ctypes.c_int64),
                ("unit_stride", ctypes.c_int64), ("d", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class _Span(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int64), ("n_sink", ctypes.c_int32), ("n_tail", ctypes.c_int32),
                ("n_gen", ctypes.c_int64)]


@dataclasses.dataclass(frozen=True)
class Span:
    """Prefill length, anchors and generated tokens (identical for all units)."""
    L: int
    n_sink: int
    n_tail: int
    n_gen: int = 0

    @property
    def L_mid(self) -> int:
        return self.L - self.n_sink - self.n_tail

    def _c(self) -> _Span:
        return _Span(self.L, self.n_sink, self.n_tail, self.n_gen)


class _PhiMlp(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("W_in", "b_in", "W_1", "b_1", "W_2", "b_2", "alpha", "W_o", "b_o")]


_lib = None
_VP, _I32, _I64, _SZ, _U32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_uint32


def lib():
    """Load librma.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m kv_cache_reads_amd.build_lib`")
    L = ctypes.CDLL(LIB_PATH)
    P_KV, P_SP = ctypes.POINTER(_KV), ctypes.POINTER(_Span)
    L.rma_phi_features.argtypes = [_VP, _I32, _I32, _I64, _I64, _I32, _VP, _VP, _I32, _I32, _VP, _I32, _VP]
    L.rma_phi_mlp_features.argtypes = [_VP, _I32, _I32, _I64, _I64, _I32, ctypes.POINTER(_PhiMlp), _I32, _I32,
                                       _VP, _I32, _VP]
    L.rma_build_summaries.argtypes = [P_KV, P_SP, _VP, _VP, _I32, _I32, _VP, _I32, _VP, _VP, _VP, _VP, _SZ, _VP]
    L.rma_build_summaries_range.argtypes = [P_KV, P_SP, _I64, _I64, _U32, _VP, _VP, _I32, _I32, _VP, _I32, _VP,
                                            _VP, _VP, _VP, _SZ, _VP]
    L.rma_decode_topk.argtypes = [_VP, _I32, P_KV, P_SP, _VP, _I32, _VP, _VP, _VP, _SZ, _VP]
    L.rma_decode_topk_static.argtypes = [_VP, _I32, P_KV, P_SP, _VP, _I32, _VP, _VP, _VP]
    L.rma_decode_merge.argtypes = [_VP, _VP, _VP, _VP, _I32, P_KV, P_SP, _VP, _VP, _I32, _VP, _I32, _VP, _VP,
                                   _I32, _I32, _VP, _VP, _U32, _VP, _VP, _VP, _SZ, _VP]
    L.rma_decode.argtypes = [_VP, _VP, _VP, _VP, _I32, P_KV, P_SP, _VP, _I32, _VP, _I32, _VP, _VP, _I32, _I32,
                             _VP, _VP, _U32, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]
    L.rma_decode_full.argtypes = [_VP, _I32, P_KV, P_SP, _VP, _I32, _VP, _VP, _VP, _VP, _SZ, _VP]
    L.rma_workspace_bytes.argtypes = [_I32, P_KV, P_SP, _I32, _I32, _I32]
    L.rma_workspace_bytes.restype = _SZ
    L.rma_status_string.argtypes = [_I32]
    L.rma_status_string.restype = ctypes.c_char_p
    L.rma_last_error.argtypes = []
    L.rma_last_error.restype = ctypes.c_char_p
    L.rma_abi_version.restype = _I32
    L.rma_trace_arm.argtypes = [ctypes.POINTER(_VP), _I32]
    L.rma_trace_arm.restype = _I32
    L.rma_trace_count.argtypes = []
    L.rma_trace_count.restype = _I32
    L.rma_trace_name.argtypes = [_I32]
    L.rma_trace_name.restype = ctypes.c_char_p
    L.rma_stream_read.argtypes = [_VP, _I64, _I32, _VP, _VP]
    L.rma_stream_read.restype = _I32
    for f in ("rma_phi_features", "rma_phi_mlp_features", "rma_build_summaries", "rma_build_summaries_range", "rma_decode_topk",
              "rma_decode_topk_static", "rma_decode_merge", "rma_decode", "rma_decode_full"):
        getattr(L, f).restype = _I32
    _lib = L
    return L


def header_functions():
    """Names of the functions include/rma.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(rma_\w+)\s*\(", text, flags=re.M)))


def _check(status: int):
    if status != RMA_OK:
        L = lib()
        raise RmaError(status, f"{L.rma_status_string(status).decode()}: {L.rma_last_error().decode()}")


def _dt(t: torch.dtype) -> int:
    if t == torch.float32:
        return RMA_F32
    if t == torch.bfloat16:
        return RMA_BF16
    raise TypeError(f"unsupported dtype {t}")


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _kv(k: torch.Tensor, v: Optional[torch.Tensor]) -> _KV:
    assert k.dim() == 3 and k.stride(2) == 1 and k.stride(1) == k.shape[2], "K must be [U, T, d] with dense rows"
    if v is not None:
        assert v.shape == k.shape and v.stride() == k.stride() and v.dtype == k.dtype
    return _KV(k.data_ptr(), 0 if v is None else v.data_ptr(), _dt(k.dtype), k.shape[0], k.shape[1],
               k.stride(0), k.shape[2], 0)


class Workspace:
    """A device buffer reused across calls on one stream.  It holds per-call
    scratch only (every byte a call reads is written earlier in that call), so
    it needs no initialisation."""

    def __init__(self, device=None):
        self.device = device
        self.buf: Optional[torch.Tensor] = None

    def get(self, nbytes: int) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(max(nbytes, 4096), dtype=torch.uint8,
                                   device=self.device or torch.device("cuda"))
        return self.buf


_default_ws = {}


def _ws(ws: Optional[Workspace], nbytes: int) -> torch.Tensor:
    if ws is None:
        dev = torch.cuda.current_device()
        ws = _default_ws.setdefault(dev, Workspace(torch.device("cuda", dev)))
    return ws.get(nbytes)


def rma_workspace_bytes(op: int, k: torch.Tensor, span: Span, G: int = 1, K: int = 0, m: int = 128) -> int:
    kv = _kv(k, None)
    sp = span._c()
    return int(lib().rma_workspace_bytes(op, ctypes.byref(kv), ctypes.byref(sp), G, K, m))


def rma_phi_features(x: torch.Tensor, W: torch.Tensor, b: torch.Tensor,
                     phi_dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None):
    """phi[u, r] = elu(W[u % P] x[u, r] + b[u % P]) + 1;  x: [U, rows, d]."""
    U, rows, d = x.shape
    P, m, _ = W.shape
    if out is None:
        out = torch.empty(U, rows, m, dtype=phi_dtype, device=x.device)
    assert x.stride(2) == 1 and x.stride(1) == d
    _check(lib().rma_phi_features(_p(x), _dt(x.dtype), U, rows, x.stride(0), d, _p(W), _p(b), m, P,
                                  _p(out), _dt(out.dtype), _stream()))
    return out


PHI_MLP_WIDTH = 512
_MLP_MATS = ("W_in", "W_1", "W_2", "W_o")
_MLP_VECS = ("b_in", "b_1", "b_2", "alpha", "b_o")


def mlp_tile_order(W: torch.Tensor) -> torch.Tensor:
    """[P][N][K] -> the matrix-core tile order of rma.h, [P][K/32][N/16][64][8]:
    lane l = n%16 + 16 * ((k%32) / 8) of tile (k/32, n/16) holds k%8 = 0..7."""
    P, N, K = W.shape
    return W.reshape(P, N // 16, 16, K // 32, 4, 8).permute(0, 3, 1, 4, 2, 5).contiguous()


class PhiMlpWeights:
    """Device weights of n_param_sets MLP feature maps (rma_phi_mlp_features):
    the matrices as bf16 (round to nearest even from the given values) in the
    tile order rma.h defines, biases and the ReZero scalars as fp32.  `params`
    maps the names of rma_phi_mlp to tensors with a leading [n_param_sets] axis
    and [out][in] matrices."""

    def __init__(self, params: dict, device="cuda"):
        for n in _MLP_MATS:
            W = params[n].to(device=device, dtype=torch.float32).to(torch.bfloat16)
            setattr(self, n, mlp_tile_order(W))
        for n in _MLP_VECS:
            setattr(self, n, params[n].to(device=device, dtype=torch.float32).contiguous())
        self.alpha = self.alpha.reshape(-1)
        self.P, self.width, self.d = params["W_in"].shape
        self.m = params["W_o"].shape[1]
        assert self.width == PHI_MLP_WIDTH and tuple(params["W_1"].shape[1:]) == (512, 512)
        self._c = _PhiMlp(*(getattr(self, n).data_ptr() for n, _ in _PhiMlp._fields_))


def rma_phi_mlp_features(x: torch.Tensor, w: PhiMlpWeights, phi_dtype: torch.dtype = torch.float32,
                         out: Optional[torch.Tensor] = None):
    """phi[u, r] = exp(W_o h1 + b_o) of the MLP map u % P (see rma.h);  x: [U, rows, d]
    with dense rows (any unit stride)."""
    U, rows, d = x.shape
    if out is None:
        out = torch.empty(U, rows, w.m, dtype=phi_dtype, device=x.device)
    assert x.stride(2) == 1 and x.stride(1) == d and d == w.d
    _check(lib().rma_phi_mlp_features(_p(x), _dt(x.dtype), U, rows, x.stride(0), d, ctypes.byref(w._c), w.m,
                                      w.P, _p(out), _dt(out.dtype), _stream()))
    return out


def rma_build_summaries(k: torch.Tensor, v: torch.Tensor, span: Span, Wk: Optional[torch.Tensor],
                        bk: Optional[torch.Tensor], m: Optional[int] = None,
                        phi_k: Optional[torch.Tensor] = None, phi_dtype: torch.dtype = torch.bfloat16,
                        n_param_sets: Optional[int] = None, ws: Optional[Workspace] = None,
                        out: Optional[tuple] = None, store_phi: bool = True):
    """Returns (phi_k [U, L_mid, m], S [U, m, d], u [U, m], kappa [U]).  `out` may
    supply preallocated (S, u, kappa).  store_phi=False (computed features only)
    keeps the phi_k rows out of memory: phi_k is returned as None and decode
    recomputes the retrieved rows."""
    U, _, d = k.shape
    if m is None:
        m = Wk.shape[1] if Wk is not None else phi_k.shape[2]
    P = n_param_sets or (Wk.shape[0] if Wk is not None else 1)
    if phi_k is None and store_phi:
        assert Wk is not None, "phi_k must be given when Wk is None"
        phi_k = torch.empty(U, span.L_mid, m, dtype=phi_dtype, device=k.device)
    if out is not None:
        S, u, kappa = out
    else:
        S = torch.empty(U, m, d, dtype=torch.float32, device=k.device)
        u = torch.empty(U, m, dtype=torch.float32, device=k.device)
        kappa = torch.empty(U, dtype=torch.float32, device=k.device)
    kv, sp = _kv(k, v), span._c()
    nb = int(lib().rma_workspace_bytes(RMA_OP_BUILD_SUMMARIES, ctypes.byref(kv), ctypes.byref(sp), 1, 0, m))
    w = _ws(ws, nb)
    pdt = _dt(phi_k.dtype) if phi_k is not None else _dt(phi_dtype)
    _check(lib().rma_build_summaries(ctypes.byref(kv), ctypes.byref(sp), _p(Wk), _p(bk), m, P, _p(phi_k),
                                     pdt, _p(S), _p(u), _p(kappa), _p(w), w.numel(), _stream()))
    return phi_k, S, u, kappa


def rma_build_summaries_range(k: torch.Tensor, v: torch.Tensor, span: Span, m_begin: int, m_end: int,
                              Wk: Optional[torch.Tensor], bk: Optional[torch.Tensor],
                              phi_k: Optional[torch.Tensor], S: torch.Tensor, u: torch.Tensor,
                              kappa: torch.Tensor, accumulate: bool = False,
                              phi_dtype: torch.dtype = torch.bfloat16, ws: Optional[Workspace] = None):
    """Summaries of the mid-region positions [m_begin, m_end): overwrite S, u,
    kappa, or (accumulate) add to them; phi_k rows of the range are written
    (phi_k may be None for bf16 keys with Wk: rows not stored)."""
    U, _, d = k.shape
    m = S.shape[1]
    P = Wk.shape[0] if Wk is not None else 1
    kv, sp = _kv(k, v), span._c()
    nb = int(lib().rma_workspace_bytes(RMA_OP_BUILD_SUMMARIES, ctypes.byref(kv), ctypes.byref(sp), 1, 0, m))
    w = _ws(ws, nb)
    pdt = _dt(phi_k.dtype) if phi_k is not None else _dt(phi_dtype)
    _check(lib().rma_build_summaries_range(ctypes.byref(kv), ctypes.byref(sp), m_begin, m_end,
                                           RMA_BUILD_ACCUMULATE if accumulate else 0, _p(Wk), _p(bk), m, P,
                                           _p(phi_k), pdt, _p(S), _p(u), _p(kappa), _p(w), w.numel(),
                                           _stream()))
    return S, u, kappa


def rma_decode_topk(q: torch.Tensor, k: torch.Tensor, span: Span, kappa: torch.Tensor, K: int,
                    ws: Optional[Workspace] = None, idx: Optional[torch.Tensor] = None,
                    sel_scores: Optional[torch.Tensor] = None):
    """q: [U, G, d] fp32.  Returns (idx [U, G, K] int32 ascending, sel_scores [U, G, K])."""
    U, G, d = q.shape
    if idx is None:
        idx = torch.empty(U, G, K, dtype=torch.int32, device=q.device)
    if sel_scores is None:
        sel_scores = torch.empty(U, G, K, dtype=torch.float32, device=q.device)
    kv, sp = _kv(k, None), span._c()
    nb = int(lib().rma_workspace_bytes(RMA_OP_DECODE_TOPK, ctypes.byref(kv), ctypes.byref(sp), G, K, 0))
    w = _ws(ws, nb)
    _check(lib().rma_decode_topk(_p(q), G, ctypes.byref(kv), ctypes.byref(sp), _p(kappa), K, _p(idx),
                                 _p(sel_scores), _p(w), w.numel(), _stream()))
    return idx, sel_scores


RMA_STATIC_SCRATCH_BYTES = 16 << 20


def rma_decode_topk_static(q: torch.Tensor, k: torch.Tensor, span: Span, kappa: torch.Tensor, K: int,
                           idx: Optional[torch.Tensor] = None, sel_scores: Optional[torch.Tensor] = None):
    """rma_decode_topk with the library's static scratch (no workspace; the
    call allocates nothing on the device when idx and sel_scores are given)."""
    U, G, d = q.shape
    if idx is None:
        idx = torch.empty(U, G, K, dtype=torch.int32, device=q.device)
    if sel_scores is None:
        sel_scores = torch.empty(U, G, K, dtype=torch.float32, device=q.device)
    kv, sp = _kv(k, None), span._c()
    _check(lib().rma_decode_topk_static(_p(q), G, ctypes.byref(kv), ctypes.byref(sp), _p(kappa), K, _p(idx),
                                        _p(sel_scores), _stream()))
    return idx, sel_scores


def rma_decode_merge(q: torch.Tensor, phi_q: Optional[torch.Tensor], k: torch.Tensor, v: torch.Tensor,
                     span: Span, idx: Optional[torch.Tensor], sel_scores: Optional[torch.Tensor], K: int,
                     phi_k: Optional[torch.Tensor], S: Optional[torch.Tensor], u: Optional[torch.Tensor],
                     flags: int = RMA_MERGE_SUB, m: Optional[int] = None, want_stats: bool = False,
                     ws: Optional[Workspace] = None, y: Optional[torch.Tensor] = None,
                     Wk: Optional[torch.Tensor] = None, bk: Optional[torch.Tensor] = None,
                     Wq: Optional[torch.Tensor] = None, bq: Optional[torch.Tensor] = None):
    """Returns y [U, G, d] (and stats [U, G, 4] = (m*, Z_E, Z_R, retrieved phi mass)).
    With phi_k None, the retrieved phi_k rows are recomputed from Wk, bk; with
    phi_q None, f = phi_q(q) is computed in the call from Wq, bq."""
    U, G, d = q.shape
    if m is None:
        m = S.shape[1] if S is not None else 128
    if y is None:
        y = torch.empty(U, G, d, dtype=torch.float32, device=q.device)
    stats = torch.empty(U, G, 4, dtype=torch.float32, device=q.device) if want_stats else None
    kv, sp = _kv(k, v), span._c()
    nb = int(lib().rma_workspace_bytes(RMA_OP_DECODE_MERGE, ctypes.byref(kv), ctypes.byref(sp), G, K, m))
    w = _ws(ws, nb)
    pdt = _dt(phi_k.dtype) if phi_k is not None else RMA_BF16
    P = Wk.shape[0] if Wk is not None else (Wq.shape[0] if Wq is not None else 1)
    _check(lib().rma_decode_merge(_p(q), _p(phi_q), _p(Wq), _p(bq), G, ctypes.byref(kv), ctypes.byref(sp), _p(idx),
                                  _p(sel_scores), K, _p(phi_k), pdt, _p(Wk), _p(bk), P, m, _p(S), _p(u),
                                  flags, _p(y), _p(stats), _p(w), w.numel(), _stream()))
    return (y, stats) if want_stats else y


def rma_decode(q: torch.Tensor, phi_q: Optional[torch.Tensor], k: torch.Tensor, v: torch.Tensor, span: Span,
               kappa: Optional[torch.Tensor], K: int, phi_k: Optional[torch.Tensor], S: Optional[torch.Tensor],
               u: Optional[torch.Tensor], flags: int = RMA_MERGE_SUB, m: Optional[int] = None,
               want_idx: bool = False, want_stats: bool = False, ws: Optional[Workspace] = None,
               y: Optional[torch.Tensor] = None, Wk: Optional[torch.Tensor] = None,
               bk: Optional[torch.Tensor] = None, Wq: Optional[torch.Tensor] = None,
               bq: Optional[torch.Tensor] = None, phi_dtype: Optional[torch.dtype] = None):
    """One decode step (Top-K + merge in one call).  Returns y [U, G, d], plus
    (idx [U, G, K], sel_scores [U, G, K]) with want_idx and stats [U, G, 4]
    with want_stats, in the order y, idx, sel, stats."""
    U, G, d = q.shape
    if m is None:
        m = S.shape[1] if S is not None else 128
    if y is None:
        y = torch.empty(U, G, d, dtype=torch.float32, device=q.device)
    idx = torch.empty(U, G, K, dtype=torch.int32, device=q.device) if want_idx else None
    sel = torch.empty(U, G, K, dtype=torch.float32, device=q.device) if want_idx else None
    stats = torch.empty(U, G, 4, dtype=torch.float32, device=q.device) if want_stats else None
    kv, sp = _kv(k, v), span._c()
    nb = int(lib().rma_workspace_bytes(RMA_OP_DECODE, ctypes.byref(kv), ctypes.byref(sp), G, K, m))
    w = _ws(ws, nb)
    pdt = _dt(phi_k.dtype) if phi_k is not None else _dt(phi_dtype or torch.bfloat16)
    P = Wk.shape[0] if Wk is not None else (Wq.shape[0] if Wq is not None else 1)
    _check(lib().rma_decode(_p(q), _p(phi_q), _p(Wq), _p(bq), G, ctypes.byref(kv), ctypes.byref(sp), _p(kappa), K,
                            _p(phi_k), pdt, _p(Wk), _p(bk), P, m, _p(S), _p(u), flags, _p(idx), _p(sel), _p(y),
                            _p(stats), _p(w), w.numel(), _stream()))
    out = (y,)
    if want_idx:
        out += (idx, sel)
    if want_stats:
        out += (stats,)
    return out[0] if len(out) == 1 else out


def rma_decode_full(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, span: Span,
                    idx: Optional[torch.Tensor] = None, K: Optional[int] = None,
                    y_cmp: Optional[torch.Tensor] = None, want_diag: bool = False,
                    ws: Optional[Workspace] = None, y: Optional[torch.Tensor] = None):
    """Full attention over [0, L + n_gen).  Returns y_full [U, G, d] (and diag
    [U, G, 8] = (log Z_full, log Z_mid, log Z_R, H_mid, rel_l1, max s, 0, 0))."""
    U, G, d = q.shape
    if K is None:
        K = idx.shape[2] if idx is not None else 0
    if y is None:
        y = torch.empty(U, G, d, dtype=torch.float32, device=q.device)
    diag = torch.empty(U, G, 8, dtype=torch.float32, device=q.device) if want_diag else None
    kv, sp = _kv(k, v), span._c()
    nb = int(lib().rma_workspace_bytes(RMA_OP_DECODE_FULL, ctypes.byref(kv), ctypes.byref(sp), G, K, 0))
    w = _ws(ws, nb)
    _check(lib().rma_decode_full(_p(q), G, ctypes.byref(kv), ctypes.byref(sp), _p(idx), K, _p(y_cmp),
                                 _p(y), _p(diag), _p(w), w.numel(), _stream()))
    return (y, diag) if want_diag else y


def rma_abi_version() -> int:
    return int(lib().rma_abi_version())


def rma_trace_arm(events) -> None:
    """Arm per-kernel timing for the next call on this thread (benchmark
    instrumentation): `events` are torch.cuda.Event(enable_timing=True), an even
    number; the call's j-th kernel is stamped with events[2j] when it starts and
    events[2j+1] when it ends (hipExtLaunchKernel)."""
    L = lib()
    handles = []
    for e in events:
        if not e.cuda_event:          # torch creates the event lazily on first record
            e.record()
        handles.append(e.cuda_event)
    arr = (_VP * max(len(handles), 1))(*handles)
    _check(L.rma_trace_arm(arr, len(handles)))


def rma_stream_read(x: torch.Tensor, blocks: int, sink: torch.Tensor) -> None:
    """Streaming-read ceiling (benchmark instrumentation): reads the bytes of the
    contiguous device tensor `x` once with `blocks` workgroups, each a contiguous
    piece; block b writes the XOR of its piece's 32-bit words to sink[b]
    (`sink`: a contiguous device int32 tensor of at least `blocks` words)."""
    if not (x.is_cuda and x.is_contiguous() and sink.is_cuda and sink.dtype == torch.int32
            and sink.is_contiguous() and sink.numel() >= int(blocks)):
        raise ValueError("x must be a contiguous device tensor and sink a device int32 tensor of >= blocks words")
    _check(lib().rma_stream_read(_p(x), x.numel() * x.element_size(), int(blocks), _p(sink), _stream()))


def rma_trace_kernels():
    """Names of the kernels the last traced call timed, in launch order."""
    L = lib()
    return [L.rma_trace_name(j).decode() for j in range(L.rma_trace_count())]
