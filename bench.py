#!/usr/bin/env python3
"""Benchmark of Top-K+phi residual-mass-accounting decode on one MI355X.

The headline is the method's decode: one timed step is one decode pass over
the workload's batch (every query head of every unit, every decode step of the
workload) through rma_decode: the exhaustive scan, then the fused selection
and merge (exact terms, retrieved-token subtraction, residual, single
normalisation), with f = phi_q(q) computed inside.  The prefill summaries
(rma_build_summaries) are built before timing and reported in a block of
their own, with their bandwidth and matrix-core use; the whole path (build +
decode per step) is reported as an extra rate.  Default workload: the
1B-shaped GQA layer at 32K context with a 1 % budget (8 kv heads x 4 query
heads, d = 64, K = 328).

Inputs are resident in HBM before timing starts.  Steps rotate over copies of
the inputs whose total exceeds 1 GB, so that no step is served from the 256 MB
last-level cache.  Steps are replayed from HIP graphs (checked against an eager
run first).  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--config c1]
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 matrix cores
MLP_WIDTH = 512
METRIC = "decode queries/s + achieved HBM GB/s (% peak), 1B-shape GQA, 32K ctx, 1% budget"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="c1")
    ap.add_argument("--K", type=int, default=None, help="override the retrieved-token count")
    ap.add_argument("--rotate-bytes", type=float, default=1.2e9)
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of graphs")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--separate", action="store_true",
                    help="decode with the two calls rma_decode_topk + rma_decode_merge instead of rma_decode")
    ap.add_argument("--separate-phi", action="store_true",
                    help="compute phi_q with rma_phi_features instead of inside the decode")
    ap.add_argument("--no-full", action="store_true", help="skip timing the full-attention reference decode")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming read / copy ceilings")
    ap.add_argument("--recompute-phi", action="store_true",
                    help="do not store the phi_k rows at prefill; decode recomputes the retrieved rows from "
                         "their keys (bf16 keys; saves the rows' HBM, costs matrix-core work per step)")
    ap.add_argument("--phi", choices=("elu", "mlp"), default="elu",
                    help="feature map: elu(Wx+b)+1 (the workloads' form, default) or the pages' MLP family "
                         "(one-block ReZero MLP, width 512, exponentiated output, d_phi = 64)")
    ap.add_argument("--copy-probe-mb", type=float, default=0.0,
                    help="first run a plain fp32 copy-like kernel (neg) of this size, for calibrating "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE against known bytes")
    return ap.parse_args()


# ------------------------------------------------------------------ measured HBM traffic
# Bytes per launch from rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; KiB per
# dispatch) of this script, each scaled by what the same counter reads for a plain
# copy of known size.  A record holds only for the kernel sources it was taken on.
TRAFFIC = {
    # (kernel, workload, K): profiles/traffic_c1.md, profiles/traffic_c4.md
    ("decode_fused_kernel", "c1", 328): {"fetch_bytes": 6298366, "write_bytes": 8192, "csrc": "4346d9d15ab6b371"},
    ("topk_scan_kernel", "c1", 328): {"fetch_bytes": 33659714, "write_bytes": 451168, "csrc": "4346d9d15ab6b371"},
    ("build_mfma_kernel", "c1", 328): {"fetch_bytes": 69255656, "write_bytes": 84056022, "csrc": "4346d9d15ab6b371"},
    ("decode_fused_kernel", "c4", 1310): {"fetch_bytes": 2352763431, "write_bytes": 1376256, "csrc": "4346d9d15ab6b371"},
    ("topk_scan_kernel", "c4", 1310): {"fetch_bytes": 30241179891, "write_bytes": 62556054, "csrc": "4346d9d15ab6b371"},
    ("build_mfma_kernel", "c4", 1310): {"fetch_bytes": 60212594223, "write_bytes": 30167620968, "csrc": "4346d9d15ab6b371"},
}


def csrc_digest():
    """Digest of the kernel sources' code (comments and whitespace ignored)."""
    import re
    d = os.path.join(ROOT, "kv_cache_reads_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".hpp")):
            code = open(os.path.join(d, f)).read()
            code = re.sub(r"/\*.*?\*/", " ", code, flags=re.S)
            code = re.sub(r"//[^\n]*", " ", code)
            h.update(f.encode())
            h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload, K):
    rec = TRAFFIC.get((kernel, workload, K))
    if rec is None or rec["csrc"] != csrc_digest():
        return None
    return int(rec["fetch_bytes"] + rec["write_bytes"])


# ------------------------------------------------------------------ byte and flop model
def kernel_bytes(cfg, K, n_gen, store_phi=True, fused_phi=True):
    """Algorithmic HBM bytes of each kernel for one batch: inputs read once,
    outputs written once; workspace scratch (chunk reports, partial sums) is
    excluded.  The scan reads the mid-region keys once; the select writes the
    indices and their scores; the merge (and the fused select-and-merge kernel)
    reads one query's exact support, its retrieved phi_k rows and the unit's
    S, u.  With fused_phi the decode computes f = phi_q(q) itself (it reads
    Wq, bq instead of f).  The fused kernel counts the 4-byte kept score of
    each retrieved entry as the two-call path does (the selection's output),
    although there it never leaves the chip."""
    U, G, d, m, P = cfg.U, cfg.G, cfg.d, cfg.m, cfg.P
    Lm, na = cfg.L_mid, cfg.n_anchor
    e = 4 if cfg.kv_dtype == "f32" else 2
    ep = 4 if cfg.phi_dtype == "f32" else 2
    params = P * (m * d * 4 + m * 4)
    phi_row = m * ep if store_phi else d * e
    merge = (U * G * (K * (d * e + phi_row + 4) + (na + n_gen) * 2 * d * e + d * 4 + m * 4 + d * 4)
             + U * (m * d * 4 + m * 4) + (0 if store_phi else params)
             + (params - U * G * m * 4 if fused_phi else 0))
    return {
        "build_mfma_kernel": U * (2 * Lm * d * e + (Lm * m * ep if store_phi else 0)) + params,
        "build_reduce_kernel": U * (m * d * 4 + m * 4 + 4),
        "phi_kernel": 0 if fused_phi else U * G * (d * 4 + m * 4) + params,
        "topk_scan_kernel": U * (Lm * d * e + 4) + U * G * d * 4,
        "topk_select_kernel": U * G * K * 8,
        "merge_kernel": merge + U * G * K * 4,       # it also reads the indices
        "decode_fused_kernel": merge,
        "merge_combine_kernel": U * G * d * 4,
        "phi_mlp_kernel": U * Lm * (d * e + m * ep) + P * mlp_weight_bytes(d, m),
        "phi_mlp_small_kernel": U * G * (d * 4 + m * 4) + P * G * mlp_weight_bytes(d, m),
        "build_valu_kernel": U * (Lm * m * ep + 2 * Lm * d * e),
        "full_partial_kernel": U * (cfg.L + n_gen) * 2 * d * e + U * G * d * 4,
    }


def decode_step_bytes(cfg, K, n_gen, store_phi=True, fused_phi=True):
    """Algorithmic bytes of one decode step of the batch (scan + selection +
    merge; the method's own minimum traffic)."""
    kb = kernel_bytes(cfg, K, n_gen, store_phi, fused_phi)
    return kb["topk_scan_kernel"] + kb["decode_fused_kernel"] + kb["phi_kernel"]


def build_bytes(cfg, store_phi=True):
    kb = kernel_bytes(cfg, 0, 0, store_phi)
    return kb["build_mfma_kernel"] + kb["build_reduce_kernel"]


def build_flops(cfg):
    """Matrix-core work of the summary build for one batch.  Algorithmic: the
    projection K W^T and the contraction Phi^T [V | 1], 2 L_mid m (d + d + 1)
    per unit.  Issued: what the builder's MFMA instructions compute, 16x16x32
    bf16 tiles (16384 flops each): per 64-token tile and 16-feature slice,
    4 (d/32) 2 for the projection (W split into bf16 high and low parts) and
    2 (1 + d/16) for S and u; tiles = ceil(L_mid / 64) per unit (chunk
    boundaries add under 1 %)."""
    U, d, m, Lm = cfg.U, cfg.d, cfg.m, cfg.L_mid
    algo = U * 2 * Lm * m * (2 * d + 1)
    per_tile = 4 * (d // 32) * 2 + 2 * (1 + d // 16)
    issued = U * math.ceil(Lm / 64) * (m // 16) * per_tile * 16 * 16 * 32 * 2
    return algo, issued


def mlp_weight_bytes(d, m):
    H = MLP_WIDTH
    return 2 * (H * d + 2 * H * H + m * H) + 4 * (3 * H + 1 + m)


def mlp_flops(cfg):
    """Matrix-core flops per launch of the MLP feature kernels (2 per multiply-add)."""
    U, G, d, m, H = cfg.U, cfg.G, cfg.d, cfg.m, MLP_WIDTH
    per_row = 2 * (d * H + 2 * H * H + H * m)
    return {"phi_mlp_kernel": U * cfg.L_mid * per_row, "phi_mlp_small_kernel": U * G * per_row}


# ------------------------------------------------------------------ runner
class PathRunner:
    """Prepared C-ABI calls for one copy of the inputs (no per-call allocation)."""

    def __init__(self, R, cfg, inp, K, ws, torch, store_phi, fused_phi=True, mlp=None, separate=False):
        self.R, self.cfg, self.K, self.t = R, cfg, K, torch
        self.mlp = mlp                      # (phi_k weights, phi_q weights) of the MLP maps, or None
        self.separate = separate            # decode with rma_decode_topk + rma_decode_merge
        L = R.lib()
        self.L = L
        dev = inp.k.device
        U, G, d, m = cfg.U, cfg.G, cfg.d, cfg.m
        self.k, self.v, self.q, self.W, self.b = inp.k, inp.v, inp.q, inp.W, inp.b
        self.phi_k = torch.empty(U, cfg.L_mid, m, dtype=cfg.torch_phi_dtype(), device=dev) if store_phi else None
        self.S = torch.empty(U, m, d, dtype=torch.float32, device=dev)
        self.u = torch.empty(U, m, dtype=torch.float32, device=dev)
        self.kappa = torch.empty(U, dtype=torch.float32, device=dev)
        self.f = torch.empty(cfg.steps, U, G, m, dtype=torch.float32, device=dev)
        self.idx = torch.empty(cfg.steps, U, G, max(K, 1), dtype=torch.int32, device=dev)
        self.sel = torch.empty(cfg.steps, U, G, max(K, 1), dtype=torch.float32, device=dev)
        self.y = torch.empty(cfg.steps, U, G, d, dtype=torch.float32, device=dev)
        self.kv = R._kv(inp.k, inp.v)
        self.sp_pre = R.Span(cfg.L, cfg.n_sink, cfg.n_tail, 0)._c()
        self.sp_dec = [R.Span(cfg.L, cfg.n_sink, cfg.n_tail, cfg.n_gen(s))._c() for s in range(cfg.steps)]
        self.ws = ws
        P = ctypes.c_void_p
        self.p = lambda t: None if t is None else P(t.data_ptr())
        self.kdt = R._dt(inp.k.dtype)
        self.pdt = R._dt(cfg.torch_phi_dtype())
        self.Wm, self.bm = (None, None) if store_phi else (inp.W, inp.b)
        self.yf = None
        self.fused_phi = fused_phi and mlp is None     # f = phi_q(q) computed inside the decode
        if mlp is not None:
            self.kmid = inp.k[:, cfg.n_sink:cfg.n_sink + cfg.L_mid]

    def phik(self, st):
        """MLP features only: phi_k rows of the keys of the mid-region."""
        cfg, wk = self.cfg, self.mlp[0]
        r = self.L.rma_phi_mlp_features(self.p(self.kmid), self.kdt, cfg.U, cfg.L_mid, self.kmid.stride(0), cfg.d,
                                        ctypes.byref(wk._c), cfg.m, wk.P, self.p(self.phi_k), self.pdt, st)
        assert r == 0, r

    def summaries(self, st):
        cfg, p = self.cfg, self.p
        W, b = (None, None) if self.mlp is not None else (self.W, self.b)   # MLP rows are given
        r = self.L.rma_build_summaries(ctypes.byref(self.kv), ctypes.byref(self.sp_pre), p(W), p(b),
                                       cfg.m, cfg.P, p(self.phi_k), self.pdt, p(self.S), p(self.u),
                                       p(self.kappa), p(self.ws), self.ws.numel(), st)
        assert r == 0, r

    def build(self, st):
        if self.mlp is not None:
            self.phik(st)
        self.summaries(st)

    def phi(self, s, st):
        cfg, p = self.cfg, self.p
        q = self.q[s]
        if self.mlp is not None:   # one map per query head: U*G one-row units
            wq = self.mlp[1]
            r = self.L.rma_phi_mlp_features(p(q), 0, cfg.U * cfg.G, 1, cfg.d, cfg.d, ctypes.byref(wq._c), cfg.m,
                                            wq.P, p(self.f[s]), 0, st)
        else:
            r = self.L.rma_phi_features(p(q), 0, cfg.U, cfg.G, q.stride(0), cfg.d, p(self.W), p(self.b), cfg.m,
                                        cfg.P, p(self.f[s]), 0, st)
        assert r == 0, r

    def topk(self, s, st):
        cfg, p = self.cfg, self.p
        r = self.L.rma_decode_topk(p(self.q[s]), cfg.G, ctypes.byref(self.kv), ctypes.byref(self.sp_dec[s]),
                                   p(self.kappa), self.K, p(self.idx[s]), p(self.sel[s]), p(self.ws),
                                   self.ws.numel(), st)
        assert r == 0, r

    def merge(self, s, st):
        cfg, p = self.cfg, self.p
        f, Wq, bq = (None, self.W, self.b) if self.fused_phi else (self.f[s], None, None)
        r = self.L.rma_decode_merge(p(self.q[s]), p(f), p(Wq), p(bq), cfg.G, ctypes.byref(self.kv),
                                    ctypes.byref(self.sp_dec[s]), p(self.idx[s]), p(self.sel[s]), self.K,
                                    p(self.phi_k), self.pdt, p(self.Wm), p(self.bm), cfg.P, cfg.m, p(self.S),
                                    p(self.u), 0, p(self.y[s]), None, p(self.ws), self.ws.numel(), st)
        assert r == 0, r

    def one_call(self, s, st):
        cfg, p = self.cfg, self.p
        f, Wq, bq = (None, self.W, self.b) if self.fused_phi else (self.f[s], None, None)
        r = self.L.rma_decode(p(self.q[s]), p(f), p(Wq), p(bq), cfg.G, ctypes.byref(self.kv),
                              ctypes.byref(self.sp_dec[s]), p(self.kappa), self.K, p(self.phi_k), self.pdt,
                              p(self.Wm), p(self.bm), cfg.P, cfg.m, p(self.S), p(self.u), 0, None, None,
                              p(self.y[s]), None, p(self.ws), self.ws.numel(), st)
        assert r == 0, r

    def decode_calls(self, s):
        """The calls of decode step s, in order, as (name, fn(stream))."""
        calls = [] if self.fused_phi else [("phi", lambda st: self.phi(s, st))]
        if self.separate:
            calls += [("topk", lambda st: self.topk(s, st)), ("merge", lambda st: self.merge(s, st))]
        else:
            calls += [("decode", lambda st: self.one_call(s, st))]
        return calls

    def decode(self, st):
        for s in range(self.cfg.steps):
            for _, fn in self.decode_calls(s):
                fn(st)

    def full(self, st):
        """The full-attention reference for every decode step (no diagnostics)."""
        cfg, p = self.cfg, self.p
        if self.yf is None:
            self.yf = self.t.empty(cfg.steps, cfg.U, cfg.G, cfg.d, dtype=self.t.float32, device=self.k.device)
        for s in range(cfg.steps):
            r = self.L.rma_decode_full(p(self.q[s]), cfg.G, ctypes.byref(self.kv), ctypes.byref(self.sp_dec[s]),
                                       None, 0, None, p(self.yf[s]), None, p(self.ws), self.ws.numel(), st)
            assert r == 0, r

    def traced(self, R, what, st):
        """The build or the decode, eager, with every kernel timed by a pair of
        HIP events that its own dispatch stamps at its start and end
        (rma_trace_arm).  Returns [(kernel name, start event, end event), ...]."""
        t = self.t
        out = []

        def one(fn):
            evs = [t.cuda.Event(enable_timing=True) for _ in range(8)]
            R.rma_trace_arm(evs)
            fn(st)
            out.extend((n, evs[2 * j], evs[2 * j + 1]) for j, n in enumerate(R.rma_trace_kernels()))

        if what == "build":
            if self.mlp is not None:
                one(self.phik)
            one(self.summaries)
        else:
            for s in range(self.cfg.steps):
                for _, fn in self.decode_calls(s):
                    one(fn)
        return out


def capture_rounds(torch, fn, n_copies, stream, start=0):
    """HIP graphs for timed runs: `round` holds one call of fn for every input copy
    (copies start, start + 1, ... mod n_copies, in turn), `single[i]` one call for
    copy i.  A graph launch has a fixed cost of a few microseconds at its
    boundary; a round pays it once per n_copies steps, as a serving loop that
    captures several decode steps in one graph does."""
    single = []
    for r_i in range(n_copies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fn(r_i)
        single.append(g)
    rnd = torch.cuda.CUDAGraph()
    with torch.cuda.graph(rnd, stream=stream):
        for j in range(n_copies):
            fn((start + j) % n_copies)
    return rnd, single


def replay_steps(rnd, single, n_copies, n, start=0):
    """Enqueues exactly n steps: whole rounds, then single steps that continue the
    rotation where the rounds left it."""
    for _ in range(n // n_copies):
        rnd.replay()
    for i in range(n % n_copies):
        single[(start + i) % n_copies].replay()


def timed_replays(fn, n_copies, n, stream, use_graphs):
    """Average microseconds of fn(i) (enqueues work for input copy i % n_copies),
    replayed from HIP graphs of whole rounds over the copies when use_graphs."""
    import torch
    with torch.cuda.stream(stream):
        fn(0)  # outputs are allocated outside any capture
    stream.synchronize()
    if use_graphs:
        rnd, single = capture_rounds(torch, fn, n_copies, stream)
        run_n = lambda k: replay_steps(rnd, single, n_copies, k)  # noqa: E731
    else:
        def run_n(k):
            for i in range(k):
                fn(i)
    with torch.cuda.stream(stream):
        run_n(3)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record()
        run_n(n)
        e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n * 1e3


def kernel_stats(recs):
    """Average duration (ms) and launches per record of each kernel name."""
    tot, cnt = {}, {}
    for rec in recs:
        for kname, a, b in rec:
            tot[kname] = tot.get(kname, 0.0) + a.elapsed_time(b)
            cnt[kname] = cnt.get(kname, 0) + 1
    return {k: tot[k] / cnt[k] for k in tot}, {k: cnt[k] / len(recs) for k in cnt}


def ceilings(torch, log, R, mb=2048):
    """Measured streaming ceilings on this GPU, over arrays well above the 256 MB
    last-level cache: the library's streaming read (rma_stream_read: 1024
    workgroups, each a contiguous piece, the scan's load form), and torch's own
    kernels, a read that writes almost nothing (the sum of an fp32 array) and a
    copy (one read, one write)."""
    n = int(mb * 1e6) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    out = torch.empty((), dtype=torch.float32, device="cuda")
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    res = {}
    for name, fn, nbytes in (("stream_read", lambda: R.rma_stream_read(a, 1024, sink), 4 * n),
                             ("read", lambda: torch.sum(a, dim=0, out=out), 4 * n),
                             ("copy", lambda: b.copy_(a), 8 * n)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = round(nbytes / (e0.elapsed_time(e1) / reps / 1e3) / 1e9, 1)
    del a, b
    log(f"[bench] streaming ceilings over {4 * n / 1e9:.2f} GB arrays: library streaming read "
        f"{res['stream_read']} GB/s, torch read {res['read']} GB/s, copy {res['copy']} GB/s (read + write)")
    return {"stream_read_GBps": res["stream_read"], "read_GBps": res["read"], "copy_GBps": res["copy"],
            "array_GB": round(4 * n / 1e9, 2),
            "kernels": "rma_stream_read with 1024 workgroups (stream_read), torch.sum (read), "
                       "Tensor.copy_ (read + write)"}


def scan_blocks(cfg):
    """The Top-K scan's grid (chunks per unit x units) by the library's planning
    rule: chunks of whole 256-thread block passes (64 tokens at d = 64, 32 at
    d = 128), about 512 blocks when the units are few (at most 256 chunks per
    unit), none longer than the fp32 scores a scan block keeps in its 54272
    bytes of LDS (G rows of ch + 8 words beside G 512-bin histograms and the
    queries)."""
    Lm, U, G, d = cfg.L_mid, cfg.U, cfg.G, cfg.d
    tile = 64 if d == 64 else 32
    ch_max = max(tile, ((54272 - G * (512 * 4 + d * 4) - 64) // (4 * G) - 8) // tile * tile)
    lo, hi = -(-Lm // ch_max), min(256, -(-Lm // tile))
    nc = max(lo, min(-(-512 // U), hi))
    ch = -(-(-(-Lm // nc)) // tile) * tile
    return -(-Lm // ch) * U


def same_shape_read(R, torch, runners, n_copies, blocks, reps):
    """The library's streaming read over each rotating copy's key cache with the
    scan's grid, timed by dispatch-stamped event pairs: what reading the scan's
    bytes with the scan's grid costs when nothing else is done.  Returns (bytes
    per launch, average microseconds)."""
    sink = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    evs = []
    for i in range(reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        R.rma_trace_arm(e)
        R.rma_stream_read(runners[i % n_copies].k, blocks, sink)
        evs.append(e)
    torch.cuda.synchronize()
    us = sum(a.elapsed_time(b) for a, b in evs[1:]) / (len(evs) - 1) * 1e3
    k = runners[0].k
    return k.numel() * k.element_size(), us


def cpu_baseline(cfg, inp, K, seconds, mlp_mode=False):
    """The oracle (numpy fp64) on host cores.  Decode queries/s: for each unit of
    a bounded sample its prefill summaries are built (timed apart, as build
    tokens/s), then every decode query of the unit is timed (exhaustive Top-K by
    a full sort with exact rationals near ties, then the merge).  With all the
    host's BLAS threads, then with one."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    import oracle as O
    ncpu = len(os.sched_getaffinity(0))

    def host(u):
        p = u % cfg.P
        return dict(k=inp.k[u].float().cpu().numpy().astype(np.float64),
                    v=inp.v[u].float().cpu().numpy().astype(np.float64),
                    q=inp.q[:, u].cpu().numpy(), W=inp.W[p].cpu().numpy(), b=inp.b[p].cpu().numpy())

    _, M, _ = O.partition(cfg.L, cfg.n_sink, cfg.n_tail)
    if mlp_mode:
        from kv_cache_reads_amd import workload as Wl
        pk, pq = (Wl.generate_phi_mlp(cfg, which, m=cfg.m) for which in "kq")
        hp = lambda par, i: {k: v[i].double().numpy() if v.dim() > 1 else float(v[i]) for k, v in par.items()}

    def run(limit, budget):
        with threadpool_limits(limits=limit):
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
            nq, units, t_dec, t_build, toks = 0, 0, 0.0, 0.0, 0
            while t_dec + t_build < budget:
                uidx = units % cfg.U
                hu = host(uidx)                      # host copy, not timed
                t0 = time.perf_counter()
                if mlp_mode:
                    P = O.phi_mlp(hu["k"][M], hp(pk, uidx % cfg.P))
                    S, uu = O.summaries(P, hu["v"][M])
                else:
                    P, S, uu = O.prefill_unit(hu["k"][M], hu["v"][M], hu["W"], hu["b"])
                t1 = time.perf_counter()
                for s in range(cfg.steps):
                    for g in range(cfg.G):
                        q = hu["q"][s, g]
                        if mlp_mode:
                            f = O.phi_mlp(q[None], hp(pq, uidx % cfg.P * cfg.G + g))[0]
                        else:
                            f = O.phi_features(q[None], hu["W"], hu["b"])[0]
                        O.decode_query(q, f, hu["k"], hu["v"], P, S, uu, cfg.L, cfg.n_sink, cfg.n_tail,
                                       cfg.n_gen(s), K)
                        nq += 1
                t2 = time.perf_counter()
                t_build += t1 - t0
                t_dec += t2 - t1
                toks += cfg.L_mid
                units += 1
        return dict(q_per_s=nq / t_dec, build_tokens_per_s=toks / t_build, units=units, queries=nq,
                    t_dec=t_dec, t_build=t_build, threads=int(threads))

    full = run(ncpu, seconds)
    one = run(1, max(seconds / 3, 3.0))
    return dict(value=round(full["q_per_s"], 2), unit="queries/s", cores=full["threads"], kind="oracle",
                sample=(f"{full['units']} units of the workload ({full['queries']} decode queries: exhaustive "
                        f"Top-K + merge, {full['t_dec']:.1f} s; their prefill summaries timed apart, "
                        f"{full['t_build']:.1f} s), numpy fp64 with {full['threads']} BLAS threads on {ncpu} "
                        f"visible cores"),
                build_tokens_per_s=round(full["build_tokens_per_s"], 1),
                single_thread={"queries_per_s": round(one["q_per_s"], 2),
                               "build_tokens_per_s": round(one["build_tokens_per_s"], 1),
                               "sample": f"{one['units']} units, {one['queries']} queries, 1 BLAS thread"})


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark times one GPU: --gpus must be 1 "
                                   "(the units of a batch shard across GPUs with no communication)"}))
        sys.exit(2)
    import torch
    from kv_cache_reads_amd import rma as R
    from kv_cache_reads_amd import workload as Wl

    torch.cuda.set_device(0)
    cfg = Wl.CONFIGS[args.config]
    mlp_mode = args.phi == "mlp"
    if mlp_mode:
        cfg = cfg.with_(m=64)          # d_phi = 64 (the pages' setting)
    K = args.K if args.K is not None else cfg.K[0]
    log = lambda *a: print(*a, file=sys.stderr, flush=True)
    log(f"[bench] workload {cfg.name}: {cfg.desc}; K={K}")
    if args.copy_probe_mb > 0:
        n = int(args.copy_probe_mb * 1e6) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: neg over {n * 4} bytes read + {n * 4} bytes written, 3 launches")
        del a, b
    ceil = None if args.no_ceiling else ceilings(torch, log, R)
    t0 = time.time()
    inp = Wl.generate(cfg, device="cuda")
    torch.cuda.synchronize()
    log(f"[bench] inputs generated in {time.time() - t0:.1f} s")

    store_phi = not args.recompute_phi or cfg.kv_dtype != "bf16"   # recomputed rows need bf16 keys
    per_copy = (inp.k.numel() + inp.v.numel()) * inp.k.element_size() + \
        (cfg.U * cfg.L_mid * cfg.m * (4 if cfg.phi_dtype == "f32" else 2) if store_phi else 0)
    n_copies = max(1, math.ceil(args.rotate_bytes / per_copy))
    free = torch.cuda.mem_get_info()[0]
    n_copies = max(1, min(n_copies, int(0.6 * free // max(per_copy, 1))))
    copies = [inp]
    for _ in range(n_copies - 1):
        copies.append(Wl.Inputs(cfg, inp.k.clone(), inp.v.clone(), inp.q.clone(), inp.W.clone(),
                                inp.b.clone(), inp.needle_pos))
    sp = R.Span(cfg.L, cfg.n_sink, cfg.n_tail, cfg.n_gen(cfg.steps - 1))
    wsb = max(R.rma_workspace_bytes(R.RMA_OP_BUILD_SUMMARIES, inp.k, sp, 1, 0, cfg.m),
              R.rma_workspace_bytes(R.RMA_OP_DECODE_TOPK, inp.k, sp, cfg.G, K, cfg.m),
              R.rma_workspace_bytes(R.RMA_OP_DECODE_MERGE, inp.k, sp, cfg.G, K, cfg.m),
              R.rma_workspace_bytes(R.RMA_OP_DECODE, inp.k, sp, cfg.G, K, cfg.m))
    if not args.no_full:
        wsb = max(wsb, R.rma_workspace_bytes(R.RMA_OP_DECODE_FULL, inp.k, sp, cfg.G, 0, cfg.m))
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    fused_phi = not args.separate_phi and not mlp_mode
    mlp = None
    if mlp_mode:
        store_phi = True
        mlp = tuple(R.PhiMlpWeights(Wl.generate_phi_mlp(cfg, which, m=cfg.m, device="cuda")) for which in "kq")
    runners = [PathRunner(R, cfg, c, K, ws, torch, store_phi, fused_phi, mlp, args.separate) for c in copies]
    log(f"[bench] {n_copies} rotating copies of {per_copy / 1e6:.1f} MB; workspace {wsb / 1e6:.1f} MB")

    stream = torch.cuda.Stream()
    st = ctypes.c_void_p(stream.cuda_stream)
    cur = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)   # noqa: E731
    # prefill summaries of every copy (the decode reads them), then the eager
    # reference of copy 0's decode for the graph check
    with torch.cuda.stream(stream):
        for r in runners:
            r.build(st)
        runners[0].decode(st)
    stream.synchronize()
    y_eager = runners[0].y.clone()

    # timed steps continue the rotation over the copies where the warm-up left it
    start = args.warmup % n_copies
    graphs = None
    if not args.eager:
        try:
            rnd, graphs = capture_rounds(torch, lambda i: runners[i].decode(cur()), n_copies, stream, start)
            # replay checks against the eager result, with eager work in between:
            # the single-step graph of copy 0, then a whole round
            for rep in range(4):
                runners[0].y.zero_()
                (graphs[0] if rep < 3 else rnd).replay()
                torch.cuda.synchronize()
                assert torch.equal(runners[0].y, y_eager), "graph replay differs from eager"
                with torch.cuda.stream(stream):
                    runners[0].decode(st)
                stream.synchronize()
            log(f"[bench] HIP graph replays match the eager run (single steps and rounds of {n_copies})")
        except Exception as ex:  # fall back to eager launches
            log(f"[bench] graph capture unavailable ({ex}); timing eager launches")
            graphs = None

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            if graphs is not None:
                graphs[i % n_copies].replay()
            else:
                runners[i % n_copies].decode(st)
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` decode steps, synchronised on both sides
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        e0.record()
        if graphs is not None:
            replay_steps(rnd, graphs, n_copies, args.steps, start)
        else:
            for i in range(args.steps):
                runners[(start + i) % n_copies].decode(st)
        e1.record()
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    queries = cfg.U * cfg.G * cfg.steps
    value = queries / (ms_per_step / 1e3)
    dec_bytes = sum(decode_step_bytes(cfg, K, cfg.n_gen(s), store_phi, fused_phi) for s in range(cfg.steps))
    dec_gbs = dec_bytes / (ms_per_step / 1e3) / 1e9
    log(f"[bench] decode {ms_per_step * 1e3:.2f} us/step, {dec_bytes / 1e6:.1f} MB algorithmic -> {dec_gbs:.1f} GB/s "
        f"({dec_gbs / PEAK_HBM_GBS:.1%} of peak); {value / 1e6:.3f} M queries/s")

    # ---- per-kernel durations (eager launches on the path's stream, queued ahead)
    n_t = int(max(5, min(200, args.steps, 2.0 / max(ms_per_step / 1e3, 1e-6))))
    with torch.cuda.stream(stream):
        drecs = [runners[i % n_copies].traced(R, "decode", st) for i in range(n_t)]
        brecs = [runners[i % n_copies].traced(R, "build", st) for i in range(min(n_t, 50))]
    torch.cuda.synchronize()
    dk_avg, dk_n = kernel_stats(drecs)
    bk_avg, _ = kernel_stats(brecs)
    kb = kernel_bytes(cfg, K, cfg.n_gen(0), store_phi, fused_phi)
    for k in dk_avg:
        log(f"[bench]   {k:22s} {dk_avg[k] * 1e3:9.2f} us/launch x{dk_n[k]:.0f}  {kb.get(k, 0) / 1e6:8.2f} MB  "
            f"{kb.get(k, 0) / (dk_avg[k] / 1e3) / 1e9:8.1f} GB/s")
    # the dominant decode kernel is the one that moves most of the step's
    # algorithmic bytes (the scan: the mid-region keys); every decode kernel's
    # own fraction is listed beside it
    dom = max(dk_avg, key=lambda k: kb.get(k, 0) * dk_n[k])
    achieved = kb[dom] / (dk_avg[dom] / 1e3) / 1e9
    traffic = measured_traffic(dom, cfg.name, K)
    per_kernel = {}
    for k in dk_avg:
        a_k = kb.get(k, 0) / (dk_avg[k] / 1e3) / 1e9
        t_k = measured_traffic(k, cfg.name, K)
        per_kernel[k] = {"algorithmic_bytes_per_launch": kb.get(k, 0), "avg_launch_us": round(dk_avg[k] * 1e3, 3),
                         "launches_per_step": round(dk_n[k], 3),
                         "achieved": round(a_k, 1), "frac": round(a_k / PEAK_HBM_GBS, 4), "traffic": t_k}
    ss_bytes, ss_us = same_shape_read(R, torch, runners, n_copies, scan_blocks(cfg), max(6, min(n_t, 60)))
    ss_gbs = ss_bytes / (ss_us / 1e6) / 1e9
    log(f"[bench] streaming read of the keys with the scan's grid ({scan_blocks(cfg)} blocks): "
        f"{ss_us:.2f} us, {ss_gbs:.1f} GB/s")
    roof = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
            "algorithmic_bytes_per_launch": kb[dom], "avg_launch_us": round(dk_avg[dom] * 1e3, 3),
            "traffic_source": None if traffic is None else f"profiles/traffic_{cfg.name}.md",
            "dominant_by": "algorithmic bytes per decode step",
            "same_shape_read": {"kernel": "rma_stream_read over the key cache with the scan's grid",
                                "blocks": scan_blocks(cfg), "bytes": ss_bytes, "us": round(ss_us, 3),
                                "GBps": round(ss_gbs, 1), "frac": round(ss_gbs / PEAK_HBM_GBS, 4),
                                "scan_over_read": round(achieved / ss_gbs, 4) if dom == "topk_scan_kernel" else None},
            "decode_kernels": per_kernel,
            "decode_step": {"algorithmic_MB": round(dec_bytes / 1e6, 3), "us": round(ms_per_step * 1e3, 2),
                            "GBps": round(dec_gbs, 1), "frac": round(dec_gbs / PEAK_HBM_GBS, 4)}}

    # ---- the prefill summary build, on its own (graph replays over the copies)
    use_graphs = graphs is not None
    build_us = timed_replays(lambda i: runners[i % n_copies].build(cur()), n_copies,
                             max(5, min(args.steps, 100)), stream, use_graphs)
    bbytes = build_bytes(cfg, store_phi)
    bgbs = bbytes / (build_us / 1e6) / 1e9
    algo_fl, issued_fl = build_flops(cfg)
    bk = "build_mfma_kernel" if "build_mfma_kernel" in bk_avg else max(bk_avg, key=bk_avg.get)
    bk_us = bk_avg[bk] * 1e3
    kb_b = kernel_bytes(cfg, K, 0, store_phi)[bk]
    build = {"call_us": round(build_us, 2), "algorithmic_MB": round(bbytes / 1e6, 3), "GBps": round(bgbs, 1),
             "frac_hbm": round(bgbs / PEAK_HBM_GBS, 4),
             "per_kernel_us": {k: round(v * 1e3, 2) for k, v in bk_avg.items()},
             "tokens_per_s": round(cfg.U * cfg.L_mid / (build_us / 1e6), 1),
             "roofline": {"bound": "hbm", "kernel": bk, "achieved": round(kb_b / (bk_us / 1e6) / 1e9, 1),
                          "peak": PEAK_HBM_GBS, "unit": "GB/s",
                          "frac": round(kb_b / (bk_us / 1e6) / 1e9 / PEAK_HBM_GBS, 4),
                          "algorithmic_bytes_per_launch": kb_b, "avg_launch_us": round(bk_us, 3),
                          "traffic": measured_traffic(bk, cfg.name, K)}}
    if bk == "build_mfma_kernel":
        build["mfma"] = {"algorithmic_TFLOP": round(algo_fl / 1e12, 4), "issued_TFLOP": round(issued_fl / 1e12, 4),
                         "algorithmic_TFLOPs": round(algo_fl / (bk_us / 1e6) / 1e12, 1),
                         "issued_TFLOPs": round(issued_fl / (bk_us / 1e6) / 1e12, 1),
                         "util_algorithmic": round(algo_fl / (bk_us / 1e6) / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "util_issued": round(issued_fl / (bk_us / 1e6) / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "peak_TFLOPs": PEAK_BF16_TFLOPS,
                         "issued_note": "W is split into bf16 high + low parts: the projection's MFMAs double"}
    log(f"[bench] build {build_us:.2f} us/call, {bbytes / 1e6:.1f} MB -> {bgbs:.1f} GB/s; kernels {build['per_kernel_us']}")

    # ---- whole path: build + decode per step
    def whole(i):
        r = runners[i % n_copies]
        r.build(cur())
        r.decode(cur())
    whole_us = timed_replays(whole, n_copies, max(5, min(args.steps, 200)), stream, use_graphs)
    log(f"[bench] whole path (build + decode) {whole_us:.2f} us/step ({queries / whole_us:.3f} M queries/s)")

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {cfg.desc}",
            "units": cfg.U, "query_heads_per_unit": cfg.G, "head_dim": cfg.d, "context": cfg.L,
            "anchors": [cfg.n_sink, cfg.n_tail], "K": K, "phi_features": cfg.m,
            "decode_steps": cfg.steps, "queries_per_step": queries,
            "step": ("one decode pass over the batch: " +
                     ("rma_decode_topk + rma_decode_merge" if args.separate else
                      "rma_decode (scan, then the fused selection and merge)") +
                     (", f = phi_q(q) inside" if fused_phi else ", phi_q by its own kernel") +
                     "; summaries built beforehand (reported under build)"),
            "phi": ("MLP family: one-block ReZero MLP, width 512, exponentiated output, d_phi 64, random "
                    "weights, bf16 matrix-core operands" if mlp_mode else "elu(Wx+b)+1"),
            "phi_k_rows": "stored" if store_phi else "recomputed at decode (not stored)",
            "kv_dtype": cfg.kv_dtype, "accumulate": "fp32",
            "rotating_copies": n_copies,
            "launch": f"hip_graph, rounds of {n_copies} steps" if graphs is not None else "eager",
            "decode_per_kernel_us": {k: round(v * 1e3, 2) for k, v in dk_avg.items()},
            "decode_per_kernel_GBps": {k: round(kb.get(k, 0) / (v / 1e3) / 1e9, 1) for k, v in dk_avg.items()},
            "decode_GBps": round(dec_gbs, 1),
            "build": build,
            "whole_path": {"us_per_step": round(whole_us, 2), "queries_per_s": round(queries / (whole_us / 1e6), 1),
                           "step": "rma_build_summaries + the decode step"},
            "ceilings": ceil,
        },
        "roofline": roof,
    }
    if mlp_mode:
        fl = mlp_flops(cfg)
        out["config"]["mlp_TFLOPs"] = {k: round(fl[k] / (v / 1e3) / 1e12, 1)
                                       for k, v in {**bk_avg, **dk_avg}.items() if k in fl}
    if not args.no_full:
        full_us = timed_replays(lambda i: runners[i % n_copies].full(cur()), n_copies,
                                max(5, min(args.steps, 200)), stream, use_graphs)
        fbytes = sum(kernel_bytes(cfg, K, cfg.n_gen(s))["full_partial_kernel"] for s in range(cfg.steps))
        out["config"]["full_exact_decode"] = {
            "us_per_step": round(full_us, 2), "queries_per_s": round(queries / (full_us / 1e6), 1),
            "algorithmic_MB": round(fbytes / 1e6, 3), "GBps": round(fbytes / (full_us / 1e6) / 1e9, 1),
            "method_decode_speedup": round(full_us / (ms_per_step * 1e3), 3)}
        log(f"[bench] full-attention decode {full_us:.2f} us/step -> method speedup "
            f"{full_us / (ms_per_step * 1e3):.3f}")
    if not args.no_cpu_baseline:
        log(f"[bench] timing the oracle on the host for ~{args.cpu_seconds:.0f} s (+ one thread)")
        out["cpu_baseline"] = cpu_baseline(cfg, inp, K, args.cpu_seconds, mlp_mode)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
