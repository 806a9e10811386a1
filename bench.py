#!/usr/bin/env python3
"""Benchmark of the Top-K+phi residual-mass-accounting path on one MI355X.

One step = one pass of the whole path over one batch of the workload:
prefill summaries (S, u; rma_build_summaries), then for every
decode step of the workload phi_q (rma_phi_features), the exhaustive Top-K
(rma_decode_topk) and the exact branch + subtraction + residual + single
normalisation (rma_decode_merge).  Default workload: the 1B-shaped GQA layer at
32K context with a 1 % budget (8 kv heads x 4 query heads, d=64, K=328).

Inputs are resident in HBM before timing starts.  Steps rotate over copies of
the inputs whose total exceeds 1 GB so that no step is served from the 256 MB
last-level cache.  Each step is replayed from a HIP graph (compared against an
eager run first).  Prints one JSON line.

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

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores
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
    ap.add_argument("--separate-phi", action="store_true",
                    help="compute phi_q with rma_phi_features instead of inside the merge")
    ap.add_argument("--no-full", action="store_true",
                    help="skip timing the full-attention reference decode")
    ap.add_argument("--recompute-phi", action="store_true",
                    help="do not store the phi_k rows at prefill; the merge recomputes the retrieved "
                         "rows from their keys (bf16 keys; saves the rows' HBM, costs MFMA/VALU work "
                         "at every decode step)")
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
    # c1 (K=328); FETCH_SIZE x 2.0 and WRITE_SIZE x 1.0 from a 1.024 GB neg copy
    ("build_mfma_kernel", "c1", 328): dict(csrc="c4f432f3331a987a", fetch_bytes=69264497, write_bytes=84049512),
    ("topk_scan_kernel", "c1", 328): dict(csrc="c4f432f3331a987a", fetch_bytes=33832736, write_bytes=636576),
    ("merge_kernel", "c1", 328): dict(csrc="c4f432f3331a987a", fetch_bytes=7074332, write_bytes=8192),
    ("full_partial_kernel", "c1", 328): dict(csrc="c4f432f3331a987a", fetch_bytes=67368312, write_bytes=589824),
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


# ------------------------------------------------------------------ byte model
def call_bytes(cfg, K, n_gen, store_phi=True, fused_phi=True, mlp=False):
    """Algorithmic HBM bytes of each call for one batch (inputs read once,
    outputs written once; workspace scratch excluded).  With mlp, the MLP
    features: phik = phi_k rows of the keys, build = summaries over those rows,
    phi = phi_q of the queries."""
    kb = kernel_bytes(cfg, K, n_gen, store_phi, fused_phi)
    out = dict(build=kb["build_mfma_kernel"] + kb["build_reduce_kernel"], phi=kb["phi_kernel"],
               topk=kb["topk_scan_kernel"] + kb["topk_select_kernel"], merge=kb["merge_kernel"], phik=0)
    if mlp:
        out.update(phik=kb["phi_mlp_kernel"], build=kb["build_valu_kernel"] + kb["build_reduce_kernel"],
                   phi=kb["phi_mlp_small_kernel"])
    return out


def kernel_bytes(cfg, K, n_gen, store_phi=True, fused_phi=True):
    """Algorithmic HBM bytes of each kernel for one batch.  The builder reads the
    mid-region K and V rows once (and writes phi_k once when the rows are stored;
    its per-chunk partial sums are scratch); the reduce writes S, u, kappa; the scan reads the mid-region K
    rows once (score bins and candidate lists are scratch); the select writes the
    indices and their scores; the merge reads what one query's exact support and
    residual need.  With fused_phi the merge computes f = phi_q(q) itself (it
    reads Wq, bq instead of f, and no phi kernel runs)."""
    U, G, d, m, P = cfg.U, cfg.G, cfg.d, cfg.m, cfg.P
    Lm, na = cfg.L_mid, cfg.n_anchor
    e = 4 if cfg.kv_dtype == "f32" else 2
    ep = 4 if cfg.phi_dtype == "f32" else 2
    params = P * (m * d * 4 + m * 4)
    # phi_k rows are either stored by the builder and gathered by the merge
    # (default), or not stored, the merge recomputing the retrieved ones from
    # their key rows (which it then reads instead)
    phi_row = m * ep if store_phi else d * e
    return {
        "build_mfma_kernel": U * (2 * Lm * d * e + (Lm * m * ep if store_phi else 0)) + params,
        "build_reduce_kernel": U * (m * d * 4 + m * 4 + 4),
        "phi_kernel": 0 if fused_phi else U * G * (d * 4 + m * 4) + params,
        "topk_scan_kernel": U * (Lm * d * e + 4) + U * G * d * 4,
        "topk_select_kernel": U * G * K * 8,
        "merge_kernel": U * G * (K * (d * e + phi_row + 8) + (na + n_gen) * 2 * d * e + d * 4 + m * 4 + d * 4)
        + U * (m * d * 4 + m * 4) + (0 if store_phi else params)
        + (params - U * G * m * 4 if fused_phi else 0),
        # with a head's entries split over several blocks, this kernel writes y
        # from their partials (scratch); the merge call's bytes are the merge's
        "merge_combine_kernel": U * G * d * 4,
        # MLP features (the pages' family): keys of the mid-region in, phi_k rows
        # out, and each map's bf16 weights and fp32 biases once
        "phi_mlp_kernel": U * Lm * (d * e + m * ep) + P * mlp_weight_bytes(d, m),
        "phi_mlp_small_kernel": U * G * (d * 4 + m * 4) + P * G * mlp_weight_bytes(d, m),
        # summaries over given phi_k rows: rows, V and (for kappa) K read once
        "build_valu_kernel": U * (Lm * m * ep + 2 * Lm * d * e),
    }


def mlp_weight_bytes(d, m):
    H = MLP_WIDTH
    return 2 * (H * d + 2 * H * H + m * H) + 4 * (3 * H + 1 + m)


def kernel_flops(cfg):
    """Matrix-core flops per launch of the MLP feature kernels (2 per multiply-add)."""
    U, G, d, m, H = cfg.U, cfg.G, cfg.d, cfg.m, MLP_WIDTH
    per_row = 2 * (d * H + 2 * H * H + H * m)
    return {"phi_mlp_kernel": U * cfg.L_mid * per_row, "phi_mlp_small_kernel": U * G * per_row}


# ------------------------------------------------------------------ runner
class PathRunner:
    """Prepared C-ABI calls for one copy of the inputs (no per-call allocation)."""

    def __init__(self, R, cfg, inp, K, ws, torch, store_phi, fused_phi=True, mlp=None):
        self.R, self.cfg, self.K, self.t = R, cfg, K, torch
        # mlp: (phi_k weights, phi_q weights) of the MLP feature maps, or None
        self.mlp = mlp
        L = R.lib()
        self.L = L
        dev = inp.k.device
        U, G, d, m = cfg.U, cfg.G, cfg.d, cfg.m
        self.k, self.v, self.q, self.W, self.b = inp.k, inp.v, inp.q, inp.W, inp.b
        # phi_k rows: stored by the builder, or (None) recomputed by the merge
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
        # f = phi_q(q): computed inside the merge (fused), or by rma_phi_features
        # (or by the MLP feature kernel)
        self.fused_phi = fused_phi and mlp is None
        if mlp is not None:
            self.kmid = inp.k[:, cfg.n_sink:cfg.n_sink + cfg.L_mid]

    def phik(self, st):
        """MLP features only: phi_k rows of the keys of the mid-region."""
        cfg, wk = self.cfg, self.mlp[0]
        r = self.L.rma_phi_mlp_features(self.p(self.kmid), self.kdt, cfg.U, cfg.L_mid, self.kmid.stride(0), cfg.d,
                                        ctypes.byref(wk._c), cfg.m, wk.P, self.p(self.phi_k), self.pdt, st)
        assert r == 0, r

    def build(self, st):
        cfg, p = self.cfg, self.p
        W, b = (None, None) if self.mlp is not None else (self.W, self.b)   # MLP rows are given
        r = self.L.rma_build_summaries(ctypes.byref(self.kv), ctypes.byref(self.sp_pre), p(W), p(b),
                                       cfg.m, cfg.P, p(self.phi_k), self.pdt, p(self.S), p(self.u),
                                       p(self.kappa), p(self.ws), self.ws.numel(), st)
        assert r == 0, r

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

    def full(self, s, st):
        """The full-attention reference for decode step s (no diagnostics)."""
        cfg, p = self.cfg, self.p
        if self.yf is None:
            self.yf = self.t.empty(cfg.steps, cfg.U, cfg.G, cfg.d, dtype=self.t.float32, device=self.k.device)
        r = self.L.rma_decode_full(p(self.q[s]), cfg.G, ctypes.byref(self.kv), ctypes.byref(self.sp_dec[s]),
                                   None, 0, None, p(self.yf[s]), None, p(self.ws), self.ws.numel(), st)
        assert r == 0, r

    def step(self, st):
        """The whole path: prefill summaries, then every decode step."""
        if self.mlp is not None:
            self.phik(st)
        self.build(st)
        for s in range(self.cfg.steps):
            if not self.fused_phi:
                self.phi(s, st)
            self.topk(s, st)
            self.merge(s, st)

    def traced_step(self, st, R):
        """The whole path, eager, with every kernel timed by a pair of HIP events
        that its own dispatch stamps at its start and end (rma_trace_arm).
        Returns one record per call: (call name, [(kernel name, start event,
        end event), ...])."""
        t = self.t
        out = []

        def traced(name, fn):
            evs = [t.cuda.Event(enable_timing=True) for _ in range(4)]
            R.rma_trace_arm(evs)
            fn()
            names = R.rma_trace_kernels()
            out.append((name, [(n, evs[2 * j], evs[2 * j + 1]) for j, n in enumerate(names)]))

        if self.mlp is not None:
            traced("phik", lambda: self.phik(st))
        traced("build", lambda: self.build(st))
        for s in range(self.cfg.steps):
            if not self.fused_phi:
                traced("phi", lambda: self.phi(s, st))
            traced("topk", lambda: self.topk(s, st))
            traced("merge", lambda: self.merge(s, st))
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


def decode_timing(args, cfg, runners, n_copies, stream, st, use_graphs, queries, log):
    """The method's decode steps alone (phi_q, top-K, merge over summaries built
    earlier) and the full-attention reference (rma_decode_full over every
    position, no diagnostics) for the same decode steps, both replayed like the
    whole step: the speed ratio of the method's decode against full attention."""
    n = max(5, min(args.steps, 200))

    def dec(i):
        r = runners[i % n_copies]
        for s in range(cfg.steps):
            if not r.fused_phi:
                r.phi(s, st)
            r.topk(s, st)
            r.merge(s, st)

    def full(i):
        r = runners[i % n_copies]
        for s in range(cfg.steps):
            r.full(s, st)

    dec_us = timed_replays(dec, n_copies, n, stream, use_graphs)
    full_us = timed_replays(full, n_copies, n, stream, use_graphs)
    e = 2 if cfg.kv_dtype == "bf16" else 4
    nbytes = sum(cfg.U * (cfg.L + cfg.n_gen(s)) * cfg.d * e * 2 + cfg.U * cfg.G * cfg.d * 8
                 for s in range(cfg.steps))
    log(f"[bench] method decode {dec_us:.2f} us/step ({queries / dec_us:.3f} M queries/s); full-attention "
        f"decode {full_us:.2f} us/step, {nbytes / 1e6:.1f} MB -> {nbytes / (full_us / 1e6) / 1e9:.1f} GB/s")
    return dec_us, {"us_per_step": round(full_us, 2), "queries_per_s": round(queries / (full_us / 1e6), 1),
                    "algorithmic_MB": round(nbytes / 1e6, 3),
                    "GBps": round(nbytes / (full_us / 1e6) / 1e9, 1),
                    "method_decode_speedup": round(full_us / dec_us, 3), "timed_steps": n}


def cpu_baseline(cfg, inp, K, seconds, mlp_mode=False):
    """The oracle (numpy fp64) on host cores: prefill + decode of whole units
    (with mlp_mode, its MLP feature maps on the same seeded weights)."""
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
    with threadpool_limits(limits=ncpu):
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        nq, units, dt = 0, 0, 0.0
        done = False
        while not done:
            for uidx in range(cfg.U):
                hu = host(uidx)                      # host copy, not timed
                t1 = time.perf_counter()
                if mlp_mode:
                    P = O.phi_mlp(hu["k"][M], hp(pk, uidx % cfg.P))
                    S, uu = O.summaries(P, hu["v"][M])
                else:
                    P, S, uu = O.prefill_unit(hu["k"][M], hu["v"][M], hu["W"], hu["b"])
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
                dt += time.perf_counter() - t1
                units += 1
                if dt >= seconds:
                    done = True
                    break
    return dict(value=nq / dt, unit="queries/s", cores=int(threads), kind="oracle",
                sample=f"{units} units of the same workload (prefill summaries + all {cfg.steps} decode "
                       f"step(s) x {cfg.G} query heads per unit), {dt:.1f} s, numpy fp64 with "
                       f"{threads} BLAS threads on {ncpu} visible cores")


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
              R.rma_workspace_bytes(R.RMA_OP_DECODE_MERGE, inp.k, sp, cfg.G, K, cfg.m))
    if not args.no_full:
        wsb = max(wsb, R.rma_workspace_bytes(R.RMA_OP_DECODE_FULL, inp.k, sp, cfg.G, 0, cfg.m))
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    fused_phi = not args.separate_phi and not mlp_mode
    mlp = None
    if mlp_mode:
        store_phi = True
        mlp = tuple(R.PhiMlpWeights(Wl.generate_phi_mlp(cfg, which, m=cfg.m, device="cuda")) for which in "kq")
    runners = [PathRunner(R, cfg, c, K, ws, torch, store_phi, fused_phi, mlp) for c in copies]
    log(f"[bench] {n_copies} rotating copies of {per_copy / 1e6:.1f} MB; workspace {wsb / 1e6:.1f} MB")

    stream = torch.cuda.Stream()
    st = ctypes.c_void_p(stream.cuda_stream)
    # eager reference outputs (copy 0) for the graph check
    with torch.cuda.stream(stream):
        runners[0].step(st)
    stream.synchronize()
    y_eager = runners[0].y.clone()
    idx_eager = runners[0].idx.clone()

    # timed steps continue the rotation over the copies where the warm-up left it
    start = args.warmup % n_copies
    graphs = None
    if not args.eager:
        try:
            rnd, graphs = capture_rounds(
                torch, lambda i: runners[i].step(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)),
                n_copies, stream, start)
            # replay checks against the eager result, with eager work in between:
            # the single-step graph of copy 0, then a whole round
            for rep in range(4):
                runners[0].y.zero_()
                (graphs[0] if rep < 3 else rnd).replay()
                torch.cuda.synchronize()
                assert torch.equal(runners[0].y, y_eager) and torch.equal(runners[0].idx, idx_eager), \
                    "graph replay differs from eager"
                with torch.cuda.stream(stream):
                    runners[0].step(st)
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
                runners[i % n_copies].step(st)
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps, synchronised on both sides
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        e0.record()
        if graphs is not None:
            replay_steps(rnd, graphs, n_copies, args.steps, start)
        else:
            for i in range(args.steps):
                runners[(start + i) % n_copies].step(st)
        e1.record()
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    queries = cfg.U * cfg.G * cfg.steps
    value = queries / (ms_per_step / 1e3)

    # ---- per-kernel durations: HIP events that each kernel's own dispatch stamps
    # at its start and end (eager launches on the path's stream, queued ahead)
    n_t = int(max(5, min(200, args.steps, 2.0 / max(ms_per_step / 1e3, 1e-6))))
    recs = []
    with torch.cuda.stream(stream):
        for i in range(n_t):
            recs.append(runners[i % n_copies].traced_step(st, R))
    torch.cuda.synchronize()
    names = ["build", "topk", "merge"] if fused_phi else ["build", "phi", "topk", "merge"]
    if mlp_mode:
        names = ["phik"] + names
    call_ms = {n: 0.0 for n in names}
    kern_ms, kern_n = {}, {}
    for rec in recs:
        for call, ks in rec:
            call_ms[call] += ks[0][1].elapsed_time(ks[-1][2])
            for kname, a, b in ks:
                kern_ms[kname] = kern_ms.get(kname, 0.0) + a.elapsed_time(b)
                kern_n[kname] = kern_n.get(kname, 0) + 1
    dur = {n: call_ms[n] / n_t for n in names}                       # ms per step
    kavg = {k: kern_ms[k] / kern_n[k] for k in kern_ms}               # ms per launch
    launches = {k: kern_n[k] / n_t for k in kern_n}                  # launches per step
    nb = call_bytes(cfg, K, cfg.n_gen(0), store_phi, fused_phi, mlp_mode)
    kb = kernel_bytes(cfg, K, cfg.n_gen(0), store_phi, fused_phi)
    step_bytes = nb["build"] + nb["phik"] + sum(call_bytes(cfg, K, cfg.n_gen(s), store_phi, fused_phi, mlp_mode)[c]
                                   for s in range(cfg.steps) for c in ("phi", "topk", "merge"))
    prefill_calls = ("build", "phik")
    gbs = {n: nb[n] * (1 if n in prefill_calls else cfg.steps) / (dur[n] / 1e3) / 1e9 for n in names}
    kgbs = {k: kb[k] / (kavg[k] / 1e3) / 1e9 for k in kavg}
    kfl = kernel_flops(cfg)
    ktf = {k: kfl[k] / (kavg[k] / 1e3) / 1e12 for k in kavg if k in kfl}      # TFLOP/s
    for n in names:
        log(f"[bench] {n:6s} {dur[n] * 1e3:9.2f} us/step  {gbs[n]:8.1f} GB/s")
    for k in kavg:
        log(f"[bench]   {k:22s} {kavg[k] * 1e3:9.2f} us/launch x{launches[k]:.0f}  "
            f"{kb[k] / 1e6:8.2f} MB  {kgbs[k]:8.1f} GB/s" + (f"  {ktf[k]:8.1f} TFLOP/s" if k in ktf else ""))
    log(f"[bench] step {ms_per_step * 1e3:.2f} us, {step_bytes / 1e6:.1f} MB algorithmic "
        f"-> {step_bytes / (ms_per_step / 1e3) / 1e9:.1f} GB/s; {value / 1e6:.3f} M queries/s")
    decode_us = sum(dur[n] for n in names if n not in prefill_calls) * 1e3
    dom = max(kavg, key=lambda k: kavg[k] * launches[k])     # most time per step
    achieved = kgbs[dom]
    traffic = measured_traffic(dom, cfg.name, K)
    if dom in ktf:   # a matrix-core contraction: its own bf16 peak
        roof = {"bound": "mfma", "kernel": dom, "achieved": round(ktf[dom], 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ktf[dom] / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "algorithmic_flops_per_launch": kfl[dom], "algorithmic_bytes_per_launch": kb[dom],
                "avg_launch_us": round(kavg[dom] * 1e3, 3),
                "traffic_source": None if traffic is None else f"profiles/traffic_{cfg.name}.md"}
    else:
        roof = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": kb[dom], "avg_launch_us": round(kavg[dom] * 1e3, 3),
                "traffic_source": None if traffic is None else f"profiles/traffic_{cfg.name}.md"}

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
            "step": ("prefill MLP phi_k + summaries over those rows + MLP phi_q + top-K + merge" if mlp_mode
                     else "prefill summaries + top-K + merge (phi_q computed inside the merge)" if fused_phi
                     else "prefill summaries + phi_q + top-K + merge"),
            "phi": ("MLP family: one-block ReZero MLP, width 512, exponentiated output, d_phi 64, random "
                    "weights, bf16 matrix-core operands" if mlp_mode else "elu(Wx+b)+1"),
            **({"per_kernel_TFLOPs": {k: round(v, 1) for k, v in ktf.items()}} if ktf else {}),
            "phi_k_rows": "stored" if store_phi else "recomputed at decode (not stored)",
            "kv_dtype": cfg.kv_dtype, "accumulate": "fp32",
            "rotating_copies": n_copies, "launch": f"hip_graph, rounds of {n_copies} steps" if graphs is not None else "eager",
            "step_algorithmic_MB": round(step_bytes / 1e6, 3),
            "step_GBps": round(step_bytes / (ms_per_step / 1e3) / 1e9, 1),
            "per_call_us": {n: round(dur[n] * 1e3, 2) for n in names},
            "per_call_GBps": {n: round(gbs[n], 1) for n in names},
            "per_kernel_us": {k: round(kavg[k] * 1e3, 2) for k in kavg},
            "per_kernel_GBps": {k: round(kgbs[k], 1) for k in kavg},
            "decode_only_queries_per_s": round(queries / (decode_us / 1e6), 1),
        },
        "roofline": roof,
    }
    if not args.no_full:
        dec_us, out["config"]["full_exact_decode"] = decode_timing(args, cfg, runners, n_copies, stream, st,
                                                                   graphs is not None, queries, log)
        out["config"]["decode_only_us_per_step"] = round(dec_us, 2)
        out["config"]["decode_only_queries_per_s"] = round(queries / (dec_us / 1e6), 1)
        dbytes = step_bytes - nb["build"] - nb["phik"]
        out["config"]["decode_only_GBps"] = round(dbytes / (dec_us / 1e6) / 1e9, 1)
    if not args.no_cpu_baseline:
        log(f"[bench] timing the oracle on the host for ~{args.cpu_seconds:.0f} s")
        out["cpu_baseline"] = cpu_baseline(cfg, inp, K, args.cpu_seconds, mlp_mode)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
