"""Shared helpers of the GPU parity tests: run the HIP path through the C-ABI
binding, run the fp64 oracle on the same inputs, compare.

Tolerances:
  * Top-K indices: bit-exact.
  * y: max |y - y_ref| <= 2e-3 and, per query, ||y - y_ref||_2 / ||y_ref||_2
    <= 1e-2 (fp32 accumulation over bf16 K/V).
  * phi_k rows: one bf16 rounding (2^-9 relative) plus the split-bf16
    projection (< 2^-16 relative) -> |dphi| <= 2^-8 |phi| + 1e-6.
  * S, u: each stored phi row carries <= 2^-9 relative rounding, so
    |dS| <= 2^-8 * (|phi|^T |V|) and |du| <= 2^-8 * u elementwise, plus fp32
    summation.
  * kappa: an upper bound of max ||k_i||_2 within 2e-5 relative.
"""
import math
import os
import sys

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import oracle as O  # noqa: E402
from kv_cache_reads_amd import rma as R  # noqa: E402
from kv_cache_reads_amd import workload as W  # noqa: E402

ABS_TOL = 2e-3
REL_TOL = 1e-2


def log(msg):
    print(msg, flush=True)


def prefill_span(cfg):
    return R.Span(cfg.L, cfg.n_sink, cfg.n_tail, 0)


def decode_span(cfg, step):
    return R.Span(cfg.L, cfg.n_sink, cfg.n_tail, cfg.n_gen(step))


def hip_prefill(inp, ws=None, store_phi=True):
    """store_phi=False: the phi_k rows are not kept; decode recomputes them."""
    cfg = inp.cfg
    return R.rma_build_summaries(inp.k, inp.v, prefill_span(cfg), inp.W, inp.b,
                                 phi_dtype=cfg.torch_phi_dtype(), ws=ws, store_phi=store_phi)


def hip_decode(inp, pre, K, step, flags=R.RMA_MERGE_SUB, ws=None, fused_phi=False):
    """fused_phi: the merge computes f = phi_q(q) from W, b itself."""
    cfg = inp.cfg
    phi_k, S, u, kappa = pre
    q = inp.q[step].contiguous()
    f = None if fused_phi else R.rma_phi_features(q, inp.W, inp.b)
    sp = decode_span(cfg, step)
    idx, sel = R.rma_decode_topk(q, inp.k, sp, kappa, K, ws=ws)
    recompute = dict(Wk=inp.W, bk=inp.b) if phi_k is None else {}
    if fused_phi:
        recompute.update(Wq=inp.W, bq=inp.b)
    y, stats = R.rma_decode_merge(q, f, inp.k, inp.v, sp, idx, sel, K, phi_k, S, u, flags=flags,
                                  want_stats=True, ws=ws, m=cfg.m, **recompute)
    return dict(idx=idx, sel=sel, y=y, stats=stats, f=f)


def host_unit(inp, u):
    cfg = inp.cfg
    p = u % cfg.P
    return dict(k=inp.k[u].float().cpu().numpy().astype(np.float64),
                v=inp.v[u].float().cpu().numpy().astype(np.float64),
                q=inp.q[:, u].cpu().numpy(),
                W=inp.W[p].cpu().numpy(), b=inp.b[p].cpu().numpy())


def oracle_prefill(cfg, hu):
    _, M, _ = O.partition(cfg.L, cfg.n_sink, cfg.n_tail)
    P, S, u = O.prefill_unit(hu["k"][M], hu["v"][M], hu["W"], hu["b"])
    return P, S, u, O.kappa_max(hu["k"][M])


def oracle_decode(cfg, hu, pre, K, step, g, variant="sub"):
    P, S, u, _ = pre
    q = hu["q"][step, g]
    f = O.phi_features(q[None], hu["W"], hu["b"])[0]
    return O.decode_query(q, f, hu["k"], hu["v"], P, S, u, cfg.L, cfg.n_sink, cfg.n_tail,
                          cfg.n_gen(step), K, variant=variant)


def check_y(y, y_ref, what=""):
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    a = float(np.abs(y - y_ref).max())
    r = float(np.linalg.norm(y - y_ref) / max(np.linalg.norm(y_ref), 1e-300))
    assert a <= ABS_TOL and r <= REL_TOL, f"{what}: abs {a:.3e} (tol {ABS_TOL}) rel {r:.3e} (tol {REL_TOL})"
    return a, r


def check_prefill(cfg, gpu_pre, u, ref_pre):
    phi_k, S, uu, kappa = gpu_pre
    P, Sr, ur, kap = ref_pre
    ph = phi_k[u].float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(ph - P) <= 2.0 ** -8 * np.abs(P) + 1e-6), "phi_k rows"
    _, M, _ = O.partition(cfg.L, cfg.n_sink, cfg.n_tail)
    return ph


def check_summaries(cfg, gpu_pre, u, ref_pre, v_mid):
    phi_k, S, uu, kappa = gpu_pre
    P, Sr, ur, kap = ref_pre
    Sg = S[u].cpu().numpy().astype(np.float64)
    ug = uu[u].cpu().numpy().astype(np.float64)
    bound_S = 2.0 ** -8 * (np.abs(P).T @ np.abs(v_mid)) + 1e-4
    assert np.all(np.abs(Sg - Sr) <= bound_S), f"S: worst ratio {np.max(np.abs(Sg - Sr) / bound_S):.3f}"
    assert np.all(np.abs(ug - ur) <= 2.0 ** -8 * ur + 1e-4), "u"
    kg = float(kappa[u].item())
    assert kap <= kg <= kap * (1 + 2e-5) + 1e-30, f"kappa {kg} vs {kap}"


def hip_decode_one_call(inp, pre, K, step, flags=R.RMA_MERGE_SUB, ws=None, fused_phi=False,
                        want_idx=True):
    """The same step as hip_decode through rma_decode (Top-K and merge in one
    call)."""
    cfg = inp.cfg
    phi_k, S, u, kappa = pre
    q = inp.q[step].contiguous()
    f = None if fused_phi else R.rma_phi_features(q, inp.W, inp.b)
    sp = decode_span(cfg, step)
    extra = dict(Wk=inp.W, bk=inp.b) if phi_k is None else {}
    if fused_phi:
        extra.update(Wq=inp.W, bq=inp.b)
    out = R.rma_decode(q, f, inp.k, inp.v, sp, kappa, K, phi_k, S, u, flags=flags, m=cfg.m,
                       want_idx=want_idx, want_stats=True, ws=ws, phi_dtype=cfg.torch_phi_dtype(), **extra)
    if want_idx:
        y, idx, sel, stats = out
        return dict(idx=idx, sel=sel, y=y, stats=stats, f=f)
    y, stats = out
    return dict(y=y, stats=stats, f=f)


def check_scan_error(sel, s_ref, q, kf, d, what):
    """The selection's certificate assumes every fp32 score of the scan lies within
    eps = 2e-6 |q| kappa of the exact q.k (kappa >= the largest key norm); the
    kept scores are those scan scores times fp32(1/sqrt(d)), which adds at most
    two roundings (3e-7 relative)."""
    qn = float(np.linalg.norm(q.double().numpy()))
    kap = float(np.linalg.norm(kf, axis=1).max())
    raw = np.abs(s_ref) * math.sqrt(d)
    bound = (2e-6 * qn * kap + 3e-7 * raw) / math.sqrt(d)
    err = np.abs(sel.astype(np.float64) - s_ref)
    assert np.all(err <= bound), f"{what}: scan score error {float((err / bound).max()):.2f}x the eps bound"
