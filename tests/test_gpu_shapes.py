"""GPU parity over the supported shape and dtype combinations that the five
workloads do not reach: every (d, m) pair, group sizes 1..8, bf16 or fp32 keys
with bf16 or fp32 stored features, two parameter sets, generated tokens.
Same bar as the workloads: bit-exact Top-K, outputs within 2e-3 abs / 1e-2 rel,
the full-attention reference within the same bar.  Inputs are the seeded
synthetic generator at small sizes with ragged mid-regions.
"""
import numpy as np
import pytest
import torch

import oracle as O
from parity_util import (R, W, check_prefill, check_summaries, check_y, decode_span, hip_decode,
                         hip_prefill, host_unit, log, oracle_decode, oracle_prefill)

pytestmark = pytest.mark.gpu
DEV = "cuda"

BASE = W.CONFIGS["c1"]
# (d, m, G, kv dtype, phi dtype, L, K, decode steps)
SHAPES = [
    (64, 64, 4, "bf16", "bf16", 2600 + 11, 31, 1),
    (128, 64, 3, "bf16", "bf16", 2600 + 5, 27, 2),
    (64, 128, 8, "bf16", "bf16", 2048 + 77, 25, 1),
    (128, 128, 5, "bf16", "bf16", 3000 + 1, 40, 2),
    (64, 128, 1, "bf16", "bf16", 1500 + 3, 15, 1),
    (128, 128, 2, "bf16", "f32", 2600 + 9, 30, 1),
    (64, 64, 6, "f32", "bf16", 1800 + 13, 20, 2),
    (128, 128, 7, "f32", "f32", 1700 + 7, 18, 1),
]


def _cfg(d, m, G, kvd, phid, L, K, steps):
    return BASE.with_(name=f"d{d}m{m}G{G}{kvd}{phid}", layers=1, h_kv=2, h_q=2 * G, d=d, m=m, L=L,
                      K=(K,), steps=steps, kv_dtype=kvd, phi_dtype=phid, seed=7)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"d{s[0]}m{s[1]}G{s[2]}{s[3]}{s[4]}")
def test_shape_matches_oracle(shape):
    cfg = _cfg(*shape)
    torch.manual_seed(0)
    inp = W.generate(cfg, device=DEV)
    pre = hip_prefill(inp)
    K = cfg.K[0]
    outs = {}
    for s in range(cfg.steps):
        for fused in (False, True):
            outs[(s, fused)] = {k: (v.cpu() if v is not None else None)
                                for k, v in hip_decode(inp, pre, K, s, fused_phi=fused).items()}
        q = inp.q[s].contiguous()
        outs[(s, "full")] = R.rma_decode_full(q, inp.k, inp.v, decode_span(cfg, s)).cpu()
    torch.cuda.synchronize()
    worst = 0.0
    for u in range(cfg.U):
        hu = host_unit(inp, u)
        ref_pre = oracle_prefill(cfg, hu)
        check_prefill(cfg, pre, u, ref_pre)
        _, M, _ = O.partition(cfg.L, cfg.n_sink, cfg.n_tail)
        check_summaries(cfg, pre, u, ref_pre, hu["v"][M])
        for s in range(cfg.steps):
            for g in range(cfg.G):
                y_ref, idx_ref, _ = oracle_decode(cfg, hu, ref_pre, K, s, g)
                for fused in (False, True):
                    out = outs[(s, fused)]
                    idx = out["idx"][u, g].numpy().astype(np.int64)
                    assert np.array_equal(idx, idx_ref), f"{cfg.name} u{u} g{g} s{s}: top-K differs"
                    a, _ = check_y(out["y"][u, g].numpy(), y_ref, f"{cfg.name} u{u} g{g} s{s} fused={fused}")
                    worst = max(worst, a)
                yf_ref = O.full_attention(hu["q"][s, g], hu["k"], hu["v"], cfg.L + cfg.n_gen(s))
                check_y(outs[(s, "full")][u, g].numpy(), yf_ref, f"{cfg.name} full u{u} g{g} s{s}")
    log(f"{cfg.name}: worst |y - oracle| {worst:.2e}")
