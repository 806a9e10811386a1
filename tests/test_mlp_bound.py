"""CPU checks of the MLP feature tolerance (tests/mlp_bound.py): rows computed
with real bfloat16 rounding at every operand (the oracle's rounding mirror)
fall inside it, and rows with a plausible mistake (a dropped output bias, a
dropped block bias) fall outside."""
import numpy as np
import pytest
import torch

import oracle as O
from mlp_bound import check_rows
from kv_cache_reads_amd import workload as W


def _case(d, m, seed=3):
    cfg = W.CONFIGS["c1"].with_(d=d, h_kv=1, h_q=1, layers=1, seed=seed)
    params = W.generate_phi_mlp(cfg, "k", m=m)
    p = {k: v[0].double().numpy() if v.dim() > 1 else float(v[0]) for k, v in params.items()}
    g = torch.Generator().manual_seed(seed)
    x = (1.5 * torch.randn(120, d, generator=g)).bfloat16().double().numpy()
    return x, p


@pytest.mark.parametrize("d,m", [(64, 64), (128, 128)])
@pytest.mark.parametrize("bf16_rows", [True, False])
def test_real_rounding_is_inside_the_tolerance(d, m, bf16_rows):
    x, p = _case(d, m)
    rows = O.phi_mlp(x, p, bf16_operands=True)
    if bf16_rows:
        rows = O.round_bf16(rows)
    ratio, _ = check_rows(rows, x, p, bf16_rows)
    assert ratio <= 0.75


@pytest.mark.parametrize("drop", ["b_o", "b_2"])
def test_dropped_bias_is_outside_the_tolerance(drop):
    x, p = _case(64, 64)
    q = dict(p)
    q[drop] = np.zeros_like(p[drop])
    with pytest.raises(AssertionError):
        check_rows(O.phi_mlp(x, q, bf16_operands=True), x, p, False)
