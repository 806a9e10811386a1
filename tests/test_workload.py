"""Synthetic workload generator: shapes, determinism and the planted structure."""
import torch

from kv_cache_reads_amd import workload as W


def test_config_table():
    c = W.CONFIGS
    assert (c["c0"].U, c["c0"].G, c["c0"].L_mid, c["c0"].K) == (1, 2, 988, (10,))
    assert (c["c1"].U, c["c1"].G, c["c1"].L_mid, c["c1"].K) == (8, 4, 32700, (328,))
    assert (c["c2"].U, c["c2"].G, c["c2"].L_mid) == (8, 3, 65468)
    assert c["c2"].K == (327, 655, 1310, 2621)
    assert (c["c3"].U, c["c3"].G, c["c3"].L_mid, c["c3"].K, c["c3"].steps) == (2048, 4, 16316, (163,), 8)
    assert (c["c4"].U, c["c4"].G, c["c4"].L_mid, c["c4"].K) == (896, 3, 131004, (1310,))
    assert c["c3"].T_cap == 16384 + 8 and c["c1"].T_cap == 32768


def test_generate_small_deterministic_and_planted():
    cfg = W.CONFIGS["c1"].with_(L=2048, batch=1, layers=2, h_q=8, h_kv=2)
    a = W.generate(cfg)
    b = W.generate(cfg)
    assert torch.equal(a.k.float(), b.k.float()) and torch.equal(a.q, b.q)
    assert a.k.shape == (cfg.U, cfg.T_cap, cfg.d) and a.k.dtype == torch.bfloat16
    assert a.q.shape == (1, cfg.U, cfg.G, cfg.d)
    assert a.W.shape == (cfg.P, cfg.m, cfg.d)
    nn = W.n_needles(cfg)
    for u in range(cfg.U):
        pos = a.needle_pos[u]
        assert len(pos) == nn == 2
        assert all(cfg.n_sink <= p < cfg.L - cfg.n_tail for p in pos)
        qh = a.q[0, u] / a.q[0, u].norm(dim=-1, keepdim=True)
        for j, p in enumerate(pos):
            # needle j aligns with query head j mod G: cosine close to 1
            cos = torch.dot(a.k[u, p].float(), qh[j % cfg.G]) / a.k[u, p].float().norm()
            assert cos > 0.95     # 4*qhat plus N(0, 0.1^2) noise per component
    # heads_half: first half of the query heads diffuse, second half peaked
    assert W.query_scale(cfg, 0) == 0.3 and W.query_scale(cfg, 1) == 2.0


def test_c0_planted_exact_ties():
    inp = W.generate(W.CONFIGS["c0"])
    pos = inp.needle_pos[0]
    assert len(pos) == 3
    k = inp.k[0]
    assert torch.equal(k[pos[0]], k[pos[1]]) and torch.equal(k[pos[1]], k[pos[2]])
    assert inp.k.dtype == torch.float32
