"""The bench's timed region enqueues exactly the requested number of steps, and
the steps keep rotating over the input copies: whole rounds (one graph holding
one step per copy, in turn from the copy the warm-up stopped at), then single
steps that continue the rotation.  Host logic only; the graphs are stand-ins
that record which copies their replays ran."""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


class _Rec:
    def __init__(self, log, copies):
        self.log, self.copies = log, copies

    def replay(self):
        self.log.extend(self.copies)


@pytest.mark.parametrize("n_copies,steps,start", [(9, 400, 2), (9, 9, 0), (9, 5, 7), (1, 13, 0),
                                                  (4, 0, 3), (12, 100, 8)])
def test_replay_steps_counts_and_rotation(n_copies, steps, start):
    log = []
    rnd = _Rec(log, [(start + j) % n_copies for j in range(n_copies)])
    single = [_Rec(log, [i]) for i in range(n_copies)]
    bench.replay_steps(rnd, single, n_copies, steps, start)
    assert len(log) == steps
    assert log == [(start + i) % n_copies for i in range(steps)]


def test_more_than_one_gpu_exits_with_a_message():
    import json
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "--gpus must be 1" in msg["error"]


def test_scan_grid_mirror_matches_the_library_plan():
    """bench.scan_blocks (the grid of the same-shape streaming read) follows the
    library's Top-K plan: the chunk count that sizes rma_workspace_bytes."""
    import ctypes

    from kv_cache_reads_amd import rma as R
    from kv_cache_reads_amd import workload as W
    if not os.path.exists(R.LIB_PATH):
        pytest.skip("librma.so not built")
    for name in ("c0", "c1", "c2", "c3", "c4"):
        cfg = W.CONFIGS[name]
        kv = R._KV(0x10000, 0x20000, R.RMA_BF16, cfg.U, cfg.T_cap, cfg.T_cap * cfg.d, cfg.d, 0)
        sp = R._Span(cfg.L, cfg.n_sink, cfg.n_tail, 0)
        blocks = bench.scan_blocks(cfg)
        assert blocks % cfg.U == 0
        nc = blocks // cfg.U
        ws = R.lib().rma_workspace_bytes(R.RMA_OP_DECODE_TOPK, ctypes.byref(kv), ctypes.byref(sp), cfg.G, cfg.K[0], 0)
        # the workspace of nc chunks: reports (r_cap slots each), the chunk table, the head parameters
        import math
        Lm, K, tile = cfg.L_mid, cfg.K[0], 64 if cfg.d == 64 else 32
        ch = -(-(-(-Lm // nc)) // tile) * tile
        assert -(-Lm // ch) == nc
        mu = K / nc
        rmin = max(16, (math.ceil(mu + 4 * math.sqrt(mu) + 4) + 7) // 8 * 8)
        r_cap = ch if K >= Lm else min(ch, 2 * min(ch, rmin) + 32)
        up = lambda x: -(-x // 256) * 256
        want = up(cfg.U * cfg.G * nc * r_cap * 8) + up(cfg.U * cfg.G * nc * 8) + up(cfg.U * cfg.G * 16)
        assert ws == want, (name, nc, ws, want)
