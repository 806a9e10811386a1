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
