"""The measurement script's command-line contract, checked without a GPU: more
than one GPU is refused with a message and exit status 2 before anything
touches the device."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 1" in r.stderr
    assert r.stdout == ""


def test_a_multi_rank_launch_is_refused():
    r = _run(["--gpus", "1"], {"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_prefill_pair_counts_match_the_oracle_mask():
    """bench.py's per-row closed form of the allowed pairs (the FLOP count of the
    prefill rows) against the oracle's mask, with and without a dilation."""
    import numpy as np

    import bench
    from oracle import prefill_allowed
    for N, wl, wr, causal, s, g in ((300, 20, 0, True, 3, ()), (257, 31, 17, False, 4, ()),
                                    (100, -1, 0, True, 7, ()), (90, 10, -1, False, 2, ()),
                                    (400, 37, 0, True, 1, ()), (500, 16, 16, False, 1, (0, 77, 499))):
        m = prefill_allowed(np.arange(N), np.arange(N), wl, wr, causal, g, dilation=s)
        assert bench.prefill_pairs(N, wl, wr, causal, g, s) == int(m.sum()), (N, wl, wr, causal, s, g)
