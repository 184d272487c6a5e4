"""The library's Admit scheduler (host code) against the oracle on random admit / advance
sequences: the same verify iterations, the same waits, the same ring contents and due lists."""
import numpy as np
import pytest

from lossless_kv_cache_vc_amd import vc
from oracle.scheduler import AdmitScheduler


@pytest.mark.parametrize("seed", range(6))
def test_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    W = int(rng.integers(8, 80))
    x = int(rng.integers(1, W + 8))
    t_iter = float(rng.uniform(0.5, 2.0))
    bw = float(rng.uniform(0.5, 4.0))
    budget = float(rng.uniform(2.0, 40.0))
    lib, ora = vc.Scheduler(W, x, t_iter, bw, budget), AdmitScheduler(W, x, t_iter, bw, budget)
    waiting = list(range(12))
    for step in range(400):
        if waiting and rng.random() < 0.6:
            r = waiting.pop(int(rng.integers(0, len(waiting))))
            kv = float(rng.uniform(0.0, 4.0 * bw * t_iter))
            got, want = lib.admit(r, kv), ora.admit(r, kv)
            assert got == want, (step, r, kv, got, want)
            if got is None:
                waiting.append(r)
        else:
            assert lib.due() == ora.due()
            _, verified = ora.due()
            lib.advance()
            ora.advance()
            waiting += verified
        assert lib.now == ora.now
        for i in range(W):
            assert lib.ring(i) == (ora.T[i], ora.B[i])


def test_rejects_bad_use():
    with pytest.raises(vc.VCError):
        vc.Scheduler(1, 4, 1.0, 1.0, 1.0)
    with pytest.raises(vc.VCError):
        vc.Scheduler(16, 4, 0.0, 1.0, 1.0)
    s = vc.Scheduler(16, 4, 1.0, 1.0, 10.0)
    assert s.admit(3, 1.0) == 4
    with pytest.raises(vc.VCError):
        s.admit(3, 1.0)          # already reserved
    with pytest.raises(vc.VCError):
        s.admit(4, -1.0)
    with pytest.raises(vc.VCError):
        s.ring(16)
