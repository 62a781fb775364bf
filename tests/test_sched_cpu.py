"""The native placement (ps_sched_*) against the oracle, on the CPU: the same
virtual-rank split, the same GPU for every rank on random admission and
release sequences, and the error paths."""
import os
import random

import pytest

from autoregressive_denoising_dit_amd import _lib
from oracle import sched as S

needs_lib = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libps.so not built")


def _pair(n_gpus, positions, B, St, slo, a, b, disc, n_ranks=0):
    from autoregressive_denoising_dit_amd.sched import Scheduler
    nat = Scheduler(n_gpus, positions, B, St, slo, a, b, disc, n_ranks)
    ora = S.Cluster(n_gpus, positions, slo, S.Model(B, St, a, b), n_ranks=n_ranks)
    return nat, ora


@needs_lib
@pytest.mark.parametrize("seed", range(12))
def test_admission_sequences_match_oracle(seed):
    rng = random.Random(seed)
    B, St = rng.choice([(2, 2), (3, 2), (4, 4), (30, 4)])
    a, b = rng.choice([(0.0, 1.0), (0.5, 0.25), (1.0, 0.3), (0.074, 0.227)])
    slo = rng.choice([2.0, 3.0, 4.5, 7.0, 12.0])
    n_gpus, positions, disc = rng.choice([2, 3, 5, 8]), rng.choice([1, 2, 4, 8]), rng.choice([0, 1, 2])
    n_ranks = rng.choice([0, 0, 1, 3, B])
    nat, ora = _pair(n_gpus, positions, B, St, slo, a, b, disc, n_ranks)
    ranks = S.split_stream(ora.model, slo, n_ranks)
    assert nat.split() == (0 if ranks is None else len(ranks))
    live = []
    for step in range(40):
        if live and rng.random() < 0.3:
            sid = live.pop(rng.randrange(len(live)))
            assert nat.release(sid) == S.release(ora, sid)
        else:
            sid = 1000 * seed + step
            got, ref = nat.admit(sid), S.admit(ora, sid, disc)
            assert got == ref, (step, got, ref)
            if got is not None:
                live.append(sid)
        for g in range(n_gpus):
            n, c = nat.gpu(g)
            assert n == len(ora.hosted[g])
            assert c == S.cycle_ms(ora.model, [e[2] for e in ora.hosted[g]])
        assert S.feasible(ora)


@needs_lib
def test_best_fit_fails_one_discrepancy_admits():
    # a = 0, b = 1: cycles are task counts.  B = 8, S = 1, SLO 5 gives two
    # ranks of 4 stages; GPUs preloaded so that Best-Fit's first choice for the
    # first rank leaves no room for the second.
    for disc, expect in ((0, None), (1, [1, 0])):
        nat, ora = _pair(2, 4, 8, 1, 5.0, 0.0, 1.0, disc)
        assert nat.split() == 2
        # preload: stream 9 on both GPUs (ranks of 4 tasks each) -> admit once
        first = nat.admit(9)
        assert first == S.admit(ora, 9, disc)
        got = nat.admit(10)
        assert got == S.admit(ora, 10, disc)


@needs_lib
def test_errors():
    from autoregressive_denoising_dit_amd.sched import Scheduler
    from autoregressive_denoising_dit_amd._lib import PsError
    with pytest.raises(PsError):
        Scheduler(0, 1, 1, 1, 1.0, 0.0, 1.0)
    with pytest.raises(PsError):
        Scheduler(1, 1, 1, 1, 1.0, 0.0, 0.0)
    s = Scheduler(2, 2, 4, 2, 10.0, 1.0, 1.0)
    assert s.admit(5) is not None
    with pytest.raises(PsError):
        s.admit(5)                       # already admitted
    assert s.release(6) == 0             # unknown id
    with pytest.raises(PsError):
        s.gpu(2)
    tiny = Scheduler(2, 2, 4, 2, 1.0, 1.0, 1.0)   # a single stage costs 2 > SLO
    assert tiny.split() == 0 and tiny.admit(1) is None


@needs_lib
def test_stage_count_limit():
    from autoregressive_denoising_dit_amd.sched import Scheduler
    from autoregressive_denoising_dit_amd._lib import PsError
    Scheduler(2, 2, 64, 64, 10.0, 0.0, 1.0)          # 4096 stages: accepted
    with pytest.raises(PsError):
        Scheduler(2, 2, 64, 65, 10.0, 0.0, 1.0)      # 4160 stages: refused
