"""Pins of the placement oracle (no GPU): hand-computed cycles and splits, a
bin-packing instance where Best-Fit fails and one discrepancy succeeds,
completeness of LDS against brute-force enumeration, and the admission
invariants (whole stream or nothing, no migration)."""
import random

import pytest

from oracle import sched as S


def _cluster(n_gpus, positions, slo, a=1.0, b=0.5, B=4, St=2):
    return S.Cluster(n_gpus, positions, slo, S.Model(B, St, a, b))


def test_cycle_hand_values():
    m = S.Model(4, 2, 1.0, 0.5)
    # block 0: 2 + 1 tasks -> 1 + 1.5; block 1: 1 task -> 1.5
    assert S.cycle_ms(m, [{0: 2, 1: 1}, {0: 1}]) == 4.0
    assert S.cycle_ms(m, []) == 0.0
    # batching: one batch of 4 is cheaper than two batches of 2 on separate blocks
    assert S.cycle_ms(m, [{0: 2}, {0: 2}]) == 3.0 and S.cycle_ms(m, [{0: 2}, {1: 2}]) == 4.0


def test_split_stream_hand_values():
    m = S.Model(4, 2, 1.0, 1.0)          # f(n) = 1 + n; 8 stages, a stage alone costs 2
    # block-major order (b0 s0, b0 s1, b1 s0, ...).  R = 1: 4 blocks x f(2) = 12;
    # R = 2: blocks {0, 1} and {2, 3}, 2 x f(2) = 6; R = 3: sizes 2, 3, 3 ->
    # {b0: 2} = 3, {b1: 2, b2: 1} = 5, {b2: 1, b3: 2} = 5
    assert len(S.split_stream(m, 12.0)) == 1
    assert S.split_stream(m, 11.9) == [{0: 2, 1: 2}, {2: 2, 3: 2}]
    assert S.split_stream(m, 5.9) == [{0: 2}, {1: 2, 2: 1}, {2: 1, 3: 2}]
    assert S.split_stream(m, 1.9) is None
    assert S.equal_split_streams(24, m, 5.9) == 8


def test_best_fit_fails_one_discrepancy_succeeds():
    # two GPUs of capacity 10 (f(n) = n), items 4, 4, 3, 3, 6 in order:
    # Best-Fit packs 4+4 | 3+3 and has no room for 6; {4, 6} | {4, 3, 3} exists
    cl = S.Cluster(2, 10, 10.0, S.Model(5, 1, 0.0, 1.0))
    ranks = [{0: 4}, {1: 4}, {2: 3}, {3: 3}, {4: 6}]
    assert S.lds_place(cl, ranks, 0) is None
    assert S.lds_place(cl, ranks, 1) == [0, 1, 0, 0, 1]
    assert S.exists_placement(cl, ranks)


def _random_cluster(rng):
    cl = _cluster(3, rng.choice([1, 2, 3]), rng.choice([6.0, 8.0, 10.0]), a=rng.choice([0.0, 1.0]), b=1.0,
                  B=3, St=1)
    # pre-load some ranks
    for g in range(cl.n_gpus):
        for k in range(rng.randrange(0, 2)):
            rk = {rng.randrange(3): rng.randrange(1, 3)}
            if len(cl.hosted[g]) < cl.positions and S.cycle_ms(cl.model, [e[2] for e in cl.hosted[g]] + [rk]) <= cl.slo_ms:
                cl.hosted[g].append((100 + g, k, rk))
    ranks = [{rng.randrange(3): rng.randrange(1, 4)} for _ in range(rng.randrange(1, 5))]
    return cl, ranks


def test_lds_is_complete_at_full_discrepancy_against_brute_force():
    rng = random.Random(7)
    found = missed = 0
    for _ in range(300):
        cl, ranks = _random_cluster(rng)
        got = S.lds_place(cl, ranks, len(ranks))
        exists = S.exists_placement(cl, ranks)
        assert (got is not None) == exists
        if got is not None:
            found += 1
            for r, g in enumerate(got):
                cl.hosted[g].append((999, r, ranks[r]))
            assert S.feasible(cl)
        else:
            missed += 1
    assert found > 50 and missed > 20      # both outcomes exercised


def test_admission_whole_stream_and_no_migration():
    m = S.Model(4, 2, 1.0, 1.0)
    cl = S.Cluster(3, 2, 5.9, m)            # a stream = 3 ranks (see the split test)
    placed = {}
    sid = 0
    while True:
        got = S.admit(cl, sid, 2)
        if got is None:
            break
        placed[sid] = got
        assert S.feasible(cl)
        # earlier streams stay where they were
        for s2, pl in placed.items():
            assert sorted((r, g) for g in range(cl.n_gpus) for (s, r, _) in cl.hosted[g] if s == s2) == \
                sorted(enumerate(pl))
        sid += 1
    assert 1 <= len(placed) <= 2
    before = [list(h) for h in cl.hosted]
    assert S.admit(cl, 77, 3) is None and cl.hosted == before      # a rejection changes nothing
    assert S.release(cl, 0) == 3
    assert S.admit(cl, 78, 2) is not None                           # freed capacity is reused


def test_joint_placement_beats_equal_split_when_batching_pays():
    # f(n) = 2 + n / 4: a block's two steps cost 2.5 as one batch.  SLO 6: a
    # stream splits into 2 ranks of 2 blocks (5 each), so an equal split
    # serves 2 streams on 4 GPUs; a GPU holding the same 2 blocks of two
    # streams batches them (2 x (2 + 1) = 6) and the pool holds 4 streams.
    m = S.Model(4, 2, 2.0, 0.25)
    slo = 6.0
    g = S.split_stream(m, slo)
    assert g == [{0: 2, 1: 2}, {2: 2, 3: 2}] and all(S.cycle_ms(m, [x]) == 5.0 for x in g)
    cl = S.Cluster(4, 8, slo, m)
    n = 0
    while S.admit(cl, n, 2) is not None:
        n += 1
    assert S.equal_split_streams(4, m, slo) == 2 and n == 4


def test_fixed_rank_count_split():
    m = S.Model(4, 2, 1.0, 1.0)
    assert S.split_stream(m, 7.0, 4) == [{0: 2}, {1: 2}, {2: 2}, {3: 2}]
    assert S.split_stream(m, 5.9, 2) is None           # two blocks x f(2) = 6 > 5.9
    assert S.split_stream(m, 7.0, 9) is None           # more ranks than stages
    # finer ranks fill capacity the fewest leave: SLO 9 on 3 GPUs.  Fewest
    # ranks: 2 of 6 -> one stream per pair of GPUs (a GPU cannot take two).
    # 4 ranks of one block (3 each): a GPU holds blocks {b, b'} of one stream
    # (6) or one block of two streams (1 + 4 = 5) plus another of one (8).
    cl = S.Cluster(3, 16, 9.0, m, n_ranks=4)
    n = 0
    while S.admit(cl, n, 1) is not None:
        n += 1
    assert S.equal_split_streams(3, m, 9.0) == 1 and n == 2
