"""The work-split specification covers every (piece, block) unit exactly once
and balances cost across chunks (CPU only; brute-force enumeration)."""
import numpy as np
import pytest

from oracle import schedule as S


def _check(lens, num_rows, next_n, lens_2d, indices, bkv, W):
    table = S.piece_table(lens, num_rows, next_n, lens_2d, indices, bkv)
    sched = S.schedule(lens, num_rows, next_n, lens_2d, indices, bkv, W)
    assert sched.shape == (W + 1, 2)
    assert tuple(sched[W]) == (num_rows, 0)
    # starts are non-decreasing in (row, block) order
    for c in range(W):
        assert tuple(sched[c]) <= tuple(sched[c + 1])
    every = [(s, b) for s, g, nblk, cost in table for b in range(nblk)]
    seen = []
    total = sum(t[3] for t in table)
    unit_cost = {s: S.COST_BASE + g for s, g, nblk, cost in table}
    for c in range(W):
        units = S.units_of_chunk(sched, table, c)
        seen += units
        load = sum(unit_cost[s] for s, b in units)
        assert load <= total / W + S.COST_BASE + S.G_MAX + 1e-9
    assert seen == every
    # pieces: groups respected, at most G_MAX rows
    vis = S.visible_lengths(lens, num_rows, next_n, lens_2d)
    for s, g, nblk, cost in table:
        assert 1 <= g <= S.G_MAX
        assert nblk == -(-int(vis[s:s + g].max()) // max(bkv, 64))
        if indices is not None:
            assert len(set(np.asarray(indices)[s:s + g].tolist())) == 1
        else:
            assert s // next_n == (s + g - 1) // next_n
    return sched


def test_hand_example():
    # two requests: 3 rows of 130 tokens, 1 row of 64 tokens; block_kv 64
    lens = np.array([128, 129, 130, 64])
    idx = np.array([7, 7, 7, 9])
    table = S.piece_table(lens, 4, 1, False, idx, 64)
    assert table == [(0, 3, 3, 3 * (S.COST_BASE + 3)), (3, 1, 1, S.COST_BASE + 1)]
    sched = _check(lens, 4, 1, False, idx, 64, 2)
    # (COST_BASE 3) total = 18 + 4 = 22; chunk 1 starts at offset 11 -> piece 0, block 11 // 6 = 1
    assert sched.tolist() == [[0, 0], [0, 1], [4, 0]]


@pytest.mark.parametrize("seed", range(6))
def test_random_varlen(seed):
    rng = np.random.default_rng(seed)
    R = int(rng.integers(1, 30))
    runs = rng.integers(1, 12, R)            # some runs exceed G_MAX
    ctx = rng.integers(0, 5000, R)
    lens = np.concatenate([np.maximum(c - n + np.arange(n) + 1, 0) for c, n in zip(ctx, runs)])
    ids = np.repeat(rng.permutation(R) % max(1, R // 2), runs)   # repeated ids in separate runs
    for W in (1, 7, 64, 513):
        _check(lens, len(lens), 1, False, ids, int(rng.choice([32, 64])), W)


@pytest.mark.parametrize("next_n,lens_2d", [(1, False), (3, False), (3, True), (10, False)])
def test_uniform(next_n, lens_2d):
    rng = np.random.default_rng(next_n)
    B = 9
    ctx = rng.integers(0, 3000, B)
    if lens_2d:
        lens = (ctx[:, None] - next_n + np.arange(next_n) + 1).clip(0, None)
    else:
        lens = ctx
    for W in (1, 5, 256):
        _check(lens, B * next_n, next_n, lens_2d, None, 64, W)


def test_all_empty():
    sched = _check(np.zeros(5, dtype=np.int64), 5, 1, False, np.arange(5), 64, 4)
    assert sched.tolist() == [[5, 0]] * 5
