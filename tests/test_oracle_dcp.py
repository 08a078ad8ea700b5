"""Pins of the oracle's exact top-k merge over decode-context-parallel shards (CPU only).

* the hand-worked fixture tests/golden/dcp_merge_hand_worked.json
* token placement against a simulation that deals runs of tokens to ranks in
  turn, plus its closed-form special cases (interleave 1 is round robin, one
  rank is the identity)
* the exactness claim of the merge: packing every rank's local top-k and
  merging gives the top-k of the whole row, as a numpy lexsort over the whole
  row computes it (ties, NaN, -inf and signed zeros included)
* the merge against an independent numpy lexsort formulation on arbitrary
  gathered arrays with padding and out-of-range ids
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import brute

GOLD = os.path.join(os.path.dirname(__file__), "golden", "dcp_merge_hand_worked.json")


def _num(x):
    if isinstance(x, str):
        return {"-inf": -math.inf, "inf": math.inf, "nan": math.nan}[x]
    return float(x)


def _shard(scores: np.ndarray, lens, world: int, interleave: int, ks=None, pad: int = 0, fill=1e30):
    """Per-rank local logits [rows][ld] (garbage outside each row's span) and span ends."""
    rows = scores.shape[0]
    held = [brute.dcp_tokens(int(L), world, interleave) for L in lens]
    n_loc = max(1, max(len(h[r]) for h in held for r in range(world)))
    ks = np.zeros(rows, np.int32) if ks is None else np.asarray(ks, np.int32)
    ld = int(ks.max()) + n_loc + pad
    out = []
    for r in range(world):
        lg = np.full((rows, ld), fill, np.float32)
        ke = np.zeros(rows, np.int32)
        for i in range(rows):
            toks = held[i][r]
            lg[i, ks[i]: ks[i] + len(toks)] = scores[i, toks]
            ke[i] = ks[i] + len(toks)
        out.append((lg, ke))
    return out, ks


def _bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def test_golden_hand_worked_merge():
    with open(GOLD) as f:
        g = json.load(f)
    W, I = g["world"], g["interleave"]
    scores = np.array([[_num(v) for v in r] for r in g["rows"]], np.float32)
    assert brute.dcp_tokens(scores.shape[1], W, I) == g["placement"]["tokens"]
    shards, ks = _shard(scores, [scores.shape[1]] * 2, W, I)
    for case in g["cases"]:
        k = case["k"]
        packed = []
        for r, (lg, ke) in enumerate(shards):
            loc = oracle.topk(lg.astype(np.float64), ke, k, ks=ks)
            assert loc.tolist() == case["local"][r], (k, r)
            packed.append(oracle.dcp_pack(lg, loc, r, W, I, ks=ks))
        if "packed" in case:
            want = np.array([[[[_num(v) for v in p] for p in row] for row in rk] for rk in case["packed"]], np.float32)
            assert np.array_equal(_bits(np.stack(packed)), _bits(want)), k
        gathered = np.stack(packed)
        assert oracle.dcp_merge(gathered, k).tolist() == case["merged"], k
        assert brute.dcp_merge(gathered, k).tolist() == case["merged"], k


@pytest.mark.parametrize("world,interleave", [(1, 1), (1, 64), (2, 1), (3, 2), (4, 64), (8, 1), (8, 16), (5, 7)])
def test_placement_deals_runs_in_turn(world, interleave):
    T = 1000
    held = brute.dcp_tokens(T, world, interleave)
    for r in range(world):
        for p, t in enumerate(held[r]):
            assert oracle.dcp_global_id(p, r, world, interleave) == t
            if interleave == 1:
                assert t == p * world + r
            if world == 1:
                assert t == p
    assert sorted(sum(held, [])) == list(range(T))


def _rows(rng, rows, T, kind):
    s = rng.standard_normal((rows, T)).astype(np.float32)
    if kind == "ties":
        s = np.round(s * 2) / 2
    elif kind == "special":
        s = np.round(s)
        m = rng.random((rows, T))
        s[m < 0.1] = np.nan
        s[(m >= 0.1) & (m < 0.2)] = -np.inf
        s[(m >= 0.2) & (m < 0.3)] = -0.0
    return s


@pytest.mark.parametrize("kind", ["normal", "ties", "special"])
@pytest.mark.parametrize("world,interleave", [(1, 1), (2, 1), (2, 64), (3, 5), (8, 1), (8, 64)])
def test_merge_of_local_topk_is_global_topk(kind, world, interleave):
    rng = np.random.default_rng(world * 131 + interleave + len(kind))
    rows, T = 6, 700
    s = _rows(rng, rows, T, kind)
    lens = rng.integers(0, T + 1, rows)
    lens[0], lens[1] = T, 0
    ks = rng.integers(0, 9, rows).astype(np.int32)
    shards, ks = _shard(s, lens, world, interleave, ks=ks, pad=3)
    for k in (1, 7, 64, 300):
        gathered = np.stack([
            oracle.dcp_pack(lg, oracle.topk(lg.astype(np.float64), ke, k, ks=ks), r, world, interleave, ks=ks)
            for r, (lg, ke) in enumerate(shards)])
        full = brute.topk(s.astype(np.float64), lens.astype(np.int32), k)
        got = oracle.dcp_merge(gathered, k)
        assert np.array_equal(got, full), (k, kind)
        assert np.array_equal(brute.dcp_merge(gathered, k), full), (k, kind)


def test_merge_matches_lexsort_on_arbitrary_candidates():
    rng = np.random.default_rng(11)
    world, rows, k = 4, 9, 50
    g = np.empty((world, rows, k, 2), np.float32)
    g[..., 0] = np.round(rng.standard_normal((world, rows, k)) * 3) / 3
    for r in range(rows):
        ids = rng.choice(1 << 20, world * k, replace=False).astype(np.float32)
        g[:, r, :, 1] = ids.reshape(world, k)
    m = rng.random((world, rows, k))
    g[..., 1][m < 0.15] = -1.0                  # padding
    g[..., 1][(m >= 0.15) & (m < 0.2)] = 2.0 ** 24   # not an exact id: ignored
    g[..., 1][(m >= 0.2) & (m < 0.22)] = np.nan
    g[..., 0][(m >= 0.3) & (m < 0.35)] = np.nan
    g[..., 0][(m >= 0.35) & (m < 0.4)] = -np.inf
    g[1, 3, :, 1] = -1.0                        # a rank with no candidates for row 3
    g[:, 5, :, 1] = -1.0                        # a row with no candidates at all
    for kk in (k,):
        a = oracle.dcp_merge(g, kk)
        assert np.array_equal(a, brute.dcp_merge(g, kk))
    assert (oracle.dcp_merge(g, k)[5] == -1).all()


def test_pack_reads_row_start_and_pads():
    rng = np.random.default_rng(5)
    rows, ld, k = 4, 40, 6
    lg = rng.standard_normal((rows, ld)).astype(np.float32)
    ks = np.array([0, 3, 39, 40], np.int32)
    tk = np.array([[0, 5, 39, -1, 40, 2],
                   [0, 36, 37, -1, -1, -1],
                   [0, 1, -1, -1, -1, -1],
                   [0, -1, -1, -1, -1, -1]], np.int32)
    p = oracle.dcp_pack(lg, tk, 1, 3, 2, ks=ks)
    for r in range(rows):
        for j in range(k):
            idx = int(tk[r, j])
            if 0 <= idx and ks[r] + idx < ld:
                assert p[r, j, 0] == lg[r, ks[r] + idx]
                assert p[r, j, 1] == (idx // 2) * 6 + 2 + idx % 2
            else:
                assert p[r, j, 0] == -np.inf and p[r, j, 1] == -1.0


def test_golden_pack_out_of_range_row_starts_are_clamped():
    """Row starts below 0 or past the row: the top-k's bound rule (start clamped
    to [0, ld]), hand-worked in tests/golden/topk_bounds_hand_worked.json."""
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "topk_bounds_hand_worked.json")))
    p = g["pack"]
    row = np.array(g["row"], dtype=np.float32)
    for c in p["cases"]:
        tk = np.array([c["topk"]], np.int32)
        got = oracle.dcp_pack(row[None, :], tk, p["rank"], p["world"], p["interleave"],
                              ks=np.array([c["ks"]], np.int32))
        want = np.array([[float(x) for x in pair] for pair in c["expected"]], np.float32)
        assert np.array_equal(got[0], want), c["derivation"]
