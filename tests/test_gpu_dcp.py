"""Exact top-k over context-parallel shards on the GPU: the pack and merge calls.

* On shared input (the same fp32 pairs on both sides) the GPU merge equals the
  oracle bit for bit, for every register and sort shape of the kernel, with
  ties, NaN, -inf, padding and out-of-range ids.
* The pack equals the oracle bit for bit (scores and float ids).
* The property the merge exists for: per-rank top_k_per_row, pack, gather and
  merge give exactly top_k_per_row over the unsharded rows, at the 120K-context
  decode size split over 8 ranks included.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import brute
import paged_mqa_logits_amd as pml
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _gathered(rng, world, rows, k, kind="mixed"):
    g = np.empty((world, rows, k, 2), np.float32)
    if kind == "mixed":
        g[..., 0] = np.round(rng.standard_normal((world, rows, k)) * 4) / 4
        m = rng.random((world, rows, k))
        g[..., 0][m < 0.03] = np.nan
        g[..., 0][(m >= 0.03) & (m < 0.06)] = -np.inf
        g[..., 0][(m >= 0.06) & (m < 0.09)] = -0.0
    elif kind == "equal":
        g[..., 0] = 1.5
    elif kind == "neginf":
        g[..., 0] = -np.inf
    elif kind == "nan":
        g[..., 0] = np.nan
    else:
        g[..., 0] = rng.standard_normal((world, rows, k))
    for r in range(rows):
        ids = (rng.choice((1 << 24) - 1, world * k, replace=False) + 1).astype(np.float32)  # 0 is set below
        g[:, r, :, 1] = ids.reshape(world, k)
    m = rng.random((world, rows, k))
    g[..., 1][m < 0.05] = -1.0
    if kind == "mixed":
        g[..., 1][(m >= 0.05) & (m < 0.07)] = 2.0 ** 24
        g[..., 1][(m >= 0.07) & (m < 0.08)] = np.nan
        g[..., 1][(m >= 0.08) & (m < 0.09)] = -0.0     # id 0 (a candidate)
    return g


def _merge_gpu(g: np.ndarray, k: int) -> np.ndarray:
    gt = torch.from_numpy(g).to(G.dev())
    out = torch.full((g.shape[1], k + 3), 777, dtype=torch.int32, device=G.dev())
    pml.stable_topk_from_gathered_candidates(gt, k, out=out[:, :k])
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert (o[:, k:] == 777).all(), "wrote past k"
    return o[:, :k]


# (world, k): every candidates-per-thread count (2..32) and sort width (1..4 per thread)
SHAPES = [(1, 64), (4, 512), (3, 1000), (8, 1024), (2, 2048), (8, 2048), (5, 3000), (16, 2048), (8, 4096),
          (1, 4096), (7, 1)]


@pytest.mark.parametrize("world,k", SHAPES)
def test_merge_matches_oracle(world, k):
    G.banner(f"dcp merge world={world} k={k}")
    rng = np.random.default_rng(world * 1000 + k)
    rows = 6
    g = _gathered(rng, world, rows, k, "mixed" if k > 1 else "plain")
    g[:, 2, :, 1] = -1.0                    # a row with no candidates
    if world > 1:
        g[1:, 3, :, 1] = -1.0               # a row with candidates on one rank only
    np.testing.assert_array_equal(_merge_gpu(g, k), oracle.dcp_merge(g, k))


@pytest.mark.parametrize("kind", ["equal", "neginf", "nan"])
@pytest.mark.parametrize("world,k", [(8, 2048), (3, 100), (16, 2048)])
def test_merge_heavy_ties(kind, world, k):
    G.banner(f"dcp merge ties {kind} world={world} k={k}")
    rng = np.random.default_rng(5 + world + k)
    g = _gathered(rng, world, 4, k, kind)
    np.testing.assert_array_equal(_merge_gpu(g, k), oracle.dcp_merge(g, k))


def test_merge_ties_at_the_boundary():
    """Distinct scores above a tied k-th value; lower ids must win the boundary."""
    G.banner("dcp merge boundary ties")
    rng = np.random.default_rng(21)
    world, rows, k = 8, 5, 2048
    g = _gathered(rng, world, rows, k, "plain")
    g[..., 0] = np.where(rng.random((world, rows, k)) < 0.3, 0.25, rng.standard_normal((world, rows, k)) + 2)
    np.testing.assert_array_equal(_merge_gpu(g, k), oracle.dcp_merge(g, k))


def test_pack_matches_oracle():
    G.banner("dcp pack")
    rng = np.random.default_rng(9)
    rows, ld, k = 37, 3000, 700
    lg = rng.standard_normal((rows, ld)).astype(np.float32)
    lg[rng.random((rows, ld)) < 0.01] = np.nan
    ks = rng.integers(-5, ld + 5, rows).astype(np.int32)
    ks[:4] = [0, -3, ld, ld + 9]
    tk = rng.integers(-3, ld, (rows, k + 5)).astype(np.int32)
    tk[:, -20:] = -1
    d = G.dev()
    for world, rank, il in ((1, 0, 1), (8, 5, 1), (4, 3, 64), (3, 1, 7)):
        for use_ks in (False, True):
            got = pml.pack_dcp_topk_candidates(torch.from_numpy(lg).to(d), torch.from_numpy(tk).to(d), rank,
                                               world, il, row_starts=torch.from_numpy(ks).to(d) if use_ks else None,
                                               k=k)
            torch.cuda.synchronize()
            want = oracle.dcp_pack(lg, tk[:, :k], rank, world, il, ks=ks if use_ks else None)
            np.testing.assert_array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32))


def _sharded_topk(full: torch.Tensor, lens: np.ndarray, k: int, world: int, interleave: int,
                  ks: np.ndarray | None = None) -> np.ndarray:
    """Per rank: its columns of the rows, top_k_per_row, pack; then gather and merge (all on the GPU)."""
    d = G.dev()
    rows, T = full.shape
    held = brute.dcp_tokens(T, world, interleave)
    lpad = max(len(h) for h in held) + (0 if ks is None else int(ks.max()))
    lpad = (lpad + 3) // 4 * 4
    packed = []
    for r in range(world):
        ids = torch.tensor(held[r], dtype=torch.long, device=d)
        local = torch.full((rows, lpad), 3e38, dtype=torch.float32, device=d)  # garbage outside the spans
        n_r = np.searchsorted(np.asarray(held[r]), lens).astype(np.int32)  # its tokens below each row's length
        if ks is None:
            local[:, : len(held[r])] = full[:, ids]
            ke = torch.from_numpy(n_r).to(d)
            kst = None
        else:
            for i in range(rows):
                local[i, ks[i]: ks[i] + len(held[r])] = full[i, ids]
            ke = torch.from_numpy(ks + n_r).to(d)
            kst = torch.from_numpy(ks).to(d)
        loc = pml.top_k_per_row(local, ke, k, ks=kst, max_width=max(1, int(n_r.max())))
        packed.append(pml.pack_dcp_topk_candidates(local, loc, r, world, interleave, row_starts=kst))
    out = pml.stable_topk_from_gathered_candidates(torch.stack(packed), k)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("world,interleave", [(2, 1), (8, 1), (8, 64), (3, 5)])
@pytest.mark.parametrize("with_ks", [False, True])
def test_sharded_equals_unsharded(world, interleave, with_ks):
    G.banner(f"dcp sharded == unsharded world={world} interleave={interleave} ks={with_ks}")
    rng = np.random.default_rng(world * 7 + interleave + with_ks)
    rows, T, k = 9, 20000, 2048
    s = rng.standard_normal((rows, T)).astype(np.float32)
    s[1] = np.round(s[1])                       # ties
    s[2, ::5] = -np.inf
    s[3, ::7] = np.nan
    lens = rng.integers(1, T + 1, rows).astype(np.int32)
    lens[0], lens[4] = T, 1500                  # a row narrower than k
    for i in range(rows):
        s[i, lens[i]:] = -np.inf                # past the row's length (never selected: outside [0, len))
    ks = rng.integers(0, 40, rows).astype(np.int32) if with_ks else None
    full = torch.from_numpy(s).to(G.dev())
    got = _sharded_topk(full, lens, k, world, interleave, ks)
    ref_gpu = pml.top_k_per_row(full, torch.from_numpy(lens).to(G.dev()), k)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got, ref_gpu.cpu().numpy())
    np.testing.assert_array_equal(got, oracle.topk(s.astype(np.float64), lens, k))


def test_sharded_equals_unsharded_at_decode_size():
    """The 120K-context varlen decode rows (about 140 rows, top-k 2048) split over 8 ranks."""
    G.banner("dcp sharded == unsharded, 140 rows x 128K, 8 ranks")
    rng = np.random.default_rng(1207)
    rows, T, k, world = 140, 131072, 2048, 8
    lens = rng.integers(100_000, T + 1, rows).astype(np.int32)
    full = torch.randn(rows, T, device=G.dev()) * 4
    col = torch.arange(T, device=G.dev())[None, :]
    full = torch.where(col < torch.from_numpy(lens).to(G.dev())[:, None], full, torch.tensor(-np.inf, device=G.dev()))
    got = _sharded_topk(full, lens, k, world, 1)
    ref = pml.top_k_per_row(full, torch.from_numpy(lens).to(G.dev()), k)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got, ref.cpu().numpy())
    # and against the oracle on sampled rows
    pick = [0, 37, 139]
    s = full[pick].cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(got[pick], oracle.topk(s, lens[pick], k))
