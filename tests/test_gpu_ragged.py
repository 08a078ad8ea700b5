"""Ragged (non-paged) prefill logits on the GPU against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
from oracle import brute
import paged_mqa_logits_amd as pml
import pml_synth as syn
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _upload(case):
    d = G.dev()
    return dict(q=case.q.to(d), k=case.k.to(d), ks_=case.k_scale.to(d), w=case.weights.to(d),
                ks=case.ks.to(d), ke=case.ke.to(d))


def run_ragged(case, t=None) -> torch.Tensor:
    """GPU logits [M, ld] on the device; columns past N must keep the sentinel."""
    t = t or _upload(case)
    ld = pml.logits_ld(case.N)
    out = torch.full((case.M, ld), G.SENTINEL, dtype=torch.float32, device=G.dev())
    pml.mqa_logits(t["q"], t["k"], t["ks_"], t["w"], t["ks"], t["ke"], logits=out)
    torch.cuda.synchronize()
    assert bool((out[:, case.N:] == G.SENTINEL).all()), "columns past N were written"
    return out


def test_causal_small_full():
    case = syn.make_ragged_case([40, 1, 23, 300, 129, 700], seed=700)
    G.banner(f"ragged causal small M={case.M}")
    gpu = run_ragged(case).cpu().numpy()[:, : case.N]
    G.assert_logits_close(gpu, oracle.ragged_logits(case), case.weights)


def test_arbitrary_bounds():
    """Bounds that are not causal: empty rows, ks > ke, ke past N, negative ks."""
    case = syn.make_ragged_case([500, 333], seed=710)
    rng = np.random.default_rng(711)
    ks = rng.integers(-50, case.N, case.M)
    ke = ks + rng.integers(-20, 900, case.M)
    ks[:5] = 0
    ke[:5] = case.N + 7
    case.ks.copy_(torch.from_numpy(ks.astype(np.int32)))
    case.ke.copy_(torch.from_numpy(ke.astype(np.int32)))
    G.banner("ragged arbitrary bounds")
    gpu = run_ragged(case).cpu().numpy()[:, : case.N]
    # the oracle clamps with n >= ks and n < min(ke, N), as the GPU clamps to [0, N]
    G.assert_logits_close(gpu, oracle.ragged_logits(case), case.weights)


def test_multi_chunk_bounds():
    """Several key chunks per row (fewer pieces than the grid aims for), N not a
    multiple of 4, and bounds that leave -inf on both sides of a row's span, in
    every chunk: the -inf columns are written a slice per block step."""
    case = syn.make_ragged_case([1100, 1103], seed=730)
    rng = np.random.default_rng(731)
    ks = rng.integers(-40, case.N, case.M)
    ke = ks + rng.integers(-10, 1500, case.M)
    ks[:3] = 0
    ke[:3] = case.N + 5
    case.ks.copy_(torch.from_numpy(ks.astype(np.int32)))
    case.ke.copy_(torch.from_numpy(ke.astype(np.int32)))
    rows = np.sort(np.concatenate([np.arange(12), np.arange(case.M - 12, case.M),
                                   rng.choice(case.M, 200, replace=False)]))
    rows = np.unique(rows)
    G.banner(f"ragged multi-chunk N={case.N} rows={len(rows)}")
    gpu = run_ragged(case).cpu().numpy()[rows, : case.N]
    G.assert_logits_close(gpu, oracle.ragged_logits(case, rows=rows), case.weights[torch.from_numpy(rows)])


def test_exact_arithmetic():
    """Exactly representable inputs: the oracle within the mass bound (tests/_gpu.py, MASS_FRAC)."""
    case = syn.make_ragged_case([600, 77], seed=720)
    g = torch.Generator().manual_seed(721)
    case.q.copy_(torch.randint(-8, 9, case.q.shape, generator=g).float().to(torch.float8_e4m3fn).view(torch.uint8))
    case.k.copy_(torch.randint(-8, 9, case.k.shape, generator=g).float().to(torch.float8_e4m3fn).view(torch.uint8))
    case.k_scale.copy_(torch.exp2(torch.randint(-4, 3, case.k_scale.shape, generator=g).float()))
    case.weights.copy_(torch.randint(-32, 33, case.weights.shape, generator=g).float() / 8)
    G.banner("ragged exact arithmetic")
    gpu = run_ragged(case).cpu().numpy()[:, : case.N]
    G.assert_within_mass(gpu, oracle.ragged_logits(case), brute.ragged_mass(case), "ragged exact")


def test_decode_rows_equal_prefill_rows():
    """Decode rows on the paged path == the same rows as ragged rows over the
    keys gathered contiguously with ks = 0, ke = vis (bitwise: same tiles)."""
    case = syn.make_paged_case([1500, 700], [3, 2], seed=730, max_ctx=1536)
    dec = G.run_paged(case)
    vis = oracle.visible_lengths(case)
    kv = case.kv_cache.numpy()
    B, D = case.block_kv, case.D
    bt = case.block_table.numpy()[0]
    nblk = -(-int(vis.max()) // B)
    for r in range(case.rows):
        bt = case.block_table.numpy()[r]
        vals = np.concatenate([kv[bt[b], : B * D].reshape(B, D) for b in range(nblk) if bt[b] >= 0])
        scl = np.concatenate([kv[bt[b], B * D: B * D + 4 * B].copy().view(np.float32) for b in range(nblk) if bt[b] >= 0])
        n = int(vis[r])
        rc = syn.RaggedCase(q=case.q[r:r + 1].clone(), weights=case.weights[r:r + 1].clone(),
                            k=torch.from_numpy(np.ascontiguousarray(vals[:n])),
                            k_scale=torch.from_numpy(scl[:n].copy()),
                            ks=torch.tensor([0], dtype=torch.int32), ke=torch.tensor([n], dtype=torch.int32),
                            topk=8)
        G.banner(f"decode == prefill row {r}")
        pre = run_ragged(rc).cpu().numpy()[0, :n]
        np.testing.assert_array_equal(pre, dec[r, :n])


def _c5_rows(case, n_random: int, seed: int) -> np.ndarray:
    """The first two and last two rows of every sequence plus n_random others."""
    starts = np.unique(case.ks.numpy())
    ends = np.append(starts[1:], case.M)
    edge = np.concatenate([[a, a + 1, b - 2, b - 1] for a, b in zip(starts, ends)])
    rest = np.setdiff1d(np.arange(case.M), edge)
    pick = np.random.default_rng(seed).choice(rest, n_random, replace=False)
    return np.sort(np.concatenate([edge, pick])).astype(np.int64)


def test_ragged_prefill_config_rows():
    case = syn.config_ragged_prefill()
    rows = _c5_rows(case, 512, 3)
    G.banner(f"ragged prefill 4x8192 M={case.M}: {len(rows)} rows against the oracle")
    t = _upload(case)
    out = run_ragged(case, t)[:, : case.N]
    # whole-output properties on the device: -inf exactly outside [ks, ke), finite inside
    cols = torch.arange(case.N, device=G.dev())
    for r0 in range(0, case.M, 4096):
        blk = out[r0: r0 + 4096]
        inside = (cols[None, :] >= t["ks"][r0: r0 + 4096, None]) & (cols[None, :] < t["ke"][r0: r0 + 4096, None])
        assert bool(torch.isneginf(blk[~inside]).all())
        assert bool(torch.isfinite(blk[inside]).all())
    ref = oracle.ragged_logits(case, rows=rows)
    G.assert_logits_close(out[torch.from_numpy(rows).to(G.dev())].cpu().numpy(), ref, case.weights[rows])


def test_ragged_prefill_config_topk_full():
    """top-k 2048 of all 32768 prefill rows on the GPU logits: bit for bit with
    the oracle's top-k over the same values, and the acceptance against the
    fp64 scores on the sampled rows (first and last rows of each sequence)."""
    case = syn.config_ragged_prefill()
    G.banner(f"ragged prefill top-k at full size M={case.M} k={case.topk}")
    t = _upload(case)
    out = run_ragged(case, t)
    got = pml.top_k_per_row(out, t["ke"], case.topk, ks=t["ks"], max_width=case.N)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    ks, ke = case.ks.numpy(), case.ke.numpy()
    for r0 in range(0, case.M, 2048):
        r1 = min(r0 + 2048, case.M)
        L = out[r0:r1, : case.N].cpu().numpy()
        np.testing.assert_array_equal(got[r0:r1], oracle.topk(L, ke[r0:r1], case.topk, ks=ks[r0:r1]),
                                      err_msg=f"rows {r0}..{r1}")
    rows = _c5_rows(case, 64, 5)
    ref = oracle.ragged_logits(case, rows=rows)
    # scores relative to each row's start, as the selection's positions are
    rel = np.full((len(rows), case.N), -np.inf)
    for i, r in enumerate(rows):
        n = max(0, int(ke[r]) - int(ks[r]))
        rel[i, :n] = ref[i, ks[r]: ks[r] + n]
    G.topk_acceptance(got[rows], rel, np.maximum(ke[rows] - ks[rows], 0), case.topk,
                      np.abs(case.weights[rows].double().numpy()).sum(1))
