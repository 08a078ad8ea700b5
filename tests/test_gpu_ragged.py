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
    vis = syn.vis_per_row(case)
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


def test_ragged_prefill_config_sampled():
    case = syn.config_ragged_prefill()
    G.banner(f"ragged prefill 4x8192 M={case.M}")
    t = _upload(case)
    out = run_ragged(case, t)[:, : case.N]
    # whole-output properties on the device: -inf exactly outside [ks, ke), finite inside
    cols = torch.arange(case.N, device=G.dev())
    for r0 in range(0, case.M, 4096):
        blk = out[r0: r0 + 4096]
        inside = (cols[None, :] >= t["ks"][r0: r0 + 4096, None]) & (cols[None, :] < t["ke"][r0: r0 + 4096, None])
        assert bool(torch.isneginf(blk[~inside]).all())
        assert bool(torch.isfinite(blk[inside]).all())
    rows = np.sort(np.random.default_rng(3).choice(case.M, 24, replace=False))
    rows[:4] = [0, 8191, 8192, case.M - 1]
    rows = np.sort(rows)
    ref = oracle.ragged_logits(case, rows=rows)
    G.assert_logits_close(out[torch.from_numpy(rows).to(G.dev())].cpu().numpy(), ref, case.weights[rows])
