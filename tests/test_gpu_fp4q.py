"""Paged logits with fp4 q (e2m1 values, per-32 e8m0 scales) over MXFP4 keys on the GPU.

* Small varlen / uniform cases and the 64K MXFP4 decode config (every row)
  within the logits tolerance of the oracle.
* Exactly representable inputs (power-of-two scales, w in (1/8)Z): bit for bit.
* The same real q given as fp8 codes and as fp4 (values, scales) scores the
  same within tolerance, and within a tight bound of each score's mass on exact inputs.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import brute
import paged_mqa_logits_amd as pml
import pml_synth as syn
from tests import _gpu as G

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("bkv", [32, 64])
def test_fp4q_varlen_small(bkv):
    ctx = [1300, 1, 64, 90, 2100, 777]
    case = syn.make_paged_case(ctx, [2, 1, 3, 1, 11, 6], seed=980 + bkv, kv_format=1, block_kv=bkv,
                               max_ctx=2200, fp4_spread=6, q_fp4=True)
    G.banner(f"fp4 q varlen small bkv={bkv}")
    G.assert_logits_close(G.run_paged(case), oracle.paged_logits(case), case.weights, f"fp4q bkv{bkv}")


def test_fp4q_uniform_next_n():
    case = syn.make_paged_case([700, 3, 129, 1500, 64], [3] * 5, seed=985, kv_format=1, block_kv=32,
                               varlen=False, next_n=3, max_ctx=1503, q_fp4=True)
    G.banner("fp4 q uniform next_n=3")
    G.assert_logits_close(G.run_paged(case), oracle.paged_logits(case), case.weights, "fp4q next_n")


def _exactify_fp4(case, seed):
    """Key scales 2^-1..2^1 (|k| <= 12, multiples of 1/4), q scales 2^-2..2^0 (|q| <= 6,
    multiples of 1/8), w in (1/8)Z within [-1, 1]: every product is a multiple of 2^-5,
    every weighted term of 2^-8 (with the exact factor 2 of the ReLU, 2^-7), and the
    sums of random rows stay near 2^12, so every partial sum is exact in fp32."""
    rng = np.random.default_rng(seed)
    kv = case.kv_cache.numpy()
    B = case.block_kv
    sc = kv[:, B * 64: B * 68]
    live = sc != syn.E8M0_NAN
    sc[live] = rng.integers(126, 129, live.sum())
    case.q_scale.copy_(torch.from_numpy(rng.integers(125, 128, tuple(case.q_scale.shape)).astype(np.uint8)))
    g = torch.Generator().manual_seed(seed)
    case.weights.copy_(torch.randint(-8, 9, case.weights.shape, generator=g).float() / 8)


@pytest.mark.parametrize("bkv", [32, 64])
def test_fp4q_exact_arithmetic(bkv):
    case = syn.make_paged_case([500, 33, 96, 1], [3, 1, 5, 1], seed=990 + bkv, kv_format=1, block_kv=bkv,
                               max_ctx=512, q_fp4=True)
    _exactify_fp4(case, 991 + bkv)
    G.banner(f"fp4 q exact arithmetic bkv={bkv}")
    G.assert_within_mass(G.run_paged(case), oracle.paged_logits(case), brute.paged_mass(case), "exact fp4 q")


def test_fp4q_equals_fp8q():
    case = syn.make_paged_case([900, 70, 400], [2, 4, 1], seed=995, kv_format=1, block_kv=32, max_ctx=900,
                               q_fp4=True)
    _exactify_fp4(case, 996)
    qv = brute.q_dequant(case)
    codes = syn.fp8_codes(torch.from_numpy(qv.astype(np.float32)))
    assert np.array_equal(codes.view(torch.float8_e4m3fn).double().numpy(), qv)  # the same real q
    c8 = syn.PagedCase(**{**case.__dict__, "q": codes, "q_scale": None})
    G.banner("fp4 q == fp8 q (same real q)")
    np.testing.assert_array_equal(G.run_paged(case), G.run_paged(c8))


def test_fp4q_config_full():
    case = G.named_case("varlen_fp4_q4")
    G.banner(f"fp4 q varlen MXFP4 64K: all {case.rows} rows")
    gpu = G.run_paged(case)
    G.check_whole_output(gpu, case)
    G.assert_logits_close(gpu, G.oracle_full("varlen_fp4_q4"), case.weights, "fp4q config")
