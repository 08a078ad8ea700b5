"""bf16 decode logits and their valid-span upcast on the GPU.

* The bf16 call computes what the fp32 call computes and rounds on the store,
  so its output equals the fp32 output rounded to bf16 (nearest, ties to even)
  bit for bit: masking, NaN for bad table entries, the -inf tail and the
  untouched columns past max_ctx included.
* Against the oracle, within the tolerance derived for bf16 in tests/_gpu.py.
* On exactly representable inputs, the oracle's value within the mass bound plus bf16 rounding.
* The upcast equals the bf16 definition on each row's span and writes nothing else.
* bf16 logits -> upcast -> top-k meets the top-k acceptance against the oracle
  with the bf16 tolerance, at the 120K varlen decode size on every row, and
  the top-k over the bf16 logits themselves selects the same, bit for bit.
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


def _same_as_rounded_fp32(case, t=None):
    t = t or G.upload(case)
    f32 = G.run_paged(case, t)
    b16 = G.run_paged_bf16(case, t)
    want = oracle.bf16_round(f32)
    nan = np.isnan(f32)
    np.testing.assert_array_equal(b16[~nan], want[~nan])
    assert np.isnan(oracle.bf16_to_f32(b16[nan])).all()
    return f32, b16


CASES = [
    ("tiny decode", lambda: syn.config_tiny_decode()),
    ("varlen fp8 bkv64", lambda: syn.make_paged_case([3000, 1200, 64, 1], [5, 2, 9, 1], seed=900, max_ctx=3072)),
    ("varlen fp8 bkv32", lambda: syn.make_paged_case([777, 33, 1500], [3, 1, 4], seed=901, block_kv=32, max_ctx=1503)),
    ("varlen mxfp4 bkv32", lambda: syn.make_paged_case([1000, 70, 2048], [2, 4, 1], seed=902, kv_format=1,
                                                       block_kv=32, max_ctx=2050)),
    ("uniform next_n 3, 2-D lengths", lambda: syn.make_paged_case([700, 3, 129, 1500, 64], [3] * 5, seed=903,
                                                                  varlen=False, next_n=3, lens_2d=True,
                                                                  max_ctx=1503)),
]


@pytest.mark.parametrize("name,mk", CASES, ids=[c[0] for c in CASES])
def test_bf16_is_fp32_rounded(name, mk):
    case = mk()
    G.banner(f"bf16 logits == rounded fp32: {name}")
    f32, b16 = _same_as_rounded_fp32(case)
    ref = oracle.paged_logits(case)
    G.assert_logits_close(oracle.bf16_to_f32(b16), ref, case.weights, f"bf16 {name}", G.REL_BF16, G.ABS_BF16)


def test_bf16_exact_arithmetic():
    case = syn.make_paged_case([900, 64, 200, 1], [4, 2, 9, 1], seed=910, max_ctx=960)
    G.exactify_fp8_case(case, seed=911)
    G.banner("bf16 exact arithmetic")
    b16 = G.run_paged_bf16(case)
    # the fp32 score within the mass bound, then rounded to bf16 (at most 2^-8 of it)
    G.assert_within_mass(oracle.bf16_to_f32(b16), oracle.paged_logits(case), brute.paged_mass(case),
                         "bf16 exact", frac=G.MASS_FRAC * (1 + G.U_BF16), rel=G.U_BF16)


def test_bf16_bad_table_entries_and_empty_rows():
    case = syn.make_paged_case([0, 200, 0, 70], [1, 2, 1, 1], seed=920, max_ctx=256)
    bt = case.block_table.clone()
    bt[1, 1] = 10 ** 6
    bt[2, 1] = -5
    c2 = syn.PagedCase(**{**case.__dict__, "block_table": bt})
    G.banner("bf16 bad table entries / empty rows")
    f32, b16 = _same_as_rounded_fp32(c2)
    assert np.all(b16[0] == 0xFF80) and np.all(b16[3] == 0xFF80)
    assert np.isnan(oracle.bf16_to_f32(b16[1, 64:128])).all()


def test_upcast_valid_span_only():
    rng = np.random.default_rng(930)
    rows, cols, ld = 23, 5000, 5008
    bits = rng.integers(0, 1 << 16, (rows, ld), dtype=np.uint32).astype(np.uint16)
    bits[0, :16] = [0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x0000, 0x8000, 0x0001, 0x8001, 0x7F7F, 0xFF7F,
                    0x3F80, 0xBF80, 0x4049, 0x0080, 0x807F, 0x7F81]
    ends = rng.integers(-10, cols + 50, rows).astype(np.int32)
    ends[:6] = [cols, 0, -3, cols + 100, 1, 8 * 37 + 5]
    d = G.dev()
    src = torch.from_numpy(bits.view(np.int16)).to(d).view(torch.bfloat16)
    out = torch.full((rows, ld), G.SENTINEL, dtype=torch.float32, device=d)
    G.banner("upcast")
    pml.as_fp32_logits(src, torch.from_numpy(ends).to(d), out=out, cols=cols)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    want = oracle.bf16_to_f32(bits)
    for r in range(rows):
        e = min(max(int(ends[r]), 0), cols)
        np.testing.assert_array_equal(o[r, :e].view(np.uint32), want[r, :e].view(np.uint32))
        assert np.all(o[r, e:] == G.SENTINEL)


def test_bf16_decode_path_topk_at_full_size():
    """The 120K varlen decode batch: bf16 logits, upcast over each row's span, top-k."""
    case = G.named_case("varlen_fp8")
    G.banner(f"bf16 decode path: {case.rows} rows, max_ctx {case.max_ctx}")
    t = G.upload(case)
    sched = pml.paged_mqa_logits_metadata(t["lens"], case.block_kv, None, indices=t["indices"])
    b16 = pml.fp8_fp4_paged_mqa_logits(t["q"], t["kv"], t["w"], t["lens"], t["bt"], sched, case.max_ctx,
                                       t["indices"], out_dtype=torch.bfloat16)
    vis = G.check_whole_output(oracle.bf16_to_f32(b16.view(torch.int16).cpu().numpy().view(np.uint16)
                                                  [:, : case.max_ctx]), case)
    ends = torch.from_numpy(vis.astype(np.int32)).to(G.dev())
    f32 = pml.as_fp32_logits(b16, ends, cols=case.max_ctx)
    got = pml.top_k_per_row(f32, ends, case.topk, max_width=case.max_ctx)
    direct = pml.top_k_per_row(b16, ends, case.topk, max_width=case.max_ctx)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    np.testing.assert_array_equal(direct.cpu().numpy(), got)
    b = b16.view(torch.int16).cpu().numpy().view(np.uint16)[:, : case.max_ctx]
    # shared input: the upcast values, bit-exact top-k
    up = oracle.bf16_to_f32(b).astype(np.float64)
    np.testing.assert_array_equal(got, oracle.topk(up, vis, case.topk))
    # every row against the fp64 oracle, with the bf16 tolerance
    ref = G.oracle_full("varlen_fp8")
    G.assert_logits_close(up.astype(np.float32), ref, case.weights, "bf16 decode rows", G.REL_BF16, G.ABS_BF16)
    # Selection bound from the per-logit bound tau: at least k GPU values are >= t_k - tau
    # (the oracle's top k, each off by at most tau), so every selected GPU value is too,
    # and its oracle score is >= t_k - 2 tau; symmetrically every score above t_k + 2 tau
    # is selected. (bf16 rounding uses most of tau, so the factor 2 is needed here.)
    wsum = np.abs(case.weights.double().numpy()).sum(1)
    G.topk_acceptance(got, ref, vis, case.topk, wsum, G.REL_BF16, G.ABS_BF16, factor=2.0)
