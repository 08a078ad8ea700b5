"""Pins of the CPU oracle against things other than itself (CPU only).

* number formats: torch's own fp8 / e8m0 conversions and the OCP MX e2m1 table
* hand-worked examples (tests/golden/paged_hand_worked.json)
* closed forms that reduce to a numpy dot / GEMV
* a numpy gather + einsum formulation on tiny inputs
* invariants of the method (grouping, padding, paging, stride, decode == prefill)
"""
import json
import math
import os
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
import pml_synth as syn

GOLD = os.path.join(os.path.dirname(__file__), "golden", "paged_hand_worked.json")


def _gold():
    with open(GOLD) as f:
        return json.load(f)


def _num(x):
    if isinstance(x, str):
        return {"-inf": -math.inf, "inf": math.inf, "nan": math.nan}[x]
    return float(x)


# --------------------------------------------------------------------------
# formats

def test_fp8_table_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.fp8_e4m3(c) for c in range(256)])
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    m = ~np.isnan(ref)
    assert np.array_equal(ref[m], got[m])
    assert got[0x7E] == 448.0 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    # numpy bit-field decoder agrees too
    nb = brute.fp8_e4m3_np(np.arange(256))
    assert np.array_equal(np.isnan(nb), np.isnan(ref)) and np.array_equal(nb[m], ref[m])


def test_e8m0_table_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).double().numpy()
    got = np.array([oracle.e8m0(c) for c in range(256)])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(ref[:255], got[:255])
    assert got[0] == 2.0 ** -127 and got[127] == 1.0


def test_e2m1_table_matches_ocp_mx():
    # OCP Microscaling Formats v1.0, FP4 E2M1 element table.
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(16):
        want = mags[c & 7] * (-1.0 if c & 8 else 1.0)
        assert oracle.e2m1(c) == want
        assert brute.e2m1_np(np.array([c]))[0] == want


def test_generator_clamps_before_fp8_cast():
    x = torch.tensor([449.0, 464.0, 480.0, 1e6, -1e6])
    got = syn.fp8_codes(x).view(torch.float8_e4m3fn).float()
    assert torch.equal(got, torch.tensor([448.0, 448.0, 448.0, 448.0, -448.0]))


def test_mx_quantizer_roundtrip_exact_values():
    # values already on the e2m1 grid times a power of two quantise exactly
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6] * 4, dtype=np.float64)
    x = (grid * np.where(np.arange(32) % 3 == 0, -1, 1) * 2.0 ** 5)[None, :]
    packed, sc = syn.mx_fp4_quantize(x)
    nib = np.empty((1, 32), dtype=np.uint8)
    nib[:, 0::2] = packed & 15
    nib[:, 1::2] = packed >> 4
    back = brute.e2m1_np(nib) * brute.e8m0_np(sc)[:, :, None].repeat(32, axis=2).reshape(1, 32)
    assert np.array_equal(back, x)


# --------------------------------------------------------------------------
# hand-worked examples

def _fp8_gold_case(g):
    c = g["fp8_case"]
    H, D, bkv = c["H"], c["D"], c["block_kv"]
    pb = bkv * (D + 4)
    kv = np.zeros((len(c["pages"]), pb), dtype=np.uint8)
    for p, page in enumerate(c["pages"]):
        kv[p, : bkv * D] = np.array(page["slot_codes"], dtype=np.uint8).reshape(-1)
        sc = np.array([_num(s) for s in page["slot_scales"]], dtype=np.float32)
        kv[p, bkv * D:] = sc.view(np.uint8)
    return syn.PagedCase(
        q=torch.tensor(c["q_codes"], dtype=torch.uint8), weights=torch.tensor(c["weights"], dtype=torch.float32),
        kv_cache=torch.from_numpy(kv), kv_format=0, block_kv=bkv,
        block_table=torch.tensor(c["block_table"], dtype=torch.int32),
        context_lens=torch.tensor(c["context_lens"], dtype=torch.int32),
        indices=torch.tensor(c["indices"], dtype=torch.int32), next_n=1, max_ctx=c["max_ctx"],
        topk=2, H=H, D=D)


def _fp4_gold_case(g):
    c = g["fp4_case"]
    H, D, bkv = c["H"], c["D"], c["block_kv"]
    pb = bkv * (D // 2 + D // 32)
    kv = np.zeros((len(c["pages"]), pb), dtype=np.uint8)
    for p, page in enumerate(c["pages"]):
        kv[p, 0] = page["packed_first_byte"]
        kv[p, D // 2] = page["e8m0"]
    q = np.zeros((1, H, D), dtype=np.uint8)
    q[0, 0, :2] = c["q_codes_first2"]
    return syn.PagedCase(
        q=torch.from_numpy(q), weights=torch.tensor(c["weights"], dtype=torch.float32),
        kv_cache=torch.from_numpy(kv), kv_format=1, block_kv=bkv,
        block_table=torch.tensor(c["block_table"], dtype=torch.int32),
        context_lens=torch.tensor(c["context_lens"], dtype=torch.int32),
        indices=None, next_n=1, max_ctx=c["max_ctx"], topk=1, H=H, D=D)


def test_golden_fp8_paged_logits_and_topk():
    g = _gold()
    case = _fp8_gold_case(g)
    want = np.array([[_num(v) for v in row] for row in g["fp8_case"]["expected_logits"]])
    got = oracle.paged_logits(case)
    assert np.array_equal(got, want)
    assert np.array_equal(brute.paged_logits(case), want)
    vis = oracle.visible_lengths(case)
    for key in ("expected_topk", "expected_topk_k3"):
        e = g["fp8_case"][key]
        assert oracle.topk(got, vis, e["k"]).tolist() == e["rows"]


def test_golden_fp4_paged_logits_nibble_order():
    g = _gold()
    case = _fp4_gold_case(g)
    want = np.array(g["fp4_case"]["expected_logits"], dtype=np.float64)
    assert np.array_equal(oracle.paged_logits(case), want)
    assert np.array_equal(brute.paged_logits(case), want)


def test_golden_topk_ties():
    t = _gold()["topk_ties"]
    s = np.array([[_num(v) for v in r] for r in t["rows"]])
    ke = np.full(2, 5, dtype=np.int32)
    for k, key in ((2, "k2"), (3, "k3"), (7, "k7")):
        assert oracle.topk(s, ke, k).tolist() == t[key]
        assert brute.topk(s, ke, k).tolist() == t[key]


# --------------------------------------------------------------------------
# closed forms

def _dequant_torch(case):
    """Independent dequantisation through torch's fp8 conversion (fp8 pages only)."""
    kv = case.kv_cache.numpy()
    B, D = case.block_kv, case.D
    vals = torch.from_numpy(kv[:, : B * D].copy()).view(torch.float8_e4m3fn).double().reshape(-1, B, D)
    sc = torch.from_numpy(kv[:, B * D: B * D + 4 * B].copy()).view(torch.float32).double().reshape(-1, B, 1)
    return (vals * sc).numpy()


def _tokens_of_row(case, r):
    pages = _dequant_torch(case)
    vis = int(oracle.visible_lengths(case)[r])
    bt = case.block_table.numpy()[r // case.next_n]
    return np.concatenate([pages[bt[b]] for b in range(-(-vis // case.block_kv))])[:vis]


def test_closed_form_single_head_is_relu_of_dot():
    case = syn.make_paged_case([300, 129], [2, 1], seed=7, H=1, max_ctx=320)
    case.weights[:] = 1.0
    got = oracle.paged_logits(case)
    q = case.q.view(torch.float8_e4m3fn).double().numpy()
    for r in range(case.rows):
        K = _tokens_of_row(case, r)
        want = np.maximum(K @ q[r, 0], 0.0)
        np.testing.assert_allclose(got[r, : len(K)], want, rtol=1e-12, atol=1e-12)
        assert np.all(np.isneginf(got[r, len(K):]))


def test_closed_form_nonnegative_is_one_gemv():
    # every dot >= 0, so the ReLU is the identity and the logits are K^ (sum_h w_h q^_h)
    case = syn.make_paged_case([200, 77, 64], [1, 3, 2], seed=8, H=8, max_ctx=256)
    case.q.copy_(case.q & 0x7F)                 # clear sign bits
    kv = case.kv_cache.numpy()
    B, D = case.block_kv, case.D
    v = kv[:, : B * D]
    v &= 0x7F
    v[v == 0x7F] = 0x7E                         # no NaN codes in the value region
    got = oracle.paged_logits(case)
    q = case.q.view(torch.float8_e4m3fn).double().numpy()
    w = case.weights.double().numpy()
    for r in range(case.rows):
        K = _tokens_of_row(case, r)
        want = K @ (w[r] @ q[r])
        np.testing.assert_allclose(got[r, : len(K)], want, rtol=1e-12, atol=1e-9)


def test_closed_form_one_hot_picks_one_element():
    case = syn.make_paged_case([150], [1], seed=9, H=4, max_ctx=192)
    d0, h0 = 37, 2
    case.q.zero_()
    case.q[0, h0, d0] = 0x38                    # 1.0
    case.weights.zero_()
    case.weights[0, h0] = 0.75
    got = oracle.paged_logits(case)
    K = _tokens_of_row(case, 0)
    np.testing.assert_array_equal(got[0, :150], 0.75 * np.maximum(K[:, d0], 0.0))


# --------------------------------------------------------------------------
# independent numpy formulation on tiny random inputs

@pytest.mark.parametrize("fmt,bkv,H", [(0, 64, 4), (0, 32, 1), (1, 32, 4), (1, 64, 64), (0, 64, 64)])
def test_oracle_matches_numpy_varlen(fmt, bkv, H):
    case = syn.make_paged_case([130, 1, 64, 90], [2, 1, 3, 1], seed=11 + fmt + bkv + H, kv_format=fmt,
                               block_kv=bkv, H=H, max_ctx=160, fp4_spread=4)
    a = oracle.paged_logits(case)
    b = brute.paged_logits(case)
    fin = np.isfinite(b)
    assert np.array_equal(np.isneginf(a), np.isneginf(b))
    np.testing.assert_allclose(a[fin], b[fin], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("lens_2d", [False, True])
def test_oracle_matches_numpy_uniform(lens_2d):
    case = syn.make_paged_case([100, 70, 3], [3, 3, 3], seed=21, varlen=False, next_n=3,
                               lens_2d=lens_2d, H=4, max_ctx=128)
    a = oracle.paged_logits(case)
    b = brute.paged_logits(case)
    assert np.array_equal(np.isneginf(a), np.isneginf(b))
    fin = np.isfinite(b)
    np.testing.assert_allclose(a[fin], b[fin], rtol=1e-12, atol=1e-12)


def test_ragged_oracle_matches_numpy():
    case = syn.make_ragged_case([40, 1, 23], seed=5, H=4)
    a = oracle.ragged_logits(case)
    b = brute.ragged_logits(case)
    assert np.array_equal(np.isneginf(a), np.isneginf(b))
    fin = np.isfinite(b)
    np.testing.assert_allclose(a[fin], b[fin], rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# invariants of the method

def test_uniform_padded_equals_flattened_varlen():
    """Padded uniform (B, next_n) rows == the same rows flattened as varlen rows,
    and 1-D lengths with next_n > 1 follow the ctx - next_n + j + 1 rule."""
    ctx = [90, 200, 65]
    a = syn.make_paged_case(ctx, [4] * 3, seed=31, varlen=False, next_n=4, H=4, max_ctx=256)
    b = syn.make_paged_case(ctx, [4] * 3, seed=31, varlen=True, H=4, max_ctx=256)
    c = syn.make_paged_case(ctx, [4] * 3, seed=31, varlen=False, next_n=4, lens_2d=True, H=4, max_ctx=256)
    la, lb, lc = (oracle.paged_logits(x) for x in (a, b, c))
    assert np.array_equal(la, lb) and np.array_equal(la, lc)


def test_decode_rows_equal_prefill_rows():
    """Decode rows == the same rows scored as non-paged rows over the gathered keys (ks = 0, ke = vis)."""
    case = syn.make_paged_case([150, 97], [3, 2], seed=41, H=4, max_ctx=160)
    dec = oracle.paged_logits(case)
    vis = oracle.visible_lengths(case)
    for r in range(case.rows):
        bt = case.block_table.numpy()[r]
        kv = case.kv_cache.numpy()
        B, D = case.block_kv, case.D
        nblk = -(-int(vis[r]) // B)
        vals = np.concatenate([kv[bt[b], : B * D].reshape(B, D) for b in range(nblk)])[: vis[r]]
        scl = np.concatenate([kv[bt[b], B * D:].copy().view(np.float32) for b in range(nblk)])[: vis[r]]
        rc = syn.RaggedCase(q=case.q[r:r + 1].clone(), weights=case.weights[r:r + 1].clone(),
                            k=torch.from_numpy(np.ascontiguousarray(vals)), k_scale=torch.from_numpy(scl.copy()),
                            ks=torch.tensor([0], dtype=torch.int32), ke=torch.tensor([int(vis[r])], dtype=torch.int32),
                            topk=8, H=case.H, D=case.D)
        pre = oracle.ragged_logits(rc)
        assert np.array_equal(pre[0], dec[r, : vis[r]])


def test_rows_are_independent():
    case = syn.make_paged_case([120, 64, 33], [2, 1, 2], seed=51, H=4, max_ctx=128)
    full = oracle.paged_logits(case)
    rows = np.array([4, 0, 3, 3, 1])
    assert np.array_equal(oracle.paged_logits(case, rows=rows), full[rows])
    assert np.array_equal(oracle.paged_logits(case, rows=[2], col_begin=10, col_end=50), full[2:3, 10:50])


def test_page_permutation_and_stride_change_nothing():
    case = syn.make_paged_case([150, 40], [2, 1], seed=61, H=4, max_ctx=192)
    base = oracle.paged_logits(case)
    kv = case.kv_cache.numpy()
    perm = np.random.default_rng(0).permutation(kv.shape[0])
    inv = np.argsort(perm)
    kv2 = kv[perm]                                 # page p now lives at inv[p]
    bt = case.block_table.numpy().copy()
    bt2 = np.where(bt >= 0, inv[np.maximum(bt, 0)], -1).astype(np.int32)
    wide = np.full((kv.shape[0], kv.shape[1] + 48), 0xAB, dtype=np.uint8)
    wide[:, : kv.shape[1]] = kv2
    c2 = syn.PagedCase(**{**case.__dict__, "kv_cache": torch.from_numpy(wide),
                          "block_table": torch.from_numpy(bt2)})
    assert np.array_equal(oracle.paged_logits(c2), base)


def test_masked_cells_are_neg_inf_and_empty_rows():
    case = syn.make_paged_case([70, 0], [1, 1], seed=71, H=2, max_ctx=128)
    out = oracle.paged_logits(case)
    assert np.all(np.isneginf(out[0, 70:])) and np.all(np.isfinite(out[0, :70]))
    assert np.all(np.isneginf(out[1]))
    tk = oracle.topk(out, oracle.visible_lengths(case), 4)
    assert tk[1].tolist() == [-1] * 4


def test_visible_lengths_hand_worked():
    """The row-length rule worked by hand: a 1-D length per batch entry with
    next_n 3 gives row j of entry b len[b] - 3 + j + 1 (never below 0); 2-D
    lengths and next_n 1 give each row its own length."""
    def vis(lens, next_n, lens_2d, rows):
        c = types.SimpleNamespace(context_lens=torch.tensor(lens, dtype=torch.int32), next_n=next_n,
                                  lens_2d=lens_2d, rows=rows)
        return oracle.visible_lengths(c).tolist()
    assert vis([10, 3, 1], 3, False, 9) == [8, 9, 10, 1, 2, 3, 0, 0, 1]
    assert vis([[4, 5, 6], [0, -2, 7]], 3, True, 6) == [4, 5, 6, 0, 0, 7]
    assert vis([5, 0, 9], 1, False, 3) == [5, 0, 9]


def test_visible_lengths_end_the_unmasked_span():
    """On generated cases the rule's bound is where the oracle's own scores turn -inf."""
    for case in (syn.make_paged_case([300, 5, 130], [3, 1, 2], seed=41, max_ctx=320),
                 syn.make_paged_case([100, 70, 3], [3, 3, 3], seed=42, varlen=False, next_n=3, H=4, max_ctx=128),
                 syn.make_paged_case([100, 70, 3], [3, 3, 3], seed=43, varlen=False, next_n=3, lens_2d=True, H=4,
                                     max_ctx=128)):
        out = oracle.paged_logits(case)
        vis = oracle.visible_lengths(case)
        cols = np.arange(case.max_ctx)[None, :]
        assert np.array_equal(np.isneginf(out), cols >= vis[:, None])


def test_topk_matches_numpy_and_torch():
    rng = np.random.default_rng(3)
    s = rng.standard_normal((6, 300))
    s[2, :] = np.round(s[2, :])                    # many ties
    ke = np.array([300, 17, 300, 0, 250, 100], dtype=np.int32)
    ks = np.array([0, 3, 10, 0, 249, 50], dtype=np.int32)
    for k in (1, 5, 64, 400):
        a = oracle.topk(s, ke, k, ks=ks)
        b = brute.topk(s, ke, k, ks=ks)
        assert np.array_equal(a, b)
    # distinct values: the same set as torch.topk
    t = oracle.topk(s[[0]], ke[[0]], 50)
    tt = torch.topk(torch.from_numpy(s[0]), 50).indices.sort().values.numpy()
    assert np.array_equal(t[0], tt)


# --------------------------------------------------------------------------
# bf16 (logits output format)

def test_bf16_helpers_match_torch():
    rng = np.random.default_rng(17)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0) ** rng.integers(-40, 40, 20000),
        np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 3.3895e38, 3.4e38, -3.4e38, 1e-40, -1e-45,
                  1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20], dtype=np.float32)])
    # exact ties: halfway between two bf16 values, both parities
    u = (rng.integers(0x00800000, 0x7f000000, 5000, dtype=np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    x = np.concatenate([x, u.view(np.float32), -u.view(np.float32)])
    got = oracle.bf16_round(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    finite = ~np.isnan(x)
    assert np.array_equal(got[finite], want[finite])
    assert np.isnan(oracle.bf16_to_f32(got[~finite])).all()
    back = torch.from_numpy(got.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(oracle.bf16_to_f32(got)[finite], back[finite])
    # the rounding error bound used for the bf16 logits tolerance: half a unit in the 8th bit
    xf = x[finite & np.isfinite(x) & (np.abs(x) > 1e-37) & (np.abs(x) < 3e38)].astype(np.float64)
    err = np.abs(oracle.bf16_to_f32(oracle.bf16_round(xf.astype(np.float32))).astype(np.float64) - xf)
    assert (err <= 2.0 ** -8 * np.abs(xf)).all()


# --------------------------------------------------------------------------
# fp4 q (values + per-32 e8m0 scales)

@pytest.mark.parametrize("fmt,bkv", [(1, 32), (1, 64), (0, 64)])
def test_fp4q_oracle_matches_numpy(fmt, bkv):
    case = syn.make_paged_case([300, 64, 130], [3, 1, 2], seed=960 + fmt + bkv, kv_format=fmt, block_kv=bkv,
                               max_ctx=320, q_fp4=True, H=8)
    assert case.q.shape == (6, 8, 64) and case.q_scale.shape == (6, 8, 4)
    a = oracle.paged_logits(case)
    b = brute.paged_logits(case)
    fin = np.isfinite(b)
    assert np.array_equal(np.isneginf(a), np.isneginf(b))
    np.testing.assert_allclose(a[fin], b[fin], rtol=1e-12, atol=1e-12)


def test_fp4q_equals_fp8q_when_exact_in_fp8():
    """e2m1 values times 2^e stay exact in e4m3 for the generator's scales, so the same
    real q given as fp8 codes (through torch's fp8 conversion) scores identically."""
    case = syn.make_paged_case([500, 90], [2, 3], seed=970, kv_format=1, block_kv=32, max_ctx=512, q_fp4=True)
    qv = brute.q_dequant(case)
    codes = syn.fp8_codes(torch.from_numpy(qv.astype(np.float32)))
    assert np.array_equal(codes.view(torch.float8_e4m3fn).double().numpy(), qv)
    c8 = syn.PagedCase(**{**case.__dict__, "q": codes, "q_scale": None})
    a, b = oracle.paged_logits(case), oracle.paged_logits(c8)
    assert np.array_equal(a, b)
    # the scales matter: one changed scale byte changes that head's scores
    c2 = syn.PagedCase(**{**case.__dict__, "q_scale": case.q_scale.clone()})
    c2.q_scale[0, 5, 1] += 1
    assert not np.array_equal(oracle.paged_logits(c2)[0], a[0])


# --------------------------------------------------------------------------
# row bounds outside the row (hand-worked, tests/golden/topk_bounds_hand_worked.json)

BOUNDS = os.path.join(os.path.dirname(__file__), "golden", "topk_bounds_hand_worked.json")


def test_golden_topk_out_of_range_bounds_are_clamped():
    g = json.load(open(BOUNDS))
    row = np.array(g["row"], dtype=np.float64)
    assert row.shape[0] == g["ld"]
    for c in g["topk"]:
        s = row[None, :]
        ke = np.array([c["ke"]], np.int32)
        ks = None if c["ks"] is None else np.array([c["ks"]], np.int32)
        got = oracle.topk(s, ke, c["k"], ks=ks)
        assert got[0].tolist() == c["expected"], c["derivation"]
        assert brute.topk(s, ke, c["k"], ks=ks)[0].tolist() == c["expected"], c["derivation"]


def test_mass_bounds_the_score_and_equals_it_for_nonnegative_terms():
    """brute.paged_mass / ragged_mass (the error scale of the exact-input GPU
    tests): |score| <= mass always, and mass == score when every q, k and w is
    non-negative (then no ReLU clips and no product is negative)."""
    case = syn.make_paged_case([300, 70], [3, 1], seed=31, max_ctx=320)
    m, L = brute.paged_mass(case), oracle.paged_logits(case)
    fin = np.isfinite(L)
    assert np.all(np.abs(L[fin]) <= m[fin] * (1 + 1e-12)) and np.all(m[~fin] == 0)
    pos = syn.make_paged_case([300, 70], [3, 1], seed=32, max_ctx=320)
    pos.q.copy_(pos.q & 0x7F)                      # clear the sign bits
    kv = pos.kv_cache.numpy()
    kv[:, : 64 * 128] &= np.where(kv[:, : 64 * 128] == syn.FP8_NAN, 0xFF, 0x7F).astype(np.uint8)
    pos.weights.abs_()
    m2, L2 = brute.paged_mass(pos), oracle.paged_logits(pos)
    f2 = np.isfinite(L2)
    np.testing.assert_allclose(m2[f2], L2[f2], rtol=1e-12)
    rc = syn.make_ragged_case([40, 30], seed=33)
    mr, Lr = brute.ragged_mass(rc), oracle.ragged_logits(rc)
    fr = np.isfinite(Lr)
    assert np.all(np.abs(Lr[fr]) <= mr[fr] * (1 + 1e-12))
