"""Paged logits and schedule on the GPU against the CPU oracle (parity tests).

Cases span several key blocks per row, ragged last blocks, groups longer than
one row-piece, uniform next_n > 1 with 1-D and 2-D lengths, fp8 and MXFP4
caches at block_kv 32 and 64, and the four paged named workloads, every row
of each compared element by element.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from oracle import schedule as spec
import paged_mqa_logits_amd as pml
import pml_synth as syn
from tests import _gpu as G

pytestmark = pytest.mark.gpu


# --------------------------------------------------------------------------
# schedule: bit-exact against the specification

def _sched_case(lens, next_n, indices, bkv, W, lens_2d=False):
    d = G.dev()
    lt = torch.as_tensor(np.asarray(lens), dtype=torch.int32).to(d)
    it = None if indices is None else torch.as_tensor(np.asarray(indices), dtype=torch.int32).to(d)
    got = pml.paged_mqa_logits_metadata(lt, bkv, W, indices=it, next_n=next_n).cpu().numpy()
    rows = lt.numel() if (lens_2d or indices is not None or next_n == 1) else lt.numel() * next_n
    assert got.shape == (W + 1, 2)  # one range per workgroup, then the end
    want = spec.schedule(np.asarray(lens), rows, next_n, lens_2d, indices, bkv, W)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("seed", range(4))
def test_schedule_varlen_matches_spec(seed):
    rng = np.random.default_rng(100 + seed)
    R = int(rng.integers(1, 300))
    runs = rng.integers(1, 12, R)
    ctx = rng.integers(0, 140000, R)
    lens = np.concatenate([np.maximum(c - n + np.arange(n) + 1, 0) for c, n in zip(ctx, runs)])
    ids = np.repeat(rng.permutation(R) % max(1, R // 2), runs)
    G.banner(f"schedule varlen seed={seed} rows={len(lens)}")
    for W in (1, 7, 256, 512, 3000, 50000):  # (chunk offsets in 32-bit arithmetic up to 46340 workers)
        _sched_case(lens, 1, ids, int(rng.choice([32, 64])), W)


@pytest.mark.parametrize("next_n,lens_2d", [(1, False), (4, False), (4, True)])
def test_schedule_uniform_matches_spec(next_n, lens_2d):
    rng = np.random.default_rng(7)
    B = 1500
    ctx = rng.integers(0, 70000, B)
    lens = (ctx[:, None] - next_n + np.arange(next_n) + 1).clip(0, None) if lens_2d else ctx
    G.banner(f"schedule uniform next_n={next_n} 2d={lens_2d}")
    for W in (1, 512):
        _sched_case(lens, next_n, None, 64, W, lens_2d)


def test_schedule_empty_rows():
    G.banner("schedule empty")
    _sched_case(np.zeros(9, dtype=np.int32), 1, np.arange(9), 64, 16)


# --------------------------------------------------------------------------
# small cases in full

def _check_case(case, **kw):
    gpu = G.run_paged(case, **kw)
    ref = oracle.paged_logits(case)
    G.assert_logits_close(gpu, ref, case.weights)
    return gpu


def test_tiny_decode_config_full():
    case = syn.config_tiny_decode()
    G.banner(f"tiny decode rows={case.rows}")
    _check_case(case)


@pytest.mark.parametrize("fmt,bkv", [(0, 64), (0, 32), (1, 32), (1, 64)])
def test_varlen_small(fmt, bkv):
    # rows per request 2, 1, 3, 1, 11 (longer than one row-piece), 6; ragged ends
    ctx = [1300, 1, 64, 90, 2100, 777]
    case = syn.make_paged_case(ctx, [2, 1, 3, 1, 11, 6], seed=200 + fmt * 10 + bkv, kv_format=fmt,
                               block_kv=bkv, max_ctx=2200, fp4_spread=6)
    G.banner(f"varlen small fmt={fmt} bkv={bkv}")
    _check_case(case)


@pytest.mark.parametrize("lens_2d", [False, True])
@pytest.mark.parametrize("fmt", [0, 1])
def test_uniform_next_n(lens_2d, fmt):
    bkv = 64 if fmt == 0 else 32
    ctx = [700, 3, 129, 1500, 64]
    case = syn.make_paged_case(ctx, [3] * 5, seed=300 + fmt, kv_format=fmt, block_kv=bkv, varlen=False,
                               next_n=3, lens_2d=lens_2d, max_ctx=1503)
    G.banner(f"uniform next_n=3 2d={lens_2d} fmt={fmt} (max_ctx not a multiple of 4)")
    _check_case(case)


def test_exact_arithmetic():
    """Integer-valued codes, power-of-two scales, weights in (1/8)Z: every sum of
    the plain evaluation is exact in fp32, so the GPU may differ from the oracle
    only by what the matrix core drops in the linear half (tests/_gpu.py,
    MASS_FRAC): this pins indexing, paging, grouping and masking independently
    of the acceptance tolerance."""
    case = syn.make_paged_case([900, 64, 200, 1], [4, 2, 9, 1], seed=400, max_ctx=960)
    G.exactify_fp8_case(case, seed=401)
    G.banner("exact arithmetic fp8")
    gpu = G.run_paged(case)
    G.assert_within_mass(gpu, oracle.paged_logits(case), brute.paged_mass(case), "exact fp8")


def test_exact_arithmetic_fp4():
    case = syn.make_paged_case([500, 33, 96], [3, 1, 5], seed=410, kv_format=1, block_kv=32, max_ctx=512)
    kv = case.kv_cache.numpy()
    sc = kv[:, 32 * 64: 32 * 68]
    live = sc != syn.E8M0_NAN
    # scales 0.5..2, |q| <= 4 and w in (1/8)Z: partial sums stay far below 2^19
    # at a resolution of 2^-5, so they are exact in fp32 in any order
    sc[live] = np.random.default_rng(0).integers(126, 129, live.sum())
    g = torch.Generator().manual_seed(411)
    case.q.copy_(torch.randint(-4, 5, case.q.shape, generator=g).float().to(torch.float8_e4m3fn).view(torch.uint8))
    case.weights.copy_(torch.randint(-32, 33, case.weights.shape, generator=g).float() / 8)
    G.banner("exact arithmetic fp4")
    gpu = G.run_paged(case)
    G.assert_within_mass(gpu, oracle.paged_logits(case), brute.paged_mass(case), "exact fp4")


# --------------------------------------------------------------------------
# invariants on the GPU (bitwise: grouping and paging never change the arithmetic)

def test_grouping_and_worker_count_do_not_change_bits():
    case = syn.make_paged_case([3000, 1200, 64], [5, 2, 9], seed=500, max_ctx=3072)
    t = G.upload(case)
    G.banner("regrouping / worker counts")
    base = G.run_paged(case, t)
    G.assert_logits_close(base, oracle.paged_logits(case), case.weights)
    per_row = torch.arange(case.rows, dtype=torch.int32, device=G.dev())
    np.testing.assert_array_equal(G.run_paged(case, t, indices=per_row), base)
    for W in (1, 5, 97, 2048):
        np.testing.assert_array_equal(G.run_paged(case, t, num_cus=W), base)


def test_schedule_is_read_only_and_shared_by_concurrent_calls():
    """One schedule serves many calls (every layer of a step), concurrent ones
    too: the logits calls only read it. Two calls on two streams that share
    the schedule, each with its own workspace, give the bits of the
    single-stream call, which matches the oracle."""
    case = syn.make_paged_case([9000, 4100, 700, 12000], [3, 1, 6, 2], seed=520, max_ctx=12288)
    other = syn.make_paged_case([9000, 4100, 700, 12000], [3, 1, 6, 2], seed=521, max_ctx=12288)
    t, u = G.upload(case), G.upload(other)
    u["lens"], u["indices"], u["bt"] = t["lens"], t["indices"], t["bt"]  # same rows: same schedule
    kv_u = u["kv"]
    G.banner("schedule shared by two streams, separate workspaces")
    d = G.dev()
    W = 37
    sched = pml.paged_mqa_logits_metadata(t["lens"], case.block_kv, W, indices=t["indices"])
    before = sched.clone()
    ld = pml.logits_ld(case.max_ctx)

    def call(x, kv, out, ws):
        pml.fp8_fp4_paged_mqa_logits(x["q"], kv, x["w"], x["lens"], x["bt"], sched, case.max_ctx, x["indices"],
                                     kv_format=case.kv_format, block_kv=case.block_kv, logits=out, workspace=ws)

    need = pml.logits_workspace_size(case.rows, W)
    ref_a = torch.full((case.rows, ld), G.SENTINEL, dtype=torch.float32, device=d)
    ref_b = torch.full_like(ref_a, G.SENTINEL)
    call(t, t["kv"], ref_a, None)
    call(u, kv_u, ref_b, None)
    torch.cuda.synchronize()
    assert torch.equal(sched, before), "the logits call wrote to the schedule"
    G.assert_logits_close(ref_a[:, : case.max_ctx].cpu().numpy(), oracle.paged_logits(case), case.weights)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        out_a = torch.full_like(ref_a, G.SENTINEL)
        out_b = torch.full_like(ref_a, G.SENTINEL)
        ws_a = torch.full((need,), 0x5A, dtype=torch.uint8, device=d)  # garbage: no initialisation needed
        ws_b = torch.full((need,), 0xA5, dtype=torch.uint8, device=d)
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            call(t, t["kv"], out_a, ws_a)
        with torch.cuda.stream(s2):
            call(u, kv_u, out_b, ws_b)
        torch.cuda.synchronize()
        assert torch.equal(out_a.view(torch.int32), ref_a.view(torch.int32)), f"stream 1, rep {rep}"
        assert torch.equal(out_b.view(torch.int32), ref_b.view(torch.int32)), f"stream 2, rep {rep}"
    assert torch.equal(sched, before)


def test_plain_decode_equals_varlen_arange():
    ctx = [5000, 17, 640, 2049]
    a = syn.make_paged_case(ctx, [1] * 4, seed=510, varlen=False, next_n=1, max_ctx=5120)
    b = syn.make_paged_case(ctx, [1] * 4, seed=510, varlen=True, max_ctx=5120)
    G.banner("plain decode == varlen arange")
    np.testing.assert_array_equal(G.run_paged(a), G.run_paged(b))


def test_padded_uniform_equals_flattened_varlen():
    ctx = [900, 2000, 65]
    a = syn.make_paged_case(ctx, [4] * 3, seed=520, varlen=False, next_n=4, max_ctx=2048)
    b = syn.make_paged_case(ctx, [4] * 3, seed=520, varlen=True, max_ctx=2048)
    c = syn.make_paged_case(ctx, [4] * 3, seed=520, varlen=False, next_n=4, lens_2d=True, max_ctx=2048)
    G.banner("padded uniform == flattened varlen")
    la, lb, lc = G.run_paged(a), G.run_paged(b), G.run_paged(c)
    np.testing.assert_array_equal(la, lb)
    np.testing.assert_array_equal(la, lc)


def test_page_permutation_and_wide_stride():
    case = syn.make_paged_case([1500, 400], [3, 1], seed=530, max_ctx=1536)
    base = G.run_paged(case)
    kv = case.kv_cache.numpy()
    perm = np.random.default_rng(1).permutation(kv.shape[0])
    inv = np.argsort(perm)
    wide = np.full((kv.shape[0], kv.shape[1] + 256), 0x7F, dtype=np.uint8)
    wide[:, : kv.shape[1]] = kv[perm]
    bt = case.block_table.numpy()
    bt2 = np.where(bt >= 0, inv[np.maximum(bt, 0)], -1).astype(np.int32)
    c2 = syn.PagedCase(**{**case.__dict__, "kv_cache": torch.from_numpy(wide), "block_table": torch.from_numpy(bt2)})
    G.banner("page permutation + stride")
    np.testing.assert_array_equal(G.run_paged(c2), base)


def test_rows_are_independent():
    case = syn.make_paged_case([800, 300, 1000], [2, 1, 3], seed=540, max_ctx=1024)
    base = G.run_paged(case)
    keep = [0, 4, 5]                         # drop rows: every kept row is its own group
    sub = syn.PagedCase(**{**case.__dict__, "q": case.q[keep].clone(), "weights": case.weights[keep].clone(),
                           "context_lens": case.context_lens[keep].clone(),
                           "indices": torch.arange(3, dtype=torch.int32),
                           "block_table": case.block_table[keep].clone()})
    G.banner("row independence")
    np.testing.assert_array_equal(G.run_paged(sub), base[keep])


# --------------------------------------------------------------------------
# edge cases

def test_empty_rows_and_bad_table_entries():
    case = syn.make_paged_case([0, 200, 0, 70], [1, 2, 1, 1], seed=600, max_ctx=256)
    G.banner("empty rows")
    gpu = _check_case(case)
    assert np.all(np.isneginf(gpu[0])) and np.all(np.isneginf(gpu[3]))
    # a visible block whose table entry is out of range scores NaN, others unaffected
    bt = case.block_table.clone()
    bt[1, 1] = 10 ** 6
    bt[2, 1] = -5
    c2 = syn.PagedCase(**{**case.__dict__, "block_table": bt})
    G.banner("bad table entry")
    g2 = G.run_paged(c2)
    assert np.all(np.isnan(g2[1, 64:128])) and np.all(np.isnan(g2[2, 64:128]))
    np.testing.assert_array_equal(g2[1, :64], gpu[1, :64])
    np.testing.assert_array_equal(g2[1, 128:], gpu[1, 128:])


def test_no_rows_is_a_no_op():
    d = G.dev()
    lens = torch.zeros(0, dtype=torch.int32, device=d)
    sched = pml.paged_mqa_logits_metadata(lens, 64, 8)
    assert sched.cpu().numpy().tolist() == [[0, 0]] * 9
    out = pml.fp8_fp4_paged_mqa_logits(torch.zeros(0, 64, 128, dtype=torch.uint8, device=d),
                                       torch.zeros(1, 64 * 132, dtype=torch.uint8, device=d),
                                       torch.zeros(0, 64, device=d), lens,
                                       torch.zeros(0, 1, dtype=torch.int32, device=d), sched, 64)
    torch.cuda.synchronize()
    assert out.shape[0] == 0


# --------------------------------------------------------------------------
# the named workloads at full size

def test_uniform_decode_config_full():
    case = syn.config_uniform_decode()
    G.banner(f"uniform decode B=64 full parity ({syn.scored_pairs(case)} pairs)")
    _check_case(case)


def _full(name):
    """Every row of a named workload against the oracle, element by element."""
    case = G.named_case(name)
    G.banner(f"{name}: all {case.rows} rows ({syn.scored_pairs(case)} pairs)")
    gpu = G.run_paged(case)
    G.check_whole_output(gpu, case)
    G.assert_logits_close(gpu, G.oracle_full(name), case.weights, name)


def test_varlen_fp8_config_full():
    _full("varlen_fp8")


def test_varlen_fp4_config_full():
    _full("varlen_fp4")
