"""Per-row top-k on the GPU.

* On shared input (the same fp32 logits on both sides) the selected set must
  equal the oracle's bit for bit, ties included.
* Against the oracle's fp64 logits the top-k acceptance holds: every
  selected index scores at least t_k - tau, every index scoring above t_k + tau
  is selected, and min(k, width) distinct in-range entries come first.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_mqa_logits_amd as pml
import pml_synth as syn
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def gpu_topk(logits: torch.Tensor, ke: torch.Tensor, k: int, ks=None, next_n=1) -> np.ndarray:
    res = pml.top_k_per_row(logits, ke, k, ks=ks, next_n=next_n)
    torch.cuda.synchronize()
    return res.cpu().numpy()


def _shared_input_check(logits_np: np.ndarray, ke: np.ndarray, k: int, ks=None, next_n=1):
    d = G.dev()
    lt = torch.from_numpy(np.ascontiguousarray(logits_np, dtype=np.float32)).to(d)
    ket = torch.from_numpy(np.asarray(ke, dtype=np.int32)).to(d)
    kst = None if ks is None else torch.from_numpy(np.asarray(ks, dtype=np.int32)).to(d)
    got = gpu_topk(lt, ket, k, kst, next_n)
    if next_n > 1:
        r = np.arange(logits_np.shape[0])
        ke = np.asarray(ke)[r // next_n] - next_n + (r % next_n) + 1
    want = oracle.topk(logits_np.astype(np.float32).astype(np.float64), ke, k, ks=ks)
    np.testing.assert_array_equal(got, want)
    return got


def test_adversarial_rows():
    rng = np.random.default_rng(800)
    W = 5000
    rows = []
    rows.append(np.zeros(W))                                  # all equal
    rows.append(np.round(rng.standard_normal(W)))             # many ties
    r = rng.standard_normal(W)
    r[::3] = 0.0
    r[1::3] = -0.0                                            # +-0 are equal
    rows.append(r)
    r = rng.standard_normal(W)
    r[100:] = -np.inf                                         # -inf tail
    rows.append(r)
    rows.append(np.full(W, -np.inf))
    rows.append(rng.standard_normal(W) * 1e-30)               # subnormal-ish spread
    r = rng.standard_normal(W)
    r[7] = np.nan                                             # NaN ranks lowest
    rows.append(r)
    rows.append(np.arange(W, dtype=np.float64)[::-1].copy())  # descending
    r = rng.standard_normal(W)
    r[rng.random(W) < 0.7] = np.nan                           # the k-th among the NaNs
    rows.append(r)
    rows.append(np.full(W, np.nan))                           # all NaN
    r = np.full(W, -np.inf)
    r[rng.random(W) < 0.5] = np.nan                           # -inf above NaN
    rows.append(r)
    L = np.stack(rows)
    n = L.shape[0]
    G.banner("top-k adversarial")
    for k, ke in ((1, [W] * n), (64, [W] * n), (2048, [W] * n), (4096, [W] * n),
                  (100, [100, 99, 101, 50, 0, 100, 5000, 1, 4999, 257, 256]),
                  (2048, [5000, 4097, 2049, 4000, 3000, 2300, 4999, 2048, 4095, 4096, 2500])):
        _shared_input_check(L, ke, k)


def test_bounds_and_next_n():
    rng = np.random.default_rng(810)
    L = rng.standard_normal((12, 9000)).astype(np.float32)
    ks = rng.integers(0, 3000, 12)
    ke = ks + rng.integers(0, 6000, 12)
    ke[0] = ks[0]          # empty
    ke[1] = ks[1] + 64     # width == k
    G.banner("top-k ks/ke")
    _shared_input_check(L, ke, 64, ks=ks)
    G.banner("top-k next_n=3")
    _shared_input_check(L, rng.integers(100, 9000, 4), 333, next_n=3)


def test_wide_rows_streaming_list_and_fallback():
    """Rows wider than the in-LDS list: the sampled path for rows of 16K+
    columns, the exact streaming passes for the narrower rows of the launch
    (10000 .. 12289 wide) and wherever the sample misjudges (ties, one wave's
    region overflowing), and the passes over the row when ties overflow the
    list."""
    rng = np.random.default_rng(830)
    W = 40000
    rows = [rng.standard_normal(W),                     # streaming, few candidates
            np.zeros(W),                                # every key equal: list overflows
            np.round(rng.standard_normal(W) * 2),       # heavy ties
            np.concatenate([rng.standard_normal(9000), np.full(W - 9000, -np.inf)]),
            rng.standard_normal(W) * 1e3,
            np.arange(W, dtype=np.float64)]             # ascending: the top is at the end
    r = rng.standard_normal(W)
    r[17000:19100] = 50.0                               # one wave's candidates overflow its region
    rows.append(r)
    L = np.stack(rows)
    G.banner("top-k wide rows")
    for k, ke in ((1, [W] * 7), (2048, [W] * 7), (4096, [W] * 7),
                  (2048, [10000, 12288, 12289, 40000, 30001, 39999, 40000])):
        _shared_input_check(L, ke, k)
    ks = np.array([0, 5, 100, 3, 17, 20000, 1])
    _shared_input_check(L, np.full(7, W), 777, ks=ks)


def test_sampled_path_rows():
    """Rows of 16K columns or more: a sampled bucket, then one append pass into
    per-wave regions (fast path); a cluster of large values that overflows one
    wave's region, and heavy ties, fall back to the exact passes."""
    rng = np.random.default_rng(840)
    W = 70000
    rows = [rng.standard_normal(W),                       # fast path
            np.arange(W, dtype=np.float64),               # ascending: all candidates at the end
            np.zeros(W),                                  # ties: region overflow, then list overflow
            np.round(rng.standard_normal(W) * 3)]         # coarse ties
    r = rng.standard_normal(W)
    r[30000:36000:4] = 1000.0                            # 1500 large values inside one wave's span
    rows.append(r)
    r = rng.standard_normal(W) * 1e-3
    r[::5000] = 5.0                                      # 14 isolated large values among tiny ones
    rows.append(r)
    L = np.stack(rows)
    n = L.shape[0]
    G.banner("top-k sampled path")
    for k, ke in ((1, [W] * n), (2048, [W] * n), (4096, [W] * n), (100, [65536, 65535, W, 69999, 66000, W])):
        _shared_input_check(L, ke, k)
    ks = np.array([0, 3, 4000, 1, 2, 0])
    _shared_input_check(L, np.full(n, W), 2048, ks=ks)


def test_sampled_path_float_threshold():
    """The sampled append tests candidates with one float compare against the
    float whose order key opens the picked bucket. Rows where that bucket lies
    among negative values, exactly at +-0, among subnormals, or at or below
    -inf (where the key compare is kept) must select exactly as the oracle."""
    rng = np.random.default_rng(850)
    W = 70000
    rows = [-np.abs(rng.standard_normal(W)) - 1.0]          # all negative: bucket among negatives
    r = rng.standard_normal(W)
    r[r > 0] = 0.0
    r[rng.random(W) < 0.5] *= -1.0                           # many +0 / -0 at the top
    rows.append(r)
    rows.append(rng.standard_normal(W) * 1e-39)              # subnormals
    r = np.full(W, -np.inf)
    r[::50] = rng.standard_normal(W // 50 + 1)[: len(r[::50])]  # 1400 finite values, the rest -inf
    rows.append(r)
    r = rng.standard_normal(W)
    r[rng.random(W) < 0.7] = np.nan                          # NaN-heavy
    rows.append(r)
    r = -np.abs(rng.standard_normal(W)) * 1e30
    r[::3] = -np.inf                                         # huge negatives and -inf
    rows.append(r)
    L = np.stack(rows)
    n = L.shape[0]
    G.banner("top-k sampled path, float threshold cases")
    for k in (1, 64, 2048, 4096):
        _shared_input_check(L, [W] * n, k)
    _shared_input_check(L, [W, 69999, 65536, W, 66001, 68000], 1500)


def _acceptance(gpu: np.ndarray, ref: np.ndarray, lo: np.ndarray, hi: np.ndarray, k: int, wsum: np.ndarray):
    for r in range(gpu.shape[0]):
        n = max(0, int(hi[r] - lo[r]))
        m = min(k, n)
        sel = gpu[r, :m]
        assert np.all(gpu[r, m:] == -1)
        assert len(np.unique(sel)) == m and np.all((sel >= 0) & (sel < n))
        if n <= k:
            continue
        sc = ref[r, lo[r]: hi[r]]
        tk = np.sort(sc)[::-1][k - 1]
        tau = 2e-3 * abs(tk) + 1e-3 * wsum[r]
        assert np.all(sc[sel] >= tk - tau)
        must = np.nonzero(sc > tk + tau)[0]
        assert np.all(np.isin(must, sel))


@pytest.mark.parametrize("name", ["tiny_decode", "varlen_fp8"])
def test_decode_configs_topk(name):
    case = G.named_case(name)
    G.banner(f"top-k decode {name} rows={case.rows} k={case.topk}")
    t = G.upload(case)
    sched = pml.paged_mqa_logits_metadata(t["lens"], case.block_kv, None, indices=t["indices"])
    logits = pml.fp8_fp4_paged_mqa_logits(t["q"], t["kv"], t["w"], t["lens"], t["bt"], sched, case.max_ctx,
                                          t["indices"], kv_format=case.kv_format, block_kv=case.block_kv)
    got = pml.top_k_per_row(logits, t["lens"], case.topk, max_width=case.max_ctx)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    L = logits.cpu().numpy()[:, : case.max_ctx]
    vis = oracle.visible_lengths(case)
    # shared input: bit-exact
    np.testing.assert_array_equal(got, oracle.topk(L.astype(np.float64), vis, case.topk))
    # every row against the fp64 oracle logits
    ref = G.oracle_full(name)
    G.topk_acceptance(got, ref, vis, case.topk, np.abs(case.weights.double().numpy()).sum(1))


def test_prefill_topk_sampled():
    case = syn.make_ragged_case([3000, 2500], seed=820)
    d = G.dev()
    G.banner("top-k prefill")
    logits = pml.mqa_logits(case.q.to(d), case.k.to(d), case.k_scale.to(d), case.weights.to(d),
                            case.ks.to(d), case.ke.to(d))
    got = pml.top_k_per_row(logits, case.ke.to(d), 2048, ks=case.ks.to(d), max_width=case.N)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    L = logits.cpu().numpy()[:, : case.N].astype(np.float64)
    ks, ke = case.ks.numpy(), case.ke.numpy()
    np.testing.assert_array_equal(got, oracle.topk(L, ke, 2048, ks=ks))
    rows = np.array([0, 1, 2047, 2048, 2049, 2999, 3000, 4500, 5499])
    ref = oracle.ragged_logits(case, rows=rows)
    _acceptance(got[rows], ref, ks[rows], ke[rows], 2048, np.abs(case.weights[rows].double().numpy()).sum(1))


@pytest.mark.parametrize("width", [32768, 65536, 131072])
def test_wide_rows_patterns(width):
    """Wide rows of several shapes (normal, ties, -inf / NaN mixed in, ascending, all
    equal, tiny values) through the sampled path and its fallbacks, bit for bit."""
    rng = np.random.default_rng(width)
    rows = []
    rows.append(rng.standard_normal(width))                       # normal
    rows.append(np.round(rng.standard_normal(width) * 2))         # ties across segments
    r = rng.standard_normal(width)
    r[::7] = -np.inf
    r[3::11] = np.nan
    rows.append(r)                                                # -inf and NaN mixed in
    rows.append(np.arange(width, dtype=np.float64))               # ascending
    rows.append(np.zeros(width))                                  # all equal: the list overflows
    rows.append(rng.standard_normal(width) * 1e-30)               # tiny values
    L = np.stack(rows).astype(np.float32)
    d = G.dev()
    lt = torch.from_numpy(L).to(d)
    ke = np.array([width, width, width - 5, width, width, width - 100], dtype=np.int32)
    kt = torch.from_numpy(ke).to(d)
    for k in (64, 2048, 4096):
        G.banner(f"wide-row top-k width={width} k={k}")
        got = pml.top_k_per_row(lt, kt, k, max_width=width)
        torch.cuda.synchronize()
        want = oracle.topk(L.astype(np.float64), ke, k)
        np.testing.assert_array_equal(got.cpu().numpy(), want)


def test_wide_rows_offsets_and_edges():
    """The sampled path with row spans that start anywhere (unaligned ks), spans from
    16K (the sample is the whole span) to 40K, a row that is mostly -inf (the bucket
    falls to -inf and the append compares order keys), and globally descending
    rows (each wave's first round over-estimates the threshold), bit for bit."""
    rng = np.random.default_rng(4242)
    ld = 48000
    widths = [16384, 16385, 17000, 20000, 33001, 40000, 24000, 30000]
    ks = np.array([0, 1, 3, 5000, 7, 2, 13, 4097], dtype=np.int32)
    ke = ks + np.array(widths, dtype=np.int32)
    L = rng.standard_normal((len(widths), ld)).astype(np.float32) * 3
    L[2] = -np.inf
    L[2, rng.choice(ld, 3000, replace=False)] = rng.standard_normal(3000)  # 3000 finite values
    L[3] = np.linspace(5, -5, ld, dtype=np.float32)                           # descending
    L[6] = np.round(L[6])                                                       # heavy ties
    L[7, ks[7]: ke[7]] = np.linspace(-1, 1, widths[7], dtype=np.float32)[::-1]  # descending span
    d = G.dev()
    lt = torch.from_numpy(L).to(d)
    for k in (1, 2048, 4096):
        G.banner(f"wide-row top-k with offsets k={k}")
        got = pml.top_k_per_row(lt, torch.from_numpy(ke).to(d), k, ks=torch.from_numpy(ks).to(d),
                                max_width=max(widths))
        torch.cuda.synchronize()
        want = oracle.topk(L.astype(np.float64), ke, k, ks=ks)
        np.testing.assert_array_equal(got.cpu().numpy(), want)


@pytest.mark.parametrize("width", [65536, 131072])
def test_wide_rows_fine_ties(width):
    """Values on a 2^-10 grid: the list's keys repeat about a dozen times each, so
    the bins the selection picks are small but hold ties at the k-th value (the
    one-wave finish then takes only some of the equal keys, the lower positions)."""
    rng = np.random.default_rng(width + 7)
    rows = 6
    L = (np.round(rng.standard_normal((rows, width)) * 1024) / 1024).astype(np.float32)
    L[1] = np.round(L[1] * 64) / 64          # coarser grid: larger tie groups
    n3 = width // 3
    L[2, 0:3 * n3:3] = L[2, 1:3 * n3:3]       # pairs of equal values side by side
    ke = np.array([width, width - 1, width, width - 333, width, width - 4096], dtype=np.int32)
    d = G.dev()
    lt = torch.from_numpy(L).to(d)
    for k in (2048, 4096, 777):
        G.banner(f"wide-row fine ties width={width} k={k}")
        got = pml.top_k_per_row(lt, torch.from_numpy(ke).to(d), k, max_width=width)
        torch.cuda.synchronize()
        want = oracle.topk(L.astype(np.float64), ke, k)
        np.testing.assert_array_equal(got.cpu().numpy(), want)
