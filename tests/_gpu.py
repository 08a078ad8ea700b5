"""Helpers of the GPU parity tests: upload seeded cases, call the HIP path
through the binding and compare with the CPU oracle (test infrastructure)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import paged_mqa_logits_amd as pml
import pml_synth as syn

SENTINEL = 12345.0  # prefilled into output buffers: any cell left unwritten shows up

# Acceptance of a logit: |gpu - oracle| <= REL * |oracle| + ABS * sum_h |w[r, h]|
REL = 2e-3
ABS = 1e-3

# bf16 logits: the fp32 logit x = oracle + e, |e| <= REL |oracle| + ABS S, is
# rounded to nearest bf16, which adds at most u |x| with u = 2^-8 (half a unit in
# the 8th significant bit). So |bf16(x) - oracle| <= u (|oracle| + |e|) + |e|
# <= (u + REL (1 + u)) |oracle| + ABS (1 + u) S.
U_BF16 = 2.0 ** -8
REL_BF16 = U_BF16 + REL * (1 + U_BF16)
ABS_BF16 = ABS * (1 + U_BF16)
SENTINEL_BF16 = 0x1234  # bf16 bits prefilled into output buffers


def dev():
    return torch.device("cuda:0")


def banner(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)


def upload(case: syn.PagedCase) -> dict:
    d = dev()
    return dict(
        q=case.q.to(d), kv=case.kv_cache.to(d), w=case.weights.to(d), lens=case.context_lens.to(d),
        bt=case.block_table.to(d), indices=None if case.indices is None else case.indices.to(d),
        qs=None if case.q_scale is None else case.q_scale.to(d))


def run_paged(case: syn.PagedCase, t: dict | None = None, *, num_cus=None, indices="case",
              ld=None) -> np.ndarray:
    """GPU logits [rows, max_ctx] as float32 numpy (checks the sentinel columns past max_ctx)."""
    t = t or upload(case)
    idx = t["indices"] if indices == "case" else indices
    sched = pml.paged_mqa_logits_metadata(t["lens"], case.block_kv, num_cus, indices=idx,
                                          next_n=case.next_n)
    ld = ld or pml.logits_ld(case.max_ctx)
    out = torch.full((case.rows, ld), SENTINEL, dtype=torch.float32, device=dev())
    pml.fp8_fp4_paged_mqa_logits(t["q"], t["kv"], t["w"], t["lens"], t["bt"], sched, case.max_ctx, idx,
                                 kv_format=case.kv_format, block_kv=case.block_kv, next_n=case.next_n,
                                 logits=out, q_scale=t["qs"])
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[:, case.max_ctx:] == SENTINEL), "columns past max_ctx were written"
    return o[:, : case.max_ctx]


def run_paged_bf16(case: syn.PagedCase, t: dict | None = None, *, ld=None, sched=None) -> np.ndarray:
    """GPU bf16 logits [rows, max_ctx] as uint16 bits (checks the sentinel columns past max_ctx)."""
    t = t or upload(case)
    if sched is None:
        sched = pml.paged_mqa_logits_metadata(t["lens"], case.block_kv, None, indices=t["indices"],
                                              next_n=case.next_n)
    ld = ld or (case.max_ctx + 7) // 8 * 8 + 8
    out = torch.full((case.rows, ld), SENTINEL_BF16, dtype=torch.int16, device=dev()).view(torch.bfloat16)
    pml.fp8_fp4_paged_mqa_logits(t["q"], t["kv"], t["w"], t["lens"], t["bt"], sched, case.max_ctx, t["indices"],
                                 kv_format=case.kv_format, block_kv=case.block_kv, next_n=case.next_n, logits=out)
    torch.cuda.synchronize()
    o = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.all(o[:, case.max_ctx:] == SENTINEL_BF16), "columns past max_ctx were written"
    return o[:, : case.max_ctx]


def abs_tol(weights: torch.Tensor, a: float = ABS) -> np.ndarray:
    return a * np.abs(weights.double().numpy()).sum(axis=1)


def assert_logits_close(gpu: np.ndarray, ref: np.ndarray, weights_rows: torch.Tensor, what: str = "",
                        rel: float = REL, abs_: float = ABS) -> None:
    """The acceptance bar: masked cells exactly -inf, the rest within tolerance."""
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert not np.any(gpu == SENTINEL), f"{what}: unwritten cells"
    masked = np.isneginf(ref)
    bad_mask = masked != np.isneginf(gpu)
    assert not bad_mask.any(), f"{what}: -inf pattern differs at {np.argwhere(bad_mask)[:5]}"
    assert not np.isnan(ref).any(), f"{what}: oracle produced NaN"
    fin = ~masked
    tol = rel * np.abs(ref) + abs_tol(weights_rows, abs_)[:, None]
    err = np.abs(gpu.astype(np.float64) - ref)
    bad = fin & ~(err <= tol)
    if fin.any():
        ratio = float(np.max(np.where(fin, err / tol, 0.0)))
        print(f"[gpu-check] {what or 'logits'}: max err/tol {ratio:.3g} over {int(fin.sum())} cells", flush=True)
    if bad.any():
        i = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} cells out of tolerance, e.g. {[(tuple(x), gpu[tuple(x)], ref[tuple(x)]) for x in i]}")


# Exactly representable inputs (exactify_*): every product and partial sum of
# the plain evaluation is exact in fp32, but the linear half of the score runs
# on the matrix core as <sum_h w_h q_h, k>, and the fp8 MFMA may drop low bits
# of products far below the largest in a dot product (by up to about 1e-4 of
# the dot product's sum of |products|, measured on full-range random operands).
# That sum is at most the cell's absolute mass (oracle.brute.paged_mass), and the
# linear half enters the score with a factor 1/2, so such cells must match the
# oracle within MASS_FRAC of their mass: far below the acceptance tolerance, and
# far below what a wrong index, page or mask produces.
MASS_FRAC = 2.0 ** -14


def assert_within_mass(gpu: np.ndarray, ref: np.ndarray, mass: np.ndarray, what: str = "",
                       frac: float = MASS_FRAC, rel: float = 0.0) -> None:
    """Masked cells exactly -inf; others |gpu - ref| <= frac * mass + rel * |ref|."""
    assert gpu.shape == ref.shape == mass.shape, (gpu.shape, ref.shape, mass.shape)
    assert not np.any(gpu == SENTINEL), f"{what}: unwritten cells"
    masked = np.isneginf(ref)
    bad_mask = masked != np.isneginf(gpu)
    assert not bad_mask.any(), f"{what}: -inf pattern differs at {np.argwhere(bad_mask)[:5]}"
    fin = ~masked
    err = np.where(fin, np.abs(gpu.astype(np.float64) - np.where(fin, ref, 0.0)), 0.0)
    bound = frac * mass + rel * np.abs(np.where(fin, ref, 0.0))
    if fin.any():
        ratio = float(np.max(np.where(fin, err / np.maximum(mass, 1e-300), 0.0)))
        print(f"[gpu-check] {what or 'logits'}: max err/mass {ratio:.3g} over {int(fin.sum())} cells, "
              f"{int((fin & (err > 0)).sum())} inexact", flush=True)
    bad = fin & ~(err <= bound)
    if bad.any():
        i = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} cells beyond the mass bound, e.g. "
                             f"{[(tuple(x), gpu[tuple(x)], ref[tuple(x)], mass[tuple(x)]) for x in i]}")


def exactify_fp8_case(case: syn.PagedCase, seed: int) -> None:
    """Make every product and partial sum exact in fp32: integer fp8 codes in
    [-8, 8], power-of-two scales 2^-4..2^2 and weights in (1/8)Z within [-4, 4]
    (valid key slots only; NaN codes of unused slots are kept)."""
    g = torch.Generator().manual_seed(seed)
    qv = torch.randint(-8, 9, case.q.shape, generator=g).float()
    case.q.copy_(qv.to(torch.float8_e4m3fn).view(torch.uint8))
    case.weights.copy_(torch.randint(-32, 33, case.weights.shape, generator=g).float() / 8)
    kv = case.kv_cache.numpy()
    B, D = case.block_kv, case.D
    vals = kv[:, : B * D]
    live = vals != syn.FP8_NAN
    ints = torch.randint(-8, 9, vals.shape, generator=g).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    vals[live] = ints[live]
    sc = kv[:, B * D: B * D + 4 * B].view(np.float32)
    e = torch.randint(-4, 3, sc.shape, generator=g).numpy().astype(np.float32)
    sc[~np.isnan(sc)] = np.exp2(e)[~np.isnan(sc)]


def oracle_rows(case, rows) -> np.ndarray:
    return oracle.paged_logits(case, rows=np.asarray(rows))


_NAMED = {
    "tiny_decode": syn.config_tiny_decode,
    "uniform_decode": syn.config_uniform_decode,
    "varlen_fp8": syn.config_varlen_fp8,
    "varlen_fp4": syn.config_varlen_fp4,
    "varlen_fp4_q4": lambda: syn.config_varlen_fp4(q_fp4=True),
}
_CASES = {}
_FULL = {}


def named_case(name: str):
    """A named workload, generated once per test session (callers must not modify it)."""
    if name not in _CASES:
        _CASES[name] = _NAMED[name]()
    return _CASES[name]


def oracle_full(name: str) -> np.ndarray:
    """fp64 oracle logits of every row of a named workload, computed once per session."""
    if name not in _FULL:
        _FULL[name] = oracle.paged_logits(named_case(name))
    return _FULL[name]


def check_whole_output(gpu: np.ndarray, case) -> np.ndarray:
    """-inf exactly past each row's visible length (the oracle's rule), finite before it."""
    vis = oracle.visible_lengths(case)
    cols = np.arange(gpu.shape[1])[None, :]
    assert np.all(np.isneginf(gpu[cols >= vis[:, None]]))
    assert np.all(np.isfinite(gpu[cols < vis[:, None]]))
    return vis


def topk_acceptance(sel: np.ndarray, ref: np.ndarray, vis, k: int, wsum, rel: float = REL, abs_: float = ABS,
                    factor: float = 1.0) -> None:
    """The top-k acceptance against fp64 scores, row by row: every selected
    index scores at least the oracle's k-th score minus tau, every score above
    the k-th plus tau is selected (tau the per-logit tolerance at the k-th
    score, times factor), and the selection has min(k, vis) distinct valid
    indices followed by -1."""
    for i in range(ref.shape[0]):
        n = int(vis[i])
        m = min(k, n)
        s = sel[i]
        assert np.all(s[m:] == -1), i
        got = s[:m]
        assert np.all((got >= 0) & (got < n)) and len(np.unique(got)) == m, i
        if m == 0:
            continue
        sc = ref[i, :n]
        tk = np.sort(sc)[::-1][m - 1]
        tau = factor * (rel * abs(tk) + abs_ * wsum[i])
        assert np.all(sc[got] >= tk - tau), i
        assert np.all(np.isin(np.nonzero(sc > tk + tau)[0], got)), i
