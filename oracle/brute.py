"""Second, numpy-only formulation of the scores for tiny inputs (test infrastructure).

It decodes the number formats with numpy bit arithmetic (not the C oracle's
functions), gathers each row's visible keys through the block table into a
dense matrix and scores them with ``einsum`` in float64. It is written
independently of ``oracle.c`` so that the two cross-check each other.
"""
from __future__ import annotations

import numpy as np


def fp8_e4m3_np(codes: np.ndarray) -> np.ndarray:
    """OCP E4M3fn by bit fields: (-1)^s * 2^(e-7) * (1 + m/8), subnormal m/8 * 2^-6."""
    c = codes.astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    v = np.where((e == 15) & ((c & 7) == 7), np.nan, v)
    return s * v


def e2m1_np(nib: np.ndarray) -> np.ndarray:
    """OCP MX E2M1 by bit fields: (-1)^s * 2^(e-1) * (1 + m/2), subnormal m/2."""
    c = nib.astype(np.int64)
    s = np.where(c & 8, -1.0, 1.0)
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    return s * np.where(e == 0, m / 2.0, (1.0 + m / 2.0) * np.exp2(e - 1.0))


def e8m0_np(code: np.ndarray) -> np.ndarray:
    c = code.astype(np.int64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def dequant_page_tokens(case, page: int) -> np.ndarray:
    """All block_kv tokens of one page as float64 [block_kv, D]."""
    kv = case.kv_cache.numpy()
    B, D = case.block_kv, case.D
    p = kv[page]
    if case.kv_format == 0:
        vals = fp8_e4m3_np(p[: B * D].reshape(B, D))
        scale = p[B * D: B * D + 4 * B].copy().view(np.float32).astype(np.float64)
        return vals * scale[:, None]
    packed = p[: B * D // 2].reshape(B, D // 2)
    nib = np.empty((B, D), dtype=np.uint8)
    nib[:, 0::2] = packed & 15
    nib[:, 1::2] = packed >> 4
    sc = p[B * D // 2: B * D // 2 + B * D // 32].reshape(B, D // 32)
    return e2m1_np(nib) * np.repeat(e8m0_np(sc), 32, axis=1)


def q_dequant(case) -> np.ndarray:
    """q as float64 [rows, H, D]: fp8 codes, or packed e2m1 times per-32 e8m0 scales."""
    if getattr(case, "q_scale", None) is None:
        return fp8_e4m3_np(case.q.numpy())
    packed = case.q.numpy()                          # [rows, H, D/2]
    rows, H, half = packed.shape
    nib = np.empty((rows, H, 2 * half), dtype=np.uint8)
    nib[..., 0::2] = packed & 15
    nib[..., 1::2] = packed >> 4
    return e2m1_np(nib) * np.repeat(e8m0_np(case.q_scale.numpy()), 32, axis=2)


def paged_logits(case) -> np.ndarray:
    """Dense [rows, max_ctx] float64 logits by gather + einsum."""
    q = q_dequant(case)                              # [rows, H, D]
    w = case.weights.numpy().astype(np.float64)      # [rows, H]
    lens = case.context_lens.numpy().astype(np.int64)
    bt = case.block_table.numpy()
    rows, nn = case.rows, case.next_n
    out = np.full((rows, case.max_ctx), -np.inf)
    for r in range(rows):
        if case.lens_2d or nn == 1:
            vis = lens.reshape(-1)[r]
        else:
            vis = lens[r // nn] - nn + (r % nn) + 1
        vis = max(0, int(vis))
        if vis == 0:
            continue
        nblk = -(-vis // case.block_kv)
        K = np.concatenate([dequant_page_tokens(case, int(bt[r // nn, b])) for b in range(nblk)])[:vis]
        dots = np.einsum("hd,sd->hs", q[r], K)
        out[r, :vis] = np.einsum("h,hs->s", w[r], np.maximum(dots, 0.0))
    return out


def ragged_logits(case) -> np.ndarray:
    q = fp8_e4m3_np(case.q.numpy())
    w = case.weights.numpy().astype(np.float64)
    K = fp8_e4m3_np(case.k.numpy()) * case.k_scale.numpy().astype(np.float64)[:, None]
    ks = case.ks.numpy()
    ke = case.ke.numpy()
    out = np.full((case.M, case.N), -np.inf)
    for r in range(case.M):
        a, b = int(ks[r]), int(ke[r])
        if b > a:
            dots = np.einsum("hd,sd->hs", q[r], K[a:b])
            out[r, a:b] = w[r] @ np.maximum(dots, 0.0)
    return out


def topk(scores: np.ndarray, ke, k: int, ks=None) -> np.ndarray:
    """lexsort by (value desc, index asc); positions relative to ks, ascending, -1 padded."""
    rows = scores.shape[0]
    out = np.full((rows, k), -1, dtype=np.int32)
    for r in range(rows):
        ld = scores.shape[1]
        lo = 0 if ks is None else min(max(int(ks[r]), 0), ld)  # bounds clamped into the row
        hi = min(max(int(ke[r]), lo), ld)
        v = scores[r, lo:hi].astype(np.float64)
        idx = np.arange(len(v))
        order = np.lexsort((idx, -v))
        sel = np.sort(order[:k])
        out[r, : len(sel)] = sel
    return out


def dcp_tokens(T: int, world: int, interleave: int) -> list:
    """Global ids held by each rank, in local order, by dealing runs of ``interleave`` tokens in turn."""
    held = [[] for _ in range(world)]
    run, t = 0, 0
    while t < T:
        for _ in range(interleave):
            if t < T:
                held[run % world].append(t)
                t += 1
        run += 1
    return held


def dcp_merge(gathered: np.ndarray, k: int) -> np.ndarray:
    """lexsort over every rank's valid pairs by (score desc, NaN last, id asc); ids ascending, -1 padded."""
    world, rows = gathered.shape[0], gathered.shape[1]
    out = np.full((rows, k), -1, dtype=np.int32)
    for r in range(rows):
        pairs = gathered[:, r].reshape(-1, 2).astype(np.float64)
        ok = (pairs[:, 1] >= 0) & (pairs[:, 1] < 2 ** 24)
        v, ids = pairs[ok, 0], np.trunc(pairs[ok, 1]).astype(np.int64)
        order = np.lexsort((ids, -v))
        sel = np.sort(ids[order[:k]])
        out[r, : len(sel)] = sel
    return out


def _row_keys(case, r: int):
    """Row r's visible keys, dequantised, as float64 [vis, D] (block-table gather)."""
    lens = case.context_lens.numpy().astype(np.int64)
    bt = case.block_table.numpy()
    nn = case.next_n
    vis = lens.reshape(-1)[r] if (case.lens_2d or nn == 1) else lens[r // nn] - nn + (r % nn) + 1
    vis = max(0, int(vis))
    if vis == 0:
        return np.zeros((0, case.D))
    nblk = -(-vis // case.block_kv)
    return np.concatenate([dequant_page_tokens(case, int(bt[r // nn, b])) for b in range(nblk)])[:vis]


def paged_mass(case) -> np.ndarray:
    """Absolute mass of every score, sum_h |w[r,h]| sum_d |q[r,h,d]| |k[s,d]|, as
    float64 [rows, max_ctx] (0 where masked): the sum of the magnitudes of all
    the products the score adds, the scale of any rounding in its evaluation."""
    q = np.abs(q_dequant(case))
    w = np.abs(case.weights.numpy().astype(np.float64))
    out = np.zeros((case.rows, case.max_ctx))
    for r in range(case.rows):
        K = np.abs(_row_keys(case, r))
        if len(K):
            out[r, : len(K)] = K @ (w[r] @ q[r])
    return out


def ragged_mass(case) -> np.ndarray:
    """paged_mass for a ragged case: [M, N], 0 outside [ks, ke)."""
    q = np.abs(fp8_e4m3_np(case.q.numpy()))
    w = np.abs(case.weights.numpy().astype(np.float64))
    K = np.abs(fp8_e4m3_np(case.k.numpy()) * case.k_scale.numpy().astype(np.float64)[:, None])
    out = np.zeros((case.M, case.N))
    for r in range(case.M):
        a, b = max(0, int(case.ks[r])), min(case.N, int(case.ke[r]))
        if b > a:
            out[r, a:b] = K[a:b] @ (w[r] @ q[r])
    return out
