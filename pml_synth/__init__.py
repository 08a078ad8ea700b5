"""Seeded synthetic inputs for the paged MQA-logits path.

This module builds inputs only: query codes, key-cache pages, block tables,
lengths, request ids and weights. It holds none of the scoring arithmetic and
is imported by both the CPU oracle's tests and the GPU path's tests and bench,
so that both sides see byte-identical inputs.

Workloads follow the shapes the indexer pages describe for DeepSeek-style
sparse-attention decode ("[Attention][DSA] Route SM100 sparse-indexer decode
through varlen paged MQA logits", Purpose; "[Bugfix][GLM-5.3-Flash] Fix
fp8_fp4_paged_mqa_logits ... speculative decode", Test Plan: 120K context,
batch 40, speculative steps) with H = 64 heads and D = 128.

Recipes (all random draws come from one seeded ``torch.Generator`` on the CPU):

* q  = fp8_e4m3fn(clamp(N(0,1), +-448))            [rows, H, D]
  or, with q_fp4, the same N(0,1) draw MX-quantised like the fp4 keys:
  packed e2m1 [rows, H, D/2] plus e8m0 scales [rows, H, D/32]
* w  = N(0,1) / 8, float32                          [rows, H]
* fp8 K, per token: x ~ N(0,1)^D, codes = fp8(clamp(448 x / max|x|)),
  scale ~ U(0.5, 2) / 448 (float32)
* fp4 K, per token: x ~ N(0,1)^D times 2^U{-spread..spread}; per 32-element
  block: shared exponent floor(log2(amax)) - 2 (OCP MX v1.0), elements rounded
  to nearest-even e2m1 and saturated at +-6, scale stored as e8m0.
* pages: ceil(ctx / block_kv) per request plus 5 % spare pages, placed by a
  random permutation of the pool; unused slots and spare pages hold NaN codes
  (fp8 0x7F, fp32 scale NaN, e8m0 0xFF) so stray reads show up as NaN.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

H_DEFAULT = 64
D_DEFAULT = 128
FP8_MAX = 448.0
MX_BLOCK = 32

KV_FP8 = 0
KV_FP4 = 1

FP8_NAN = 0x7F
E8M0_NAN = 0xFF


def page_bytes(kv_format: int, block_kv: int, D: int) -> int:
    """Bytes of one cache page: values region then scales region."""
    if kv_format == KV_FP8:
        return block_kv * (D + 4)
    return block_kv * (D // 2 + D // MX_BLOCK)


def fp8_codes(x: torch.Tensor) -> torch.Tensor:
    """Round float32 to fp8 e4m3fn codes (nearest-even) after clamping to +-448.

    The clamp matters: torch saturates 449..464 to 448 but turns >= 480 into NaN.
    """
    return x.clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn).view(torch.uint8)


# e2m1 magnitudes by 3-bit code and the midpoints between neighbours.
_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_codes(v: np.ndarray) -> np.ndarray:
    """Nearest-even rounding of float values to 4-bit e2m1 codes, saturating at +-6."""
    a = np.minimum(np.abs(v), 6.0)
    # index of the nearest magnitude; ties go to the even code
    hi = np.searchsorted(_E2M1_MAG, a, side="left").clip(0, 7)
    lo = (hi - 1).clip(0, 7)
    dlo = a - _E2M1_MAG[lo]
    dhi = _E2M1_MAG[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    sign = (np.signbit(v) & (code != 0)).astype(np.uint8) << 3
    return code | sign


def mx_fp4_quantize(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """OCP MX v1.0 quantisation of rows of D floats into packed e2m1 + e8m0.

    Returns (packed [T, D/2] uint8 with element 2i in the low nibble,
    scales [T, D/32] uint8 e8m0).
    """
    T, D = x.shape
    xb = x.reshape(T, D // MX_BLOCK, MX_BLOCK)
    amax = np.abs(xb).max(axis=2)
    amax = np.where(amax > 0, amax, 1.0)
    e = np.floor(np.log2(amax)).astype(np.int64) - 2  # emax(e2m1) = 2
    e = e.clip(-127, 127)
    codes = e2m1_codes(xb / np.exp2(e)[:, :, None].astype(np.float64)).reshape(T, D)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8)


@dataclass
class PagedCase:
    """Inputs of one paged-logits call (CPU tensors)."""
    q: torch.Tensor            # uint8 fp8 codes [rows, H, D], or packed e2m1 [rows, H, D/2]
    weights: torch.Tensor      # float32 [rows, H]
    kv_cache: torch.Tensor     # uint8 [num_pages, page_stride]
    kv_format: int
    block_kv: int
    block_table: torch.Tensor  # int32 [bt_rows, bt_cols]
    context_lens: torch.Tensor  # int32 [rows] or [B, next_n]
    indices: torch.Tensor | None  # int32 [rows] or None
    next_n: int
    max_ctx: int
    topk: int
    H: int = H_DEFAULT
    D: int = D_DEFAULT
    req_ctx: list = field(default_factory=list)  # per request (or batch entry) full length
    q_scale: torch.Tensor | None = None  # uint8 e8m0 [rows, H, D/32] when q is e2m1

    @property
    def rows(self) -> int:
        return self.q.shape[0]

    @property
    def page_stride(self) -> int:
        return self.kv_cache.shape[1]

    @property
    def lens_2d(self) -> bool:
        return self.context_lens.dim() == 2


def vis_per_row(case: PagedCase) -> np.ndarray:
    """Tokens each flattened row sees (input bookkeeping, used for sizing and bounds)."""
    lens = case.context_lens.numpy().astype(np.int64)
    if case.lens_2d:
        return lens.reshape(-1)
    if case.next_n == 1:
        return lens.copy()
    j = np.arange(case.next_n)
    return (lens[:, None] - case.next_n + j[None, :] + 1).reshape(-1).clip(0, None)


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator()
    g.manual_seed(seed)
    return g


def _fill_nan_pages(kv: np.ndarray, kv_format: int, block_kv: int, D: int) -> None:
    if kv_format == KV_FP8:
        kv[:, : block_kv * D] = FP8_NAN
        nan4 = np.frombuffer(np.float32(np.nan).tobytes(), dtype=np.uint8)
        kv[:, block_kv * D: block_kv * (D + 4)] = np.tile(nan4, block_kv)
    else:
        kv[:, : block_kv * D // 2] = 0x77  # finite codes; the e8m0 NaN scale poisons them
        kv[:, block_kv * D // 2: block_kv * (D // 2 + D // MX_BLOCK)] = E8M0_NAN


def _write_request_tokens(kv, pages, ctx, kv_format, block_kv, D, gen, fp4_spread):
    """Quantise ctx tokens of one request into its pages."""
    x = torch.randn(ctx, D, generator=gen, dtype=torch.float32)
    if kv_format == KV_FP8:
        amax = x.abs().amax(dim=1, keepdim=True).clamp_min(1e-30)
        codes = fp8_codes(x * (FP8_MAX / amax)).numpy()
        scale = ((torch.rand(ctx, generator=gen, dtype=torch.float32) * 1.5 + 0.5) / FP8_MAX).numpy()
        sbytes = scale.view(np.uint8).reshape(ctx, 4)
        for i, p in enumerate(pages):
            t0 = i * block_kv
            t1 = min(ctx, t0 + block_kv)
            n = t1 - t0
            kv[p, : n * D] = codes[t0:t1].reshape(-1)
            kv[p, block_kv * D: block_kv * D + n * 4] = sbytes[t0:t1].reshape(-1)
    else:
        if fp4_spread:
            ex = torch.randint(-fp4_spread, fp4_spread + 1, (ctx, 1), generator=gen).float()
            x = x * torch.exp2(ex)
        packed, sc = mx_fp4_quantize(x.numpy().astype(np.float64))
        vb = D // 2
        sb = D // MX_BLOCK
        for i, p in enumerate(pages):
            t0 = i * block_kv
            t1 = min(ctx, t0 + block_kv)
            n = t1 - t0
            kv[p, : n * vb] = packed[t0:t1].reshape(-1)
            kv[p, block_kv * vb: block_kv * vb + n * sb] = sc[t0:t1].reshape(-1)


def make_paged_case(
    req_ctx: list[int],
    req_rows: list[int],
    *,
    seed: int,
    kv_format: int = KV_FP8,
    block_kv: int = 64,
    max_ctx: int | None = None,
    varlen: bool = True,
    next_n: int = 1,
    lens_2d: bool = False,
    H: int = H_DEFAULT,
    D: int = D_DEFAULT,
    topk: int = 2048,
    page_stride: int | None = None,
    spare_frac: float = 0.05,
    fp4_spread: int = 0,
    row_ctx: list[int] | None = None,
    q_fp4: bool = False,
) -> PagedCase:
    """Build a paged case.

    ``req_ctx[i]`` is request i's full cached length and ``req_rows[i]`` its
    number of query rows (accepted draft length). Row j (0-based) of request i
    sees ``ctx - rows + j + 1`` tokens.

    * ``varlen=True``: rows are flattened (next_n = 1), ``indices`` holds the
      request id of each row and the block table has one row per query row.
    * ``varlen=False``: every request has ``next_n`` rows, ``indices`` is None,
      the block table has one row per request and ``context_lens`` is 1-D (the
      full length) or, with ``lens_2d``, [B, next_n] per-row lengths.
    ``row_ctx`` overrides the per-row visible lengths (varlen only).
    ``q_fp4`` MX-quantises q (packed e2m1 + e8m0 per 32 elements) instead of fp8.
    """
    g = _gen(seed)
    B = len(req_ctx)
    if not varlen:
        assert all(r == next_n for r in req_rows)
    if max_ctx is None:
        max_ctx = max(req_ctx) if req_ctx else 0
    pb = page_bytes(kv_format, block_kv, D)
    stride = pb if page_stride is None else page_stride
    assert stride >= pb and stride % 16 == 0
    npages_req = [math.ceil(c / block_kv) for c in req_ctx]
    total = sum(npages_req)
    num_pages = max(1, total + int(math.ceil(total * spare_frac)))
    perm = torch.randperm(num_pages, generator=g).numpy().astype(np.int32)
    kv = np.zeros((num_pages, stride), dtype=np.uint8)
    _fill_nan_pages(kv, kv_format, block_kv, D)
    bt_cols = max(1, math.ceil(max_ctx / block_kv))
    req_table = np.full((B, bt_cols), -1, dtype=np.int32)
    pos = 0
    for i in range(B):
        pages = perm[pos: pos + npages_req[i]]
        pos += npages_req[i]
        req_table[i, : len(pages)] = pages
        _write_request_tokens(kv, pages, req_ctx[i], kv_format, block_kv, D, g, fp4_spread)

    rows = sum(req_rows)
    qf = torch.randn(rows, H, D, generator=g, dtype=torch.float32)
    q_scale = None
    if q_fp4:
        packed, sc = mx_fp4_quantize(qf.reshape(rows * H, D).numpy().astype(np.float64))
        q = torch.from_numpy(packed.reshape(rows, H, D // 2).copy())
        q_scale = torch.from_numpy(sc.reshape(rows, H, D // MX_BLOCK).copy())
    else:
        q = fp8_codes(qf)
    w = torch.randn(rows, H, generator=g, dtype=torch.float32) / 8
    req_of_row = np.repeat(np.arange(B, dtype=np.int32), req_rows)
    if varlen:
        if row_ctx is None:
            lens = np.concatenate([
                np.asarray(req_ctx[i] - req_rows[i] + np.arange(req_rows[i]) + 1, dtype=np.int64)
                for i in range(B)
            ]) if rows else np.zeros(0, dtype=np.int64)
            lens = lens.clip(0, None)
        else:
            lens = np.asarray(row_ctx, dtype=np.int64)
        context_lens = torch.from_numpy(lens.astype(np.int32))
        indices = torch.from_numpy(req_of_row.copy())
        block_table = torch.from_numpy(req_table[req_of_row].copy()) if rows else torch.zeros(0, bt_cols, dtype=torch.int32)
    else:
        if lens_2d:
            j = np.arange(next_n)
            l2 = (np.asarray(req_ctx, dtype=np.int64)[:, None] - next_n + j[None, :] + 1).clip(0, None)
            context_lens = torch.from_numpy(l2.astype(np.int32))
        else:
            context_lens = torch.tensor(req_ctx, dtype=torch.int32)
        indices = None
        block_table = torch.from_numpy(req_table)
    return PagedCase(q=q, weights=w, kv_cache=torch.from_numpy(kv), kv_format=kv_format,
                     block_kv=block_kv, block_table=block_table, context_lens=context_lens,
                     indices=indices, next_n=(1 if varlen else next_n), max_ctx=max_ctx,
                     topk=topk, H=H, D=D, req_ctx=list(req_ctx), q_scale=q_scale)


@dataclass
class RaggedCase:
    """Inputs of one non-paged (prefill) logits call (CPU tensors)."""
    q: torch.Tensor        # uint8 fp8 codes [M, H, D]
    weights: torch.Tensor  # float32 [M, H]
    k: torch.Tensor        # uint8 fp8 codes [N, D]
    k_scale: torch.Tensor  # float32 [N]
    ks: torch.Tensor       # int32 [M]
    ke: torch.Tensor       # int32 [M]
    topk: int
    H: int = H_DEFAULT
    D: int = D_DEFAULT

    @property
    def M(self) -> int:
        return self.q.shape[0]

    @property
    def N(self) -> int:
        return self.k.shape[0]


def make_ragged_case(seq_lens: list[int], *, seed: int, H: int = H_DEFAULT, D: int = D_DEFAULT,
                     topk: int = 2048) -> RaggedCase:
    """Concatenated causal prefill: row r of sequence i sees keys
    [start_i, start_i + pos + 1)."""
    g = _gen(seed)
    N = sum(seq_lens)
    x = torch.randn(N, D, generator=g, dtype=torch.float32)
    amax = x.abs().amax(dim=1, keepdim=True).clamp_min(1e-30)
    k = fp8_codes(x * (FP8_MAX / amax))
    k_scale = (torch.rand(N, generator=g, dtype=torch.float32) * 1.5 + 0.5) / FP8_MAX
    q = fp8_codes(torch.randn(N, H, D, generator=g, dtype=torch.float32))
    w = torch.randn(N, H, generator=g, dtype=torch.float32) / 8
    ks = np.zeros(N, dtype=np.int32)
    ke = np.zeros(N, dtype=np.int32)
    start = 0
    for L in seq_lens:
        ks[start: start + L] = start
        ke[start: start + L] = start + np.arange(L) + 1
        start += L
    return RaggedCase(q=q, weights=w, k=k, k_scale=k_scale, ks=torch.from_numpy(ks),
                      ke=torch.from_numpy(ke), topk=topk, H=H, D=D)


# ---------------------------------------------------------------------------
# The five named workloads. Ranges "U[a,b]" are inclusive integer ranges;
# "K" means 1024.

def _randint(g, lo, hi, n):
    return torch.randint(lo, hi + 1, (n,), generator=g).tolist()


def config_tiny_decode(seed: int = 1001) -> PagedCase:
    """B=4 plain decode rows, ctx U[100,4096], fp8 K, block_kv 64, top-k 64."""
    g = _gen(seed)
    ctx = _randint(g, 100, 4096, 4)
    return make_paged_case(ctx, [1] * 4, seed=seed + 100, kv_format=KV_FP8, block_kv=64,
                           max_ctx=4096, varlen=True, topk=64)


def config_uniform_decode(seed: int = 1002, B: int = 64) -> PagedCase:
    """B=64 plain decode rows (non-varlen), ctx U[16K,32K], fp8 K, top-k 2048."""
    g = _gen(seed)
    ctx = _randint(g, 16384, 32768, B)
    return make_paged_case(ctx, [1] * B, seed=seed + 100, kv_format=KV_FP8, block_kv=64,
                           max_ctx=32768, varlen=False, next_n=1, topk=2048)


def config_varlen_fp8(seed: int = 1003, R: int = 40, lo: int = 102400, hi: int = 131072,
                      max_ctx: int = 131072) -> PagedCase:
    """40 requests, ctx U[100K,128K], accepted lengths U{1..6}, flattened varlen rows."""
    g = _gen(seed)
    ctx = _randint(g, lo, hi, R)
    nrows = _randint(g, 1, 6, R)
    return make_paged_case(ctx, nrows, seed=seed + 100, kv_format=KV_FP8, block_kv=64,
                           max_ctx=max_ctx, varlen=True, topk=2048)


def config_varlen_fp4(seed: int = 1004, R: int = 64, lo: int = 32768, hi: int = 65536,
                      max_ctx: int = 65536, q_fp4: bool = False) -> PagedCase:
    """64 requests, ctx U[32K,64K], lengths U{1..4}, MXFP4 K, block_kv 32
    (with q_fp4, q MX-quantised from the same draw)."""
    g = _gen(seed)
    ctx = _randint(g, lo, hi, R)
    nrows = _randint(g, 1, 4, R)
    return make_paged_case(ctx, nrows, seed=seed + 100, kv_format=KV_FP4, block_kv=32,
                           max_ctx=max_ctx, varlen=True, topk=2048, q_fp4=q_fp4)


def config_ragged_prefill(seed: int = 1005, nseq: int = 4, L: int = 8192) -> RaggedCase:
    """4 sequences of 8192 tokens, contiguous fp8 K, causal bounds, top-k 2048."""
    return make_ragged_case([L] * nseq, seed=seed, topk=2048)


def scored_pairs(case: PagedCase) -> int:
    return int(vis_per_row(case).sum())
