"""Python binding of libpml, the gfx950 paged MQA-logits library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (``include/pml.h``). Tensors must already live on the
GPU; work is enqueued on torch's current stream and nothing synchronises.
There is no CPU fallback: if ``libpml.so`` is missing the calls raise.

Calls (names follow the indexer pages: get_paged_mqa_logits_metadata,
fp8_fp4_paged_mqa_logits, mqa_logits and the per-row top-k selector):

* ``paged_mqa_logits_metadata(context_lens, block_kv, num_cus, indices=None, next_n=1)``
* ``fp8_fp4_paged_mqa_logits(q, kv_cache, weights, context_lens, block_table, schedule,
  max_model_len, indices=None, q_scale=None, workspace=None, ...)``
* ``mqa_logits(q, k, k_scale, weights, cu_seqlen_ks, cu_seqlen_ke)``
* ``top_k_per_row(logits, ke, k, ks=None, next_n=1, max_width=None)``
"""
from __future__ import annotations

import ctypes
from pathlib import Path

import torch

KV_FP8 = 0
KV_MXFP4 = 1
HEADS = 64
HEAD_DIM = 128
MAX_TOPK = 4096
WORKERS_PER_CU = 2

_LIB_PATH = Path(__file__).resolve().parent / "libpml.so"
_lib = None

# status codes that mean "bad argument" (ValueError); the rest are RuntimeError
_ARG_ERRORS = {1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 12}


class PmlError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class PmlArgError(PmlError, ValueError):
    pass


def library_path() -> Path:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded libpml.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not _LIB_PATH.exists():
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with paged_mqa_logits_amd.build.build() "
                               "(or __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(str(_LIB_PATH))
        P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        L.paged_mqa_logits_metadata.argtypes = [P, I, I, I, P, I, I, P, P]
        L.paged_mqa_logits_schedule_rows.argtypes = [I]
        L.paged_mqa_logits_schedule_rows.restype = I
        # (q, q_scale), rows .. logits_ld, workspace, bytes, stream
        body = [I, I, I, I, P, I, I, I64, I64, P, P, I, P, I64, I, P, I, P, I, P, I64]
        L.fp8_fp4_paged_mqa_logits.argtypes = [P, P] + body + [P, SZ, P]
        L.fp8_fp4_paged_mqa_logits_workspace_size.argtypes = [I, I]
        L.fp8_fp4_paged_mqa_logits_workspace_size.restype = SZ
        if hasattr(L, "fp8_fp4_paged_mqa_logits_noalloc"):
            L.fp8_fp4_paged_mqa_logits_noalloc.argtypes = [P, P] + body + [P]
        if hasattr(L, "fp8_fp4_paged_mqa_logits_bf16"):
            L.fp8_fp4_paged_mqa_logits_bf16.argtypes = [P] + body + [P, SZ, P]
            L.as_fp32_logits.argtypes = [P, I, I64, I, P, P, I64, P]
        if hasattr(L, "fp8_fp4_paged_mqa_logits_topk"):
            L.fp8_fp4_paged_mqa_logits_topk.argtypes = [P] + body + [I, P, I64, P, SZ, P]
            L.fp8_fp4_paged_mqa_logits_topk_workspace_size.argtypes = [I, I, I, I, I]
            L.fp8_fp4_paged_mqa_logits_topk_workspace_size.restype = SZ
        if hasattr(L, "fp8_fp4_paged_mqa_logits_fp4q"):
            L.fp8_fp4_paged_mqa_logits_fp4q.argtypes = L.fp8_fp4_paged_mqa_logits.argtypes
        if hasattr(L, "mqa_logits"):
            L.mqa_logits.argtypes = [P, I, I, I, P, P, I, P, P, P, P, I64, P]
        if hasattr(L, "top_k_per_row"):
            L.top_k_per_row_workspace_size.argtypes = [I, I, I]
            L.top_k_per_row_workspace_size.restype = SZ
            L.top_k_per_row.argtypes = [P, I, I64, P, P, I, I, I, P, I64, P, SZ, P]
        if hasattr(L, "top_k_per_row_bf16"):
            L.top_k_per_row_bf16.argtypes = L.top_k_per_row.argtypes
        if hasattr(L, "stable_topk_from_gathered_candidates"):
            L.pack_dcp_topk_candidates.argtypes = [P, I, I64, P, P, I64, I, I, I, I, P, P]
            L.stable_topk_from_gathered_candidates.argtypes = [P, I, I, I, P, I64, P]
        for name in ("paged_mqa_logits_metadata", "fp8_fp4_paged_mqa_logits", "mqa_logits", "top_k_per_row",
                     "top_k_per_row_bf16", "pack_dcp_topk_candidates", "stable_topk_from_gathered_candidates",
                     "fp8_fp4_paged_mqa_logits_bf16", "as_fp32_logits", "fp8_fp4_paged_mqa_logits_fp4q",
                     "fp8_fp4_paged_mqa_logits_topk", "fp8_fp4_paged_mqa_logits_noalloc"):
            if hasattr(L, name):
                getattr(L, name).restype = I
        L.pml_status_string.argtypes = [I]
        L.pml_status_string.restype = ctypes.c_char_p
        L.pml_version.restype = I
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().pml_status_string(status).decode()


def _check(status: int, call: str) -> None:
    if status != 0:
        msg = f"{call}: {status_string(status)} (status {status})"
        raise (PmlArgError if status in _ARG_ERRORS else PmlError)(status, msg)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, name: str, dtypes) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype} not in {dtypes}")
    return t


_FP8_TYPES = (torch.uint8, torch.float8_e4m3fn)
_I32 = (torch.int32,)
_F32 = (torch.float32,)


def default_num_workers(device=None) -> int:
    """Persistent workgroups for the paged-logits call: WORKERS_PER_CU per compute unit."""
    props = torch.cuda.get_device_properties(device if device is not None else torch.cuda.current_device())
    return WORKERS_PER_CU * props.multi_processor_count


def _rows_of(context_lens: torch.Tensor, next_n: int, indices) -> tuple[int, int]:
    """(flattened rows, 2-D flag) implied by the lengths and next_n."""
    if context_lens.dim() == 2:
        if indices is not None:
            raise ValueError("2-D context_lens cannot be combined with indices")
        if context_lens.shape[1] != next_n:
            raise ValueError("2-D context_lens must be [batch, next_n]")
        return context_lens.numel(), 1
    if indices is not None or next_n == 1:
        return context_lens.numel(), 0
    return context_lens.numel() * next_n, 0


def paged_mqa_logits_metadata(context_lens: torch.Tensor, block_kv: int, num_cus: int | None = None,
                              indices: torch.Tensor | None = None, next_n: int = 1,
                              out: torch.Tensor | None = None) -> torch.Tensor:
    """Work split of the paged-logits call for num_cus workgroups: int32
    [num_cus + 1, 2] on the device (one range start per workgroup, then the
    end); read only by the logits calls."""
    _dev(context_lens, "context_lens", _I32)
    context_lens = context_lens.contiguous()
    if indices is not None:
        indices = _dev(indices, "indices", _I32).contiguous()
    if num_cus is None:
        num_cus = default_num_workers(context_lens.device)
    rows, l2d = _rows_of(context_lens, next_n, indices)
    n = schedule_rows(num_cus)
    if out is None:
        out = torch.empty(n, 2, dtype=torch.int32, device=context_lens.device)
    elif out.shape != (n, 2) or not out.is_contiguous():
        raise ValueError(f"schedule buffer must be a contiguous [{n}, 2] tensor")
    _check(lib().paged_mqa_logits_metadata(_p(context_lens), rows, next_n, l2d, _p(indices), block_kv,
                                           num_cus, _p(out), _stream()), "paged_mqa_logits_metadata")
    return out


def schedule_rows(num_cus: int) -> int:
    """Rows of the [rows, 2] schedule tensor for num_cus logits workgroups (num_cus + 1)."""
    n = lib().paged_mqa_logits_schedule_rows(int(num_cus))
    if n < 0:
        raise ValueError(f"num_cus {num_cus} outside 1 .. 2^20")
    return n


def schedule_workers(schedule: torch.Tensor) -> int:
    """Workgroups a schedule tensor was made for: schedule.shape[0] - 1."""
    if schedule.dim() != 2 or schedule.shape[1] != 2 or schedule.shape[0] < 2:
        raise ValueError(f"schedule of shape {tuple(schedule.shape)} is not a metadata output")
    return schedule.shape[0] - 1


def logits_ld(max_ctx: int) -> int:
    """Row stride used when the binding allocates the logits (a multiple of 4 floats)."""
    return max(4, (max_ctx + 3) // 4 * 4)


def logits_workspace_size(rows: int, num_cus: int) -> int:
    """Bytes of scratch one paged-logits call needs."""
    return int(lib().fp8_fp4_paged_mqa_logits_workspace_size(rows, num_cus))


def _workspace(ws, need: int, device) -> tuple:
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    _dev(ws, "workspace", (torch.uint8,))
    return ws, ws.numel()


def fp8_fp4_paged_mqa_logits(q: torch.Tensor, kv_cache: torch.Tensor, weights: torch.Tensor,
                             context_lens: torch.Tensor, block_table: torch.Tensor,
                             schedule: torch.Tensor, max_model_len: int,
                             indices: torch.Tensor | None = None, *, kv_format: int = KV_FP8,
                             block_kv: int = 64, next_n: int = 1,
                             logits: torch.Tensor | None = None,
                             out_dtype: torch.dtype = torch.float32,
                             q_scale: torch.Tensor | None = None,
                             workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Paged logits [rows, ld >= max_model_len], fp32 or bf16 (``out_dtype``, or
    the dtype of a given ``logits``); columns past each row's visible length are
    -inf. ``kv_cache`` is [num_pages, page_stride_bytes] uint8 (a row stride
    larger than the page is allowed). With ``q_scale`` (uint8 e8m0 [rows, heads,
    head_dim / 32]) q is packed e2m1 [rows, heads, head_dim / 2] (MXFP4 keys,
    fp32 logits). ``workspace``: uint8 scratch of at least
    ``logits_workspace_size(rows, schedule rows - 1)`` bytes (allocated when
    None), or ``"static"`` for the allocation-free call
    (fp8_fp4_paged_mqa_logits_noalloc: the library's per-GPU scratch, up to
    4096 rows and 4096 workgroups)."""
    _dev(q, "q", _FP8_TYPES)
    _dev(kv_cache, "kv_cache", (torch.uint8,))
    _dev(weights, "weights", _F32)
    _dev(context_lens, "context_lens", _I32)
    _dev(block_table, "block_table", _I32)
    _dev(schedule, "schedule", _I32)
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [rows, heads, head_dim] tensor")
    head_dim = q.shape[2]
    if q_scale is not None:
        _dev(q_scale, "q_scale", (torch.uint8,))
        head_dim = 2 * q.shape[2]
        if tuple(q_scale.shape) != (q.shape[0], q.shape[1], head_dim // 32) or not q_scale.is_contiguous():
            raise ValueError("q_scale must be a contiguous uint8 [rows, heads, head_dim / 32] tensor")
        if out_dtype != torch.float32 or (logits is not None and logits.dtype != torch.float32):
            raise ValueError("fp4 q writes fp32 logits")
    if kv_cache.dim() != 2 or kv_cache.stride(1) != 1:
        raise ValueError("kv_cache must be [num_pages, page_stride] with unit inner stride")
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be 2-D with unit inner stride")
    weights = weights.contiguous()
    context_lens = context_lens.contiguous()
    if indices is not None:
        indices = _dev(indices, "indices", _I32).contiguous()
    rows, l2d = _rows_of(context_lens, next_n, indices)
    if rows != q.shape[0]:
        raise ValueError(f"q has {q.shape[0]} rows but the lengths describe {rows}")
    if logits is None:
        if out_dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("out_dtype must be float32 or bfloat16")
        ld = logits_ld(max_model_len) if out_dtype == torch.float32 else (max_model_len + 7) // 8 * 8
        logits = torch.empty(rows, max(ld, 8), dtype=out_dtype, device=q.device)
    if logits.dim() != 2 or logits.stride(1) != 1 or logits.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("logits must be a 2-D float32 or bfloat16 tensor with unit inner stride")
    num_cus = schedule_workers(schedule)
    if not schedule.is_contiguous():
        raise ValueError("schedule must be contiguous")
    args = (rows, next_n, q.shape[1], head_dim, _p(kv_cache), kv_format, block_kv,
            kv_cache.stride(0), kv_cache.shape[0], _p(weights), _p(context_lens), l2d, _p(block_table),
            block_table.stride(0), block_table.shape[1], _p(schedule), num_cus, _p(indices),
            max_model_len, _p(logits), logits.stride(0))
    if isinstance(workspace, str):
        if workspace != "static" or logits.dtype != torch.float32:
            raise ValueError('workspace="static" (the allocation-free call) writes fp32 logits')
        _check(lib().fp8_fp4_paged_mqa_logits_noalloc(_p(q), _p(q_scale), *args, _stream()),
               "fp8_fp4_paged_mqa_logits_noalloc")
        return logits
    ws, wbytes = _workspace(workspace, logits_workspace_size(rows, num_cus), q.device)
    tail = args + (_p(ws), wbytes, _stream())
    if logits.dtype == torch.float32:
        st = lib().fp8_fp4_paged_mqa_logits(_p(q), _p(q_scale), *tail)
    else:
        st = lib().fp8_fp4_paged_mqa_logits_bf16(_p(q), *tail)
    _check(st, "fp8_fp4_paged_mqa_logits")
    return logits


def as_fp32_logits(logits: torch.Tensor, row_ends: torch.Tensor, out: torch.Tensor | None = None,
                   cols: int | None = None) -> torch.Tensor:
    """fp32 copy of bf16 logits over each row's columns [0, row_end), with the
    same row stride; other columns of ``out`` are left as they are."""
    _dev(logits, "logits", (torch.bfloat16,))
    _dev(row_ends, "row_ends", _I32)
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be 2-D with unit inner stride")
    rows = logits.shape[0]
    cols = logits.shape[1] if cols is None else cols
    if row_ends.numel() != rows:
        raise ValueError("row_ends needs one entry per row")
    if out is None:
        out = torch.empty_strided(logits.shape, (logits.stride(0), 1), dtype=torch.float32, device=logits.device)
    _check(lib().as_fp32_logits(_p(logits), rows, logits.stride(0), cols, _p(row_ends.contiguous()), _p(out),
                                out.stride(0), _stream()), "as_fp32_logits")
    return out


def mqa_logits(q: torch.Tensor, k: torch.Tensor, k_scale: torch.Tensor, weights: torch.Tensor,
               cu_seqlen_ks: torch.Tensor, cu_seqlen_ke: torch.Tensor,
               logits: torch.Tensor | None = None) -> torch.Tensor:
    """Ragged (non-paged) logits fp32 [M, ld >= N]; row r is scored on keys [ks[r], ke[r])."""
    _dev(q, "q", _FP8_TYPES)
    _dev(k, "k", _FP8_TYPES)
    _dev(k_scale, "k_scale", _F32)
    _dev(weights, "weights", _F32)
    _dev(cu_seqlen_ks, "cu_seqlen_ks", _I32)
    _dev(cu_seqlen_ke, "cu_seqlen_ke", _I32)
    if q.dim() != 3 or not q.is_contiguous() or k.dim() != 2 or not k.is_contiguous():
        raise ValueError("q must be contiguous [M, heads, head_dim] and k contiguous [N, head_dim]")
    M, N = q.shape[0], k.shape[0]
    if logits is None:
        logits = torch.empty(M, logits_ld(N), dtype=torch.float32, device=q.device)
    _check(lib().mqa_logits(_p(q), M, q.shape[1], q.shape[2], _p(k), _p(k_scale.contiguous()), N,
                            _p(weights.contiguous()), _p(cu_seqlen_ks.contiguous()),
                            _p(cu_seqlen_ke.contiguous()), _p(logits), logits.stride(0), _stream()),
           "mqa_logits")
    return logits


def top_k_workspace_size(rows: int, max_width: int, k: int) -> int:
    return int(lib().top_k_per_row_workspace_size(rows, max_width, k))


def top_k_per_row(logits: torch.Tensor, ke: torch.Tensor, k: int, ks: torch.Tensor | None = None,
                  next_n: int = 1, max_width: int | None = None, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None) -> torch.Tensor:
    """int32 [rows, k]: per row the positions (minus ks) of the k largest logits
    among columns [ks, ke), ascending, then -1. fp32 or bf16 logits (bf16 are
    selected by their exact fp32 values: the same result as on as_fp32_logits)."""
    _dev(logits, "logits", (torch.float32, torch.bfloat16))
    _dev(ke, "ke", _I32)
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be 2-D with unit inner stride")
    rows = logits.shape[0]
    if ks is not None:
        ks = _dev(ks, "ks", _I32).contiguous()
    if max_width is None:
        max_width = logits.shape[1]
    if out is None:
        out = torch.empty(rows, max(k, 1), dtype=torch.int32, device=logits.device)
    need = top_k_workspace_size(rows, max_width, k)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=logits.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    fn = lib().top_k_per_row_bf16 if logits.dtype == torch.bfloat16 else lib().top_k_per_row
    _check(fn(_p(logits), rows, logits.stride(0), _p(ks), _p(ke.contiguous()), next_n, k,
              max_width, _p(out), out.stride(0), _p(workspace), wbytes, _stream()),
           "top_k_per_row")
    return out


def pack_dcp_topk_candidates(logits: torch.Tensor, topk: torch.Tensor, rank: int, world: int, interleave: int,
                             row_starts: torch.Tensor | None = None, k: int | None = None,
                             out: torch.Tensor | None = None) -> torch.Tensor:
    """fp32 [rows, k, 2]: this rank's (score, global token id) pairs from its local
    top-k positions; padding entries become (-inf, -1)."""
    _dev(logits, "logits", _F32)
    _dev(topk, "topk", _I32)
    if logits.dim() != 2 or logits.stride(1) != 1 or topk.dim() != 2 or topk.stride(1) != 1:
        raise ValueError("logits and topk must be 2-D with unit inner stride")
    rows = topk.shape[0]
    if logits.shape[0] != rows:
        raise ValueError("logits and topk must have the same rows")
    k = topk.shape[1] if k is None else k
    if row_starts is not None:
        row_starts = _dev(row_starts, "row_starts", _I32).contiguous()
    if out is None:
        out = torch.empty(rows, max(k, 1), 2, dtype=torch.float32, device=logits.device)
    elif not out.is_contiguous() or tuple(out.shape) != (rows, k, 2) or out.dtype != torch.float32:
        raise ValueError("out must be a contiguous fp32 [rows, k, 2] tensor")
    _check(lib().pack_dcp_topk_candidates(_p(logits), rows, logits.stride(0), _p(row_starts), _p(topk),
                                          topk.stride(0), k, rank, world, interleave, _p(out), _stream()),
           "pack_dcp_topk_candidates")
    return out


def stable_topk_from_gathered_candidates(gathered: torch.Tensor, k: int,
                                         out: torch.Tensor | None = None) -> torch.Tensor:
    """int32 [rows, k]: ids of the k best (score, id) pairs of each row over all
    ranks of gathered [world, rows, k, 2], ascending, then -1."""
    _dev(gathered, "gathered", _F32)
    if gathered.dim() != 4 or gathered.shape[2] != k or gathered.shape[3] != 2 or not gathered.is_contiguous():
        raise ValueError("gathered must be a contiguous fp32 [world, rows, k, 2] tensor")
    world, rows = gathered.shape[0], gathered.shape[1]
    if out is None:
        out = torch.empty(rows, max(k, 1), dtype=torch.int32, device=gathered.device)
    _check(lib().stable_topk_from_gathered_candidates(_p(gathered), world, rows, k, _p(out), out.stride(0),
                                                      _stream()),
           "stable_topk_from_gathered_candidates")
    return out


def fused_topk_workspace_size(rows: int, max_model_len: int, block_kv: int, k: int, num_cus: int) -> int:
    return int(lib().fp8_fp4_paged_mqa_logits_topk_workspace_size(rows, max_model_len, block_kv, k, num_cus))


def fp8_fp4_paged_mqa_logits_topk(q: torch.Tensor, kv_cache: torch.Tensor, weights: torch.Tensor,
                                  context_lens: torch.Tensor, block_table: torch.Tensor,
                                  schedule: torch.Tensor, max_model_len: int, k: int,
                                  indices: torch.Tensor | None = None, *, kv_format: int = KV_FP8,
                                  block_kv: int = 64, next_n: int = 1, logits: torch.Tensor | None = None,
                                  out: torch.Tensor | None = None,
                                  workspace: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """Paged logits (fp32, as fp8_fp4_paged_mqa_logits writes them) and their per-row
    top-k (as top_k_per_row over them, max_width = max_model_len) in one call, the
    top-k taken from candidates the logits kernel keeps. Returns (logits, topk)."""
    _dev(q, "q", _FP8_TYPES)
    _dev(kv_cache, "kv_cache", (torch.uint8,))
    _dev(weights, "weights", _F32)
    _dev(context_lens, "context_lens", _I32)
    _dev(block_table, "block_table", _I32)
    _dev(schedule, "schedule", _I32)
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [rows, heads, head_dim] tensor")
    weights = weights.contiguous()
    context_lens = context_lens.contiguous()
    if indices is not None:
        indices = _dev(indices, "indices", _I32).contiguous()
    rows, l2d = _rows_of(context_lens, next_n, indices)
    if rows != q.shape[0]:
        raise ValueError(f"q has {q.shape[0]} rows but the lengths describe {rows}")
    if logits is None:
        logits = torch.empty(rows, logits_ld(max_model_len), dtype=torch.float32, device=q.device)
    if out is None:
        out = torch.empty(rows, max(k, 1), dtype=torch.int32, device=q.device)
    num_cus = schedule_workers(schedule)
    ws, wbytes = _workspace(workspace, fused_topk_workspace_size(rows, max_model_len, block_kv, k, num_cus),
                            q.device)
    _check(lib().fp8_fp4_paged_mqa_logits_topk(
        _p(q), rows, next_n, q.shape[1], q.shape[2], _p(kv_cache), kv_format, block_kv,
        kv_cache.stride(0), kv_cache.shape[0], _p(weights), _p(context_lens), l2d, _p(block_table),
        block_table.stride(0), block_table.shape[1], _p(schedule), num_cus, _p(indices),
        max_model_len, _p(logits), logits.stride(0), k, _p(out), out.stride(0), _p(ws), wbytes,
        _stream()), "fp8_fp4_paged_mqa_logits_topk")
    return logits, out
