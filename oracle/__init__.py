"""CPU oracle for the paged MQA-logits path (TEST INFRASTRUCTURE ONLY).

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package. It never imports the GPU package, and the GPU package never
imports it; the two share only the seeded input generator ``pml_synth``.

``oracle.c`` holds the fp64 reference of the scores, the masking and the
top-k; ``brute.py`` is a second, numpy-only formulation for tiny inputs;
``schedule.py`` is the specification of the work split that the metadata
call produces.

The pages print no worked example and no numeric value for this path, so no
stored value comes from them. Every function here is pinned by something other
than itself: the fp8 / e2m1 / e8m0 format definitions, hand-worked fixtures
(tests/golden), closed forms, invariants and the independent numpy brute force
(tests/test_oracle.py, tests/test_schedule_spec.py).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "oracle.c"
_LIB = _HERE / "liboracle.so"
_lib = None


def build(force: bool = False) -> Path:
    """Compile oracle.c with gcc (-O2, OpenMP) into liboracle.so next to it."""
    if force or not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB.with_suffix(".so.tmp")
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", str(_SRC), "-o", str(tmp), "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path) -> ctypes.CDLL:
    L = ctypes.CDLL(str(path))
    u8p = ctypes.c_void_p
    L.pml_oracle_fp8_e4m3.restype = ctypes.c_double
    L.pml_oracle_fp8_e4m3.argtypes = [ctypes.c_uint8]
    L.pml_oracle_e2m1.restype = ctypes.c_double
    L.pml_oracle_e2m1.argtypes = [ctypes.c_uint8]
    L.pml_oracle_e8m0.restype = ctypes.c_double
    L.pml_oracle_e8m0.argtypes = [ctypes.c_uint8]
    L.pml_oracle_paged_logits.restype = None
    L.pml_oracle_paged_logits.argtypes = [
        u8p, u8p, ctypes.c_int, ctypes.c_int, u8p, u8p, ctypes.c_int, ctypes.c_int,
        ctypes.c_int64, ctypes.c_int64, u8p, ctypes.c_int, ctypes.c_int, u8p,
        ctypes.c_int64, u8p, ctypes.c_int, ctypes.c_int, ctypes.c_int, u8p]
    L.pml_oracle_ragged_logits.restype = None
    L.pml_oracle_ragged_logits.argtypes = [
        u8p, ctypes.c_int, ctypes.c_int, u8p, u8p, u8p, ctypes.c_int, u8p, u8p,
        u8p, ctypes.c_int, ctypes.c_int, ctypes.c_int, u8p]
    L.pml_oracle_topk.restype = None
    L.pml_oracle_topk.argtypes = [u8p, ctypes.c_int, ctypes.c_int64, u8p, u8p, ctypes.c_int, u8p]
    L.pml_oracle_num_threads.restype = ctypes.c_int
    L.pml_oracle_set_num_threads.restype = None
    L.pml_oracle_set_num_threads.argtypes = [ctypes.c_int]
    L.pml_oracle_visible_lengths.restype = None
    L.pml_oracle_visible_lengths.argtypes = [u8p, ctypes.c_int, ctypes.c_int, ctypes.c_int, u8p]
    L.pml_oracle_dcp_global_id.restype = ctypes.c_int64
    L.pml_oracle_dcp_global_id.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    L.pml_oracle_dcp_pack.restype = None
    L.pml_oracle_dcp_pack.argtypes = [
        u8p, ctypes.c_int, ctypes.c_int64, u8p, u8p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, u8p]
    L.pml_oracle_dcp_merge.restype = None
    L.pml_oracle_dcp_merge.argtypes = [u8p, ctypes.c_int, ctypes.c_int, ctypes.c_int, u8p]
    return L


def lib():
    """The oracle library; ``use_library`` can point it at another build."""
    global _lib
    if _lib is None:
        build()
        _lib = _bind(_LIB)
    return _lib


def use_library(path) -> None:
    """Bind the wrappers below to another compiled oracle (the mutation tests do)."""
    global _lib
    _lib = _bind(path) if path is not None else None


def _np(t, dtype):
    a = t.numpy() if hasattr(t, "numpy") else np.asarray(t)
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def fp8_e4m3(code: int) -> float:
    return lib().pml_oracle_fp8_e4m3(code)


def e2m1(nib: int) -> float:
    return lib().pml_oracle_e2m1(nib)


def e8m0(code: int) -> float:
    return lib().pml_oracle_e8m0(code)


def paged_logits(case, rows=None, col_begin: int = 0, col_end: int | None = None) -> np.ndarray:
    """fp64 logits of a ``pml_synth.PagedCase`` for the given rows and columns."""
    q = _np(case.q, np.uint8)
    w = _np(case.weights, np.float32)
    kv = _np(case.kv_cache, np.uint8)
    lens = _np(case.context_lens, np.int32)
    bt = _np(case.block_table, np.int32)
    if rows is None:
        rows = np.arange(case.rows)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    if col_end is None:
        col_end = case.max_ctx
    out = np.empty((len(rows), col_end - col_begin), dtype=np.float64)
    qs = None if getattr(case, "q_scale", None) is None else _np(case.q_scale, np.uint8)
    if out.size:
        lib().pml_oracle_paged_logits(
            _ptr(q), None if qs is None else _ptr(qs), case.H, case.D, _ptr(w), _ptr(kv), case.kv_format, case.block_kv,
            kv.shape[1], kv.shape[0], _ptr(lens), int(case.lens_2d), case.next_n,
            _ptr(bt), bt.shape[1] if bt.ndim == 2 else 0, _ptr(rows), len(rows),
            col_begin, col_end, _ptr(out))
    return out


def visible_lengths(case) -> np.ndarray:
    """Tokens each row of a ``pml_synth.PagedCase`` sees (int64 [rows]): the
    end of its unmasked span, the bound its top-k takes."""
    lens = _np(case.context_lens, np.int32)
    out = np.empty(case.rows, dtype=np.int64)
    if case.rows:
        lib().pml_oracle_visible_lengths(_ptr(lens), int(case.lens_2d), case.next_n, case.rows, _ptr(out))
    return out


def ragged_logits(case, rows=None, col_begin: int = 0, col_end: int | None = None) -> np.ndarray:
    """fp64 logits of a ``pml_synth.RaggedCase`` for the given rows and columns."""
    q = _np(case.q, np.uint8)
    w = _np(case.weights, np.float32)
    k = _np(case.k, np.uint8)
    ksc = _np(case.k_scale, np.float32)
    ks = _np(case.ks, np.int32)
    ke = _np(case.ke, np.int32)
    if rows is None:
        rows = np.arange(case.M)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    if col_end is None:
        col_end = case.N
    out = np.empty((len(rows), col_end - col_begin), dtype=np.float64)
    if out.size:
        lib().pml_oracle_ragged_logits(
            _ptr(q), case.H, case.D, _ptr(w), _ptr(k), _ptr(ksc), case.N, _ptr(ks), _ptr(ke),
            _ptr(rows), len(rows), col_begin, col_end, _ptr(out))
    return out


def topk(scores: np.ndarray, ke, k: int, ks=None) -> np.ndarray:
    """Per-row top-k positions (relative to ks) in ascending order, -1 padded."""
    s = np.ascontiguousarray(scores, dtype=np.float64)
    rows = s.shape[0]
    ke_a = np.ascontiguousarray(ke, dtype=np.int32)
    ks_a = None if ks is None else np.ascontiguousarray(ks, dtype=np.int32)
    out = np.empty((rows, k), dtype=np.int32)
    if rows:
        lib().pml_oracle_topk(_ptr(s), rows, s.shape[1], None if ks_a is None else _ptr(ks_a),
                              _ptr(ke_a), k, _ptr(out))
    return out


def dcp_global_id(p: int, rank: int, world: int, interleave: int) -> int:
    """Global token id of local position p on ``rank`` (runs of ``interleave`` tokens dealt in turn)."""
    return lib().pml_oracle_dcp_global_id(p, rank, world, interleave)


def dcp_pack(logits: np.ndarray, topk_local: np.ndarray, rank: int, world: int, interleave: int,
             ks=None) -> np.ndarray:
    """One rank's (score, global id) float32 pairs [rows][k][2]; padding is (-inf, -1)."""
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    tk = np.ascontiguousarray(topk_local, dtype=np.int32)
    rows, k = tk.shape
    ks_a = None if ks is None else np.ascontiguousarray(ks, dtype=np.int32)
    out = np.empty((rows, k, 2), dtype=np.float32)
    if rows and k:
        lib().pml_oracle_dcp_pack(_ptr(lg), rows, lg.shape[1], None if ks_a is None else _ptr(ks_a),
                                  _ptr(tk), tk.shape[1], k, rank, world, interleave, _ptr(out))
    return out


def dcp_merge(gathered: np.ndarray, k: int) -> np.ndarray:
    """Global top-k ids [rows][k] (ascending, -1 padded) from [world][rows][k][2] candidates."""
    g = np.ascontiguousarray(gathered, dtype=np.float32)
    world, rows = g.shape[0], g.shape[1]
    assert g.shape == (world, rows, k, 2)
    out = np.empty((rows, k), dtype=np.int32)
    if rows and k:
        lib().pml_oracle_dcp_merge(_ptr(g), world, rows, k, _ptr(out))
    return out


def bf16_round(x) -> np.ndarray:
    """bf16 bits (uint16) of float32 values, rounded to nearest, ties to even.

    bf16 is the upper half of an IEEE binary32 (1 sign, 8 exponent, 7 mantissa
    bits). Rounding the binary32 magnitude to a multiple of 2^16 units in the
    last place, ties to the even result, is rounding to the nearest bf16; a
    carry out of the mantissa moves to the next binade or to infinity, as it
    should. NaN maps to the quiet NaN 0x7fc0 with the input's sign."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    return np.where(nan, ((u >> 16) & 0x8000).astype(np.uint16) | np.uint16(0x7FC0), r).astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    """float32 value of bf16 bits: the 16 bits as the upper half of a binary32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def num_threads() -> int:
    return lib().pml_oracle_num_threads()


def set_num_threads(n: int) -> None:
    lib().pml_oracle_set_num_threads(int(n))
