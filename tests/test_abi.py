"""The C-ABI library loads, exports every call its header declares, and rejects
bad arguments on the host before launching anything (CPU only: every call here
returns an error status before it would touch a GPU)."""
import ctypes
import re
from pathlib import Path

import pytest

import paged_mqa_logits_amd as pml

HEADER = Path(__file__).resolve().parents[1] / "include" / "pml.h"


def _declared():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_four_calls():
    names = _declared()
    for n in ("paged_mqa_logits_metadata", "fp8_fp4_paged_mqa_logits", "mqa_logits", "top_k_per_row",
              "top_k_per_row_workspace_size", "pml_status_string", "pml_version",
              "pack_dcp_topk_candidates", "stable_topk_from_gathered_candidates",
              "fp8_fp4_paged_mqa_logits_bf16", "as_fp32_logits", "fp8_fp4_paged_mqa_logits_fp4q",
              "fp8_fp4_paged_mqa_logits_workspace_size", "paged_mqa_logits_schedule_rows"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = pml.lib()
    missing = [n for n in _declared() if not hasattr(L, n)]
    assert not missing, missing


def test_schedule_rows():
    """The schedule has one row per worker plus the end, so a caller reads the
    worker count back as schedule.shape[0] - 1 (sparse_attn_indexer page,
    _varlen_decode_rows)."""
    L = pml.lib()
    for W in (1, 7, 512, 1 << 20):
        assert L.paged_mqa_logits_schedule_rows(W) == W + 1
        assert pml.schedule_rows(W) == W + 1
    for W in (0, -3, (1 << 20) + 1):
        assert L.paged_mqa_logits_schedule_rows(W) == -1
    import torch
    sched = torch.empty(pml.schedule_rows(37), 2)
    assert pml.schedule_workers(sched) == 37 == sched.shape[0] - 1
    with pytest.raises(ValueError):
        pml.schedule_workers(torch.empty(1, 2))


def _ws_bytes(rows, W):
    r = lambda b: (b + 255) // 256 * 256
    # pieces of u per row (4 x 128 fp8 codes, then 4 x 4 e8m0 scale bytes), a split
    # point per range (2 x int32) and 8 pool counters 128 bytes apart
    return r(512 * rows) + r(16 * rows) + r(8 * W) + r(8 * 128)


def test_logits_workspace_size():
    f = pml.lib().fp8_fp4_paged_mqa_logits_workspace_size
    for rows in (0, 1, 135, 4097):
        for W in (1, 4, 512, 1 << 20):
            assert f(rows, W) == _ws_bytes(rows, W)
    assert f(-1, 512) == 0 and f(4, 0) == 0 and f(4, (1 << 20) + 1) == 0


def test_status_strings_and_version():
    assert pml.status_string(0) == "ok"
    for code in range(1, 12):
        assert pml.status_string(code) != "unknown status"
    assert pml.status_string(999) == "unknown status"
    assert pml.lib().pml_version() >= 10000


P = ctypes.c_void_p
FAKE = P(0x1000)  # never dereferenced: every call below fails validation first


WS = P(0x100000)  # 256-B aligned, never dereferenced


def _paged(**kw):
    a = dict(q=FAKE, qs=None, rows=4, next_n=1, H=64, D=128, kv=FAKE, fmt=0, bkv=64, stride=64 * 132, pages=10,
             w=FAKE, lens=FAKE, l2d=0, bt=FAKE, bt_ld=8, bt_cols=8, sched=FAKE, cus=4, idx=None,
             max_ctx=512, out=FAKE, ld=512, ws=WS, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return pml.lib().fp8_fp4_paged_mqa_logits(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(H=32), 2), (dict(D=64), 2), (dict(rows=-1), 2), (dict(cus=0), 2), (dict(cus=(1 << 20) + 1), 2),
    (dict(fmt=2), 9), (dict(bkv=16), 3), (dict(idx=FAKE, next_n=2, rows=4), 4),
    (dict(rows=5, next_n=2), 2), (dict(q=None), 1), (dict(bt=None), 1),
    (dict(stride=64 * 132 - 16), 5), (dict(stride=64 * 132 + 4), 5), (dict(ld=500), 5),
    (dict(ld=514, max_ctx=513), 5), (dict(pages=0), 5), (dict(bt_cols=9), 5),
    (dict(fmt=1, bkv=32, stride=32 * 68 - 16), 5),
    (dict(q=P(0x1001)), 6), (dict(out=P(0x1004)), 6), (dict(sched=P(0x1008)), 6),
    # q_scale (fp4 q) needs MXFP4 keys and 16-B alignment
    (dict(qs=FAKE), 10), (dict(qs=P(0x1008), fmt=1, bkv=32, stride=32 * 68), 6),
    # the workspace: missing, one byte too small for 4 rows and 4 workgroups, misaligned
    (dict(ws=None), 8), (dict(ws_bytes=_ws_bytes(4, 4) - 1), 8), (dict(ws=P(0x100010)), 6),
])
def test_paged_validation(kw, code):
    assert _paged(**kw) == code


def test_paged_workspace_exact_size_passes_validation():
    # the smallest valid workspace gets past every host check (a NULL block table is then the first error)
    assert _paged(ws_bytes=_ws_bytes(4, 4), bt=None) == 1


def test_paged_zero_rows_is_ok_without_gpu():
    assert _paged(rows=0) == 0


def test_metadata_validation():
    f = pml.lib().paged_mqa_logits_metadata
    assert f(FAKE, 4, 1, 0, None, 64, 4, None, None) == 1
    assert f(FAKE, 4, 1, 0, None, 48, 4, FAKE, None) == 3
    assert f(FAKE, 4, 2, 0, FAKE, 64, 4, FAKE, None) == 4
    assert f(FAKE, 5, 2, 0, None, 64, 4, FAKE, None) == 2
    assert f(FAKE, 4, 1, 0, None, 64, 0, FAKE, None) == 2
    assert f(FAKE, 4, 1, 0, None, 64, (1 << 20) + 1, FAKE, None) == 2
    assert f(None, 4, 1, 0, None, 64, 4, FAKE, None) == 1
    assert f(FAKE, 4, 1, 0, None, 64, 4, P(0x1008), None) == 6


def _pack(**kw):
    a = dict(logits=FAKE, rows=4, ld=1024, rs=None, topk=FAKE, topk_ld=64, k=64, rank=1, world=4, il=1,
             packed=FAKE, stream=None)
    a.update(kw)
    return pml.lib().pack_dcp_topk_candidates(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(rows=-1), 2), (dict(ld=-4), 2), (dict(k=0), 7), (dict(k=4097, topk_ld=5000), 7),
    (dict(world=0, rank=0), 2), (dict(rank=4), 2), (dict(rank=-1), 2), (dict(il=0), 2),
    (dict(logits=None), 1), (dict(topk=None), 1), (dict(packed=None), 1), (dict(topk_ld=63), 5),
    (dict(packed=P(0x1004)), 6),
    # ids must stay exact in float32: local position 2^21 of rank 0 of 8, interleave 1, is id 2^24
    (dict(ld=(1 << 21) + 1, world=8, rank=0), 2),
])
def test_pack_validation(kw, code):
    assert _pack(**kw) == code


def test_pack_id_limit_edge_and_zero_rows():
    # local position 2^21 - 1 on rank 7 of 8, interleave 1: global id 2^24 - 1, the largest allowed
    assert _pack(rows=0, ld=(1 << 21), world=8, rank=7) == 0
    assert _pack(rows=0, ld=(1 << 21) + 1, world=8, rank=7) == 2
    assert _pack(rows=0) == 0


def _merge(**kw):
    a = dict(g=FAKE, world=8, rows=4, k=2048, out=FAKE, out_ld=2048, stream=None)
    a.update(kw)
    return pml.lib().stable_topk_from_gathered_candidates(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(rows=-1), 2), (dict(world=0), 2), (dict(k=0), 7), (dict(k=4097, out_ld=5000), 7),
    (dict(world=9, k=4096, out_ld=4096), 2), (dict(g=None), 1), (dict(out=None), 1),
    (dict(out_ld=2047), 5), (dict(g=P(0x1004)), 6),
])
def test_merge_validation(kw, code):
    assert _merge(**kw) == code


def test_merge_zero_rows_and_largest_pairs():
    assert _merge(rows=0) == 0
    assert _merge(rows=0, world=8, k=4096, out_ld=4096) == 0


def _paged_bf16(**kw):
    a = dict(q=FAKE, rows=4, next_n=1, H=64, D=128, kv=FAKE, fmt=0, bkv=64, stride=64 * 132, pages=10,
             w=FAKE, lens=FAKE, l2d=0, bt=FAKE, bt_ld=8, bt_cols=8, sched=FAKE, cus=4, idx=None,
             max_ctx=512, out=FAKE, ld=512, ws=WS, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return pml.lib().fp8_fp4_paged_mqa_logits_bf16(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(H=32), 2), (dict(fmt=2), 9), (dict(bkv=16), 3), (dict(q=None), 1), (dict(out=None), 1),
    (dict(ld=508), 5), (dict(ld=516, max_ctx=512), 5), (dict(ld=500), 5), (dict(out=P(0x1008)), 6),
    (dict(ws=None), 8),
])
def test_paged_bf16_validation(kw, code):
    assert _paged_bf16(**kw) == code


def test_paged_bf16_zero_rows():
    assert _paged_bf16(rows=0) == 0


def _upcast(**kw):
    a = dict(src=FAKE, rows=4, ld=1024, cols=1000, ends=FAKE, out=FAKE, out_ld=1024, stream=None)
    a.update(kw)
    return pml.lib().as_fp32_logits(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(rows=-1), 2), (dict(cols=-1), 2), (dict(src=None), 1), (dict(ends=None), 1), (dict(out=None), 1),
    (dict(ld=1020), 5), (dict(ld=996), 5), (dict(out_ld=998), 5), (dict(out_ld=996), 5),
    (dict(src=P(0x1008)), 6), (dict(out=P(0x1004)), 6),
    # one chunk past 65535 x 2048 columns
    (dict(cols=134215681, ld=134215688, out_ld=134215688), 2),
])
def test_upcast_validation(kw, code):
    assert _upcast(**kw) == code


def _ragged(**kw):
    a = dict(q=FAKE, M=16, heads=64, dim=128, k=FAKE, k_scale=FAKE, N=1000, w=FAKE, ks=FAKE, ke=FAKE,
             out=FAKE, ld=1000, stream=None)
    a.update(kw)
    return pml.lib().mqa_logits(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), 2), (dict(N=-1), 2), (dict(heads=32), 2), (dict(dim=64), 2),
    (dict(M=524281), 2), (dict(N=2 ** 31 - 256, ld=2 ** 31), 2),
    (dict(q=None), 1), (dict(k_scale=None), 1), (dict(ke=None), 1), (dict(out=None), 1),
    (dict(ld=996), 5), (dict(ld=1002), 5),
    (dict(q=P(0x1008)), 6), (dict(k=P(0x1004)), 6), (dict(out=P(0x1008)), 6), (dict(k_scale=P(0x1002)), 6),
])
def test_ragged_validation(kw, code):
    assert _ragged(**kw) == code


def test_ragged_empty_is_ok_without_gpu():
    assert _ragged(M=0) == 0
    assert _ragged(N=0) == 0
    assert _ragged(M=0, q=None, out=None) == 0


def test_upcast_empty_is_ok():
    assert _upcast(rows=0) == 0
    assert _upcast(cols=0) == 0


def _paged_fp4q(**kw):
    a = dict(q=FAKE, qs=FAKE, rows=4, next_n=1, H=64, D=128, kv=FAKE, fmt=1, bkv=32, stride=32 * 68, pages=10,
             w=FAKE, lens=FAKE, l2d=0, bt=FAKE, bt_ld=8, bt_cols=8, sched=FAKE, cus=4, idx=None,
             max_ctx=256, out=FAKE, ld=256, ws=WS, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return pml.lib().fp8_fp4_paged_mqa_logits_fp4q(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(fmt=0, bkv=64, stride=64 * 132), 10), (dict(fmt=0, bkv=64, stride=64 * 132, rows=0), 10),
    (dict(ws=None), 8),
    (dict(qs=None), 1), (dict(q=None), 1), (dict(qs=P(0x1008)), 6), (dict(H=32), 2), (dict(bkv=16), 3),
    (dict(ld=252), 5),
])
def test_paged_fp4q_validation(kw, code):
    assert _paged_fp4q(**kw) == code


def test_paged_fp4q_zero_rows():
    assert _paged_fp4q(rows=0, qs=None) == 0


def _fused(**kw):
    a = dict(q=FAKE, rows=4, next_n=1, H=64, D=128, kv=FAKE, fmt=0, bkv=64, stride=64 * 132, pages=10,
             w=FAKE, lens=FAKE, l2d=0, bt=FAKE, bt_ld=8, bt_cols=8, sched=FAKE, cus=4, idx=None,
             max_ctx=512, out=FAKE, ld=512, k=64, topk=FAKE, topk_ld=64, ws=P(0x100000),
             ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return pml.lib().fp8_fp4_paged_mqa_logits_topk(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(k=0), 7), (dict(k=4097), 7), (dict(H=32), 2), (dict(bkv=16), 3), (dict(topk=None), 1),
    (dict(topk_ld=63), 5), (dict(ws=None), 8), (dict(ws_bytes=100), 8), (dict(ws=P(0x100010)), 6),
    (dict(q=None), 1), (dict(ld=500), 5),
])
def test_fused_validation(kw, code):
    assert _fused(**kw) == code


def test_fused_workspace_size():
    f = pml.lib().fp8_fp4_paged_mqa_logits_topk_workspace_size
    # the logits call's workspace, then 3 x [rows] int32 regions + counts [rows][nb]
    # + pairs [rows][nb * bkv][2], each 256-B aligned
    rows, mc, bkv, k, W = 135, 131072, 64, 2048, 512
    nb = mc // bkv
    r = lambda b: (b + 255) // 256 * 256
    logits_ws = pml.lib().fp8_fp4_paged_mqa_logits_workspace_size(rows, W)
    assert f(rows, mc, bkv, k, W) == logits_ws + 3 * r(4 * rows) + r(4 * rows * nb) + r(8 * rows * nb * bkv)
    assert f(rows, mc, 48, k, W) == 0 and f(rows, mc, bkv, 0, W) == 0 and f(-1, mc, bkv, k, W) == 0
    assert _fused(rows=0, topk=None, ws=None) == 0


def _noalloc(**kw):
    a = dict(q=FAKE, qs=None, rows=4, next_n=1, H=64, D=128, kv=FAKE, fmt=0, bkv=64, stride=64 * 132, pages=10,
             w=FAKE, lens=FAKE, l2d=0, bt=FAKE, bt_ld=8, bt_cols=8, sched=FAKE, cus=4, idx=None,
             max_ctx=512, out=FAKE, ld=512, stream=None)
    a.update(kw)
    return pml.lib().fp8_fp4_paged_mqa_logits_noalloc(*a.values())


def test_noalloc_limits_and_validation_without_gpu():
    # beyond the static scratch: rejected on the host, nothing launched
    assert _noalloc(rows=4097) == 12 and _noalloc(cus=4097) == 12
    assert pml.status_string(12) != "unknown status"
    # the checks of the main call, before any device query
    assert _noalloc(rows=0) == 0 and _noalloc(rows=-1) == 2 and _noalloc(H=32, rows=0) == 2

def _topk_bf16(**kw):
    a = dict(logits=FAKE, rows=4, ld=1024, ks=None, ke=FAKE, next_n=1, k=64, max_width=1024, out=FAKE, out_ld=64,
             ws=None, wbytes=0, stream=None)
    a.update(kw)
    return pml.lib().top_k_per_row_bf16(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(rows=-1), 2), (dict(next_n=0), 2), (dict(max_width=-1), 2), (dict(k=0), 7), (dict(k=4097), 7),
    (dict(logits=None), 1), (dict(ke=None), 1), (dict(out=None), 1), (dict(out_ld=63), 5),
    (dict(ld=1020), 5), (dict(ld=1028), 5), (dict(logits=P(0x1008)), 6),
])
def test_topk_bf16_validation(kw, code):
    assert _topk_bf16(**kw) == code


def test_topk_bf16_zero_rows():
    assert _topk_bf16(rows=0) == 0
