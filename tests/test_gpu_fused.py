"""The fused logits + top-k call on the GPU.

The call must write the same logits as fp8_fp4_paged_mqa_logits and the same
top-k as top_k_per_row over them, bit for bit, whichever way each row is
settled: from the candidates the logits kernel keeps, or by the full top-k
when the candidates cannot settle it (too few, too many, too wide). The done
flags in the workspace tell which rows took which way; the cases are chosen
so that both ways occur. The top-k is also checked against the oracle's
top-k over the same logits.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_mqa_logits_amd as pml
import pml_synth as syn
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _ws_done(ws: torch.Tensor, rows: int, num_cus: int) -> np.ndarray:
    base = pml.logits_workspace_size(rows, num_cus)  # the logits call's region comes first
    reg = (4 * rows + 255) // 256 * 256  # then thresholds, widths, done flags: [rows] each
    return ws[base + 2 * reg: base + 2 * reg + 4 * rows].view(torch.int32).cpu().numpy()


def _check(case, k, t=None):
    t = t or G.upload(case)
    d = G.dev()
    sched = pml.paged_mqa_logits_metadata(t["lens"], case.block_kv, None, indices=t["indices"], next_n=case.next_n)
    ref_logits = pml.fp8_fp4_paged_mqa_logits(t["q"], t["kv"], t["w"], t["lens"], t["bt"], sched, case.max_ctx,
                                              t["indices"], kv_format=case.kv_format, block_kv=case.block_kv,
                                              next_n=case.next_n)
    ke = t["lens"].reshape(-1)
    nn = 1 if case.lens_2d else case.next_n
    ref_topk = pml.top_k_per_row(ref_logits, ke, k, next_n=nn, max_width=case.max_ctx)
    need = pml.fused_topk_workspace_size(case.rows, case.max_ctx, case.block_kv, k, pml.schedule_workers(sched))
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=d)  # garbage-filled: no initialisation needed
    logits, topk = pml.fp8_fp4_paged_mqa_logits_topk(t["q"], t["kv"], t["w"], t["lens"], t["bt"], sched,
                                                     case.max_ctx, k, t["indices"], kv_format=case.kv_format,
                                                     block_kv=case.block_kv, next_n=case.next_n, workspace=ws)
    torch.cuda.synchronize()
    L = logits.cpu().numpy()[:, : case.max_ctx]
    np.testing.assert_array_equal(L.view(np.uint32), ref_logits.cpu().numpy()[:, : case.max_ctx].view(np.uint32))
    got = topk.cpu().numpy()
    np.testing.assert_array_equal(got, ref_topk.cpu().numpy())
    vis = np.minimum(oracle.visible_lengths(case), case.max_ctx)
    np.testing.assert_array_equal(got, oracle.topk(L.astype(np.float64), vis, k))
    done = _ws_done(ws, case.rows, pml.schedule_workers(sched))
    print(f"[gpu-check] fused top-k k={k}: {int(done.sum())} of {case.rows} rows from candidates", flush=True)
    return done, vis


PATHS = {"cand": 0, "full": 0}


def _count(done, vis, k):
    wide = vis > k
    PATHS["cand"] += int((done[wide] == 1).sum())
    PATHS["full"] += int((done[wide] == 0).sum())


@pytest.mark.parametrize("fmt,bkv,k", [(0, 64, 64), (0, 32, 128), (1, 32, 64), (1, 64, 100)])
def test_fused_varlen_small(fmt, bkv, k):
    ctx = [1300, 1, 64, 90, 2100, 777, 3000]
    case = syn.make_paged_case(ctx, [2, 1, 3, 1, 11, 6, 2], seed=1100 + fmt * 10 + bkv, kv_format=fmt,
                               block_kv=bkv, max_ctx=3072, fp4_spread=6)
    G.banner(f"fused varlen small fmt={fmt} bkv={bkv} k={k}")
    _count(*_check(case, k), k)


@pytest.mark.parametrize("lens_2d", [False, True])
def test_fused_uniform_next_n(lens_2d):
    case = syn.make_paged_case([700, 3, 1290, 1500, 64], [3] * 5, seed=1120, varlen=False, next_n=3,
                               lens_2d=lens_2d, max_ctx=1503)
    G.banner(f"fused uniform next_n=3 2d={lens_2d}")
    _count(*_check(case, 50), 50)


def test_fused_tiny_config():
    case = syn.config_tiny_decode()
    G.banner("fused tiny decode")
    _count(*_check(case, case.topk), case.topk)


def test_fused_ties_and_bad_entries_fall_back():
    """Rows whose q is all zero score 0 everywhere (every column ties at the
    threshold: too many candidates); a bad table entry makes NaN logits."""
    case = syn.make_paged_case([3000, 2500, 2800, 900], [1, 1, 1, 1], seed=1130, max_ctx=3072)
    case.q[1].zero_()
    bt = case.block_table.clone()
    bt[2, 3] = -7
    c2 = syn.PagedCase(**{**case.__dict__, "block_table": bt})
    G.banner("fused ties / NaN rows")
    done, vis = _check(c2, 64)
    assert done[1] == 0, "an all-tied row cannot be settled by candidates"
    _count(done, vis, 64)


@pytest.mark.parametrize("k", [2048, 4096])
def test_fused_uniform_config(k):
    case = syn.config_uniform_decode()
    G.banner(f"fused uniform 32K k={k}")
    _count(*_check(case, k), k)


def test_fused_varlen_120k_config():
    case = G.named_case("varlen_fp8")
    G.banner(f"fused varlen 120K rows={case.rows}")
    done, vis = _check(case, case.topk)
    _count(done, vis, case.topk)
    assert done.all(), "the 120K decode rows should all be settled by candidates"


def test_fused_mxfp4_config():
    case = G.named_case("varlen_fp4")
    G.banner(f"fused MXFP4 64K rows={case.rows}")
    _count(*_check(case, case.topk), case.topk)


def test_zz_both_paths_were_taken():
    if PATHS["cand"] + PATHS["full"] == 0:
        pytest.skip("needs the other tests of this file in the same run")
    assert PATHS["cand"] > 0 and PATHS["full"] > 0, PATHS
