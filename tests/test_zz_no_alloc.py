"""The allocation-free logits call (fp8_fp4_paged_mqa_logits_noalloc) against
the workspace call, through the C ABI: the same kernels with the library's
static per-GPU scratch, so the logits must be the same bits. Two calls in a
row, the second with fewer rows and workgroups, so that scratch contents left
by the first call cannot leak into the second."""
import numpy as np
import pytest
import torch

import oracle
import paged_mqa_logits_amd as pml
import pml_synth as syn
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _both(case, W):
    t = G.upload(case)
    sched = pml.paged_mqa_logits_metadata(t["lens"], case.block_kv, W, indices=t["indices"], next_n=case.next_n)
    outs = []
    for ws in (None, "static"):
        out = torch.full((case.rows, pml.logits_ld(case.max_ctx)), G.SENTINEL, dtype=torch.float32, device=G.dev())
        pml.fp8_fp4_paged_mqa_logits(t["q"], t["kv"], t["w"], t["lens"], t["bt"], sched, case.max_ctx, t["indices"],
                                     kv_format=case.kv_format, block_kv=case.block_kv, next_n=case.next_n,
                                     logits=out, q_scale=t["qs"], workspace=ws)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    return outs


def test_noalloc_equals_workspace_call_twice_shrinking():
    big = syn.make_paged_case([3000, 700, 5000, 64, 1200], [3, 1, 6, 2, 4], seed=940, max_ctx=5120)
    small = syn.make_paged_case([900, 33], [2, 1], seed=941, max_ctx=1024)
    G.banner(f"no-alloc call: {big.rows} rows, W 512, then {small.rows} rows, W 37")
    a, b = _both(big, 512)
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))
    G.assert_logits_close(b[:, : big.max_ctx], oracle.paged_logits(big), big.weights, "no-alloc big")
    a, b = _both(small, 37)
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))
    G.assert_logits_close(b[:, : small.max_ctx], oracle.paged_logits(small), small.weights, "no-alloc small")


def test_noalloc_mxfp4_fp4q_and_limit():
    case = syn.make_paged_case([700, 64, 1500], [2, 4, 1], seed=942, kv_format=1, block_kv=32, max_ctx=1536,
                               q_fp4=True)
    G.banner("no-alloc call: MXFP4 keys with fp4 q")
    a, b = _both(case, 64)
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))
    # more rows than the static scratch holds: refused before anything runs
    d = G.dev()
    q = torch.zeros(4097, 64, 128, dtype=torch.uint8, device=d)
    lens = torch.ones(4097, dtype=torch.int32, device=d)
    sched = pml.paged_mqa_logits_metadata(lens, 64, 8)
    with pytest.raises(ValueError, match="allocation-free"):
        pml.fp8_fp4_paged_mqa_logits(q, torch.zeros(4, 64 * 132, dtype=torch.uint8, device=d),
                                     torch.zeros(4097, 64, device=d), lens,
                                     torch.zeros(4097, 1, dtype=torch.int32, device=d), sched, 64,
                                     workspace="static")
