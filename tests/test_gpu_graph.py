"""The decode step (schedule -> logits -> top-k) captured in a HIP graph.

The calls allocate nothing, never synchronise and clear nothing with memset,
so a captured step must reproduce the eager step bit for bit on every replay,
also with other work on the stream between the replays.
"""
import numpy as np
import pytest
import torch

import paged_mqa_logits_amd as pml
import pml_synth as syn
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def test_captured_step_matches_eager_on_every_replay():
    case = syn.make_paged_case([3000, 700, 5000, 64], [3, 1, 6, 2], seed=900, max_ctx=5120)
    other = syn.make_paged_case([4000, 100], [2, 5], seed=901, max_ctx=5120)
    d = G.dev()
    t = G.upload(case)
    u = G.upload(other)
    W = pml.default_num_workers()
    sched = torch.empty(pml.schedule_rows(W), 2, dtype=torch.int32, device=d)
    logits = torch.empty(case.rows, pml.logits_ld(case.max_ctx), dtype=torch.float32, device=d)
    topk = torch.empty(case.rows, 64, dtype=torch.int32, device=d)
    ws = torch.empty(pml.logits_workspace_size(case.rows, W), dtype=torch.uint8, device=d)

    def step(x, c):
        pml.paged_mqa_logits_metadata(x["lens"], c.block_kv, W, indices=x["indices"], out=sched)
        pml.fp8_fp4_paged_mqa_logits(x["q"], x["kv"], x["w"], x["lens"], x["bt"], sched, c.max_ctx, x["indices"],
                                     kv_format=c.kv_format, block_kv=c.block_kv, logits=logits, workspace=ws)
        pml.top_k_per_row(logits, x["lens"], 64, max_width=c.max_ctx, out=topk)

    G.banner("graph capture of the decode step")
    step(t, case)
    torch.cuda.synchronize()
    want = (sched.clone(), logits.clone(), topk.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(t, case)
    torch.cuda.synchronize()
    for rep in range(4):
        # other eager work on the same buffers between replays
        sched.fill_(-7)
        logits.fill_(123.0)
        topk.fill_(-5)
        ws.fill_(0x7F)
        if rep % 2:
            oth = torch.empty(other.rows, pml.logits_ld(other.max_ctx), dtype=torch.float32, device=d)
            pml.fp8_fp4_paged_mqa_logits(u["q"], u["kv"], u["w"], u["lens"], u["bt"],
                                         pml.paged_mqa_logits_metadata(u["lens"], other.block_kv, W,
                                                                       indices=u["indices"]),
                                         other.max_ctx, u["indices"], kv_format=other.kv_format,
                                         block_kv=other.block_kv, logits=oth)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(sched, want[0]), f"replay {rep}: schedule differs"
        np.testing.assert_array_equal(logits.cpu().numpy(), want[1].cpu().numpy(), err_msg=f"replay {rep}")
        assert torch.equal(topk, want[2]), f"replay {rep}: top-k differs"


def test_captured_prefill_step_matches_eager_on_every_replay():
    """The prefill step (ragged logits -> top-k) and the bf16 decode top-k in
    one graph: no memsets, no allocation, the same bits on every replay."""
    case = syn.make_ragged_case([300, 1, 700, 129], seed=905)
    dec = syn.make_paged_case([2000, 90], [2, 3], seed=906, max_ctx=2048)
    d = G.dev()
    q, k, ksc, w = case.q.to(d), case.k.to(d), case.k_scale.to(d), case.weights.to(d)
    ks, ke = case.ks.to(d), case.ke.to(d)
    logits = torch.empty(case.M, pml.logits_ld(case.N), dtype=torch.float32, device=d)
    topk = torch.empty(case.M, 64, dtype=torch.int32, device=d)
    mw = int((case.ke - case.ks).clamp_min(0).max())
    u = G.upload(dec)
    sched = pml.paged_mqa_logits_metadata(u["lens"], dec.block_kv, None, indices=u["indices"])
    b16 = pml.fp8_fp4_paged_mqa_logits(u["q"], u["kv"], u["w"], u["lens"], u["bt"], sched, dec.max_ctx,
                                       u["indices"], out_dtype=torch.bfloat16)
    topk16 = torch.empty(dec.rows, 100, dtype=torch.int32, device=d)

    def step():
        pml.mqa_logits(q, k, ksc, w, ks, ke, logits=logits)
        pml.top_k_per_row(logits, ke, 64, ks=ks, max_width=mw, out=topk)
        pml.top_k_per_row(b16, u["lens"], 100, max_width=dec.max_ctx, out=topk16)

    G.banner("graph capture of the prefill step and the bf16 top-k")
    step()
    torch.cuda.synchronize()
    want = (logits.clone(), topk.clone(), topk16.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        logits.fill_(123.0)
        topk.fill_(-5)
        topk16.fill_(-5)
        if rep % 2:
            pml.mqa_logits(q, k, ksc, w, ks, ks + 1, logits=torch.empty_like(logits))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        # (columns past N are never written: compare the written ones)
        np.testing.assert_array_equal(logits[:, : case.N].cpu().numpy().view(np.uint32),
                                      want[0][:, : case.N].cpu().numpy().view(np.uint32), err_msg=f"replay {rep}")
        assert torch.equal(topk, want[1]), f"replay {rep}: prefill top-k differs"
        assert torch.equal(topk16, want[2]), f"replay {rep}: bf16 top-k differs"
