"""Per-row top-k over bf16 logits on the GPU (top_k_per_row_bf16).

A bf16 is the upper half of the fp32 with the same value, so the selection
over bf16 logits must equal, bit for bit, both the fp32 call's selection over
the exact upcast values and the oracle's top-k over those values. The rows
cover every path of the two kernels: rows of at most 8192 columns (registers),
rows that fit the candidate list, the exact streaming passes, the sampled
path of rows of 16K columns or more, and the list overflow of heavy ties
(bf16's 8-bit significand makes ties common), with NaN, -0 and -inf.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_mqa_logits_amd as pml
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _bf16_tensor(bits: np.ndarray, ld: int) -> torch.Tensor:
    rows, w = bits.shape
    buf = np.full((rows, ld), 0xFFC1, dtype=np.uint16)  # a NaN past each row's columns
    buf[:, :w] = bits
    return torch.from_numpy(buf.view(np.int16)).to(G.dev()).view(torch.bfloat16)


def _check(bits: np.ndarray, ke, k: int, ks=None, next_n: int = 1, max_width=None):
    rows, w = bits.shape
    ld = (w + 7) // 8 * 8 + 8
    d = G.dev()
    b16 = _bf16_tensor(bits, ld)
    f32 = b16.float()  # exact: the upcast values
    ket = torch.from_numpy(np.asarray(ke, dtype=np.int32)).to(d)
    kst = None if ks is None else torch.from_numpy(np.asarray(ks, dtype=np.int32)).to(d)
    mw = w if max_width is None else max_width
    got = pml.top_k_per_row(b16, ket, k, ks=kst, next_n=next_n, max_width=mw)
    via = pml.top_k_per_row(f32, ket, k, ks=kst, next_n=next_n, max_width=mw)
    torch.cuda.synchronize()
    got, via = got.cpu().numpy(), via.cpu().numpy()
    np.testing.assert_array_equal(got, via)
    ke_rows = np.asarray(ke)
    if next_n > 1:
        r = np.arange(rows)
        ke_rows = ke_rows[r // next_n] - next_n + (r % next_n) + 1
    vals = oracle.bf16_to_f32(bits).astype(np.float64)
    np.testing.assert_array_equal(got, oracle.topk(vals, np.minimum(ke_rows, w), k, ks=ks))
    return got


def _rows(rng, w):
    rows = [rng.standard_normal(w),
            np.round(rng.standard_normal(w) * 4),            # heavy ties
            np.zeros(w)]                                     # every value equal
    r = rng.standard_normal(w)
    r[::3] = 0.0
    r[1::3] = -0.0
    rows.append(r)
    r = rng.standard_normal(w)
    r[w // 3:] = -np.inf
    rows.append(r)
    r = rng.standard_normal(w)
    r[rng.random(w) < 0.4] = np.nan
    rows.append(r)
    rows.append(np.arange(w, dtype=np.float64))              # ascending
    return oracle.bf16_round(np.stack(rows).astype(np.float32))


@pytest.mark.parametrize("w", [700, 5000, 8192])
def test_bf16_rows_in_registers(w):
    rng = np.random.default_rng(1000 + w)
    bits = _rows(rng, w)
    n = bits.shape[0]
    G.banner(f"bf16 top-k, {w}-column rows (registers)")
    for k in (1, 64, 2048):
        _check(bits, [w] * n, k)
    ke = rng.integers(0, w + 1, n)
    _check(bits, ke, 100)
    ks = rng.integers(0, w // 2, n)
    _check(bits, np.full(n, w), 333, ks=ks)


@pytest.mark.parametrize("w", [12288, 15000, 40000, 70000])
def test_bf16_wide_rows(w):
    """List path (<= 12288), exact streaming passes, sampled path (>= 16K),
    and the overflow of ties."""
    rng = np.random.default_rng(1100 + w)
    bits = _rows(rng, w)
    n = bits.shape[0]
    G.banner(f"bf16 top-k, {w}-column rows")
    for k in (1, 2048, 4096):
        _check(bits, [w] * n, k)
    ke = np.maximum(rng.integers(w // 2, w + 1, n), 1)
    _check(bits, ke, 2048)


def test_bf16_random_bits_and_next_n():
    """Every bf16 bit pattern (NaNs of both signs, infinities, subnormals) and
    next_n rows."""
    rng = np.random.default_rng(1200)
    bits = rng.integers(0, 1 << 16, (12, 20000), dtype=np.uint32).astype(np.uint16)
    G.banner("bf16 top-k, random bits")
    _check(bits, [20000] * 12, 2048)
    _check(bits, rng.integers(5000, 20001, 4), 777, next_n=3)
    _check(bits[:, :6000], [6000] * 12, 512)
