"""Specification of the work split returned by the metadata call (test infrastructure).

The pages size this output by the number of persistent workers (the caller
reads the SM count back from the schedule's first dimension, sparse_attn_indexer
page, _varlen_decode_rows) and give a row slice a schedule of its own. The
content is this library's own definition, stated here in plain Python:

* Rows are grouped as the varlen decode path groups them ("[Bugfix]
  [GLM-5.3-Flash] ...", Purpose: consecutive equal request indices are one
  request): with ``indices`` a group is a maximal run of equal consecutive ids;
  without, a group is the ``next_n`` rows of one batch entry.
* A group is cut into pieces of at most ``G_MAX`` consecutive rows.
* A piece's extent is the largest visible length among its rows; it has
  ``nblk = ceil(extent / step)`` key blocks of ``step = max(block_kv, 64)``
  tokens (a step of a 32-token cache is two pages), each costing ``COST_BASE + g``
  (g = rows in the piece: a page read and the fixed work of a step, then g
  rows of scoring; a one-row block takes about half the time of a six-row
  one).
* Units (piece, block) are ordered by piece then block and cut into C
  ranges, one per logits workgroup. Range c starts at the unit holding cost
  offset floor(c * T / C) of the total T; entry C is the end sentinel
  (num_rows, 0).

Entries are (first row of the piece, block offset within the piece).
"""
from __future__ import annotations

import numpy as np

G_MAX = 8
COST_BASE = 3
MIN_STEP = 64  # tokens per unit: a block_kv 32 cache is taken two pages at a time


def step_tokens(block_kv: int) -> int:
    return max(block_kv, MIN_STEP)


def visible_lengths(context_lens: np.ndarray, num_rows: int, next_n: int, lens_2d: bool) -> np.ndarray:
    lens = np.asarray(context_lens, dtype=np.int64).reshape(-1)
    if lens_2d or next_n == 1:
        v = lens[:num_rows].copy()
    else:
        r = np.arange(num_rows)
        v = lens[r // next_n] - next_n + (r % next_n) + 1
    return np.maximum(v, 0)


def pieces(num_rows: int, next_n: int, indices) -> list[tuple[int, int]]:
    """(first row, row count) of every piece, in row order."""
    out = []
    r = 0
    while r < num_rows:
        if indices is not None:
            end = r
            while end < num_rows and indices[end] == indices[r]:
                end += 1
        else:
            end = min(num_rows, (r // next_n + 1) * next_n)
        s = r
        while s < end:
            g = min(G_MAX, end - s)
            out.append((s, g))
            s += g
        r = end
    return out


def piece_table(context_lens, num_rows, next_n, lens_2d, indices, block_kv):
    vis = visible_lengths(context_lens, num_rows, next_n, lens_2d)
    idx = None if indices is None else np.asarray(indices).reshape(-1)
    table = []
    for s, g in pieces(num_rows, next_n, idx):
        ext = int(vis[s: s + g].max())
        nblk = -(-ext // step_tokens(block_kv))
        table.append((s, g, nblk, nblk * (COST_BASE + g)))
    return table


def schedule(context_lens, num_rows: int, next_n: int, lens_2d: bool, indices, block_kv: int,
             num_chunks: int) -> np.ndarray:
    table = piece_table(context_lens, num_rows, next_n, lens_2d, indices, block_kv)
    total = sum(t[3] for t in table)
    out = np.zeros((num_chunks + 1, 2), dtype=np.int32)
    out[num_chunks] = (num_rows, 0)
    if total == 0:
        out[:] = (num_rows, 0)
        return out
    # targets grow with c, so one forward walk over the pieces finds them all
    p, cum = 0, 0
    for c in range(num_chunks):
        target = c * total // num_chunks
        while not (cum <= target < cum + table[p][3]):
            cum += table[p][3]
            p += 1
        s, g, nblk, cost = table[p]
        out[c] = (s, (target - cum) // (COST_BASE + g))
    return out


def units_of_chunk(sched: np.ndarray, table, c: int) -> list[tuple[int, int]]:
    """Enumerate the (first row, block) units of chunk c."""
    start = tuple(sched[c])
    end = tuple(sched[c + 1])
    units = []
    for s, g, nblk, cost in table:
        for b in range(nblk):
            if start <= (s, b) < end:
                units.append((s, b))
    return units
