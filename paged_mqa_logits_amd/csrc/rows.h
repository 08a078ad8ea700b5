// Row bookkeeping of the decode path: visible lengths, groups and row-pieces.
//
// Groups follow the varlen decode rule ("[Bugfix][GLM-5.3-Flash] Fix
// fp8_fp4_paged_mqa_logits MQA kpool varlen path", Purpose): rows with equal
// consecutive request ids belong together; without ids, the next_n rows of a
// batch entry do. A row-piece is at most kGMax consecutive rows of one group,
// counted from the group's first row; its rows are scored against each key
// block that is read once for all of them.
//
// Everything here is wave-uniform and read through the scalar cache, so that
// the vector-memory counter only ever counts the key-page loads in flight.
#pragma once

#include "pml_device.h"

namespace pml {

// Load through the scalar data cache (constant address space). `idx` must be
// wave-uniform; the pointed-to data must not change during the kernel.
template <typename T>
__device__ __forceinline__ T sload(const T *base, int64_t idx) {
    typedef __attribute__((address_space(4))) const T cT;
    return ((cT *)base)[idx];
}


struct RowView {
    const int32_t *lens;
    const int32_t *indices;  // nullable
    int lens_2d;
    int next_n;
    int num_rows;

    // Tokens row r sees: its own length (varlen / next_n == 1 / 2-D lengths),
    // else len[b] - next_n + j + 1 for row j of entry b. Per-lane (vector) read.
    __device__ __forceinline__ int visible(int r) const {
        int v;
        if (lens_2d || next_n == 1)
            v = lens[r];
        else
            v = lens[r / next_n] - next_n + (r % next_n) + 1;
        return v > 0 ? v : 0;
    }
    // The same for a wave-uniform row, through the scalar cache.
    __device__ __forceinline__ int visible_s(int r) const {
        int v;
        if (lens_2d || next_n == 1)
            v = sload(lens, r);
        else
            v = sload(lens, r / next_n) - next_n + (r % next_n) + 1;
        return v > 0 ? v : 0;
    }
    __device__ __forceinline__ bool same_group(int r, int r0) const {
        return indices ? (indices[r] == indices[r0]) : (r / next_n == r0 / next_n);
    }
    __device__ __forceinline__ bool same_group_s(int r, int r0) const {
        return indices ? (sload(indices, r) == sload(indices, r0)) : (r / next_n == r0 / next_n);
    }
};

// Rows and key-block count of the piece starting at row r0 (r0 < num_rows,
// wave-uniform). The piece extent is the largest visible length of its rows.
// The lengths and ids of all kGMax candidate rows are requested up front (rows
// past the end re-read row r0), so their scalar loads overlap.
template <int BKV>
__device__ __forceinline__ void piece_at(const RowView &v, int r0, int &g, int &nblk) {
    int vis[kGMax];
    bool same[kGMax];
    const int id0 = v.indices ? sload(v.indices, r0) : 0;
#pragma unroll
    for (int i = 0; i < kGMax; ++i) {
        const int r = r0 + i < v.num_rows ? r0 + i : r0;
        vis[i] = v.visible_s(r);
        same[i] = r0 + i < v.num_rows &&
                  (v.indices ? sload(v.indices, r) == id0 : r / v.next_n == r0 / v.next_n);
    }
    int gg = 1, e = vis[0];
    bool go = true;
#pragma unroll
    for (int i = 1; i < kGMax; ++i) {
        go = go && same[i];
        if (go) {
            e = max(e, vis[i]);
            gg = i + 1;
        }
    }
    g = uni(gg);
    nblk = uni((e + BKV - 1) / BKV);
}

}  // namespace pml
