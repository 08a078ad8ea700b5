// Workgroup helpers of the radix selections (per-row top-k and the merge of
// gathered candidates): the order-preserving key of a float, a block-wide
// scan, and the search for the histogram bin that holds the kk-th largest key.
#pragma once
#include "pml_device.h"

namespace pml {

// Order-preserving 32-bit key of a float: larger float, larger key; NaN below
// every number; -0 equal to +0.
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN sorts below every number
    if (u == 0x80000000u) u = 0u;                    // -0 counts as +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive scan of one uint32 per lane over the wave, by DPP moves (no LDS
// traffic): shifts by 1, 2, 4, 8 lanes inside each row of 16, then row 0's
// and row 2's last lanes into rows 1 and 3 (row_bcast:15), then lane 31 into
// rows 2 and 3 (row_bcast:31). A lane whose source lies outside its row, or
// whose row the row mask leaves out, adds 0.
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}

// Inclusive scan of one uint32 per thread over the workgroup; *total gets the
// sum. Each wave scans its lanes, publishes its total, and every thread adds
// the totals of the waves before its own.
template <int NT>
__device__ __forceinline__ uint32_t block_scan(uint32_t x, uint32_t *s_wave, uint32_t *total) {
    constexpr int NW = NT / kWave;
    const int wave = threadIdx.x / kWave;
    const uint32_t incl = wave_scan_incl(x);
    if (lane_id() == kWave - 1) s_wave[wave] = incl;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint32_t t = s_wave[w];
        before += w < wave ? t : 0u;
        tot += t;
    }
    *total = tot;
    __syncthreads();  // s_wave is free for the next scan
    return incl + before;
}

// Exclusive prefix over the wave's lanes of c (0 <= c <= 4), and the wave total.
__device__ __forceinline__ void wave_prefix4(uint32_t c, uint32_t &pre, uint32_t &tot) {
    pre = 0;
    tot = 0;
#pragma unroll
    for (int b = 0; b < 3; ++b) {
        const uint64_t m = __ballot((c >> b) & 1u);
        const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        pre += below << b;
        tot += (uint32_t)__popcll(m) << b;
    }
}

// Find the bin holding the kk-th largest key among bins [0, nbins) whose
// counts count(b) gives: writes (bin, count of keys in higher bins) to s_pick.
template <int NT, typename C>
__device__ __forceinline__ void pick_bin_by(C count, int nbins, uint32_t kk, uint32_t *s_wave, uint32_t *s_pick) {
    const int per = (nbins + NT - 1) / NT;
    const int t = threadIdx.x;
    // thread t owns bins top - t*per - j, j < per (descending)
    uint32_t own = 0;
    for (int j = 0; j < per; ++j) {
        const int b = nbins - 1 - (t * per + j);
        if (b >= 0) own += count(b);
    }
    uint32_t tot;
    uint32_t above = block_scan<NT>(own, s_wave, &tot) - own;
    for (int j = 0; j < per; ++j) {
        const int b = nbins - 1 - (t * per + j);
        if (b < 0) break;
        const uint32_t h = count(b);
        if (above < kk && kk <= above + h) {
            s_pick[0] = (uint32_t)b;
            s_pick[1] = above;
        }
        above += h;
    }
    __syncthreads();
}

template <int NT>
__device__ __forceinline__ void pick_bin(const uint32_t *s_hist, int nbins, uint32_t kk, uint32_t *s_wave,
                                         uint32_t *s_pick) {
    pick_bin_by<NT>([&](int b) { return s_hist[b]; }, nbins, kk, s_wave, s_pick);
}

}  // namespace pml
