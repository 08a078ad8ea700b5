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

// Maximum of one uint32 per lane over the wave (DPP row shifts, then row
// broadcasts); the result is valid in lane 63.
__device__ __forceinline__ uint32_t wave_max_to_last(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false));  // row_shr:1
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false));  // row_shr:2
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false));  // row_shr:4
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false));  // row_shr:8
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));  // row_bcast:15
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));  // row_bcast:31
    return v;
}

// Workgroup maxima of (a, b) (s_wave: 2 * NT / 64 words; all threads get them).
template <int NT>
__device__ __forceinline__ void block_max2(uint32_t &a, uint32_t &b, uint32_t *s_wave) {
    constexpr int NW = NT / kWave;
    const int wave = threadIdx.x / kWave;
    const uint32_t wa = wave_max_to_last(a), wb = wave_max_to_last(b);
    if (lane_id() == kWave - 1) {
        s_wave[wave] = wa;
        s_wave[NW + wave] = wb;
    }
    __syncthreads();
    a = 0;
    b = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        a = max(a, s_wave[w]);
        b = max(b, s_wave[NW + w]);
    }
    __syncthreads();
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

// pick_bin for nbins = NT * PER (PER 2, 4 or 8): thread t's bins, the PER
// consecutive ones ending at nbins - t * PER, read once with 8- or 16-byte
// loads and kept in registers for both the sum and the search (pick_bin reads
// each bin twice, one word at a time). Same result as pick_bin. s_hist must be
// 16-byte aligned.
template <int NT, int PER>
__device__ __forceinline__ void pick_bin_vec(const uint32_t *s_hist, uint32_t kk, uint32_t *s_wave,
                                             uint32_t *s_pick) {
    static_assert(PER == 2 || PER == 4 || PER == 8, "8- or 16-byte loads");
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    const int base = (NT - 1 - (int)threadIdx.x) * PER;  // bins [base, base + PER)
    uint32_t h[PER];
    if constexpr (PER == 2) {
        const u2 v = *(const u2 *)(s_hist + base);
        h[0] = v[0];
        h[1] = v[1];
    } else {
#pragma unroll
        for (int c = 0; c < PER / 4; ++c) {
            const u4 v = *(const u4 *)(s_hist + base + 4 * c);
            h[4 * c] = v[0]; h[4 * c + 1] = v[1]; h[4 * c + 2] = v[2]; h[4 * c + 3] = v[3];
        }
    }
    uint32_t own = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) own += h[j];
    uint32_t tot;
    uint32_t above = block_scan<NT>(own, s_wave, &tot) - own;
#pragma unroll
    for (int j = PER - 1; j >= 0; --j) {  // descending bins
        if (above < kk && kk <= above + h[j]) {
            s_pick[0] = (uint32_t)(base + j);
            s_pick[1] = above;
        }
        above += h[j];
    }
    __syncthreads();
}

template <int NT>
__device__ __forceinline__ void pick_bin(const uint32_t *s_hist, int nbins, uint32_t kk, uint32_t *s_wave,
                                         uint32_t *s_pick) {
    pick_bin_by<NT>([&](int b) { return s_hist[b]; }, nbins, kk, s_wave, s_pick);
}

// One radix pass: histogram of bits [shift, shift + log2(nbins)) of key(i)
// over the pairs live(i) whose key matches prefix under mask, then the bin of
// the kk-th largest. Returns that bin's count; s_pick holds (bin, count above).
template <int NT, int P, typename K, typename L>
__device__ __forceinline__ uint32_t radix_pass(K key, L live, uint32_t prefix, uint32_t mask, int shift, int nbins,
                                               uint32_t kk, uint32_t *s_hist, uint32_t *s_wave, uint32_t *s_pick) {
    for (int b = threadIdx.x; b < nbins; b += NT) s_hist[b] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const uint32_t x = key(i);
        if (live(i) && (x & mask) == prefix) atomicAdd(&s_hist[(x >> shift) & (nbins - 1)], 1u);
    }
    __syncthreads();
    pick_bin<NT>(s_hist, nbins, kk, s_wave, s_pick);
    const uint32_t cnt = s_hist[s_pick[0]];
    __syncthreads();
    return cnt;
}

// Value of lane (lane ^ m) of the wave, m a power of two below 64 (a
// constant once the caller's loops are unrolled).
__device__ __forceinline__ int32_t lane_xor(int32_t v, int m) {
    switch (m) {
        case 1: return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xf, 0xf, false);   // quad_perm [1,0,3,2]
        case 2: return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xf, 0xf, false);   // quad_perm [2,3,0,1]
        case 4: return __builtin_amdgcn_ds_swizzle(v, 0x101F);                       // xor 4 in 32 lanes
        case 8: return __builtin_amdgcn_update_dpp(0, v, 0x128, 0xf, 0xf, false);  // row_ror:8 = xor 8
        case 16: return __builtin_amdgcn_ds_swizzle(v, 0x401F);                      // xor 16 in 32 lanes
        default: return __shfl_xor(v, 32, kWave);
    }
}

constexpr int kSortThreads = 256;  // the four waves that run the sort

// Ascending bitonic sort of s[0, kSortThreads * E): every thread of the
// workgroup calls it (it holds the barriers); threads below kSortThreads load
// entries t * E .. t * E + E - 1 from s, sort, and leave them in x.
template <int E>
__device__ __forceinline__ void bitonic_sort(int32_t (&x)[E], int32_t *s) {
    constexpr int NS = kSortThreads * E;
    const int t = threadIdx.x;
    const bool active = t < kSortThreads;
    if (active) {
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = s[t * E + e];
    }
#pragma unroll
    for (int sz = 2; sz <= NS; sz <<= 1) {
#pragma unroll
        for (int j = sz >> 1; j > 0; j >>= 1) {
            if (j < E) {
                if (active) {
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        if ((e & j) == 0) {
                            const bool asc = ((t * E + e) & sz) == 0;
                            const int32_t lo = min(x[e], x[e | j]), hi = max(x[e], x[e | j]);
                            x[e] = asc ? lo : hi;
                            x[e | j] = asc ? hi : lo;
                        }
                }
                continue;
            }
            int32_t y[E];
            if (j < kWave * E) {
                if (!active) continue;
#pragma unroll
                for (int e = 0; e < E; ++e) y[e] = lane_xor(x[e], j / E);
            } else {
                __syncthreads();  // earlier reads of s are done
                if (active) {
#pragma unroll
                    for (int e = 0; e < E; ++e) s[t * E + e] = x[e];
                }
                __syncthreads();
                if (!active) continue;
#pragma unroll
                for (int e = 0; e < E; ++e) y[e] = s[(t * E + e) ^ j];
            }
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int i = t * E + e;
                const bool keep_low = ((i & j) == 0) == ((i & sz) == 0);
                x[e] = keep_low ? min(x[e], y[e]) : max(x[e], y[e]);
            }
        }
    }
}

}  // namespace pml
