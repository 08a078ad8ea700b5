// mqa_logits: non-paged (ragged prefill) logits. Query row r is scored on the
// keys [cu_seqlen_ks[r], cu_seqlen_ke[r]) of a contiguous fp8 key array and is
// -inf on every other column of the dense [M][N] output (the dense M*N logits
// tensor whose size the prefill chunking bounds, sparse_attn_indexer page,
// forward_cpu: per-row lengths ke - ks).
//
// Grid (x = chunk of key blocks, y = piece of kGMax consecutive rows; the chunk
// is as wide as still gives about kTargetWGs workgroups: whole rows at prefill sizes).
// A workgroup stages q and w of its rows in LDS; its 4 waves take the chunk's
// blocks that intersect the union of the rows' key ranges in turn, loading 64
// keys at a time into VGPRs (three buffers deep) and scoring them with the
// core of logits_core.h, as in the paged kernel. The chunk's other columns of
// its rows are filled with -inf, a slice per block step, and nothing is read
// for them, so a causal prefill does about half the work of the dense
// product.
#include <type_traits>

#include "logits_core.h"
#include "rows.h"

namespace pml {

constexpr int kMinChunk = 32;      // key blocks per workgroup, at least
constexpr int kTargetWGs = 4096;   // workgroups the grid aims for (about 8 per CU, in turn)

struct RaggedArgs {
    const uint8_t *q;
    const float *w;
    const uint8_t *k;
    const float *k_scale;
    int N;
    const int32_t *ks;
    const int32_t *ke;
    int M;
    float *out;
    int64_t out_ld;
    int chunk;  // key blocks per workgroup
};

// A wave's share of a piece's -inf columns, written a slice per step of its
// block loop, so the fill's stores spread over the scoring instead of
// preceding it (they go out before the step's key loads, like the logit
// stores). The wave takes rows i = wave, wave + kCW, ... of the piece; each
// row has a left region [c0, lend) and a right region [rs, re), both starting
// on a multiple of 64 columns, re a multiple of 4 (a row's last columns past
// re are stored at set-up). One store instruction covers 256 columns of a
// region. All fields are wave-uniform.
struct NegFill {
    float *out;
    int64_t out_ld;
    int row0, g, wave;
    int c0, lend, rs, re;  // the piece's regions (the same for every row)
    int item;              // next region: row wave + kCW * (item / 2), side item % 2
    float *base;           // current row
    int col, end;          // current region [col, end)
    bool active;

    __device__ bool next_region() {
        while (true) {
            const int i = wave + kCW * (item >> 1);
            if (i >= g) return false;
            const int side = item & 1;
            ++item;
            const int s = side ? rs : c0, e = side ? re : lend;
            if (e > s) {
                base = out + (int64_t)(row0 + i) * out_ld;
                col = s;
                end = e;
                return true;
            }
        }
    }
    // store instructions for all of this wave's regions
    __device__ int count() const {
        const int rows = g > wave ? (g - wave + kCW - 1) / kCW : 0;
        const int per_row = (max(lend - c0, 0) + 255) / 256 + (max(re - rs, 0) + 255) / 256;
        return rows * per_row;
    }
    __device__ void init() {
        item = 0;
        active = next_region();
    }
    // up to n store instructions
    __device__ void slice(int n) {
        const int lane = lane_id();
        const float ninf = -__builtin_inff();
        const v4f pat = {ninf, ninf, ninf, ninf};
        for (int t = 0; t < n && active; ++t) {
            const int c = col + 4 * lane;
            if (c < end) store_v4f_async(base + c, pat);
            col += 256;
            if (col >= end) active = next_region();
        }
    }
};

// One step of a wave's block loop (see wave_step of the paged kernel); every
// row of the piece is stored, -inf outside its [lo, hi) (lane i of lo_lane /
// hi_lane holds the bounds of row i). Rows go in quads, the linear half of a
// quad scored once (lin_quad).
template <bool PF>
__device__ __forceinline__ void ragged_step(const RaggedArgs &a, int row0, int g, int b,
                                            const KeyRegs<false, 64> &kc, int bp, KeyRegs<false, 64> &kp,
                                            const uint8_t *s_q, const float *s_w, const uint8_t *s_u,
                                            const uint8_t *s_us, int lo_lane, int hi_lane, WaveSlot<64> &sl,
                                            int &mask, int &col0p, NegFill &fill, int fill_per) {
    touch<false, 64>(kc);
    flush_slot<64>(sl, mask, row0, col0p, a.N, a.out, a.out_ld);
    fill.slice(fill_per);
    if constexpr (PF) load_contig(a.k, a.k_scale, a.N, bp * 64, kp);
    const int lane = lane_id();
    const int s = b * 64 + lane;
    const float scale = 0.5f * __uint_as_float(kc.sc[0]);  // 1/2: see score_row
    // (both quads unrolled: the rows' LDS operand addresses become immediates)
#pragma unroll
    for (int q0 = 0; q0 < kGMax; q0 += 4) {
        if (q0 >= g) break;
        float M[4];
#pragma unroll
        for (int G = 0; G < 4; ++G) {
            const int i = q0 + G;
            if (i >= g) break;
            const int lo = __builtin_amdgcn_readlane(lo_lane, i);
            const int hi = __builtin_amdgcn_readlane(hi_lane, i);
            const float sr = G == 0 ? score_row<false, 64, false, true>(kc, s_q + i * kQBytes, s_w + i * PML_HEADS,
                                                                        s_u, s_us, q0 >> 2, M)
                                    : score_row<false, 64>(kc, s_q + i * kQBytes, s_w + i * PML_HEADS);
            float v = (sr + M[G]) * scale;
            if (b * 64 < lo || b * 64 + 64 > hi)  // (wave-uniform: only blocks that cross a bound are masked)
                if (s < lo || s >= hi) v = -__builtin_inff();
            lds_st<float>(&sl.v[i][lane], v);
        }
    }
    mask = (1 << g) - 1;
    col0p = b * 64;
}

__global__ __launch_bounds__(kLThreads, 2) void ragged_logits_kernel(RaggedArgs a) {
    constexpr int BKV = 64;
    __shared__ __attribute__((aligned(16))) uint8_t s_q[kGMax * kQBytes];
    __shared__ __attribute__((aligned(16))) float s_w[kGMax * PML_HEADS];
    __shared__ __attribute__((aligned(16))) uint8_t s_u[kGMax * kUBytes];
    __shared__ __attribute__((aligned(16))) uint8_t s_us[kGMax * kUScales];
    __shared__ int s_lo[kGMax];
    __shared__ int s_hi[kGMax];
    __shared__ __attribute__((aligned(16))) WaveSlot<BKV> s_slot[kCW];

    const int tid = threadIdx.x;
    const int wave = uni(tid / kWave);
    const int N = a.N;
    // pieces go out last-rows-first: in a causal prefill those see the most
    // keys, so the longest workgroups start first and the short ones fill the tail
    const int row0 = (gridDim.y - 1 - blockIdx.y) * kGMax;
    const int g = uni(min(kGMax, a.M - row0));

    // the union of the piece's key ranges, as key blocks
    int lo_min = N, hi_max = 0;
    for (int i = 0; i < g; ++i) {
        const int lo = min(max(sload(a.ks, row0 + i), 0), N);
        const int hi = min(max(sload(a.ke, row0 + i), lo), N);
        if (hi > lo) {
            lo_min = min(lo_min, lo);
            hi_max = max(hi_max, hi);
        }
    }
    const int nb = (N + BKV - 1) / BKV;
    const int c0 = blockIdx.x * a.chunk;
    const int c1 = min(c0 + a.chunk, nb);
    int u_lo = c0, u_hi = c0;  // blocks of this chunk to score
    if (hi_max > lo_min) {
        u_lo = uni(max(lo_min / BKV, c0));
        u_hi = uni(min((hi_max + BKV - 1) / BKV, c1));
        if (u_hi < u_lo) u_hi = u_lo;
    }

    // -inf on the chunk's columns that are not scored: all at once when
    // nothing is scored, else a slice per step (NegFill) plus, here, each
    // row's last columns past a multiple of 4
    const int cend = min(c1 * BKV, N);
    if (u_hi <= u_lo) {
        for (int i = 0; i < g; ++i) fill_neg_inf(a.out + (int64_t)(row0 + i) * a.out_ld, c0 * BKV, cend);
        return;
    }
    const int rs = min(u_hi * BKV, cend);       // a multiple of 64, or cend
    const int re = max(rs, cend & ~3);
    if (tid < g * 4 && re + (tid & 3) < cend)    // at most 3 columns a row
        a.out[(int64_t)(row0 + (tid >> 2)) * a.out_ld + re + (tid & 3)] = -__builtin_inff();
    NegFill fill{a.out, a.out_ld, row0, g, wave, c0 * BKV, u_lo * BKV, rs, re};
    fill.init();

    stage_rows(a.q, a.w, row0, g, s_q, s_w);
    if (tid < g) {
        const int lo = min(max(a.ks[row0 + tid], 0), N);
        s_lo[tid] = lo;
        s_hi[tid] = min(max(a.ke[row0 + tid], lo), N);
    }
    barrier_lds();
    derive_pieces<false>(s_q, s_w, g, s_u, s_us);
    barrier_lds();

    const int lo_lane = lds_ld<int>(&s_lo[lane_id() % kGMax]);  // lane i: bounds of row i
    const int hi_lane = lds_ld<int>(&s_hi[lane_id() % kGMax]);
    const int b0 = u_lo + wave;
    if (b0 >= u_hi) {
        fill.slice(fill.count());  // no blocks for this wave: its share of the fill at once
        return;
    }
    const int nmy = (u_hi - b0 + kCW - 1) / kCW;  // this wave's blocks
    const int fill_per = (fill.count() + nmy - 1) / nmy;  // fill stores per step
    WaveSlot<BKV> &sl = s_slot[wave];
    KeyRegs<false, BKV> k0, k1, k2;
    int mask = 0, col0p = 0;
    auto step = [&](const KeyRegs<false, BKV> &kc, int j, KeyRegs<false, BKV> &kp, auto pf) {
        ragged_step<decltype(pf)::value>(a, row0, g, b0 + kCW * j, kc, b0 + kCW * (j + 2), kp, s_q, s_w, s_u, s_us,
                                         lo_lane, hi_lane, sl, mask, col0p, fill, fill_per);
    };
    constexpr std::true_type PF{};
    constexpr std::false_type NOPF{};
    if (nmy >= 3) {
        // every step of the main loop requests a block (see the paged kernel)
        load_contig(a.k, a.k_scale, N, b0 * BKV, k0);
        load_contig(a.k, a.k_scale, N, (b0 + kCW) * BKV, k1);
        for (int j = 0;;) {
            if (j + 2 >= nmy) {
                step(k0, j, k2, NOPF);
                step(k1, j + 1, k2, NOPF);
                break;
            }
            step(k0, j, k2, PF);
            ++j;
            if (j + 2 >= nmy) {
                step(k1, j, k0, NOPF);
                step(k2, j + 1, k0, NOPF);
                break;
            }
            step(k1, j, k0, PF);
            ++j;
            if (j + 2 >= nmy) {
                step(k2, j, k1, NOPF);
                step(k0, j + 1, k1, NOPF);
                break;
            }
            step(k2, j, k1, PF);
            ++j;
        }
    } else {
        load_contig(a.k, a.k_scale, N, b0 * BKV, k0);
        if (nmy > 1) load_contig(a.k, a.k_scale, N, (b0 + kCW) * BKV, k1);
        step(k0, 0, k2, NOPF);
        if (nmy > 1) step(k1, 1, k2, NOPF);
    }
    flush_slot<BKV>(sl, mask, row0, col0p, N, a.out, a.out_ld);
    fill.slice(fill.count());  // (nothing is left: every step took its share)
}

}  // namespace pml

static inline bool al16r(const void *p) { return ((uintptr_t)p & 15) == 0; }

extern "C" int mqa_logits(const void *q, int M, int num_heads, int head_dim, const void *k,
                          const float *k_scale, int N, const float *weights,
                          const int32_t *cu_seqlen_ks, const int32_t *cu_seqlen_ke, float *logits,
                          int64_t logits_ld, void *stream) {
    if (M < 0 || N < 0) return PML_ERR_SHAPE;
    if (num_heads != PML_HEADS || head_dim != PML_HEAD_DIM) return PML_ERR_SHAPE;
    if (M == 0 || N == 0) return PML_OK;  // nothing to write
    if (!q || !k || !k_scale || !weights || !cu_seqlen_ks || !cu_seqlen_ke || !logits) return PML_ERR_NULL;
    if (logits_ld < N || logits_ld % 4 != 0) return PML_ERR_STRIDE;
    if (!al16r(q) || !al16r(k) || !al16r(weights) || !al16r(logits)) return PML_ERR_ALIGN;
    if (((uintptr_t)k_scale & 3) != 0) return PML_ERR_ALIGN;
    // Key chunks per row: as few as give about kTargetWGs workgroups, at least
    // kMinChunk blocks wide. Few, long workgroups keep the CUs on scoring work;
    // a grid of many chunks spends its time starting workgroups that only fill
    // -inf (measured: a causal 32K x 32K prefill took 3.5 ms in 32-block chunks,
    // 1.3 ms in whole rows).
    const int nb = (N + 63) / 64;
    const int pieces = (M + pml::kGMax - 1) / pml::kGMax;
    const int max_chunks = (nb + pml::kMinChunk - 1) / pml::kMinChunk;
    const int want = (pml::kTargetWGs + pieces - 1) / pieces;
    const int nchunks = want < max_chunks ? want : max_chunks;
    const int chunk = (nb + nchunks - 1) / nchunks;
    pml::RaggedArgs a{(const uint8_t *)q, weights, (const uint8_t *)k, k_scale, N, cu_seqlen_ks,
                      cu_seqlen_ke, M, logits, logits_ld, chunk};
    const dim3 grid((nb + chunk - 1) / chunk, pieces);
    if (grid.y > 65535) return PML_ERR_SHAPE;
    hipLaunchKernelGGL(pml::ragged_logits_kernel, grid, dim3(pml::kLThreads), 0, (hipStream_t)stream, a);
    return hipGetLastError() == hipSuccess ? PML_OK : PML_ERR_HIP;
}
