// mqa_logits: non-paged (ragged prefill) logits. Query row r is scored on the
// keys [cu_seqlen_ks[r], cu_seqlen_ke[r]) of a contiguous fp8 key array and is
// -inf on every other column of the dense [M][N] output (the dense M*N logits
// tensor whose size the prefill chunking bounds, sparse_attn_indexer page,
// forward_cpu: per-row lengths ke - ks).
//
// Grid (x = chunk of kChunk key blocks, y = piece of kGMax consecutive rows).
// A workgroup scores the blocks of its chunk that intersect the union of its
// rows' key ranges with the shared tile pipeline (logits_core.h), and fills the
// chunk's other columns of its rows with -inf. Nothing is read for masked
// blocks, so a causal prefill does about half the work of the dense product.
#include "logits_core.h"
#include "rows.h"

namespace pml {

constexpr int kChunk = 32;  // key blocks per workgroup

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
};

__global__ __launch_bounds__(kThreads, 2) void ragged_logits_kernel(RaggedArgs a) {
    constexpr int BKV = 64;
    using C = TileCfg<false, BKV>;
    __shared__ __attribute__((aligned(16))) uint8_t s_stage[kStages][C::TILE];
    __shared__ __attribute__((aligned(16))) float s_red[kGMax][kWaves][BKV];
    __shared__ int s_lo[kGMax];
    __shared__ int s_hi[kGMax];

    const int tid = threadIdx.x;
    const int N = a.N;
    const int row0 = blockIdx.y * kGMax;
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
    const int c0 = blockIdx.x * kChunk;
    const int c1 = min(c0 + kChunk, nb);
    int u_lo = c0, u_hi = c0;  // blocks of this chunk to score
    if (hi_max > lo_min) {
        u_lo = uni(max(lo_min / BKV, c0));
        u_hi = uni(min((hi_max + BKV - 1) / BKV, c1));
        if (u_hi < u_lo) u_hi = u_lo;
    }

    // -inf on the chunk's columns that are not scored
    const int cend = min(c1 * BKV, N);
    for (int i = 0; i < g; ++i) {
        float *row = a.out + (int64_t)(row0 + i) * a.out_ld;
        if (u_hi > u_lo) {
            fill_neg_inf(row, c0 * BKV, u_lo * BKV);
            fill_neg_inf(row, min(u_hi * BKV, cend), cend);
        } else {
            fill_neg_inf(row, c0 * BKV, cend);
        }
    }
    const int nunits = u_hi - u_lo;
    if (nunits <= 0) return;

    v8i qa[kGMax];
    v4f w4[kGMax];
#pragma unroll
    for (int i = 0; i < kGMax; ++i)
        if (i < g) load_row<false>(a.q, a.w, row0 + i, qa[i], w4[i]);
    int lo = 0, hi = 0;
    if (tid < g) {
        lo = min(max(a.ks[row0 + tid], 0), N);
        hi = min(max(a.ke[row0 + tid], lo), N);
    }
    // Everything above has landed before the first key tile is requested, so
    // the per-tile waits below count tile loads (and logit stores) only.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    asm volatile("" ::: "memory");
    if (tid < g) {
        lds_write_i32(lds_addr(&s_lo[tid]), lo);
        lds_write_i32(lds_addr(&s_hi[tid]), hi);
    }

#pragma unroll
    for (int k = 0; k < kStages - 1; ++k)
        if (k < nunits) issue_contig<BKV>(a.k, a.k_scale, N, (u_lo + k) * BKV, s_stage[k]);

    for (int u = 0; u < nunits; ++u) {
        // tile u has landed once at most (kStages - 2) tiles issued after it are in flight
        const int ahead = min(nunits, u + kStages - 1) - (u + 1);
        if (ahead >= kStages - 2)
            wait_vmcnt<(kStages - 2) * C::NLD>();
        else
            wait_vmcnt<0>();
        barrier_lds();
        if (u + kStages - 1 < nunits)
            issue_contig<BKV>(a.k, a.k_scale, N, (u_lo + u + kStages - 1) * BKV,
                              s_stage[(u + kStages - 1) % kStages]);
        const uint8_t *st = s_stage[u % kStages];
        score_tile<false, BKV>(st, qa, w4, g, s_red);
        barrier_lds();
        store_tile<false, BKV>(st, s_red, s_lo, s_hi, g, row0, (u_lo + u) * BKV, N, true, false, a.out,
                               a.out_ld);
    }
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
    pml::RaggedArgs a{(const uint8_t *)q, weights, (const uint8_t *)k, k_scale, N, cu_seqlen_ks,
                      cu_seqlen_ke, M, logits, logits_ld};
    const int nb = (N + 63) / 64;
    const dim3 grid((nb + pml::kChunk - 1) / pml::kChunk, (M + pml::kGMax - 1) / pml::kGMax);
    if (grid.y > 65535) return PML_ERR_SHAPE;
    hipLaunchKernelGGL(pml::ragged_logits_kernel, grid, dim3(pml::kThreads), 0, (hipStream_t)stream, a);
    return hipGetLastError() == hipSuccess ? PML_OK : PML_ERR_HIP;
}
