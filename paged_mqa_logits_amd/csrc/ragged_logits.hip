// mqa_logits: non-paged (ragged prefill) logits. Query row r is scored on the
// keys [cu_seqlen_ks[r], cu_seqlen_ke[r]) of a contiguous fp8 key array and is
// -inf on every other column of the dense [M][N] output (the dense M*N logits
// tensor whose size the prefill chunking bounds, sparse_attn_indexer page,
// forward_cpu: per-row lengths ke - ks).
//
// Grid (x = chunk of kChunk key blocks, y = piece of kGMax consecutive rows).
// A workgroup stages q and w of its rows in LDS; its 4 waves take the chunk's
// blocks that intersect the union of the rows' key ranges in turn, loading 64
// keys at a time into VGPRs (double-buffered) and scoring them with the core
// of logits_core.h. The chunk's other columns of its rows are filled with
// -inf, and nothing is read for them, so a causal prefill does about half the
// work of the dense product.
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

__device__ __forceinline__ void ragged_block(int g, int b, const KeyRegs<false, 64> &k, const uint8_t *s_q,
                                             const float *s_w, const int *s_lo, const int *s_hi, Pending &p) {
    const int s = b * 64 + lane_id();
    const float scale = __uint_as_float(k.sc[0]);
    p.mask = 0;
    p.col0 = b * 64;
#pragma unroll
    for (int i = 0; i < kGMax; ++i) {
        if (i < g) {
            const int lo = uni(lds_ld<int>(&s_lo[i]));
            const int hi = uni(lds_ld<int>(&s_hi[i]));
            float v = score_row<false, 64>(k, s_q + i * kQBytes, s_w + i * PML_HEADS) * scale;
            if (s < lo || s >= hi) v = -__builtin_inff();
            p.v[i] = v;
            p.mask |= 1 << i;
        }
    }
}

__device__ __forceinline__ void ragged_store(const RaggedArgs &a, int row0, const Pending &p) {
    const int s = p.col0 + lane_id();
#pragma unroll
    for (int i = 0; i < kGMax; ++i)
        if ((p.mask >> i) & 1)
            if (s < a.N) a.out[(int64_t)(row0 + i) * a.out_ld + s] = p.v[i];
}

// One step of a wave's block loop: wait for the current block, store the
// previous block's logits, request the next block, score the current one.
__device__ __forceinline__ void ragged_step(const RaggedArgs &a, int row0, int g, int u_hi,
                                            const KeyRegs<false, 64> &kc, int bc, KeyRegs<false, 64> &kn, int bn,
                                            const uint8_t *s_q, const float *s_w, const int *s_lo, const int *s_hi,
                                            Pending &p) {
    touch<false, 64>(kc);
    ragged_store(a, row0, p);
    if (bn < u_hi) load_contig(a.k, a.k_scale, a.N, bn * 64, kn);
    ragged_block(g, bc, kc, s_q, s_w, s_lo, s_hi, p);
}

__global__ __launch_bounds__(kThreads, 2) void ragged_logits_kernel(RaggedArgs a) {
    constexpr int BKV = 64;
    __shared__ __attribute__((aligned(16))) uint8_t s_q[kGMax * kQBytes];
    __shared__ __attribute__((aligned(16))) float s_w[kGMax * PML_HEADS];
    __shared__ int s_lo[kGMax];
    __shared__ int s_hi[kGMax];

    const int tid = threadIdx.x;
    const int wave = uni(tid / kWave);
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
    if (u_hi <= u_lo) return;

    stage_rows(a.q, a.w, row0, g, s_q, s_w);
    if (tid < g) {
        const int lo = min(max(a.ks[row0 + tid], 0), N);
        s_lo[tid] = lo;
        s_hi[tid] = min(max(a.ke[row0 + tid], lo), N);
    }
    barrier_lds();

    int b = u_lo + wave;
    if (b >= u_hi) return;
    KeyRegs<false, BKV> k0, k1;
    load_contig(a.k, a.k_scale, N, b * BKV, k0);
    Pending p;
    p.mask = 0;
    p.col0 = 0;
    for (;;) {
        const int b1 = b + kWaves;
        ragged_step(a, row0, g, u_hi, k0, b, k1, b1, s_q, s_w, s_lo, s_hi, p);
        if (b1 >= u_hi) break;
        const int b2 = b1 + kWaves;
        ragged_step(a, row0, g, u_hi, k1, b1, k0, b2, s_q, s_w, s_lo, s_hi, p);
        if (b2 >= u_hi) break;
        b = b2;
    }
    ragged_store(a, row0, p);
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
