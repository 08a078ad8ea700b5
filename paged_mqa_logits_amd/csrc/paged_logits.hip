// fp8_fp4_paged_mqa_logits: score every visible token of a paged fp8 / MXFP4
// key cache for each query row (the tile pipeline is in logits_core.h).
//
// Design (gfx950):
//  * Persistent grid: one workgroup per schedule entry. Each walks its
//    contiguous run of (row-piece, key-block) units. A row-piece is up to 8
//    rows of one request ("[Bugfix][GLM-5.3-Flash] ...", Purpose: rows of a
//    request are processed together), so each key page is read from HBM once
//    for all of them.
//  * Key pages stream HBM -> LDS with direct-to-LDS loads (global_load_lds
//    _dwordx4), kStages deep, with 16-byte chunks XOR-swizzled per token so the
//    MFMA operand reads are free of bank conflicts. All per-unit metadata
//    (schedule, block table, lengths, request ids) comes through the scalar
//    cache, so the vector-memory counter holds only page loads and logit
//    stores and the wait before a page never drains the loads behind it.
//  * Columns past each row's last visible block are filled with -inf by the
//    workgroups after their units (row-strided).
#include "logits_core.h"
#include "rows.h"

namespace pml {

struct PagedArgs {
    const uint8_t *q;
    const float *w;
    const uint8_t *kv;
    int64_t page_stride;
    int64_t num_pages;
    RowView rows;
    const int32_t *bt;
    int64_t bt_ld;
    int bt_cols;
    const int32_t *sched;
    int max_ctx;
    float *out;
    int64_t out_ld;
};

// Walks one worker's units in order: pieces, then blocks inside a piece.
// Every field is wave-uniform.
template <int BKV>
struct UnitIter {
    int r0, g, nblk, blk;
    int end_r, end_b;
    bool valid;

    __device__ __forceinline__ bool in_range() const {
        return r0 < end_r || (r0 == end_r && blk < end_b);
    }
    __device__ __forceinline__ void settle(const RowView &v) {
        for (;;) {
            if (!in_range()) {
                valid = false;
                return;
            }
            if (blk < nblk) {
                valid = true;
                return;
            }
            r0 += g;
            blk = 0;
            if (r0 >= v.num_rows) {
                valid = false;
                return;
            }
            piece_at<BKV>(v, r0, g, nblk);
        }
    }
    __device__ __forceinline__ void init(const PagedArgs &a, int c) {
        const int n = a.rows.num_rows;
        r0 = min(max(sload(a.sched, 2 * c), 0), n);
        blk = max(sload(a.sched, 2 * c + 1), 0);
        end_r = min(max(sload(a.sched, 2 * c + 2), 0), n);
        end_b = max(sload(a.sched, 2 * c + 3), 0);
        g = 0;
        nblk = 0;
        valid = false;
        if (r0 >= n || !in_range()) return;
        piece_at<BKV>(a.rows, r0, g, nblk);
        settle(a.rows);
    }
    __device__ __forceinline__ void next(const RowView &v) {
        ++blk;
        settle(v);
    }
    // Page of the current unit; false when the table entry is unusable (then
    // page 0 is read and the unit's logits are written as NaN).
    __device__ __forceinline__ bool page(const PagedArgs &a, const uint8_t *&pg) const {
        int32_t e = -1;
        if (blk < a.bt_cols) e = sload(a.bt, (int64_t)(r0 / a.rows.next_n) * a.bt_ld + blk);
        const bool ok = e >= 0 && e < a.num_pages;
        pg = a.kv + (ok ? (int64_t)e : 0) * a.page_stride;
        return ok;
    }
};

template <bool FP4, int BKV>
__global__ __launch_bounds__(kThreads, 2) void paged_logits_kernel(PagedArgs a) {
    using C = TileCfg<FP4, BKV>;
    __shared__ __attribute__((aligned(16))) uint8_t s_stage[kStages][C::TILE];
    __shared__ __attribute__((aligned(16))) float s_red[kGMax][kWaves][BKV];
    __shared__ int s_lo[kGMax];
    __shared__ int s_vis[kGMax];

    const int tid = threadIdx.x;
    const int W = gridDim.x;
    const int c = blockIdx.x;

    UnitIter<BKV> ld, cp;
    ld.init(a, c);
    cp = ld;

    int issued = 0;
#pragma unroll
    for (int k = 0; k < kStages - 1; ++k) {
        if (ld.valid) {
            const uint8_t *pg;
            ld.page(a, pg);
            issue_page<FP4, BKV>(pg, s_stage[k]);
            ++issued;
            ld.next(a.rows);
        }
    }

    v8i qa[kGMax];
    v4f w4[kGMax];
    int cur_r0 = -1, cur_g = 0;

    for (int u = 0; cp.valid; ++u) {
        // Page u has landed once at most (kStages - 2) pages issued after it
        // are still in flight (loads complete in order; stores issued in
        // between only make the wait stricter).
        if (issued - (u + 1) >= kStages - 2)
            wait_vmcnt<(kStages - 2) * C::NLD>();
        else
            wait_vmcnt<0>();
        barrier_lds();
        if (ld.valid) {
            const uint8_t *pg;
            ld.page(a, pg);
            issue_page<FP4, BKV>(pg, s_stage[(u + kStages - 1) % kStages]);
            ++issued;
            ld.next(a.rows);
        }
        if (cp.r0 != cur_r0) {
            cur_r0 = cp.r0;
            cur_g = cp.g;
#pragma unroll
            for (int i = 0; i < kGMax; ++i)
                if (i < cur_g) load_row<FP4>(a.q, a.w, cur_r0 + i, qa[i], w4[i]);
            int vis = 0;
            if (tid < cur_g) vis = a.rows.visible(cur_r0 + tid);
            // Drain here, on the rare piece change, so that the compiler does
            // not wait for every load in flight before each use of q and w.
            // The empty asm statements keep the loads above the wait (the
            // builtin alone does not order memory operations); the builtin is
            // the form the compiler's wait tracking understands.
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt(kVmcnt0);
            asm volatile("" ::: "memory");
            if (tid < cur_g) {
                lds_write_i32(lds_addr(&s_vis[tid]), vis);
                lds_write_i32(lds_addr(&s_lo[tid]), 0);
            }
        }
        const uint8_t *unused;
        const bool ok = cp.page(a, unused);
        const uint8_t *st = s_stage[u % kStages];
        score_tile<FP4, BKV>(st, qa, w4, cur_g, s_red);
        barrier_lds();
        store_tile<FP4, BKV>(st, s_red, s_lo, s_vis, cur_g, cur_r0, cp.blk * BKV, a.max_ctx, ok, true,
                             a.out, a.out_ld);
        cp.next(a.rows);
    }

    // -inf past each row's last visible block: rows c, c + W, ...
    for (int r = c; r < a.rows.num_rows; r += W) {
        const int vis = a.rows.visible_s(r);
        const int start = min((vis + BKV - 1) / BKV * BKV, a.max_ctx);
        fill_neg_inf(a.out + (int64_t)r * a.out_ld, start, a.max_ctx);
    }
}

template <bool FP4, int BKV>
static int launch_paged(const PagedArgs &a, int W, hipStream_t st) {
    hipLaunchKernelGGL((paged_logits_kernel<FP4, BKV>), dim3(W), dim3(kThreads), 0, st, a);
    return hipGetLastError() == hipSuccess ? PML_OK : PML_ERR_HIP;
}

}  // namespace pml

static inline bool al16(const void *p) { return ((uintptr_t)p & 15) == 0; }

extern "C" int fp8_fp4_paged_mqa_logits(const void *q, int num_rows, int next_n, int num_heads,
                                        int head_dim, const void *kv_cache, int kv_format,
                                        int block_kv, int64_t page_stride_bytes, int64_t num_pages,
                                        const float *weights, const int32_t *context_lens,
                                        int context_lens_2d, const int32_t *block_table,
                                        int64_t block_table_ld, int block_table_cols,
                                        const int32_t *schedule, int num_CUs,
                                        const int32_t *indices, int max_ctx, float *logits,
                                        int64_t logits_ld, void *stream) {
    if (num_rows < 0 || next_n < 1 || num_CUs < 1 || max_ctx < 0) return PML_ERR_SHAPE;
    if (num_heads != PML_HEADS || head_dim != PML_HEAD_DIM) return PML_ERR_SHAPE;
    if (kv_format != PML_KV_FP8 && kv_format != PML_KV_MXFP4) return PML_ERR_FORMAT;
    if (block_kv != 32 && block_kv != 64) return PML_ERR_BLOCK_KV;
    if (indices && next_n != 1) return PML_ERR_VARLEN_NEXT_N;
    if (num_rows % next_n != 0) return PML_ERR_SHAPE;
    if (num_rows == 0) return PML_OK;
    if (!q || !kv_cache || !weights || !context_lens || !block_table || !schedule || !logits)
        return PML_ERR_NULL;
    if (num_pages < 1 || block_table_cols < 0 || block_table_ld < block_table_cols)
        return PML_ERR_STRIDE;
    const int64_t pb = kv_format == PML_KV_FP8 ? (int64_t)block_kv * (head_dim + 4)
                                               : (int64_t)block_kv * (head_dim / 2 + head_dim / 32);
    if (page_stride_bytes < pb || page_stride_bytes % 16 != 0) return PML_ERR_STRIDE;
    if (logits_ld < max_ctx || logits_ld % 4 != 0) return PML_ERR_STRIDE;
    if (!al16(q) || !al16(kv_cache) || !al16(weights) || !al16(logits)) return PML_ERR_ALIGN;
    pml::PagedArgs a;
    a.q = (const uint8_t *)q;
    a.w = weights;
    a.kv = (const uint8_t *)kv_cache;
    a.page_stride = page_stride_bytes;
    a.num_pages = num_pages;
    a.rows = pml::RowView{context_lens, indices, context_lens_2d ? 1 : 0, next_n, num_rows};
    a.bt = block_table;
    a.bt_ld = block_table_ld;
    a.bt_cols = block_table_cols;
    a.sched = schedule;
    a.max_ctx = max_ctx;
    a.out = logits;
    a.out_ld = logits_ld;
    hipStream_t st = (hipStream_t)stream;
    if (kv_format == PML_KV_FP8)
        return block_kv == 64 ? pml::launch_paged<false, 64>(a, num_CUs, st)
                              : pml::launch_paged<false, 32>(a, num_CUs, st);
    return block_kv == 64 ? pml::launch_paged<true, 64>(a, num_CUs, st)
                          : pml::launch_paged<true, 32>(a, num_CUs, st);
}
