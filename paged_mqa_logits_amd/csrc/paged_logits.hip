// fp8_fp4_paged_mqa_logits: score every visible token of a paged fp8 / MXFP4
// key cache for each query row (scoring core in logits_core.h).
//
// Design (gfx950):
//  * Persistent grid of num_CUs workgroups. The schedule cuts the ordered
//    (row-piece, key-block) units into one range of about equal cost per
//    workgroup; workgroup c walks range c up to its split point, and the
//    ranges' last eighths are dealt out at run time from 8 counters in the
//    call's workspace, so the grid stays balanced whatever slows one
//    workgroup down. A row-piece is up to 8 rows of one request
//    ("[Bugfix][GLM-5.3-Flash] ...", Purpose: rows of a request are processed
//    together), so each key page is read from HBM once for all of them.
//  * The 4 waves take the current piece's blocks in turn (wave w: blocks
//    w, w + 4, ...). Each loads its pages from HBM straight into VGPRs, two
//    buffers deep (one block in flight while one is scored), and scores them
//    against every row of the piece, whose q and w sit in LDS. Waves meet at
//    a barrier only when the piece changes.
//  * Logit stores are issued as inline asm one step after the block is
//    scored, so the compiler waits for a page exactly and the page behind
//    it stays in flight.
//  * All per-unit metadata (chunk entries, block table, lengths, request ids)
//    is read through the scalar cache; the counters only by vector atomics.
//  * Columns past each row's last visible block are filled with -inf by the
//    workgroups after their units (row-strided).
#include <mutex>

#include "logits_core.h"
#include "rows.h"
#include "select.h"
#include "fused.h"

namespace pml {

struct PagedArgs {
    const uint8_t *q;  // fp8 codes, or packed e2m1 values (fp4 q)
    const float *w;
    const uint8_t *kv;
    int64_t page_stride;
    int64_t num_pages;
    RowView rows;
    const int32_t *bt;
    int64_t bt_ld;
    int bt_cols;
    const int32_t *sched;  // range entries (read through the scalar cache)
    int max_ctx;
    void *out;  // float, or uint16_t bf16 bits
    int64_t out_ld;
    const uint8_t *qs;      // fp4 q: e8m0 scales [rows][H][D/32]
    const uint8_t *ucodes;  // pieces of u = sum_h w_h q_h: [rows][4][128] fp8 codes
    const uint8_t *uscales; // and their e8m0 scales [rows][4][4]
    int32_t *split;         // [num_CUs][2]: where the last 1/kDynDiv of each range starts
    int32_t *pools;         // kPools work counters, kPoolStride int32 apart
    // fused top-k: per-row threshold; per (row, block) a candidate count and
    // a list of up to block_kv (logit, column) pairs, compacted at its start
    const float *theta;
    int32_t *ccount;  // [rows][count_ld]
    float *cand;      // [rows][cand_ld][2], block b's pairs from b * block_kv
    int64_t count_ld, cand_ld;
};

__device__ __forceinline__ void store_i32_async(int32_t *p, int v) {
    asm volatile("global_store_dword %0, %1, off" ::"v"(p), "v"(v) : "memory");
}

__device__ __forceinline__ void store_v2f_async(float *p, float x, float y) {
    typedef float v2f_s __attribute__((ext_vector_type(2)));
    const v2f_s v = {x, y};
    asm volatile("global_store_dwordx2 %0, %1, off" ::"v"(p), "v"(v) : "memory");
}

// Load block b (BKV tokens) of the piece whose table row is bt_row, from its
// BKV / PG pages: table entries b * (BKV / PG) + i. Bit i of the result says
// page i's entry is usable; an unusable entry reads page 0 instead, and its
// tokens score NaN.
template <bool FP4, int BKV, int PG = BKV>
__device__ __forceinline__ int fetch_block(const PagedArgs &a, int64_t bt_row, int b, KeyRegs<FP4, BKV> &k) {
    constexpr int NP = BKV / PG;
    if constexpr (NP == 1) {
        int32_t e = -1;
        if (b < a.bt_cols) e = sload(a.bt, bt_row * a.bt_ld + b);
        const bool ok = e >= 0 && e < a.num_pages;
        load_page<FP4, BKV>(a.kv + (ok ? (int64_t)e : 0) * a.page_stride, k);
        return ok ? 1 : 0;
    } else {
        const uint8_t *pg[NP];
        int ok = 0;
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int pb = b * NP + i;
            int32_t e = -1;
            if (pb < a.bt_cols) e = sload(a.bt, bt_row * a.bt_ld + pb);
            const bool oki = e >= 0 && e < a.num_pages;
            pg[i] = a.kv + (oki ? (int64_t)e : 0) * a.page_stride;
            ok |= (oki ? 1 : 0) << i;
        }
        load_pages<FP4, BKV, PG>(pg, k);
        return ok;
    }
}

// One step of a wave's block loop: wait for block b, store the previous
// block's logits, request block bp (the depth ahead; with PF) into the
// buffer freed by the previous step, and score block b against the g staged
// rows into the wave's LDS slot. Rows go in quads: the linear half of a quad
// (lin_quad) is scored once for its rows, the first time one of them needs
// the block. Rows whose visible length ends before the block are skipped
// (their tail is filled separately). Lane i of vis_lane holds the visible
// length of row i.
template <bool FP4, int BKV, int PG, typename OT, bool Q4, bool CAND, bool PF>
__device__ __forceinline__ void wave_step(const PagedArgs &a, int r0, int g, int64_t bt_row, int b,
                                          const KeyRegs<FP4, BKV> &kc, int okc, int bp, KeyRegs<FP4, BKV> &kp,
                                          int &okp, const uint8_t *s_q, const float *s_w, const uint8_t *s_u,
                                          const uint8_t *s_us, int vis_lane, WaveSlot<BKV> &sl, int &mask,
                                          int &col0p, const float *s_th) {
    touch<FP4, BKV>(kc);
    flush_slot<BKV, OT>(sl, mask, r0, col0p, a.max_ctx, (OT *)a.out, a.out_ld);
    if constexpr (PF) okp = fetch_block<FP4, BKV, PG>(a, bt_row, bp, kp);
    const int lane = lane_id();
    const int col0 = b * BKV;
    const int tok = out_token<BKV>(lane);
    const int s = col0 + tok;
    const float scale = FP4 ? 0.5f : 0.5f * __uint_as_float(kc.sc[0]);  // 1/2: see score_row
    int m = 0;
    for (int q0 = 0; q0 < g; q0 += 4) {
        // the quad's rows with G known at compile time, so M[G] stays in registers
        float M[4] = {0.f, 0.f, 0.f, 0.f};
        bool have = false;  // M holds the quad's linear halves
#pragma unroll
        for (int G = 0; G < 4; ++G) {
            const int i = q0 + G;
            if (i >= g) break;
            const int vis = __builtin_amdgcn_readlane(vis_lane, i);
            if (col0 >= vis) continue;
            float sr;
            if (G == 0) {
                // (the quad's first row is skipped only at the end of a piece)
                sr = score_row<FP4, BKV, Q4, true>(kc, s_q + i * kQBytes, s_w + i * PML_HEADS, s_u, s_us, q0 >> 2, M);
                have = true;
            } else {
                if (!have) {
                    lin_quad<FP4, BKV>(kc, s_u, s_us, q0 >> 2, M);
                    have = true;
                }
                sr = score_row<FP4, BKV, Q4>(kc, s_q + i * kQBytes, s_w + i * PML_HEADS);
            }
            float v = (sr + M[G]) * scale;
            if (!((okc >> (tok / PG)) & 1)) v = __builtin_nanf("");  // the token's page is unusable
            if (col0 + BKV > vis)  // (wave-uniform: only a row's last block is masked)
                if (s >= vis) v = -__builtin_inff();
            if (out_lane<BKV>(lane)) lds_st<float>(&sl.v[i][tok], v);
            if constexpr (CAND) {
                // candidates (logit at or above the row's threshold) to the block's
                // region of the row's list, in lane order, and their count
                const bool pred = out_lane<BKV>(lane) && v >= lds_ld<float>(&s_th[i]);
                const uint64_t cm = __ballot(pred);
                const int64_t row = r0 + i;
                if (lane == 0) store_i32_async(a.ccount + row * a.count_ld + b, (int)__popcll(cm));
                const int pos = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(cm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)cm, 0u));
                if (pred) store_v2f_async(a.cand + (row * a.cand_ld + col0 + pos) * 2, v, (float)s);
            }
            m |= 1 << i;
        }
    }
    mask = m;
    col0p = col0;
}

constexpr int kPW = kCW;            // waves per workgroup
constexpr int kDynDiv = 8;          // each range's last 1/kDynDiv (by cost) is dealt out at run time
constexpr int kPools = 8;           // counters those parts are drawn from
constexpr int kPoolStride = 32;     // int32 between counters (one 128-byte line each)
constexpr int kSplitPieces = 16;    // ranges of more pieces keep no dynamic part
constexpr int kPThreads = kPW * kWave;
constexpr int kDepth = 1;          // key blocks in flight per wave while one is scored
constexpr int kBufs = kDepth + 1;  // key-block buffers per wave

// LDS of a logits workgroup. (q last: the small arrays read per row sit
// below 64 KB, within reach of an LDS instruction's immediate offset from one
// base address.)
template <int BKV>
struct PagedShared {
    float w[kGMax * PML_HEADS];
    uint8_t u[kGMax * kUBytes];
    uint8_t us[kGMax * kUScales];
    int vis[kGMax];
    float th[kGMax];
    WaveSlot<BKV> slot[kPW];
    uint8_t q[kGMax * kQBytes];
};

// One piece (the whole workgroup): stage its rows, then every wave scores its
// blocks b0, b0 + kPW, ... (nmy of them; the 4 waves take the piece's blocks in
// turn). kDepth blocks are in flight per wave while one is scored: step s
// waits for block s, then requests block s + kDepth (near the end the last
// block again, an L2 hit, so every step has the same loads behind its wait).
// The caller has requested the first block (kb0) before it knew the piece's
// size, so that load overlaps the length reads; the piece's q, w and pieces
// are then staged, so those round trips overlap too.
template <bool FP4, int BKV, int PG, typename OT, bool Q4, bool CAND>
__device__ __forceinline__ void run_piece(const PagedArgs &a, int r0, int g, int64_t bt_row, int b0, int nmy,
                                          const KeyRegs<FP4, BKV> &kb0, int okb0, PagedShared<BKV> &sh,
                                          WaveSlot<BKV> &sl) {
    constexpr int NB = kBufs;
    static_assert(kDepth == 1, "the first block comes from the caller");
    const int tid = threadIdx.x;
    const int last = nmy - 1;
    KeyRegs<FP4, BKV> kb[NB];
    int okb[NB];
    kb[0] = kb0;
    okb[0] = okb0;
    // The piece's loads (q, w, pieces, lengths) are all issued before the
    // barrier at which every wave is done with the previous piece's rows, so
    // waiting for the slowest wave overlaps their latency.
    const int vis_t = tid < g ? a.rows.visible(r0 + tid) : 0;
    float th_t = 0.f;
    if constexpr (CAND) th_t = tid < g ? a.theta[r0 + tid] : 0.f;
    auto wait_prev = [] { barrier_lds(); };
    auto pieces_then_wait = [&] { stage_pieces<kPThreads>(a.ucodes, a.uscales, r0, g, sh.u, sh.us, wait_prev); };
    if constexpr (Q4)
        stage_rows_q4<kPThreads>(a.q, a.qs, a.w, r0, g, sh.q, sh.w, pieces_then_wait);
    else
        stage_rows<kPThreads>(a.q, a.w, r0, g, sh.q, sh.w, pieces_then_wait);
    if (tid < g) sh.vis[tid] = vis_t;
    if constexpr (CAND)
        if (tid < g) sh.th[tid] = th_t;
    barrier_lds();
    const int vis_lane = lds_ld<int>(&sh.vis[lane_id() % kGMax]);  // lane i: visible length of row i
    if (nmy > 0) {
        int mask = 0, col0p = 0;
        for (int j = 0; j < nmy; j += NB) {
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                if (j + u >= nmy) break;
                wave_step<FP4, BKV, PG, OT, Q4, CAND, true>(a, r0, g, bt_row, b0 + kPW * (j + u), kb[u], okb[u],
                                                        b0 + kPW * min(j + u + kDepth, last), kb[(u + kDepth) % NB],
                                                        okb[(u + kDepth) % NB], sh.q, sh.w, sh.u, sh.us, vis_lane,
                                                        sl, mask, col0p, sh.th);
            }
        }
        flush_slot<BKV, OT>(sl, mask, r0, col0p, a.max_ctx, (OT *)a.out, a.out_ld);
    }
}

// The units from (r0, blk_lo) up to (end_r, end_b) (the whole workgroup).
template <bool FP4, int BKV, int PG, typename OT, bool Q4, bool CAND>
__device__ __forceinline__ void run_range(const PagedArgs &a, int r0, int blk_lo, int end_r, int end_b,
                                          PagedShared<BKV> &sh, WaveSlot<BKV> &sl) {
    const int tid = threadIdx.x;
    const int wave = uni(tid / kWave);
    const int n = a.rows.num_rows;
    r0 = min(max(r0, 0), n);
    blk_lo = max(blk_lo, 0);
    end_r = min(max(end_r, 0), n);
    end_b = max(end_b, 0);
    while (r0 < n && (r0 < end_r || (r0 == end_r && blk_lo < end_b))) {
        const int64_t bt_row = r0 / a.rows.next_n;
        // this wave's blocks: blk_lo + wave, + kPW, ...; the first is requested
        // before the piece's size is known (if it lies past the range, its
        // table entry and page are read but not used)
        const int b0 = blk_lo + wave;
        KeyRegs<FP4, BKV> kb0;
        const int okb0 = fetch_block<FP4, BKV, PG>(a, bt_row, b0, kb0);
        int g, nblk;
        piece_at<BKV>(a.rows, r0, g, nblk);
        const int blk_hi = r0 == end_r ? min(end_b, nblk) : nblk;
        if (blk_lo < blk_hi) {
            // (run_piece holds the barrier after which the previous piece's rows are free)
            const int nmy = b0 < blk_hi ? (blk_hi - b0 + kPW - 1) / kPW : 0;
            run_piece<FP4, BKV, PG, OT, Q4, CAND>(a, r0, g, bt_row, b0, nmy, kb0, okb0, sh, sl);
        }
        r0 += g;
        blk_lo = 0;
    }
}

// Workgroup c first runs range c up to its split point (split[c], the start
// of the range's last 1/kDynDiv by cost). The ranges' last parts are then
// dealt out at run time: pool x holds those of ranges x, x + P, x + 2P, ...
// (P = min(W, kPools)) and serves the workgroups c with c % P == x, each
// drawing from its pool's counter until the pool is empty. So workgroups
// that run fast (on a compute unit shared with lighter work, say) take more
// of them. The counters are zeroed by the call's first kernel.
template <bool FP4, int BKV, int PG, typename OT, bool Q4, bool CAND>
__global__ __launch_bounds__(kPThreads, 8 / kPW) void paged_logits_kernel(PagedArgs a) {
    __shared__ __attribute__((aligned(16))) PagedShared<BKV> sh;
    __shared__ int s_take;
    const int tid = threadIdx.x;
    const int wave = uni(tid / kWave);
    const int W = gridDim.x;
    const int c = blockIdx.x;
    const int n = a.rows.num_rows;
    const int P = min(W, kPools);
    const int x = c % P;
    const int cnt = (W - x + P - 1) / P;
    int r0 = sload(a.sched, 2 * c), b0 = sload(a.sched, 2 * c + 1);
    int r1 = sload(a.split, 2 * c), b1 = sload(a.split, 2 * c + 1);
    for (;;) {
        run_range<FP4, BKV, PG, OT, Q4, CAND>(a, r0, b0, r1, b1, sh, sh.slot[wave]);
        __syncthreads();  // every wave is done reading s_take
        if (tid == 0) s_take = atomicAdd(a.pools + kPoolStride * x, 1);
        __syncthreads();
        const int t = uni(s_take);
        if (t >= cnt) break;
        const int e = x + P * t;
        r0 = sload(a.split, 2 * e);
        b0 = sload(a.split, 2 * e + 1);
        r1 = sload(a.sched, 2 * e + 2);
        b1 = sload(a.sched, 2 * e + 3);
    }
    // -inf past each row's last visible block: rows c, c + W, ...
    for (int r = c; r < n; r += W) {
        const int vis = a.rows.visible_s(r);
        const int start = min((vis + BKV - 1) / BKV * BKV, a.max_ctx);
        fill_neg_inf<kPThreads, OT>((OT *)a.out + (int64_t)r * a.out_ld, start, a.max_ctx);
    }
}

// block_kv 64: steps of one 64-token page; block_kv 32: steps of 64 tokens
// from two 32-token pages (step_tokens), which doubles a wave's bytes in
// flight and halves the per-step work per token.
template <bool FP4, int BKV, typename OT, bool Q4 = false, bool CAND = false>
static int launch_paged(const PagedArgs &a, int W, hipStream_t st) {
    constexpr int S = BKV < kMinStep ? kMinStep : BKV;
    hipLaunchKernelGGL((paged_logits_kernel<FP4, S, BKV, OT, Q4, CAND>), dim3(W), dim3(kPThreads), 0, st, a);
    return hipGetLastError() == hipSuccess ? PML_OK : PML_ERR_HIP;
}

// The pieces of u = sum_h w_h q_h for every row (kGMax rows per workgroup),
// written to the call's workspace ahead of the logits kernel, which stages
// them with q.
// Split point of range e (thread-per-range walk, vector loads): the first
// unit at or past the range's cost offset total - total / kDynDiv. Ranges of
// more than kSplitPieces pieces keep no dynamic part.
__device__ __forceinline__ void range_split(const PagedArgs &a, int block_kv, int e, int &sr, int &sb) {
    const int n = a.rows.num_rows;
    int r = min(max(a.sched[2 * e], 0), n), b = max(a.sched[2 * e + 1], 0);
    const int re = min(max(a.sched[2 * e + 2], 0), n), be = max(a.sched[2 * e + 3], 0);
    int pr[kSplitPieces], plo[kSplitPieces], phi[kSplitPieces], pg[kSplitPieces];
    int np = 0;
    long long total = 0;
    bool many = false;
    while (r < n && (r < re || (r == re && b < be))) {
        if (np == kSplitPieces) {
            many = true;
            break;
        }
        // rows of the piece at r (as piece_at, per thread)
        int g = 1, ext = a.rows.visible(r);
        for (int i = 1; i < kGMax && r + i < n && a.rows.same_group(r + i, r); ++i) {
            ext = max(ext, a.rows.visible(r + i));
            g = i + 1;
        }
        const int nblk = (ext + block_kv - 1) / block_kv;
        const int hi = r == re ? min(be, nblk) : nblk;
        pr[np] = r;
        plo[np] = b;
        phi[np] = max(hi, b);
        pg[np] = g;
        total += (long long)(phi[np] - b) * (kCostBase + g);
        ++np;
        r += g;
        b = 0;
    }
    sr = re;
    sb = be;
    if (many || total == 0) return;
    long long target = total - total / kDynDiv, cum = 0;
    for (int p = 0; p < np; ++p) {
        const long long cp = (long long)(phi[p] - plo[p]) * (kCostBase + pg[p]);
        if (cum + cp > target) {
            const int per = kCostBase + pg[p];
            const int blk = plo[p] + (int)((target - cum + per - 1) / per);
            if (blk < phi[p]) {
                sr = pr[p];
                sb = blk;
            } else if (p + 1 < np) {
                sr = pr[p + 1];
                sb = plo[p + 1];
            }
            return;
        }
        cum += cp;
    }
}

// First kernel of every logits call. Workgroups [0, rows): the pieces of
// u = sum_h w_h q_h of one row each (a short chain per workgroup: the row's q
// staged, 8 head steps per thread, the pieces written), to the workspace for
// the logits kernel to stage with q. The following workgroups: one split point
// per range (a thread each), and the pool counters set to zero.
template <bool Q4>
__global__ __launch_bounds__(kPThreads) void pieces_kernel(PagedArgs a, uint8_t *codes, uint8_t *scales,
                                                           int block_kv, int W) {
    const int nrow_wg = a.rows.num_rows;
    if ((int)blockIdx.x >= nrow_wg) {
        const int e = (blockIdx.x - nrow_wg) * kPThreads + threadIdx.x;
        if (e < W) {
            int sr, sb;
            range_split(a, block_kv, e, sr, sb);
            a.split[2 * e] = sr;
            a.split[2 * e + 1] = sb;
        }
        if (blockIdx.x == nrow_wg && threadIdx.x < kPools) a.pools[kPoolStride * threadIdx.x] = 0;
        return;
    }
    __shared__ __attribute__((aligned(16))) uint8_t s_q[kQBytes];
    __shared__ __attribute__((aligned(16))) float s_w[PML_HEADS];
    __shared__ __attribute__((aligned(16))) uint8_t s_u[kUBytes];
    __shared__ __attribute__((aligned(16))) uint8_t s_us[kUScales];
    const int r0 = blockIdx.x;
    const int g = 1;
    if constexpr (Q4)
        stage_rows_q4<kPThreads>(a.q, a.qs, a.w, r0, g, s_q, s_w);
    else
        stage_rows<kPThreads>(a.q, a.w, r0, g, s_q, s_w);
    barrier_lds();
    derive_pieces<Q4, kPThreads>(s_q, s_w, g, s_u, s_us);
    barrier_lds();
    constexpr int kChunks = kUBytes / 16;
    for (int i = threadIdx.x; i < g * (kChunks + 1); i += kPThreads) {
        const int row = i / (kChunks + 1), c = i % (kChunks + 1);
        if (c < kChunks)
            *(v4i *)(codes + (int64_t)(r0 + row) * kUBytes + c * 16) =
                lds_ld<v4i>(s_u + q_lds_off(kPieces * row + c / 8, c % 8));
        else
            *(v4i *)(scales + (int64_t)(r0 + row) * kUScales) = lds_ld<v4i>(s_us + row * kUScales);
    }
}

// Threshold of the fused top-k, one workgroup per row. A row with at most cap
// visible columns takes every finite logit as a candidate (threshold
// -FLT_MAX). A wider row scores an evenly spaced sample of its blocks
// (kSampleTokens tokens) and takes the lower bound of the radix bin that holds
// the jr-th largest sampled value as the threshold, jr chosen so that about
// 2k of the row's columns are expected at or above it (the search stops once
// the bin adds at most a quarter of jr). Any threshold gives the exact
// result: the selection falls back to the full top-k when the candidates
// number fewer than k or more than cap. Also writes the row's width.
constexpr int kThThreads = 512;
constexpr int kSampleTokens = 1024;

template <bool FP4, int BKV>
__global__ __launch_bounds__(kThThreads) void threshold_kernel(PagedArgs a, int k, int cap, float *theta,
                                                               int32_t *width) {
    constexpr int S = kSampleTokens / BKV;  // sampled blocks
    constexpr int NW = kThThreads / kWave;
    constexpr int PER = S / NW;             // blocks per wave
    constexpr int NPT = kSampleTokens / kThThreads;
    __shared__ __attribute__((aligned(16))) uint8_t s_q[kQBytes];
    __shared__ __attribute__((aligned(16))) float s_w[PML_HEADS];
    __shared__ __attribute__((aligned(16))) uint8_t s_u[kUBytes];
    __shared__ __attribute__((aligned(16))) uint8_t s_us[kUScales];
    __shared__ uint32_t s_key[kSampleTokens];
    __shared__ __attribute__((aligned(16))) uint32_t s_hist[2048];
    __shared__ __attribute__((aligned(16))) uint32_t s_wave[NW];
    __shared__ uint32_t s_pick[2];
    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = uni(tid / kWave);
    const int vis = min(a.rows.visible_s(r), a.max_ctx);
    if (tid == 0) width[r] = vis;
    if (vis <= cap) {
        if (tid == 0) theta[r] = -__FLT_MAX__;
        return;
    }
    const int nblk = (vis + BKV - 1) / BKV;  // (narrow rows may sample a block twice)
    const int64_t bt_row = r / a.rows.next_n;
    auto blk = [&](int t) { return (int)((int64_t)(2 * (wave + NW * t) + 1) * nblk / (2 * S)); };
    KeyRegs<FP4, BKV> kb[2];
    bool okb[2];
    okb[0] = fetch_block<FP4, BKV>(a, bt_row, blk(0), kb[0]);
    stage_rows<kThThreads>(a.q, a.w, r, 1, s_q, s_w);
    barrier_lds();
    derive_pieces<false, kThThreads>(s_q, s_w, 1, s_u, s_us);
    barrier_lds();
    const int tok = out_token<BKV>(lane);

#pragma unroll
    for (int t = 0; t < PER; ++t) {
        if (t + 1 < PER) okb[(t + 1) & 1] = fetch_block<FP4, BKV>(a, bt_row, blk(t + 1), kb[(t + 1) & 1]);
        const KeyRegs<FP4, BKV> &kc = kb[t & 1];
        const float scale = FP4 ? 0.5f : 0.5f * __uint_as_float(kc.sc[0]);
        float M[4];
        const float sr = score_row<FP4, BKV, false, true>(kc, s_q, s_w, s_u, s_us, 0, M);
        float v = (sr + M[0]) * scale;
        if (!okb[t & 1]) v = __builtin_nanf("");
        if (blk(t) * BKV + tok >= vis) v = -__builtin_inff();
        if (out_lane<BKV>(lane)) s_key[(wave + NW * t) * BKV + tok] = order_key(v);
    }
    barrier_lds();
    uint32_t key[NPT];
#pragma unroll
    for (int i = 0; i < NPT; ++i) key[i] = s_key[i * kThThreads + tid];
    const uint32_t jr = (uint32_t)max(1, (int)(((int64_t)2 * k * kSampleTokens + vis - 1) / vis));
    uint32_t prefix = 0, mask = 0, kk = jr;
    auto kf = [&](int i) { return key[i]; };
    auto live = [&](int) { return true; };
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const int nbins = pass == 2 ? 1024 : 2048;
        const uint32_t cnt = radix_pass<kThThreads, NPT>(kf, live, prefix, mask, shift, nbins, kk, s_hist, s_wave, s_pick);
        prefix |= s_pick[0] << shift;
        mask |= (uint32_t)(nbins - 1) << shift;
        kk -= s_pick[1];
        if (cnt == kk || 4 * cnt <= jr) break;
    }
    if (tid == 0) {
        // the float whose order key is prefix (key 0, NaN, gives NaN: no candidates, the row falls back)
        const uint32_t bits = (prefix & 0x80000000u) ? (prefix & 0x7fffffffu) : ~prefix;
        theta[r] = __uint_as_float(bits);
    }
}

}  // namespace pml

static inline bool al16(const void *p) { return ((uintptr_t)p & 15) == 0; }
static size_t region256(size_t bytes) { return (bytes + 255) / 256 * 256; }

// Workspace of the logits call: the pieces of u = sum_h w_h q_h per row,
// codes [num_rows][4][128] then e8m0 scales [num_rows][4][4], each region
// 256-B aligned.
extern "C" size_t fp8_fp4_paged_mqa_logits_workspace_size(int num_rows, int num_CUs) {
    if (num_rows < 0 || num_CUs < 1 || num_CUs > (1 << 20)) return 0;
    return region256((size_t)num_rows * pml::kUBytes) + region256((size_t)num_rows * pml::kUScales) +
           region256((size_t)num_CUs * 8) + region256(pml::kPools * pml::kPoolStride * 4);
}

// Validate the arguments shared by the paged-logits entry points and fill a
// (bf16: logits are uint16_t bits and rows must be 16-B aligned, logits_ld a
// multiple of 8; q_scale: fp4 q with its scales, MXFP4 keys only). PML_OK with
// *empty set when there is nothing to launch.
static int prepare_paged(pml::PagedArgs &a, bool &empty, const void *q, const uint8_t *q_scale, int num_rows,
                         int next_n, int num_heads, int head_dim, const void *kv_cache, int kv_format,
                         int block_kv, int64_t page_stride_bytes, int64_t num_pages, const float *weights,
                         const int32_t *context_lens, int context_lens_2d, const int32_t *block_table,
                         int64_t block_table_ld, int block_table_cols, const int32_t *schedule, int num_CUs,
                         const int32_t *indices, int max_ctx, void *logits, int64_t logits_ld, bool bf16,
                         void *workspace, size_t workspace_bytes) {
    empty = false;
    const bool q4 = q_scale != nullptr;
    if (num_rows < 0 || next_n < 1 || max_ctx < 0) return PML_ERR_SHAPE;
    if (paged_mqa_logits_schedule_rows(num_CUs) < 0) return PML_ERR_SHAPE;
    if (num_heads != PML_HEADS || head_dim != PML_HEAD_DIM) return PML_ERR_SHAPE;
    if (kv_format != PML_KV_FP8 && kv_format != PML_KV_MXFP4) return PML_ERR_FORMAT;
    if (block_kv != 32 && block_kv != 64) return PML_ERR_BLOCK_KV;
    if (indices && next_n != 1) return PML_ERR_VARLEN_NEXT_N;
    if (num_rows % next_n != 0) return PML_ERR_SHAPE;
    if (q4 && kv_format != PML_KV_MXFP4) return PML_ERR_UNSUPPORTED;
    if (num_rows == 0) {
        empty = true;
        return PML_OK;
    }
    if (q4 && !al16(q_scale)) return PML_ERR_ALIGN;
    if (!q || !kv_cache || !weights || !context_lens || !block_table || !schedule || !logits)
        return PML_ERR_NULL;
    if (num_pages < 1 || block_table_cols < 0 || block_table_ld < block_table_cols)
        return PML_ERR_STRIDE;
    const int64_t pb = kv_format == PML_KV_FP8 ? (int64_t)block_kv * (head_dim + 4)
                                               : (int64_t)block_kv * (head_dim / 2 + head_dim / 32);
    if (page_stride_bytes < pb || page_stride_bytes % 16 != 0) return PML_ERR_STRIDE;
    if (logits_ld < max_ctx || logits_ld % (bf16 ? 8 : 4) != 0) return PML_ERR_STRIDE;
    if (!al16(q) || !al16(kv_cache) || !al16(weights) || !al16(logits) || !al16(schedule)) return PML_ERR_ALIGN;
    if (!workspace || workspace_bytes < fp8_fp4_paged_mqa_logits_workspace_size(num_rows, num_CUs))
        return PML_ERR_WORKSPACE;
    if ((uintptr_t)workspace % 256) return PML_ERR_ALIGN;
    a = pml::PagedArgs{};
    a.q = (const uint8_t *)q;
    a.qs = q_scale;
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
    uint8_t *ws = (uint8_t *)workspace;
    const size_t rc = region256((size_t)num_rows * pml::kUBytes), rs = region256((size_t)num_rows * pml::kUScales);
    a.ucodes = ws;
    a.uscales = ws + rc;
    a.split = (int32_t *)(ws + rc + rs);
    a.pools = (int32_t *)(ws + rc + rs + region256((size_t)num_CUs * 8));
    return PML_OK;
}

// The first kernel of each logits call: every row's pieces, every range's
// split point and zeroed pool counters, into the workspace.
static int launch_pieces(const pml::PagedArgs &a, int block_kv, int W, hipStream_t st) {
    const dim3 grid(a.rows.num_rows + (W + pml::kPThreads - 1) / pml::kPThreads);
    uint8_t *codes = (uint8_t *)a.ucodes, *scales = (uint8_t *)a.uscales;
    if (a.qs)
        hipLaunchKernelGGL(pml::pieces_kernel<true>, grid, dim3(pml::kPThreads), 0, st, a, codes, scales, block_kv, W);
    else
        hipLaunchKernelGGL(pml::pieces_kernel<false>, grid, dim3(pml::kPThreads), 0, st, a, codes, scales, block_kv,
                           W);
    return hipGetLastError() == hipSuccess ? PML_OK : PML_ERR_HIP;
}

// The fp32, bf16 and fp4-q logits calls.
static int paged_logits(const void *q, const uint8_t *q_scale, int num_rows, int next_n, int num_heads,
                        int head_dim, const void *kv_cache, int kv_format, int block_kv, int64_t page_stride_bytes,
                        int64_t num_pages, const float *weights, const int32_t *context_lens,
                        int context_lens_2d, const int32_t *block_table, int64_t block_table_ld,
                        int block_table_cols, const int32_t *schedule, int num_CUs, const int32_t *indices,
                        int max_ctx, void *logits, int64_t logits_ld, bool bf16, void *workspace,
                        size_t workspace_bytes, void *stream) {
    pml::PagedArgs a;
    bool empty;
    const int st0 = prepare_paged(a, empty, q, q_scale, num_rows, next_n, num_heads, head_dim, kv_cache, kv_format,
                                  block_kv, page_stride_bytes, num_pages, weights, context_lens, context_lens_2d,
                                  block_table, block_table_ld, block_table_cols, schedule, num_CUs, indices,
                                  max_ctx, logits, logits_ld, bf16, workspace, workspace_bytes);
    if (st0 != PML_OK || empty) return st0;
    if (q_scale && bf16) return PML_ERR_UNSUPPORTED;
    hipStream_t st = (hipStream_t)stream;
    const int rp = launch_pieces(a, pml::step_tokens(block_kv), num_CUs, st);
    if (rp != PML_OK) return rp;
    if (q_scale)
        return block_kv == 64 ? pml::launch_paged<true, 64, float, true>(a, num_CUs, st)
                              : pml::launch_paged<true, 32, float, true>(a, num_CUs, st);
    if (bf16) {
        if (kv_format == PML_KV_FP8)
            return block_kv == 64 ? pml::launch_paged<false, 64, uint16_t>(a, num_CUs, st)
                                  : pml::launch_paged<false, 32, uint16_t>(a, num_CUs, st);
        return block_kv == 64 ? pml::launch_paged<true, 64, uint16_t>(a, num_CUs, st)
                              : pml::launch_paged<true, 32, uint16_t>(a, num_CUs, st);
    }
    if (kv_format == PML_KV_FP8)
        return block_kv == 64 ? pml::launch_paged<false, 64, float>(a, num_CUs, st)
                              : pml::launch_paged<false, 32, float>(a, num_CUs, st);
    return block_kv == 64 ? pml::launch_paged<true, 64, float>(a, num_CUs, st)
                          : pml::launch_paged<true, 32, float>(a, num_CUs, st);
}

extern "C" int fp8_fp4_paged_mqa_logits(const void *q, const uint8_t *q_scale, int num_rows, int next_n,
                                        int num_heads, int head_dim, const void *kv_cache, int kv_format,
                                        int block_kv, int64_t page_stride_bytes, int64_t num_pages,
                                        const float *weights, const int32_t *context_lens, int context_lens_2d,
                                        const int32_t *block_table, int64_t block_table_ld, int block_table_cols,
                                        const int32_t *schedule, int num_CUs, const int32_t *indices, int max_ctx,
                                        float *logits, int64_t logits_ld, void *workspace, size_t workspace_bytes,
                                        void *stream) {
    return paged_logits(q, q_scale, num_rows, next_n, num_heads, head_dim, kv_cache, kv_format, block_kv,
                        page_stride_bytes, num_pages, weights, context_lens, context_lens_2d, block_table,
                        block_table_ld, block_table_cols, schedule, num_CUs, indices, max_ctx, logits, logits_ld,
                        false, workspace, workspace_bytes, stream);
}

// ---- the allocation-free variant -------------------------------------------
//
// The logits call's scratch in a file-scope device array, for callers that
// cannot allocate (code under graph capture, tight serving loops). Each GPU the
// library runs on holds its own copy until the process ends. Its address is
// looked up once per device with hipGetSymbolAddress (the array's name is not
// a device address in host code) and that pointer is what the kernels get.
// Every call on one GPU shares the array: the call's first kernel rewrites
// all of it that the call reads (pieces, split points, zeroed counters), and
// calls that overlap on one GPU race.
constexpr int kNoAllocMaxRows = 4096;
constexpr int kNoAllocMaxCUs = 4096;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[(kNoAllocMaxRows * (pml::kUBytes + pml::kUScales) +
                                                  kNoAllocMaxCUs * 8 + pml::kPools * pml::kPoolStride * 4 + 4 * 256 +
                                                  255) / 256 * 256];
static void *g_scratch[kMaxDevices];
static int g_scratch_rc[kMaxDevices];
static std::once_flag g_scratch_once[kMaxDevices];

// The current device's scratch pointer (looked up on its first use), or NULL
// with *rc set when the lookup failed.
static void *device_scratch(int *rc) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *rc = PML_ERR_HIP;
        return nullptr;
    }
    std::call_once(g_scratch_once[dev], [dev] {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        g_scratch[dev] = e == hipSuccess ? ptr : nullptr;
        g_scratch_rc[dev] = e == hipSuccess ? PML_OK : PML_ERR_HIP;
    });
    *rc = g_scratch_rc[dev];
    return g_scratch[dev];
}

extern "C" int fp8_fp4_paged_mqa_logits_noalloc(const void *q, const uint8_t *q_scale, int num_rows, int next_n,
                                                int num_heads, int head_dim, const void *kv_cache, int kv_format,
                                                int block_kv, int64_t page_stride_bytes, int64_t num_pages,
                                                const float *weights, const int32_t *context_lens,
                                                int context_lens_2d, const int32_t *block_table,
                                                int64_t block_table_ld, int block_table_cols,
                                                const int32_t *schedule, int num_CUs, const int32_t *indices,
                                                int max_ctx, float *logits, int64_t logits_ld, void *stream) {
    if (num_rows > kNoAllocMaxRows || num_CUs > kNoAllocMaxCUs) return PML_ERR_SCRATCH;
    const size_t need = fp8_fp4_paged_mqa_logits_workspace_size(num_rows < 0 ? 0 : num_rows, num_CUs < 1 ? 1 : num_CUs);
    if (need > sizeof(scratch)) return PML_ERR_SCRATCH;
    if (num_rows <= 0) {  // nothing to score (or a bad size): no scratch needed, same checks as the main call
        return fp8_fp4_paged_mqa_logits(q, q_scale, num_rows, next_n, num_heads, head_dim, kv_cache, kv_format,
                                        block_kv, page_stride_bytes, num_pages, weights, context_lens,
                                        context_lens_2d, block_table, block_table_ld, block_table_cols, schedule,
                                        num_CUs, indices, max_ctx, logits, logits_ld, nullptr, 0, stream);
    }
    int rc = PML_OK;
    void *ptr = device_scratch(&rc);
    if (!ptr) return rc == PML_OK ? PML_ERR_HIP : rc;
    return fp8_fp4_paged_mqa_logits(q, q_scale, num_rows, next_n, num_heads, head_dim, kv_cache, kv_format, block_kv,
                                    page_stride_bytes, num_pages, weights, context_lens, context_lens_2d,
                                    block_table, block_table_ld, block_table_cols, schedule, num_CUs, indices, max_ctx,
                                    logits, logits_ld, ptr, sizeof(scratch), stream);
}

extern "C" int fp8_fp4_paged_mqa_logits_bf16(const void *q, int num_rows, int next_n, int num_heads,
                                             int head_dim, const void *kv_cache, int kv_format, int block_kv,
                                             int64_t page_stride_bytes, int64_t num_pages, const float *weights,
                                             const int32_t *context_lens, int context_lens_2d,
                                             const int32_t *block_table, int64_t block_table_ld,
                                             int block_table_cols, const int32_t *schedule, int num_CUs,
                                             const int32_t *indices, int max_ctx, uint16_t *logits,
                                             int64_t logits_ld, void *workspace, size_t workspace_bytes,
                                             void *stream) {
    return paged_logits(q, nullptr, num_rows, next_n, num_heads, head_dim, kv_cache, kv_format, block_kv,
                        page_stride_bytes, num_pages, weights, context_lens, context_lens_2d, block_table,
                        block_table_ld, block_table_cols, schedule, num_CUs, indices, max_ctx, logits, logits_ld,
                        true, workspace, workspace_bytes, stream);
}

extern "C" int fp8_fp4_paged_mqa_logits_fp4q(const uint8_t *q_values, const uint8_t *q_scales, int num_rows,
                                             int next_n, int num_heads, int head_dim, const void *kv_cache,
                                             int kv_format, int block_kv, int64_t page_stride_bytes,
                                             int64_t num_pages, const float *weights,
                                             const int32_t *context_lens, int context_lens_2d,
                                             const int32_t *block_table, int64_t block_table_ld,
                                             int block_table_cols, const int32_t *schedule, int num_CUs,
                                             const int32_t *indices, int max_ctx, float *logits,
                                             int64_t logits_ld, void *workspace, size_t workspace_bytes,
                                             void *stream) {
    if (num_rows > 0 && !q_scales) return PML_ERR_NULL;
    return fp8_fp4_paged_mqa_logits(q_values, q_scales, num_rows, next_n, num_heads, head_dim, kv_cache,
                                    kv_format, block_kv, page_stride_bytes, num_pages, weights, context_lens,
                                    context_lens_2d, block_table, block_table_ld, block_table_cols, schedule,
                                    num_CUs, indices, max_ctx, logits, logits_ld, workspace, workspace_bytes,
                                    stream);
}

// Workspace of the fused call: the logits call's workspace, then thresholds,
// row widths and done flags (fp32 / int32 [num_rows] each), the candidate
// counts (int32 [num_rows][nb]) and the candidate lists (fp32
// [num_rows][nb * S][2]), S = max(block_kv, 64) tokens per step and
// nb = ceil(max_ctx / S); every region 256-B aligned.
extern "C" size_t fp8_fp4_paged_mqa_logits_topk_workspace_size(int num_rows, int max_ctx, int block_kv, int k,
                                                               int num_CUs) {
    if (num_rows < 0 || max_ctx < 0 || (block_kv != 32 && block_kv != 64) || k < 1 || k > PML_MAX_TOPK ||
        num_CUs < 1)
        return 0;
    const size_t rows = (size_t)num_rows;
    const size_t S = (size_t)pml::step_tokens(block_kv);  // candidate regions are per step
    const size_t nb = ((size_t)max_ctx + S - 1) / S;
    return fp8_fp4_paged_mqa_logits_workspace_size(num_rows, num_CUs) + 3 * region256(4 * rows) +
           region256(rows * nb * 4) + region256(rows * nb * S * 8);
}

extern "C" int fp8_fp4_paged_mqa_logits_topk(const void *q, int num_rows, int next_n, int num_heads,
                                             int head_dim, const void *kv_cache, int kv_format,
                                             int block_kv, int64_t page_stride_bytes, int64_t num_pages,
                                             const float *weights, const int32_t *context_lens,
                                             int context_lens_2d, const int32_t *block_table,
                                             int64_t block_table_ld, int block_table_cols,
                                             const int32_t *schedule, int num_CUs,
                                             const int32_t *indices, int max_ctx, float *logits,
                                             int64_t logits_ld, int k, int32_t *topk, int64_t topk_ld,
                                             void *workspace, size_t workspace_bytes, void *stream) {
    if (k < 1 || k > PML_MAX_TOPK) return PML_ERR_K;
    pml::PagedArgs a;
    bool empty;
    const int st0 = prepare_paged(a, empty, q, nullptr, num_rows, next_n, num_heads, head_dim, kv_cache,
                                  kv_format, block_kv, page_stride_bytes, num_pages, weights, context_lens,
                                  context_lens_2d, block_table, block_table_ld, block_table_cols, schedule,
                                  num_CUs, indices, max_ctx, logits, logits_ld, false, workspace, workspace_bytes);
    if (st0 != PML_OK || empty) return st0;
    if (!topk) return PML_ERR_NULL;
    if (topk_ld < k) return PML_ERR_STRIDE;
    if (workspace_bytes < fp8_fp4_paged_mqa_logits_topk_workspace_size(num_rows, max_ctx, block_kv, k, num_CUs))
        return PML_ERR_WORKSPACE;
    const size_t rows = (size_t)num_rows;
    const int S = pml::step_tokens(block_kv);  // candidate regions are per step
    const int64_t nb = ((int64_t)max_ctx + S - 1) / S;
    uint8_t *ws = (uint8_t *)workspace + fp8_fp4_paged_mqa_logits_workspace_size(num_rows, num_CUs);
    const size_t reg = region256(4 * rows);
    float *theta = (float *)ws;
    int32_t *width = (int32_t *)(ws + reg);
    int32_t *done = (int32_t *)(ws + 2 * reg);
    int32_t *count = (int32_t *)(ws + 3 * reg);
    float *cand = (float *)(ws + 3 * reg + region256(rows * nb * 4));
    a.theta = theta;
    a.ccount = count;
    a.cand = cand;
    a.count_ld = nb;
    a.cand_ld = nb * S;
    const int cap = pml::kCandPerK * k;
    hipStream_t st = (hipStream_t)stream;
    const dim3 tg(num_rows), tb(pml::kThThreads);
    int rc = launch_pieces(a, pml::step_tokens(block_kv), num_CUs, st);
    if (rc != PML_OK) return rc;
    if (kv_format == PML_KV_FP8) {
        if (block_kv == 64) {
            hipLaunchKernelGGL((pml::threshold_kernel<false, 64>), tg, tb, 0, st, a, k, cap, theta, width);
            rc = pml::launch_paged<false, 64, float, false, true>(a, num_CUs, st);
        } else {
            hipLaunchKernelGGL((pml::threshold_kernel<false, 32>), tg, tb, 0, st, a, k, cap, theta, width);
            rc = pml::launch_paged<false, 32, float, false, true>(a, num_CUs, st);
        }
    } else {
        if (block_kv == 64) {
            hipLaunchKernelGGL((pml::threshold_kernel<true, 64>), tg, tb, 0, st, a, k, cap, theta, width);
            rc = pml::launch_paged<true, 64, float, false, true>(a, num_CUs, st);
        } else {
            hipLaunchKernelGGL((pml::threshold_kernel<true, 32>), tg, tb, 0, st, a, k, cap, theta, width);
            rc = pml::launch_paged<true, 32, float, false, true>(a, num_CUs, st);
        }
    }
    if (rc != PML_OK) return rc;
    pml::CandSelectArgs cs{cand, count, width, nb, nb * S, S, cap, k, topk, topk_ld, done};
    rc = pml::launch_cand_select(cs, num_rows, st);
    if (rc != PML_OK) return rc;
    // rows the candidates could not settle: the full top-k over the written logits
    pml::TopkArgs ta{logits, logits_ld, nullptr, context_lens, context_lens_2d ? 1 : next_n, k, max_ctx,
                     topk, topk_ld, done};
    return pml::launch_topk(ta, num_rows, st);
}
