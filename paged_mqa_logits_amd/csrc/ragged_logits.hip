// mqa_logits: non-paged (ragged prefill) logits. Query row r is scored on the
// keys [cu_seqlen_ks[r], cu_seqlen_ke[r]) of a contiguous fp8 key array and is
// -inf on every other column of the dense [M][N] output (the dense M*N logits
// tensor whose size the prefill chunking bounds, sparse_attn_indexer page,
// forward_cpu: per-row lengths ke - ks).
//
// Grid (x = chunk of key blocks, y = piece of kGMax consecutive rows; the chunk
// is as wide as still gives about kTargetWGs workgroups: whole rows at prefill
// sizes). A workgroup of kGMax waves scores its piece against the chunk's
// blocks that intersect the union of the rows' key ranges, one wave per row
// (ragged_rows_kernel below). The chunk's other columns of the rows are filled
// with -inf, a slice per block step, and nothing is read for them, so a causal
// prefill does about half the dense product.
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

// ---- one row per wave ------------------------------------------------------
//
// ragged_rows_kernel: a workgroup of kGMax waves scores a piece of kGMax
// rows, wave i owning row i: the A operands of its q (4 head tiles) and its w
// stay in registers for the whole piece, so a wave needs no LDS for q and
// about half the registers of the decode kernel's block-per-wave layout (4
// waves per SIMD instead of 2). Each 64-token key block is read once for the
// workgroup (one 16-byte load per thread, kRLook blocks ahead, in registers)
// and staged in LDS, where every wave reads its B operands; one barrier per
// block. The
// linear half of a quad (rows 4m .. 4m+3, one MFMA per 16-token slice) is
// scored by the quad's 4 waves, one slice each, and exchanged through LDS, so
// a row's logits of a block are finished one step later. Every sum is taken
// in the order of score_row and lin_quad: the logits are bit-identical to
// those of the paged kernel for the same row and keys.

constexpr int kRW = kGMax;              // waves per workgroup, one per row
constexpr int kRThreads = kRW * kWave;  // 512
constexpr int kRLook = 3;               // key blocks in flight per thread
constexpr int kStageCodes = 64 * PML_HEAD_DIM;
constexpr int kStage = kStageCodes + 64 * 4;  // a block's codes, then its fp32 scales
static_assert(kGMax == 8 && kRW * kWave == 512 && PML_HEADS == kWave,
              "two quads of rows, one 16-byte load per thread and block, one weight per lane");

struct RowsShared {
    union {
        struct {
            uint8_t q[kGMax * kQBytes];
            float w[kGMax * PML_HEADS];
        } in;                     // set-up: q and w of the piece
        uint8_t stage[2][kStage]; // then: key blocks n (even / odd)
    };
    uint8_t u[kGMax * kUBytes];
    uint8_t us[kGMax * kUScales];
    float lin[2][kGMax][64];  // the linear halves of a block, by row and token
};

// A stage holds token j's 16-byte chunk c at chunk position 8 j + (c ^ (j & 7)),
// so that the 16 tokens of a B-operand read land in distinct banks. Thread t
// loads chunk (t & 7) ^ ((t >> 3) & 7) of token t >> 3, which it stores at
// position t.
__device__ __forceinline__ v8i stage_b(const uint8_t *st, int t) {
    const int lane = lane_id();
    const int jl = lane & 15, grp = lane >> 4;
    const uint8_t *tok = st + (16 * t + jl) * PML_HEAD_DIM;
    const v4i lo = lds_ld<v4i>(tok + ((grp ^ (jl & 7)) << 4));
    const v4i hi = lds_ld<v4i>(tok + (((4 + grp) ^ (jl & 7)) << 4));
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// score_row for a row whose A operands (aq) and weights (wv) are in
// registers and whose keys are in a stage: the same MFMAs (slice by slice,
// head tiles in order within a slice) and the same sums in the same order.
__device__ __forceinline__ float score_row_staged(const v8i *aq, const v4f *wv, const uint8_t *st) {
    // B operands one slice ahead (two register buffers): slice t + 1 is read
    // when slice t's first MFMA issues
    v8i bb[2];
    bb[0] = stage_b(st, 0);
    asm volatile("" ::: "memory");
    float p[4];
    v4f d[16];
    float last = 0.f;
#pragma unroll
    for (int k = 0; k < 16 + kPipe; ++k) {
        if (k < 16) {
            const int t = k >> 2;
            asm volatile("" : "+v"(bb[t & 1]) : "v"(last));
            d[k] = mfma_fp8(aq[k & 3], bb[t & 1]);
            if ((k & 3) == 0 && t < 3) {
                bb[(t + 1) & 1] = stage_b(st, t + 1);
                asm volatile("" ::: "memory");
            }
        }
        if (k >= kPipe) {
            const int e = k - kPipe, t = e >> 2, ht = e & 3;
            asm volatile("" : "+v"(d[e]));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (ht == 0 && i == 0)
                    p[t] = wv[ht][i] * __builtin_fabsf(d[e][i]);
                else
                    p[t] = __builtin_fmaf(wv[ht][i], __builtin_fabsf(d[e][i]), p[t]);
            }
            last = p[t];
        }
    }
    return reduce_slices<false, 64>(p);
}

// -inf on one row's unscored columns of the chunk: the left region [c, lend),
// then the right one [rs, re) (both start on a multiple of 64 columns and end
// on a multiple of 4), one 256-column store instruction at a time.
struct RowFill {
    float *row;
    int col, end, rs, re;
    bool right_next, active;
    int cnt;  // store instructions in all
    __device__ void init(float *r, int l0, int l1, int r0, int r1, bool own) {
        row = r;
        rs = r0;
        re = r1;
        cnt = own ? (max(l1 - l0, 0) + 255) / 256 + (max(r1 - r0, 0) + 255) / 256 : 0;
        active = own && (l1 > l0 || r1 > r0);
        right_next = l1 > l0;
        col = l1 > l0 ? l0 : r0;
        end = l1 > l0 ? l1 : r1;
    }
    __device__ void slice(int n) {
        const int lane = lane_id();
        const float ninf = -__builtin_inff();
        const v4f pat = {ninf, ninf, ninf, ninf};
        for (int t = 0; t < n && active; ++t) {
            const int c = col + 4 * lane;
            if (c < end) store_v4f_async(row + c, pat);
            col += 256;
            if (col >= end) {
                if (right_next && re > rs) {
                    col = rs;
                    end = re;
                    right_next = false;
                } else {
                    active = false;
                }
            }
        }
    }
};

__global__ __launch_bounds__(kRThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void ragged_rows_kernel(
    RaggedArgs a) {
    constexpr int BKV = 64;
    __shared__ __attribute__((aligned(16))) RowsShared sh;

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = uni(tid / kWave);
    const int N = a.N;
    // pieces go out last-rows-first: in a causal prefill those see the most
    // keys, so the longest workgroups start first and the short ones fill the tail
    const int row0 = (gridDim.y - 1 - blockIdx.y) * kGMax;
    const int g = uni(min(kGMax, a.M - row0));

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
    int u_lo = c0, u_hi = c0;
    if (hi_max > lo_min) {
        u_lo = uni(max(lo_min / BKV, c0));
        u_hi = uni(min((hi_max + BKV - 1) / BKV, c1));
        if (u_hi < u_lo) u_hi = u_lo;
    }
    const int cend = min(c1 * BKV, N);
    if (u_hi <= u_lo) {
        for (int i = 0; i < g; ++i)
            fill_neg_inf<kRThreads>(a.out + (int64_t)(row0 + i) * a.out_ld, c0 * BKV, cend);
        return;
    }
    const int nblk = u_hi - u_lo;

    // the first blocks' keys, in flight during the set-up
    const int jt = tid >> 3;
    const int kofs = ((tid & 7) ^ (jt & 7)) << 4;
    v4i kb[kRLook];
    float kz[kRLook];
    // (every thread issues the same loads every step, the scale too, so that
    // the compiler's wait for a block leaves the blocks behind it in flight;
    // blocks past the last one read the last one again)
    auto load_blk = [&](int j, v4i &kv, float &sv) {
        const int t0 = (u_lo + min(j, nblk - 1)) * BKV;
        kv = *(const v4i *)(a.k + (int64_t)min(t0 + jt, N - 1) * PML_HEAD_DIM + kofs);
        sv = a.k_scale[min(t0 + lane, N - 1)];
    };
    auto put_blk = [&](int j, const v4i &kv, float sv) {
        uint8_t *st = sh.stage[j & 1];
        lds_st<v4i>(st + 16 * tid, kv);
        if (tid < 64) lds_st<float>(st + kStageCodes + 4 * tid, sv);
    };
#pragma unroll
    for (int i = 0; i < kRLook; ++i) load_blk(i, kb[i], kz[i]);

    // this wave's row, its bounds and its -inf columns
    const bool own = wave < g;
    const int ri = min(wave, g - 1);
    const int lo = min(max(sload(a.ks, row0 + ri), 0), N);
    const int hi = min(max(sload(a.ke, row0 + ri), lo), N);
    float *orow = a.out + (int64_t)(row0 + ri) * a.out_ld;
    const int rs = min(u_hi * BKV, cend);  // a multiple of 64, or cend
    const int re = max(rs, cend & ~3);
    if (own && lane < 4 && re + lane < cend) orow[re + lane] = -__builtin_inff();  // at most 3 columns
    RowFill fill;
    fill.init(orow, c0 * BKV, u_lo * BKV, rs, re, own);
    const int fill_per = (fill.cnt + nblk - 1) / nblk;

    // q and w of the piece, the pieces of u, then each wave's operands
    {
        // wave i stages row i (8 loads of 16 bytes and one weight per lane)
        const uint8_t *src = a.q + (int64_t)(row0 + ri) * kQBytes;
        v4i x[kQBytes / 16 / kWave];
#pragma unroll
        for (int k = 0; k < kQBytes / 16 / kWave; ++k) x[k] = *(const v4i *)(src + 16 * (kWave * k + lane));
        const float wl = a.w[(int64_t)(row0 + ri) * PML_HEADS + lane];
        if (own) {
#pragma unroll
            for (int k = 0; k < kQBytes / 16 / kWave; ++k) {
                const int c = kWave * k + lane;  // head c / 8, chunk c % 8
                lds_st<v4i>(sh.in.q + ri * kQBytes + q_lds_off(c >> 3, c & 7), x[k]);
            }
            sh.in.w[ri * PML_HEADS + lane] = wl;
        }
    }
    barrier_lds();
    derive_pieces<false, kRThreads>(sh.in.q, sh.in.w, g, sh.u, sh.us);
    barrier_lds();
    const int grp = lane >> 4;
    v8i aq[4];
    v4f wv[4];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
        aq[ht] = load_a<false>(sh.in.q + ri * kQBytes, ht);
        wv[ht] = lds_ld<v4f>(sh.in.w + ri * PML_HEADS + 16 * ht + 4 * grp);
    }
    const int m = wave >> 2, tl = wave & 3;  // this wave's share of the linear half: quad m, slice tl
    barrier_lds();  // every wave holds its operands: the q image becomes the stages
    put_blk(0, kb[0], kz[0]);
    load_blk(kRLook, kb[0], kz[0]);

    float sr_prev = 0.f, sc_prev = 0.f;
    // the row's logits of block j (scored the step before) with the linear
    // halves the quad's waves left in LDS
    auto finish = [&](int j) {
        if (!own) return;
        const int b = u_lo + j;
        const int s = b * BKV + lane;
        float v = (sr_prev + lds_ld<float>(&sh.lin[j & 1][wave][lane])) * sc_prev;
        if (b * BKV < lo || b * BKV + BKV > hi)  // (wave-uniform: only blocks that cross a bound are masked)
            if (s < lo || s >= hi) v = -__builtin_inff();
        if (s < N) store_f32_async(orow + s, v);
    };
    auto step = [&](int n, v4i &kv, float &sv) {
        barrier_lds();  // block n is staged; every wave is done with step n - 1
        if (n > 0) finish(n - 1);
        fill.slice(fill_per);
        const uint8_t *st = sh.stage[n & 1];
        // (the quad's pieces are read again every step: registers are short)
        const v8i au = load_a<false>(sh.u, m);
        const int aus = lds_ld<uint8_t>(sh.us + (16 * m + (lane & 15)) * 4 + grp);
        const v8i bl = stage_b(st, tl);
        v4f dl = mfma_scaled<0>(au, bl, aus, 127);
        asm volatile("" : "+v"(dl));  // (finished here: its operands' registers are free for the rows')
        const float L = (dl[0] + dl[1]) + (dl[2] + dl[3]);
        lds_st<float>(&sh.lin[n & 1][4 * m + grp][16 * tl + (lane & 15)], L);
        const float sc = 0.5f * lds_ld<float>(st + kStageCodes + 4 * lane);  // 1/2: see score_row
        float sr = 0.f;
        if (own) sr = score_row_staged(aq, wv, st);
        asm volatile("" ::: "memory");  // the stage of block n + 1 is written after this step's reads
        put_blk(n + 1, kv, sv);  // (after the last block: a stage nobody reads)
        load_blk(n + 1 + kRLook, kv, sv);
        sr_prev = sr;
        sc_prev = sc;
    };
    for (int n = 0; n < nblk; n += kRLook) {
        step(n, kb[1], kz[1]);
        if (n + 1 >= nblk) break;
        step(n + 1, kb[2], kz[2]);
        if (n + 2 >= nblk) break;
        step(n + 2, kb[0], kz[0]);
    }
    barrier_lds();
    finish(nblk - 1);
    fill.slice(fill.cnt);  // (nothing is left: every step took its share)
}

}  // namespace pml

static inline bool al16r(const void *p) { return ((uintptr_t)p & 15) == 0; }

extern "C" int mqa_logits(const void *q, int M, int num_heads, int head_dim, const void *k,
                          const float *k_scale, int N, const float *weights,
                          const int32_t *cu_seqlen_ks, const int32_t *cu_seqlen_ke, float *logits,
                          int64_t logits_ld, void *stream) {
    if (M < 0 || N < 0) return PML_ERR_SHAPE;
    // (pieces of 8 rows fill at most 65535 grid rows; key positions plus a
    // block stay inside int32)
    if (M > 65535 * pml::kGMax || N > 0x7fffffff - 256) return PML_ERR_SHAPE;
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
    hipLaunchKernelGGL(pml::ragged_rows_kernel, grid, dim3(pml::kRThreads), 0, (hipStream_t)stream, a);
    return hipGetLastError() == hipSuccess ? PML_OK : PML_ERR_HIP;
}
