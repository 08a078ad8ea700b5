// Scoring core shared by the paged (decode) and ragged (prefill) logits
// kernels.
//
//   logit[r, s] = scale_k[s] * sum_h w[r,h] * max(0, <q[r,h,:], k[s,:]>)
//
// The fp8 per-token scale is positive, so it moves out of the ReLU; MXFP4
// pages carry per-32-element e8m0 scales that the scaled MFMA applies.
//
// The ReLU is split as 2 max(0, x) = x + |x|. The linear half summed over the
// heads is one dot product, sum_h w_h <q_h, k> = <u, k> with u = sum_h w_h q_h,
// which runs on the matrix core: u is held as four fp8 pieces with one e8m0
// scale per 32 elements each (u = p0 + p1 + p2 + p3 up to about 2^-16 of each
// element), and one MFMA scores the 4 pieces of 4 rows against a 16-token
// slice. The other half costs one VALU instruction per (head, token) value
// (an FMA with an abs modifier): on gfx950 a wave64 VALU instruction takes
// about 4.6 SIMD cycles and every MFMA about 10 of the same issue port, so
// the epilogue, not the matrix core, set the speed of the two-instruction
// ReLU-and-weight form.
//
// Work split of the paged kernel (gfx950; the ragged kernel instead gives each
// wave one row, see ragged_logits.hip): a workgroup of 4 waves scores a
// row-piece (up to kGMax rows of one request) against key blocks; q and w of
// the piece sit in LDS, shared by the 4 waves. Each wave takes whole key
// blocks on its own: the block's keys go from HBM straight into VGPRs,
// already laid out as the B operand of v_mfma_f32_16x16x128_f8f6f4 (lane l
// holds token l % 16 of a 16-token slice), two buffers deep so one block is
// in flight while one is scored. For every row the wave runs 4 head tiles x
// (BKV / 16) token slices of MFMAs, folds ReLU and w into per-lane partial
// sums in registers, and a transpose-reduce with v_permlane32/16_swap leaves
// one finished token per lane; the block's logits wait in LDS and go out one
// step later as coalesced row segments, 16 bytes per lane and four rows per
// store instruction. No barrier is taken per block, only at piece changes.
#pragma once

#include "pml_device.h"

namespace pml {

constexpr int kQBytes = PML_HEADS * PML_HEAD_DIM;  // q of one row: 8 KB
constexpr int kCW = 4;                             // waves per workgroup
constexpr int kLThreads = kCW * kWave;

template <bool FP4, int BKV>
struct BlockCfg {
    static constexpr int D = PML_HEAD_DIM;
    static constexpr int TOKB = FP4 ? D / 2 : D;   // value bytes per token
    static constexpr int VBYTES = BKV * TOKB;      // values region of a page
    static constexpr int NT = BKV / 16;            // 16-token slices per block
    static constexpr int NV = FP4 ? 1 : 2;         // 16-B value loads per lane per slice
    static constexpr int NS = FP4 ? NT : 1;        // scale dwords per lane
    static_assert(NT == 2 || NT == 4, "block_kv 32 or 64");
};

// One key block in VGPRs in B-operand layout, plus the scales this lane needs:
// fp8: the fp32 scale of the token this lane finishes; MXFP4: per slice, the
// e8m0 byte of (token 16t + lane % 16, k-block lane / 16) in bits 0..7.
template <bool FP4, int BKV>
struct KeyRegs {
    using C = BlockCfg<FP4, BKV>;
    v4i v[C::NT][C::NV];
    uint32_t sc[C::NS];
};

// Token this lane holds after the transpose-reduce of a block.
template <int BKV>
__device__ __forceinline__ int out_token(int lane) {
    return BKV == 64 ? lane : ((lane >> 5) * 16 + (lane & 15));
}
template <int BKV>
__device__ __forceinline__ bool out_lane(int lane) {
    return BKV == 64 ? true : ((lane >> 4) & 1) == 0;
}

// Load a cache page (values region [BKV][TOKB], then scales) into registers.
// Lane group g takes the hardware's k order (see load_a): fp8 bytes
// 16g .. 16g+15 and 64+16g .. 64+16g+15 of its token, MXFP4 bytes 16g .. 16g+15
// (the 32 fp4 values of k-block g). Each load instruction then reads one
// contiguous 64-byte run per token.
template <bool FP4, int BKV>
__device__ __forceinline__ void load_page(const uint8_t *pg, KeyRegs<FP4, BKV> &k) {
    using C = BlockCfg<FP4, BKV>;
    const int lane = lane_id();
    const int tl = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int t = 0; t < C::NT; ++t) {
        const uint8_t *tok = pg + (16 * t + tl) * C::TOKB;
        if constexpr (FP4) {
            k.v[t][0] = *(const v4i *)(tok + 16 * grp);
            k.sc[t] = *(const uint32_t *)(pg + C::VBYTES + (16 * t + tl) * 4) >> (8 * grp);
        } else {
            k.v[t][0] = *(const v4i *)(tok + 16 * grp);
            k.v[t][1] = *(const v4i *)(tok + 64 + 16 * grp);
        }
    }
    if (!FP4) k.sc[0] = *(const uint32_t *)(pg + C::VBYTES + 4 * out_token<BKV>(lane));
}

// A block of BKV tokens from BKV / PG cache pages of PG tokens each (pg[i]
// holds tokens PG * i .. PG * i + PG - 1), in the register layout load_page
// gives a page of BKV tokens: slice t comes from page t / (PG / 16), and an
// fp8 lane's token scale from the page of the token it finishes.
template <bool FP4, int BKV, int PG>
__device__ __forceinline__ void load_pages(const uint8_t *const *pg, KeyRegs<FP4, BKV> &k) {
    using C = BlockCfg<FP4, BKV>;
    constexpr int PVB = PG * C::TOKB;  // values region of one page
    constexpr int SPP = PG / 16;       // slices per page
    const int lane = lane_id();
    const int tl = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int t = 0; t < C::NT; ++t) {
        const uint8_t *p = pg[t / SPP];
        const int tok = 16 * (t % SPP) + tl;
        if constexpr (FP4) {
            k.v[t][0] = *(const v4i *)(p + tok * C::TOKB + 16 * grp);
            k.sc[t] = *(const uint32_t *)(p + PVB + tok * 4) >> (8 * grp);
        } else {
            k.v[t][0] = *(const v4i *)(p + tok * C::TOKB + 16 * grp);
            k.v[t][1] = *(const v4i *)(p + tok * C::TOKB + 64 + 16 * grp);
        }
    }
    if constexpr (!FP4) {
        const int s = out_token<BKV>(lane);
        k.sc[0] = *(const uint32_t *)(pg[s / PG] + PVB + 4 * (s % PG));
    }
}

// Load keys [t0, t0 + 64) of a contiguous fp8 key array k[N][D] and their fp32
// scales. Tokens at or past N are read as token N - 1 (their logits are never
// stored), so no load leaves the arrays.
__device__ __forceinline__ void load_contig(const uint8_t *k, const float *k_scale, int N, int t0,
                                            KeyRegs<false, 64> &kr) {
    const int lane = lane_id();
    const int tl = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint8_t *tok = k + (int64_t)min(t0 + 16 * t + tl, N - 1) * PML_HEAD_DIM;
        kr.v[t][0] = *(const v4i *)(tok + 16 * grp);
        kr.v[t][1] = *(const v4i *)(tok + 64 + 16 * grp);
    }
    kr.sc[0] = __float_as_uint(k_scale[min(t0 + lane, N - 1)]);
}

// LDS image of q for one row: head h's 128 bytes at h * 128, its 16-B chunk c
// stored at chunk position c ^ (h & 7), so that the 16 heads of an A-operand
// read land in distinct banks.
__device__ __forceinline__ int q_lds_off(int h, int c) { return h * PML_HEAD_DIM + ((c ^ (h & 7)) << 4); }

struct NoWait {
    __device__ void operator()() const {}
};

// Stage q and w of rows r0 .. r0 + g - 1 into LDS (the whole workgroup). All
// loads are issued before the first LDS store, so staging costs one memory
// latency rather than one per round of the thread loop. before_store runs
// between the loads and the stores (a barrier that frees the LDS rows, say,
// which the loads then overlap).
template <int NTH = kLThreads, typename B = NoWait>
__device__ __forceinline__ void stage_rows(const uint8_t *q, const float *w, int64_t r0, int g, uint8_t *s_q,
                                           float *s_w, B before_store = B()) {
    constexpr int kChunks = kQBytes / 16;               // 16-B chunks per row
    constexpr int kPer = (kGMax * kChunks + NTH - 1) / NTH;  // chunks per thread, at most
    constexpr int kWPer = (kGMax * PML_HEADS + NTH - 1) / NTH;
    const int tid = threadIdx.x;
    const int nchunk = g * kChunks;
    const uint8_t *src = q + r0 * kQBytes;
    v4i x[kPer];
    float wv[kWPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k)
        if (tid + k * NTH < nchunk) x[k] = *(const v4i *)(src + (tid + k * NTH) * 16);
#pragma unroll
    for (int k = 0; k < kWPer; ++k)
        if (tid + k * NTH < g * PML_HEADS) wv[k] = w[r0 * PML_HEADS + tid + k * NTH];
    before_store();
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int i = tid + k * NTH;
        if (i < nchunk) {
            const int row = i / kChunks, rem = i % kChunks;
            *(v4i *)(s_q + row * kQBytes + q_lds_off(rem / 8, rem % 8)) = x[k];
        }
    }
#pragma unroll
    for (int k = 0; k < kWPer; ++k)
        if (tid + k * NTH < g * PML_HEADS) s_w[tid + k * NTH] = wv[k];
}

// fp4 q (packed e2m1 values [H][D/2] and e8m0 scales [H][D/32] per row, the
// MXFP4 key layout) in the same 8-KB LDS row: head h's 64 value bytes at
// h * 64, its 16-B chunk c (k-block c) at chunk position c ^ ((h >> 2) & 3) so
// that the 16 heads of an A-operand read land in distinct banks, then the
// scales, 4 bytes per head, from byte 4096.
constexpr int kQ4Values = PML_HEADS * PML_HEAD_DIM / 2;  // 4096
constexpr int kQ4Scales = PML_HEADS * PML_HEAD_DIM / 32;  // 256
__device__ __forceinline__ int q4_lds_off(int h, int c) { return h * (PML_HEAD_DIM / 2) + ((c ^ ((h >> 2) & 3)) << 4); }

// Stage fp4 q (values and scales) and w of rows r0 .. r0 + g - 1 into LDS,
// every load issued before the first store (before_store as in stage_rows).
template <int NTH = kLThreads, typename B = NoWait>
__device__ __forceinline__ void stage_rows_q4(const uint8_t *qv, const uint8_t *qs, const float *w, int64_t r0,
                                              int g, uint8_t *s_q, float *s_w, B before_store = B()) {
    constexpr int kVC = kQ4Values / 16, kSC = kQ4Scales / 16, kRow = kVC + kSC;  // 16-B chunks
    constexpr int kPer = (kGMax * kRow + NTH - 1) / NTH;
    constexpr int kWPer = (kGMax * PML_HEADS + NTH - 1) / NTH;
    const int tid = threadIdx.x;
    const int nchunk = g * kRow;
    v4i x[kPer];
    float wv[kWPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int i = tid + k * NTH;
        if (i < nchunk) {
            const int row = i / kRow, rem = i % kRow;
            const uint8_t *src = rem < kVC ? qv + (r0 + row) * kQ4Values + rem * 16
                                           : qs + (r0 + row) * kQ4Scales + (rem - kVC) * 16;
            x[k] = *(const v4i *)src;
        }
    }
#pragma unroll
    for (int k = 0; k < kWPer; ++k)
        if (tid + k * NTH < g * PML_HEADS) wv[k] = w[r0 * PML_HEADS + tid + k * NTH];
    before_store();
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int i = tid + k * NTH;
        if (i < nchunk) {
            const int row = i / kRow, rem = i % kRow;
            const int off = rem < kVC ? q4_lds_off(rem / 4, rem % 4) : kQ4Values + (rem - kVC) * 16;
            *(v4i *)(s_q + row * kQBytes + off) = x[k];
        }
    }
#pragma unroll
    for (int k = 0; k < kWPer; ++k)
        if (tid + k * NTH < g * PML_HEADS) s_w[tid + k * NTH] = wv[k];
}

// ---- the linear half: u = sum_h w_h q_h as four scaled fp8 pieces ----------
//
// Piece image of a row in LDS: 4 pseudo-heads (the pieces) of 128 fp8 codes,
// laid out and swizzled as q (pseudo-head 4 i + p of row i at q_lds_off), so
// that the A operand of pieces of rows 4m .. 4m+3 is load_a(s_u, m); then one
// e8m0 byte per (pseudo-head, 32-element block), 4 per pseudo-head.
// In HBM (the logits call's workspace) a row's pieces are [4][128] codes
// followed, in a second array, by [4][4] scale bytes.
constexpr int kPieces = 4;
constexpr int kUBytes = kPieces * PML_HEAD_DIM;          // codes of one row: 512
constexpr int kUScales = kPieces * (PML_HEAD_DIM / 32);  // scale bytes of one row: 16

// Stage the pieces of rows r0 .. r0 + g - 1 (codes [rows][512], scales
// [rows][16]) into the LDS image (the whole workgroup; loads first, then
// before_store, then the stores).
template <int NTH = kLThreads, typename B = NoWait>
__device__ __forceinline__ void stage_pieces(const uint8_t *codes, const uint8_t *scales, int64_t r0, int g,
                                             uint8_t *s_u, uint8_t *s_us, B before_store = B()) {
    constexpr int kChunks = kUBytes / 16;                          // 32 per row
    constexpr int kPer = (kGMax * (kChunks + 1) + NTH - 1) / NTH;  // + one chunk of scales per row
    const int tid = threadIdx.x;
    const int n = g * (kChunks + 1);
    v4i x[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int i = tid + k * NTH;
        if (i < n) {
            const int row = i / (kChunks + 1), c = i % (kChunks + 1);
            x[k] = c < kChunks ? *(const v4i *)(codes + (r0 + row) * kUBytes + c * 16)
                               : *(const v4i *)(scales + (r0 + row) * kUScales);
        }
    }
    before_store();
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int i = tid + k * NTH;
        if (i < n) {
            const int row = i / (kChunks + 1), c = i % (kChunks + 1);
            if (c < kChunks)
                lds_st<v4i>(s_u + q_lds_off(kPieces * row + c / 8, c % 8), x[k]);
            else
                lds_st<v4i>(s_us + row * kUScales, x[k]);
        }
    }
}

// u[d] = sum_h w_h q_h[d] (fp32) of the staged rows 0 .. g-1 and its four
// pieces, written to the LDS image (s_u, s_us). Threads 0..255 run it, one row
// at a time: thread 8 dq + hp sums heads 8 hp .. 8 hp + 7 (in order) of
// elements 4 dq .. 4 dq + 3, and the 8 head parts of an element are added by
// lanes xor 1, 2, 4 (every lane of the group gets the same bits), so each row
// costs 8 dependent steps per thread instead of 64. Every path that derives
// pieces uses this order, so a row's pieces do not depend on which kernel made
// them. Piece p of a 32-element block (one wave: dq 8c .. 8c + 7) takes the
// e8m0 scale 2^e with e = floor(log2 m) - 7 for the largest magnitude m of what
// the earlier pieces left (so its codes stay below 256, within e4m3), rounds
// the rest over 2^e to fp8 and subtracts the rounded value, which is exact in
// fp32. Each piece removes about 4 significant bits, so after four the
// remainder is about 2^-16 of the element or less.
// Q4: q is fp4 (values and e8m0 scales, stage_rows_q4's image).
// With NTH >= 512 the rows are taken NTH / 256 at a time (thread t serves
// rows t / 256, t / 256 + NTH / 256, ...), each in the same order.
// Callers put a barrier between the staging of q / w and this, and between
// this and reads of the image.
template <bool Q4, int NTH = kLThreads>
__device__ __forceinline__ void derive_pieces(const uint8_t *s_q, const float *s_w, int g, uint8_t *s_u,
                                              uint8_t *s_us) {
    static_assert(NTH >= 256, "256 threads per row");
    constexpr int kPar = NTH / 256;  // rows at a time
    const int tid = threadIdx.x;
    if (tid >= 256 * kPar) return;
    const int t8 = tid & 255;
    const int dq = t8 >> 3, hp = t8 & 7;  // elements 4 dq .. 4 dq + 3, heads 8 hp .. 8 hp + 7
    for (int row = tid >> 8; row < g; row += kPar) {
        const uint8_t *qr = s_q + row * kQBytes;
        const float *wr = s_w + row * PML_HEADS;
        float u[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int h = 8 * hp + j;
            const float wh = lds_ld<float>(wr + h);
            float qv[4];
            if constexpr (Q4) {
                const int c = dq >> 3;  // 32-element block
                const int sb = lds_ld<uint8_t>(qr + kQ4Values + 4 * h + c);
                const float sc = sb == 255 ? __builtin_nanf("") : __builtin_amdgcn_ldexpf(1.0f, sb - 127);
                const uint32_t two = lds_ld<uint16_t>(qr + q4_lds_off(h, c) + 2 * (dq & 7));
                const v2f lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(two, sc, 0);
                const v2f hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(two, sc, 1);
                qv[0] = lo[0]; qv[1] = lo[1]; qv[2] = hi[0]; qv[3] = hi[1];
            } else {
                const uint32_t four = lds_ld<uint32_t>(qr + q_lds_off(h, dq >> 2) + 4 * (dq & 3));
                const v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8(four, false);
                const v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8(four, true);
                qv[0] = lo[0]; qv[1] = lo[1]; qv[2] = hi[0]; qv[3] = hi[1];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) u[e] = __builtin_fmaf(wh, qv[e], u[e]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            u[e] += __shfl_xor(u[e], 1, kWave);
            u[e] += __shfl_xor(u[e], 2, kWave);
            u[e] += __shfl_xor(u[e], 4, kWave);
        }
#pragma unroll
        for (int p = 0; p < kPieces; ++p) {
            float m = fmaxf(fmaxf(__builtin_fabsf(u[0]), __builtin_fabsf(u[1])),
                            fmaxf(__builtin_fabsf(u[2]), __builtin_fabsf(u[3])));
            // the 8 elements-of-4 of a 32-element block are lanes xor 8, 16, 32 of one wave
            m = fmaxf(m, __shfl_xor(m, 8, kWave));
            m = fmaxf(m, __shfl_xor(m, 16, kWave));
            m = fmaxf(m, __shfl_xor(m, 32, kWave));
            int e = m > 0.f ? __builtin_amdgcn_frexp_expf(m) - 8 : -127;  // m in [2^(e+7), 2^(e+8))
            e = max(e, -127);
            const float inv = __builtin_amdgcn_ldexpf(1.0f, -e);
            const int lo2 = __builtin_amdgcn_cvt_pk_fp8_f32(u[0] * inv, u[1] * inv, 0, false);
            const int codes = __builtin_amdgcn_cvt_pk_fp8_f32(u[2] * inv, u[3] * inv, lo2, true);
            const v2f d01 = __builtin_amdgcn_cvt_pk_f32_fp8(codes, false);
            const v2f d23 = __builtin_amdgcn_cvt_pk_f32_fp8(codes, true);
            u[0] -= __builtin_amdgcn_ldexpf(d01[0], e);
            u[1] -= __builtin_amdgcn_ldexpf(d01[1], e);
            u[2] -= __builtin_amdgcn_ldexpf(d23[0], e);
            u[3] -= __builtin_amdgcn_ldexpf(d23[1], e);
            if (hp == 0) {
                const int ph = kPieces * row + p;  // pseudo-head
                lds_st<int>(s_u + q_lds_off(ph, dq >> 2) + 4 * (dq & 3), codes);
                if ((dq & 7) == 0) lds_st<uint8_t>(s_us + ph * 4 + (dq >> 3), (uint8_t)(e + 127));
            }
        }
    }
}

// A operand of fp4 q (heads 16 ht + lane % 16, k-block lane / 16: one 16-B
// chunk, the upper half of the operand unused) and its e8m0 scale in bits 0-7.
__device__ __forceinline__ v8i load_a_q4(const uint8_t *s_qrow, int ht, int &scale) {
    const int lane = lane_id();
    const int h = 16 * ht + (lane & 15), grp = lane >> 4;
    const v4i v = lds_ld<v4i>(s_qrow + q4_lds_off(h, grp));
    scale = (int)((lds_ld<uint32_t>(s_qrow + kQ4Values + 4 * h) >> (8 * grp)) & 0xffu);
    return v8i{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
}

// A operand (q of heads 16 ht + lane % 16) of one staged row, in the
// hardware's k order for v_mfma_scale_f32_16x16x128_f8f6f4 as measured on
// gfx950: an fp8 operand holds k = 16g .. 16g+15 in bytes 0-15 and
// k = 64+16g .. 64+16g+15 in bytes 16-31 of lane group g, an fp4 operand holds
// k = 32g .. 32g+31 in order (low nibble first), and the e8m0 scale of
// k-block g comes from lane group g. (fp8 x fp8 only needs A and B in the
// same order; the hardware order also keeps the key loads contiguous.)
template <bool FP4>
__device__ __forceinline__ v8i load_a(const uint8_t *s_qrow, int ht) {
    const int lane = lane_id();
    const int h = 16 * ht + (lane & 15), grp = lane >> 4;
    const int c0 = grp;
    const int c1 = 4 + grp;
    const v4i lo = lds_ld<v4i>(s_qrow + q_lds_off(h, c0));
    const v4i hi = lds_ld<v4i>(s_qrow + q_lds_off(h, c1));
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Lane l holds partial sums p[t] of token 16t + l % 16 over the heads of lane
// group l / 16; transpose slices against lane groups and add, leaving token
// out_token(l)'s total in lane l.
template <bool FP4, int BKV>
__device__ __forceinline__ float reduce_slices(float *p) {  // p[BlockCfg::NT]
    using C = BlockCfg<FP4, BKV>;
    if (C::NT == 4) {
        swap32(p[0], p[2 % C::NT]);
        swap32(p[1 % C::NT], p[3 % C::NT]);
        float x = p[0] + p[2 % C::NT];
        float y = p[1 % C::NT] + p[3 % C::NT];
        swap16(x, y);
        return x + y;
    } else {
        swap32(p[0], p[1 % C::NT]);
        float x = p[0] + p[1 % C::NT];
        float y = x;
        swap16(x, y);
        return x + y;
    }
}

constexpr int kPipe = 3;  // MFMAs issued ahead of the epilogue that reads them

// MFMA of one 16-token slice t. fp8 x fp8 takes the unscaled opcode: the
// scaled form costs an extra VALU instruction per MFMA (it loads the scales).
// MXFP4 keys need their e8m0 block scales, with fp8 A at unit scale (`a_scale`
// = 127) or fp4 A (Q4) at its own e8m0 scale: e2m1 x e2m1 runs at twice the
// fp8 rate.
template <bool FP4, int BKV, bool Q4 = false>
__device__ __forceinline__ v4f mfma_slice(const KeyRegs<FP4, BKV> &k_, const v8i &a, int t, int a_scale) {
    if constexpr (FP4) {
        const v8i b = v8i{k_.v[t][0][0], k_.v[t][0][1], k_.v[t][0][2], k_.v[t][0][3], 0, 0, 0, 0};
        if constexpr (Q4)
            return mfma_scaled_ab<4, 4>(a, b, a_scale, (int)(k_.sc[t] & 0xffu));
        else
            return mfma_scaled<4>(a, b, a_scale, (int)(k_.sc[t] & 0xffu));
    } else {
        const v8i b = v8i{k_.v[t][0][0], k_.v[t][0][1], k_.v[t][0][2], k_.v[t][0][3],
                          k_.v[t][1][0], k_.v[t][1][1], k_.v[t][1][2], k_.v[t][1][3]};
        return mfma_fp8(a, b);
    }
}

// The transpose of the linear half: L[t] (lane group G = quad row G, tokens
// 16t + j) to M[G] (token out_token(lane) in lane `lane`).
template <int NT>
__device__ __forceinline__ void lin_transpose(float *L, float *M) {
    if constexpr (NT == 4) {
        // L[t] row G = values of quad row G at tokens 16t + j; after the swaps,
        // M[G] row t holds them, i.e. token 16t + j sits in lane 16t + j
        swap32(L[0], L[2]);
        swap32(L[1], L[3]);
        swap16(L[0], L[1]);
        swap16(L[2], L[3]);
        M[0] = L[0];
        M[1] = L[1];
        M[2] = L[2];
        M[3] = L[3];
    } else {
        // block_kv 32: token 16t + j belongs in lane 32t + j (out_token)
        float A = L[0], B = L[1 % NT];
        swap32(A, B);  // A: rows (0, 1, 0, 1) of quad rows 0/1; B: quad rows 2/3
        float A2 = A, B2 = B;
        swap16(A, A2);  // A: quad row 0 in lane groups 0 and 2; A2: quad row 1
        swap16(B, B2);
        M[0] = A;
        M[1] = A2;
        M[2] = B;
        M[3] = B2;
    }
}

// The linear half of rows 4m .. 4m+3 against the block: A is their pieces
// (row 4m + G's piece p in A-row 4G + p, with its e8m0 scale), so lane group G
// of the result of slice t holds row 4m + G's four piece dots for token
// 16t + lane % 16 in its four registers; their sum is <u, k> of that row and
// token (before the key scale). A transpose of lane groups against slices
// (permlane swaps, as in reduce_slices) then leaves row 4m + G's values in
// M[G] with token out_token(lane) in lane `lane`, the layout score_row
// returns, so a row adds its own M[G] after its reduction, whatever its place
// in the quad. fp8 keys take unit B scales (their fp32 per-token scale is
// applied with the rest of the score).
template <bool FP4, int BKV>
__device__ __forceinline__ void lin_quad(const KeyRegs<FP4, BKV> &k_, const uint8_t *s_u, const uint8_t *s_us,
                                         int m, float *M) {  // M[4]
    using C = BlockCfg<FP4, BKV>;
    const int lane = lane_id();
    v8i a = load_a<false>(s_u, m);
    int sc = lds_ld<uint8_t>(s_us + (16 * m + (lane & 15)) * 4 + (lane >> 4));
    v4f d[C::NT];
#pragma unroll
    for (int t = 0; t < C::NT; ++t) {
        if constexpr (FP4) {
            const v8i b = v8i{k_.v[t][0][0], k_.v[t][0][1], k_.v[t][0][2], k_.v[t][0][3], 0, 0, 0, 0};
            d[t] = mfma_scaled<4>(a, b, sc, (int)(k_.sc[t] & 0xffu));
        } else {
            const v8i b = v8i{k_.v[t][0][0], k_.v[t][0][1], k_.v[t][0][2], k_.v[t][0][3],
                              k_.v[t][1][0], k_.v[t][1][1], k_.v[t][1][2], k_.v[t][1][3]};
            d[t] = mfma_scaled<0>(a, b, sc, 127);
        }
    }
    float L[C::NT];
#pragma unroll
    for (int t = 0; t < C::NT; ++t) L[t] = (d[t][0] + d[t][1]) + (d[t][2] + d[t][3]);
    lin_transpose<C::NT>(L, M);
}


// Score one staged row against the block in registers: this lane's
// sum_h w_h |x_h|, x_h = <q_h, k>, for token out_token(lane), before the key
// scale. With the linear half <u, k> (lin_quad) it gives twice the score,
//   2 sum_h w_h max(0, x_h) = <u, k> + sum_h w_h |x_h|;
// the factor 2 is exact and the caller folds 1/2 into the scale. The sum here
// costs one FMA with an abs modifier per (head, token) value.
//
// With LIN the row also scores the linear half of its quad m (as lin_quad,
// into M[0..3]): its MFMAs lead the row's MFMA stream and their sums and
// transpose trail it, so they overlap the row's own work instead of forming a
// dependent chain of their own.
template <bool FP4, int BKV, bool Q4 = false, bool LIN = false>
__device__ __forceinline__ float score_row(const KeyRegs<FP4, BKV> &k_, const uint8_t *s_qrow,
                                           const float *s_wrow, const uint8_t *s_u = nullptr,
                                           const uint8_t *s_us = nullptr, int m = 0, float *M = nullptr) {
    static_assert(!Q4 || FP4, "fp4 q pairs with MXFP4 keys");
    using C = BlockCfg<FP4, BKV>;
    const int lane = lane_id();
    const int grp = lane >> 4;
    constexpr int NL = LIN ? C::NT : 0;  // leading MFMAs of the linear half
    float p[C::NT];
    // LDS operands in the order of use (the linear half's, then head tile 0,
    // 1, ...): compiler barriers keep the reads in this order, so each MFMA
    // waits only for the reads before it
    [[maybe_unused]] v8i al = {};
    int sl = 0;
    if constexpr (LIN) {
        al = load_a<false>(s_u, m);
        sl = lds_ld<uint8_t>(s_us + (16 * m + (lane & 15)) * 4 + (lane >> 4));
        asm volatile("" ::: "memory");
    }
    v8i av[4];
    v4f wv[4];
    [[maybe_unused]] int asc[4];  // fp4 q: A scale per head tile
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
        if constexpr (Q4)
            av[ht] = load_a_q4(s_qrow, ht, asc[ht]);
        else
            av[ht] = load_a<FP4>(s_qrow, ht);
        wv[ht] = lds_ld<v4f>(s_wrow + 16 * ht + 4 * grp);
        asm volatile("" ::: "memory");
    }
    // MFMA k (after the NL linear ones: head tile (k - NL) / NT, slice
    // (k - NL) % NT) is issued kPipe steps before its epilogue, so the matrix
    // core works while the VALU folds earlier results, and enough independent
    // instructions separate an MFMA from its reader that few wait states are
    // padded. The MFMA intrinsics have no side effects, so empty volatile asm
    // statements pin the order: each MFMA takes an operand (its A tile, or for
    // MXFP4 the unit A scale) that an asm before it claims to rewrite, and that
    // asm also reads the previous epilogue's result, so epilogues stay between
    // the MFMAs. (fp4 q: the operand is the head tile's A scale.)
    constexpr int NK = 4 * C::NT;
    v4f d[NL + NK];
    [[maybe_unused]] float L[C::NT];
    int unit = 127;  // e8m0 1.0
    float last = 0.f;  // the accumulator the previous epilogue wrote
#pragma unroll
    for (int k = 0; k < NL + NK + kPipe; ++k) {
        if (k < NL) {
            asm volatile("" : "+v"(sl) : "v"(last));
            if constexpr (FP4) {
                const v8i b = v8i{k_.v[k][0][0], k_.v[k][0][1], k_.v[k][0][2], k_.v[k][0][3], 0, 0, 0, 0};
                d[k] = mfma_scaled<4>(al, b, sl, (int)(k_.sc[k] & 0xffu));
            } else {
                const v8i b = v8i{k_.v[k][0][0], k_.v[k][0][1], k_.v[k][0][2], k_.v[k][0][3],
                                  k_.v[k][1][0], k_.v[k][1][1], k_.v[k][1][2], k_.v[k][1][3]};
                d[k] = mfma_scaled<0>(al, b, sl, 127);
            }
        } else if (k < NL + NK) {
            const int j = k - NL;
            if constexpr (Q4) {
                asm volatile("" : "+v"(asc[j / C::NT]) : "v"(last));
                d[k] = mfma_slice<FP4, BKV, true>(k_, av[j / C::NT], j % C::NT, asc[j / C::NT]);
            } else {
                if constexpr (FP4)
                    asm volatile("" : "+v"(unit) : "v"(last));
                else
                    asm volatile("" : "+v"(av[j / C::NT]) : "v"(last));
                d[k] = mfma_slice<FP4, BKV>(k_, av[j / C::NT], j % C::NT, unit);
            }
        }
        if (k >= kPipe) {
            const int e = k - kPipe;
            asm volatile("" : "+v"(d[e]));
            if (e < NL) {
                L[e] = (d[e][0] + d[e][1]) + (d[e][2] + d[e][3]);
                last = L[e];
            } else {
                const int j = e - NL, ht = j / C::NT, t = j % C::NT;
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
    }
    if constexpr (LIN) lin_transpose<C::NT>(L, M);
    return reduce_slices<FP4, BKV>(p);
}

// An empty use of the block's registers. The compiler places its wait for
// the block's loads here, at the top of a step, where only those loads (and
// stores issued a step earlier) are outstanding; the next block's loads are
// issued after it and stay in flight while this block is scored.
template <bool FP4, int BKV>
__device__ __forceinline__ void touch(const KeyRegs<FP4, BKV> &k) {
    using C = BlockCfg<FP4, BKV>;
#pragma unroll
    for (int t = 0; t < C::NT; ++t)
#pragma unroll
        for (int j = 0; j < C::NV; ++j) asm volatile("" ::"v"(k.v[t][j]));
#pragma unroll
    for (int j = 0; j < C::NS; ++j) asm volatile("" ::"v"(k.sc[j]));
}

// Global stores issued as inline asm. The compiler's wait tracking then
// counts only key-block loads in the vector-memory counter and waits for a
// block exactly, leaving the blocks behind it in flight; in hardware the
// stores still count, which can only make those waits stricter (loads
// complete in order among themselves). A store reads its data registers when
// it issues, so no hazard guard is needed around it.
__device__ __forceinline__ void store_f32_async(float *p, float v) {
    asm volatile("global_store_dword %0, %1, off" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void store_v4f_async(float *p, v4f v) {
    asm volatile("global_store_dwordx4 %0, %1, off" ::"v"(p), "v"(v) : "memory");
}
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_v2u_async(uint16_t *p, v2u v) {
    asm volatile("global_store_dwordx2 %0, %1, off" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void store_u16_async(uint16_t *p, uint32_t v) {
    asm volatile("global_store_short %0, %1, off" ::"v"(p), "v"(v) : "memory");
}

// Two floats rounded to bf16 (nearest even, NaN kept), lo in bits 0-15.
typedef float v2f_t __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    const v2f_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, v2bf_t));
}

// One block's logits for up to kGMax rows, parked in the wave's own LDS slot
// until the next step stores them ahead of the key loads it issues.
template <int BKV>
struct WaveSlot {
    float v[kGMax][BKV];
};

// Store rows (bit i of mask) of the parked block at columns [col0, col0 + BKV),
// never at or past ncols. Each lane moves 4 consecutive columns of one row, so
// one store instruction (16 bytes of fp32, or 8 of bf16) covers 64 * 4 / BKV
// rows; a 4-column group that crosses ncols is stored column by column. OT is
// float, or uint16_t for bf16 logits (rounded to nearest even).
template <int BKV, typename OT = float>
__device__ __forceinline__ void flush_slot(const WaveSlot<BKV> &sl, int mask, int64_t row0, int col0, int ncols,
                                           OT *out, int64_t out_ld) {
    constexpr int kLanesPerRow = BKV / 4;
    constexpr int kRowsPer = kWave / kLanesPerRow;  // rows per instruction: 4 (BKV 64) or 8 (BKV 32)
    const int lane = lane_id();
    const int c4 = 4 * (lane % kLanesPerRow);
    const int s = col0 + c4;
#pragma unroll
    for (int m = 0; m < kGMax; m += kRowsPer) {
        if ((mask >> m) == 0) break;
        const int i = m + lane / kLanesPerRow;
        if (i < kGMax && ((mask >> i) & 1)) {
            const v4f v = lds_ld<v4f>(&sl.v[i][c4]);
            OT *p = out + (row0 + i) * out_ld + s;
            if constexpr (sizeof(OT) == 4) {
                if (s + 4 <= ncols) {
                    store_v4f_async(p, v);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (s + j < ncols) store_f32_async(p + j, v[j]);
                }
            } else {
                const v2u h = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
                if (s + 4 <= ncols) {
                    store_v2u_async(p, h);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (s + j < ncols) store_u16_async(p + j, h[j / 2] >> (16 * (j % 2)));
                }
            }
        }
    }
}

// Fill columns [c0, c1) of one row with -inf (the whole workgroup of NTH
// threads), fp32 or bf16 (OT = uint16_t); rows are 16-B aligned.
template <int NTH = kLThreads, typename OT = float>
__device__ __forceinline__ void fill_neg_inf(OT *row, int c0, int c1) {
    if (c0 >= c1) return;
    constexpr int V = 16 / sizeof(OT);  // columns per 16-B store
    constexpr uint32_t kBits = sizeof(OT) == 4 ? 0xff800000u : 0xff80ff80u;  // -inf (fp32 / two bf16)
    OT ninf;
    if constexpr (sizeof(OT) == 4)
        ninf = -__builtin_inff();
    else
        ninf = (OT)0xff80u;
    const int tid = threadIdx.x;
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    const v4u pat = {kBits, kBits, kBits, kBits};
    const int a = min((c0 + V - 1) & ~(V - 1), c1);  // first 16-B aligned column
    const int b = max(a, c1 & ~(V - 1));
    if (c0 + tid < a) row[c0 + tid] = ninf;
    for (int col = a + V * tid; col < b; col += V * NTH) *(v4u *)(row + col) = pat;
    if (b + tid < c1) row[b + tid] = ninf;
}

}  // namespace pml
