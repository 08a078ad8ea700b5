// Scoring core shared by the paged (decode) and ragged (prefill) logits
// kernels.
//
//   logit[r, s] = scale_k[s] * sum_h w[r,h] * max(0, <q[r,h,:], k[s,:]>)
//
// The fp8 per-token scale is positive, so it moves out of the ReLU; MXFP4
// pages carry per-32-element e8m0 scales that the scaled MFMA applies.
//
// Work split (gfx950): a workgroup of 4 waves scores a row-piece (up to kGMax
// rows of one request) against key blocks; q and w of the piece sit in LDS,
// shared by the 4 waves. Each wave takes whole key blocks on its own: the
// block's keys go from HBM straight into VGPRs, already laid out as the B
// operand of v_mfma_f32_16x16x128_f8f6f4 (lane l holds token l % 16 of a
// 16-token slice), two buffers deep so one block is in flight while one is
// scored. For every row the wave runs 4 head tiles x (BKV / 16) token
// slices of MFMAs, folds ReLU and w into per-lane partial sums in registers,
// and a transpose-reduce with v_permlane32/16_swap leaves one finished token
// per lane; the block's logits wait in LDS and go out as coalesced
// 4-byte-per-lane row segments one step later. No barrier is taken per
// block, only at piece changes.
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

// Score one staged row against the block in registers; returns twice this
// lane's sum over all 64 heads for token out_token(lane) (before the key
// scale; the factor 2 is exact and the caller folds 1/2 into the scale).
constexpr int kPipe = 2;  // MFMAs issued ahead of the epilogue that reads them

// MFMA of one 16-token slice t. fp8 x fp8 takes the unscaled opcode: the
// scaled form costs an extra VALU instruction per MFMA (it loads the scales),
// measured as about a fifth more SIMD time for MFMA plus epilogue. MXFP4 keys
// need their e8m0 block scales, with fp8 A at unit scale (`a_scale` = 127) or
// fp4 A (Q4) at its own e8m0 scale: e2m1 x e2m1 runs at twice the fp8 rate.
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

template <bool FP4, int BKV, bool Q4 = false>
__device__ __forceinline__ float score_row(const KeyRegs<FP4, BKV> &k_, const uint8_t *s_qrow,
                                           const float *s_wrow) {
    static_assert(!Q4 || FP4, "fp4 q pairs with MXFP4 keys");
    using C = BlockCfg<FP4, BKV>;
    const int lane = lane_id();
    const int grp = lane >> 4;
    float p[C::NT];
#pragma unroll
    for (int t = 0; t < C::NT; ++t) p[t] = 0.f;
    // all LDS operands of the row first: one wait instead of one per head tile
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
    }
    // MFMA k = (head tile k / NT, slice k % NT) is issued kPipe steps before
    // its epilogue, so the matrix core works while the VALU folds earlier
    // results and few wait states are padded between an MFMA and its reader.
    // The MFMA intrinsics have no side effects, so empty volatile asm
    // statements pin the order: each MFMA takes an operand (its A tile, or
    // for MXFP4 the unit A scale) that the asm before it claims to rewrite,
    // and each epilogue reads its result only after the asm that follows the
    // next MFMAs. (fp4 q: the operand is the head tile's A scale.)
    constexpr int NK = 4 * C::NT;
    v4f d[NK];
    int unit = 127;  // e8m0 1.0
#pragma unroll
    for (int k = 0; k < NK + kPipe; ++k) {
        if (k < NK) {
            if constexpr (Q4) {
                asm volatile("" : "+v"(asc[k / C::NT]));
                d[k] = mfma_slice<FP4, BKV, true>(k_, av[k / C::NT], k % C::NT, asc[k / C::NT]);
            } else {
                if constexpr (FP4)
                    asm volatile("" : "+v"(unit));
                else
                    asm volatile("" : "+v"(av[k / C::NT]));
                d[k] = mfma_slice<FP4, BKV>(k_, av[k / C::NT], k % C::NT, unit);
            }
        }
        if (k >= kPipe) {
            const int e = k - kPipe, ht = e / C::NT, t = e % C::NT;
            asm volatile("" : "+v"(d[e]));
            // d + |d| = 2 ReLU(d) is one add with an abs modifier (fmaxf would
            // canonicalise its input first); the factor 2 is taken out at the end
#pragma unroll
            for (int i = 0; i < 4; ++i) p[t] = __builtin_fmaf(wv[ht][i], d[e][i] + __builtin_fabsf(d[e][i]), p[t]);
        }
    }
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
