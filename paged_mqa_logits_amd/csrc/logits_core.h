// Tile pipeline shared by the paged (decode) and ragged (prefill) logits
// kernels: a key tile of BKV tokens is staged in LDS and scored against up to
// kGMax query rows whose q stays in VGPRs.
//
//   logit[r, s] = scale_k[s] * sum_h w[r,h] * max(0, <q[r,h,:], k[s,:]>)
//
// The fp8 per-token scale is positive, so it moves out of the ReLU; MXFP4
// tiles carry per-32-element e8m0 scales that the scaled MFMA applies.
//
// Workgroup: 4 waves; wave w owns heads [16w, 16w+16). Its q rows are the A
// operand of v_mfma_f32_16x16x128_f8f6f4 (16 heads x the whole D = 128) and the
// tile's 16-token slices are the B operand. Epilogue in registers: ReLU, x w,
// sum over the lane's 4 heads, then a transpose-reduce over the 4 lane groups
// with v_permlane32/16_swap that leaves one token per lane; the 4 waves'
// partials meet in LDS and each lane stores 4 consecutive logits (16 B).
#pragma once

#include "pml_device.h"

namespace pml {

constexpr int kStages = 4;
constexpr int kVmcnt0 = 0x0F70;  // s_waitcnt encoding: vmcnt(0), other counters untouched

template <bool FP4, int BKV>
struct TileCfg {
    static constexpr int D = PML_HEAD_DIM;
    static constexpr int TOKB = FP4 ? D / 2 : D;   // value bytes per token
    static constexpr int CPT = TOKB / 16;          // 16-B chunks per token
    static constexpr int VBYTES = BKV * TOKB;      // values region of a tile
    static constexpr int SBYTES = BKV * 4;         // fp32 scale or 4 e8m0 per token
    static constexpr int TILE = VBYTES + SBYTES;
    static constexpr int VC = VBYTES / 16;
    static constexpr int RV = (VC + kThreads - 1) / kThreads;  // DMA rounds for values
    static constexpr int VCW = VC / (kWaves * RV);            // chunks per wave per round
    static constexpr int SCW = SBYTES / 16 / kWaves;          // 16-B scale chunks per wave
    static constexpr int NLD = RV + 1;                        // DMA instructions per wave per tile
    static constexpr int NT = BKV / 16;                       // 16-token slices per tile
    static_assert(VCW >= 1 && VCW <= kWave && VC == VCW * kWaves * RV, "value DMA split");
    static_assert(SCW >= 1 && SCW * 16 * kWaves == SBYTES, "scale DMA split");
    static_assert(TILE % 16 == 0, "tile size");
    static_assert(kGMax * BKV / 4 <= 2 * kThreads, "epilogue covers a piece in two rounds");
};

// Position of 16-B chunk c of token s inside the LDS copy of a tile.
template <bool FP4>
__device__ __forceinline__ int swz(int s, int c) {
    if (FP4) return c ^ (((s >> 2) ^ (s >> 1)) & 3);
    return c ^ ((s & 7) ^ ((s >> 3) & 1));
}

// Stage one cache page (values region then scales region, contiguous) into
// LDS. Every wave issues exactly TileCfg::NLD load instructions.
template <bool FP4, int BKV>
__device__ __forceinline__ void issue_page(const uint8_t *pg, uint8_t *stage) {
    using C = TileCfg<FP4, BKV>;
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
#pragma unroll
    for (int i = 0; i < C::RV; ++i) {
        const int base = (i * kWaves + wave) * C::VCW;
        const int ch = base + lane;
        const int s = ch / C::CPT;
        const int c = swz<FP4>(s, ch % C::CPT);  // the swizzle is an involution
        if (lane < C::VCW) dma16(pg + s * C::TOKB + c * 16, stage + base * 16);
    }
    const int sbase = wave * C::SCW;
    if (lane < C::SCW) dma16(pg + C::VBYTES + (sbase + lane) * 16, stage + C::VBYTES + sbase * 16);
}

// Stage keys [t0, t0 + BKV) of a contiguous fp8 key array k[N][D] with its
// fp32 scales k_scale[N]. Tokens at or past N are read as token N - 1 (they
// are never stored), so no load leaves the arrays. Every wave issues exactly
// TileCfg::NLD load instructions (the scales go 4 bytes per lane).
template <int BKV>
__device__ __forceinline__ void issue_contig(const uint8_t *k, const float *k_scale, int N, int t0,
                                             uint8_t *stage) {
    using C = TileCfg<false, BKV>;
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
#pragma unroll
    for (int i = 0; i < C::RV; ++i) {
        const int base = (i * kWaves + wave) * C::VCW;
        const int ch = base + lane;
        const int s = ch / C::CPT;
        const int c = swz<false>(s, ch % C::CPT);
        const int tok = min(t0 + s, N - 1);
        if (lane < C::VCW) dma16(k + (int64_t)tok * C::D + c * 16, stage + base * 16);
    }
    constexpr int SPW = BKV / kWaves;  // scales per wave
    const int tok = min(t0 + wave * SPW + lane, N - 1);
    if (lane < SPW) dma4(k_scale + tok, stage + C::VBYTES + wave * SPW * 4);
}

// q (A operands) and w of row r for this lane: heads 16*wave + (lane % 16) and
// 4*(lane / 16) .. +3 within the wave's 16.
//
// Order of the 128 k-values of an operand over lane group g = lane / 16, as
// measured on gfx950 for v_mfma_scale_f32_16x16x128_f8f6f4: an fp8 operand
// holds k = 16g .. 16g+15 in its bytes 0-15 and k = 64+16g .. 64+16g+15 in
// bytes 16-31; an fp4 operand holds k = 32g .. 32g+31 in order (low nibble
// first), and the e8m0 scale of k-block g comes from lane group g. fp8 x fp8
// tiles only need A and B in the same order, so both take d = 32g .. 32g+31;
// against fp4 keys q must follow the hardware's fp8 order.
template <bool FP4>
__device__ __forceinline__ void load_row(const uint8_t *q, const float *w, int64_t r, v8i &qa, v4f &w4) {
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int tl = lane & 15;
    const int grp = lane >> 4;
    const uint8_t *qrow = q + ((size_t)r * PML_HEADS + 16 * wave + tl) * PML_HEAD_DIM;
    const v4i lo = *(const v4i *)(qrow + (FP4 ? 16 * grp : 32 * grp));
    const v4i hi = *(const v4i *)(qrow + (FP4 ? 64 + 16 * grp : 32 * grp + 16));
    qa = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    w4 = *(const v4f *)(w + (size_t)r * PML_HEADS + 16 * wave + 4 * grp);
}

// Score the staged tile against rows 0..g-1 of the piece and leave each wave's
// per-token partial sums in red[i][wave][token].
template <bool FP4, int BKV>
__device__ __forceinline__ void score_tile(const uint8_t *st, const v8i (&qa)[kGMax], const v4f (&w4)[kGMax],
                                           int g, float (*red)[kWaves][BKV]) {
    using C = TileCfg<FP4, BKV>;
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int tl = lane & 15;
    const int grp = lane >> 4;

    v8i kb[C::NT];
    int ksc[C::NT];
#pragma unroll
    for (int t = 0; t < C::NT; ++t) {
        const int s = 16 * t + tl;
        if (FP4) {
            const v4i x = lds_read_b128(lds_addr(st + s * C::TOKB + swz<FP4>(s, grp) * 16));
            kb[t] = v8i{x[0], x[1], x[2], x[3], 0, 0, 0, 0};
            ksc[t] = (int)lds_read_u8(lds_addr(st + C::VBYTES + s * 4 + grp));
        } else {
            const v4i x = lds_read_b128(lds_addr(st + s * C::TOKB + swz<FP4>(s, 2 * grp) * 16));
            const v4i y = lds_read_b128(lds_addr(st + s * C::TOKB + swz<FP4>(s, 2 * grp + 1) * 16));
            kb[t] = v8i{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
            ksc[t] = 0;
        }
    }
    wait_lgkm0();

#pragma unroll
    for (int i = 0; i < kGMax; ++i) {
        if (i < g) {
            float p[C::NT];
#pragma unroll
            for (int t = 0; t < C::NT; ++t) {
                const v4f d = FP4 ? mfma_fp8_fp4(qa[i], kb[t], ksc[t]) : mfma_fp8(qa[i], kb[t]);
                p[t] = w4[i][0] * fmaxf(d[0], 0.f) + w4[i][1] * fmaxf(d[1], 0.f) +
                       w4[i][2] * fmaxf(d[2], 0.f) + w4[i][3] * fmaxf(d[3], 0.f);
            }
            float tot;
            int tok;
            bool wr;
            if (C::NT == 4) {
                swap32(p[0], p[2 % C::NT]);
                swap32(p[1 % C::NT], p[3 % C::NT]);
                float x = p[0] + p[2 % C::NT];
                float y = p[1 % C::NT] + p[3 % C::NT];
                swap16(x, y);
                tot = x + y;
                tok = lane;
                wr = true;
            } else {
                swap32(p[0], p[1 % C::NT]);
                float x = p[0] + p[1 % C::NT];
                float y = x;
                swap16(x, y);
                tot = x + y;
                tok = (lane >> 5) * 16 + tl;
                wr = (grp & 1) == 0;
            }
            if (wr) lds_write_f32(lds_addr(&red[i][wave][tok]), tot);
        }
    }
}

// Sum the waves' partials, apply the per-token scale and the row bounds
// [lo[i], hi[i]) (-inf outside; NaN everywhere when !ok) and store columns
// [col0, col0 + BKV) of rows row0 .. row0 + g - 1, never at or past ncols.
// With skip_past_end, rows whose bound ends before col0 are not stored at all
// (their tail is filled separately).
template <bool FP4, int BKV>
__device__ __forceinline__ void store_tile(const uint8_t *st, float (*red)[kWaves][BKV], const int *s_lo,
                                           const int *s_hi, int g, int64_t row0, int col0, int ncols,
                                           bool ok, bool skip_past_end, float *out, int64_t out_ld) {
    using C = TileCfg<FP4, BKV>;
    const int tid = threadIdx.x;
    const int nvec = g * (BKV / 4);
#pragma unroll
    for (int rnd = 0; rnd < 2; ++rnd) {
        const int idx = tid + rnd * kThreads;
        if (idx < nvec) {
            const int i = idx / (BKV / 4);
            const int tok = (idx % (BKV / 4)) * 4;
            const int s = col0 + tok;
            const int lo = lds_read_i32(lds_addr(&s_lo[i]));
            const int hi = lds_read_i32(lds_addr(&s_hi[i]));
            const v4i r0v = lds_read_b128(lds_addr(&red[i][0][tok]));
            const v4i r1v = lds_read_b128(lds_addr(&red[i][1][tok]));
            const v4i r2v = lds_read_b128(lds_addr(&red[i][2][tok]));
            const v4i r3v = lds_read_b128(lds_addr(&red[i][3][tok]));
            v4i scv = {0x3f800000, 0x3f800000, 0x3f800000, 0x3f800000};
            if (!FP4) scv = lds_read_b128(lds_addr(st + C::VBYTES + tok * 4));
            wait_lgkm0();
            if (!skip_past_end || col0 < hi) {
                v4f val;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float v = ((__int_as_float(r0v[j]) + __int_as_float(r1v[j])) +
                               (__int_as_float(r2v[j]) + __int_as_float(r3v[j]))) *
                              __int_as_float(scv[j]);
                    if (!ok) v = __builtin_nanf("");
                    if (s + j < lo || s + j >= hi) v = -__builtin_inff();
                    val[j] = v;
                }
                float *dst = out + (row0 + i) * out_ld + s;
                if (s + 4 <= ncols) {
                    *(v4f *)dst = val;
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (s + j < ncols) dst[j] = val[j];
                }
            }
        }
    }
}

// Fill columns [c0, c1) of one row with -inf (the whole workgroup).
__device__ __forceinline__ void fill_neg_inf(float *row, int c0, int c1) {
    if (c0 >= c1) return;
    const int tid = threadIdx.x;
    const v4f ninf = {-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
    const int a4 = min((c0 + 3) & ~3, c1);  // first 16-B aligned column (rows are 16-B aligned)
    const int b4 = max(a4, c1 & ~3);
    if (c0 + tid < a4) row[c0 + tid] = -__builtin_inff();
    for (int col = a4 + 4 * tid; col < b4; col += 4 * kThreads) *(v4f *)(row + col) = ninf;
    if (b4 + tid < c1) row[b4 + tid] = -__builtin_inff();
}

}  // namespace pml
