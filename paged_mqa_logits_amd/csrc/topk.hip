// top_k_per_row: the k largest logits of each row among its valid columns
// [lo, hi), returned as int32 positions relative to lo in ascending order and
// padded with -1 (the indexer's top-k selector; output preset to -1 and
// request-local positions as in the CPU decode path of the sparse_attn_indexer
// page). Selection order: larger value first, equal values by lower position.
//
// One workgroup per row, radix select on an order-preserving 32-bit key (NaN
// lowest, -0 == +0) followed by an ordered compaction, so positions come out
// ascending without a sort:
//  * When every row has at most 8192 columns (max_width <= 8192) a compact
//    256-thread kernel holds the row's keys in registers and selects there
//    (topk_small_kernel: 8.7 KB of LDS and 48 VGPRs per 256-thread row).
//  * Otherwise a row that fits the LDS candidate list is read once into it.
//  * A row of 16K columns or more first takes a sampled pass: a histogram of
//    the top 11 key bits over each wave's first 512 positions (16 places
//    spread over the row) picks a bucket b with a margin (about 1.5 k of the
//    row's keys at or above it, by the sample's share). Then one streaming
//    pass, which starts from the sample's registers, appends in position
//    order every element whose top digit is >= b into its wave's region of
//    the list (each wave's span of the row is contiguous). Any key outside
//    the regions is then below every key in them, so if they hold at least k
//    keys the top k are among them: every wave lifts its region into
//    registers (forming the order keys there), and the selection and the
//    placement run on those registers, placing by ballots over 64-entry
//    chunks in (wave, entry) order, which is position order. When the sample
//    holds, the row is read once rather than three times. When the bucket
//    lies above -inf the pass walks the row in words (lane l holds positions
//    r + 64 j + l): per word index one float compare, a ballot whose popcount
//    advances the wave's count, a slot from mbcnt and one LDS store of value
//    and position (lanes that are not candidates store into a spare entry of
//    their own, so no word takes a branch).
//  * Narrower rows, and rows where the sample misjudges (fewer than k
//    candidates, or a region overflows), take the exact streaming passes: a
//    full histogram fixes b, then every wave counts, then appends, the
//    candidates.
//  * The key bits are selected among the candidates (registers or list):
//    radix digits from the highest bit where the live keys differ, until the
//    picked bin is taken whole or holds at most 64 keys (one wave then sorts
//    those). One block scan over the candidates' counts places every selected
//    element.
//  * If the candidates overflow the list (heavy ties), the selection finishes
//    with passes over the row itself.
#include "select.h"
#include "fused.h"

namespace pml {

constexpr int kBins = 2048;
constexpr int kUnroll = 4;  // float4 loads in flight per lane in the streaming passes

template <int NT>
struct TopkCfg {
    static constexpr int NW = NT / kWave;
    static constexpr int CAP = NT == 1024 ? 12288 : 8192;  // candidate list entries
    static constexpr int RCAP = CAP / NW;                   // one wave's region of the list
};
constexpr int kSmallMaxCols = 8192;  // rows up to this wide take topk_small_kernel
constexpr int kSampledMin = 16384;  // rows at least this wide take the sampled path (measured:
                                    // 32K-64K rows 47 -> 35 us; narrower rows gain nothing)

// Logit elements: fp32, or bf16 bits (E = uint16_t). A bf16 is the upper half
// of the fp32 with the same value, so the selection on bf16 logits is the
// selection on their exact fp32 values.
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
template <typename E>
__device__ __forceinline__ float elem(const E *p, int64_t i) {
    return to_f32(p[i]);
}
// The 4 elements at 4q .. 4q + 3 (16 bytes of fp32, 8 of bf16: element 4q in
// the low half of the first word).
template <typename E>
__device__ __forceinline__ v4f group4(const E *base, int64_t q) {
    if constexpr (sizeof(E) == 4) {
        return *(const v4f *)(base + 4 * q);
    } else {
        typedef uint32_t v2u32 __attribute__((ext_vector_type(2)));
        const v2u32 u = *(const v2u32 *)(base + 4 * q);
        return v4f{__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xffff0000u), __uint_as_float(u[1] << 16),
                   __uint_as_float(u[1] & 0xffff0000u)};
    }
}


// Float4 walk of one wave's share [q0, q1) of the row's 16-B groups:
// f(q, x, all_in) gets every group index q (lanes at or past q1 included: they
// must check q < q1, unless the wave-uniform all_in says the whole round lies
// below q1) with its 4 values, in position order across the wave (round, j,
// lane).
//
// Two register buffers of kUnroll groups per lane alternate: the next round's
// loads are issued before the current round is processed, so a wave always
// has a round in flight. Loads are unconditional, with addresses clamped to
// the share's last group, which keeps the compiler's wait counts exact:
// processing a round waits for that round only.
template <typename E, typename F>
__device__ __forceinline__ void wave_walk_raw(const E *rowbase, int q0, int q1, F &&f) {
    if (q0 >= q1) return;
    const int lane = lane_id();
    const int qlast = q1 - 1;
    constexpr int kStep = kWave * kUnroll;
    auto load = [&](v4f *x, int g) {
#pragma unroll
        for (int j = 0; j < kUnroll; ++j)
            x[j] = group4(rowbase, (int64_t)min(g + j * kWave + lane, qlast));
    };
    auto process = [&](const v4f *x, int g) {
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) f(g + j * kWave + lane, x[j], g + kStep <= q1);
    };
    v4f xa[kUnroll], xb[kUnroll];
    load(xa, q0);
    for (int g = q0;; g += 2 * kStep) {
        load(xb, g + kStep);
        process(xa, g);
        if (g + kStep >= q1) break;
        load(xa, g + 2 * kStep);
        process(xb, g + kStep);
        if (g + 2 * kStep >= q1) break;
    }
}

// Word walk of positions [ps, pe) of a row: in a round starting at r, lane l
// holds the kWords values at r + j * kWave + l, so for each j the wave's 64
// lanes hold consecutive positions and the (j, lane) order is position order.
// f(p - bias, x, full) gets each of them, where the wave-uniform `full` says the
// whole round lies below pe (otherwise lanes must check p < pe). Rounds alternate
// between two register buffers as in wave_walk_raw; only a round that reaches
// pe clamps its addresses, so the others load at a base plus fixed offsets.
// The caller loads the first round (load_words at ps) into xa.
constexpr int kWords = 16;
constexpr int kRound = kWave * kWords;
constexpr int kSampleWords = 8;  // of a wave's first round, the words the bucket is sampled from

// The round of words at r, for r < pe (addresses clamped to pe - 1 in a round that reaches pe).
template <typename E>
__device__ __forceinline__ void load_words(const E *rowbase, int r, int pe, float *x) {
    const int lane = lane_id();
    if (r + kRound <= pe) {
        const E *src = rowbase + r + lane;
#pragma unroll
        for (int j = 0; j < kWords; ++j) x[j] = elem(src, j * kWave);
    } else {
#pragma unroll
        for (int j = 0; j < kWords; ++j) x[j] = elem(rowbase, min(r + j * kWave + lane, pe - 1));
    }
}

template <typename E, typename F>
__device__ __forceinline__ void wave_walk_words(const E *rowbase, int ps, int pe, int bias, float *xa, F &&f) {
    if (ps >= pe) return;
    const int lane = lane_id();
    auto load = [&](float *x, int r) { load_words(rowbase, r, pe, x); };
    auto process = [&](const float *x, int r) {
        const int rb = r + lane - bias;
        if (r + kRound <= pe) {  // two copies, so f sees `full` as a constant
#pragma unroll
            for (int j = 0; j < kWords; ++j) f(rb + j * kWave, x[j], true);
        } else {
#pragma unroll
            for (int j = 0; j < kWords; ++j) f(rb + j * kWave, x[j], false);
        }
    };
    float xb[kWords];
    for (int r = ps;; r += 2 * kRound) {
        load(xb, r + kRound);
        process(xa, r);
        if (r + kRound >= pe) break;
        load(xa, r + 2 * kRound);
        process(xb, r + kRound);
        if (r + 2 * kRound >= pe) break;
    }
}

// The same walk with order keys and validity: f(p, key, valid) for the 4
// elements at positions p .. p + 3.
template <typename E, typename F>
__device__ __forceinline__ void wave_walk(const E *rowbase, int lo, int hi, int q0, int q1, F &&f) {
    wave_walk_raw(rowbase, q0, q1, [&](int q, const v4f &x, bool) {
        uint32_t key[4];
        bool ok[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int p = 4 * q + e;
            ok[e] = q < q1 && p >= lo && p < hi;
            key[e] = order_key(x[e]);
        }
        f(4 * q, key, ok);
    });
}

// Float whose order key is `prefix`, for prefix >= 0x00800000 (above the key of
// -inf): for every non-NaN f, order_key(f) >= prefix exactly when f >= it
// (-0 and +0 compare equal both ways; NaN fails both tests).
__device__ __forceinline__ float key_floor_float(uint32_t prefix) {
    return (prefix & 0x80000000u) ? __uint_as_float(prefix & 0x7fffffffu) : __uint_as_float(~prefix);
}

template <int NT, typename E>
__global__ __launch_bounds__(NT) void topk_kernel(TopkArgs a) {
    using Cfg = TopkCfg<NT>;
    constexpr int NW = Cfg::NW;
    constexpr int CAP = Cfg::CAP;
    __shared__ __attribute__((aligned(16))) uint32_t s_hist[kBins];
    // keys, then positions: one array, so an entry's two stores share an
    // address; entries CAP + lane take the sampled append's non-candidates
    __shared__ uint32_t s_list[2 * (CAP + kWave)];
    uint32_t *const s_key = s_list;
    int32_t *const s_pos = (int32_t *)(s_list + CAP + kWave);
    __shared__ __attribute__((aligned(16))) uint32_t s_wave[2 * NW];  // (block_max2 uses two words per wave)
    __shared__ uint32_t s_wcnt[NW];
    __shared__ uint32_t s_pick[2];
    __shared__ uint32_t s_small[kWave];  // the keys of a small picked bin
    __shared__ uint32_t s_nsmall;

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform, and known to be
    const int r = blockIdx.x;
    if (a.skip && a.skip[r]) return;
    int lo = a.ks ? a.ks[r] : 0;
    int hi;
    if (a.ks || a.next_n == 1)
        hi = a.ke[r];
    else
        hi = a.ke[r / a.next_n] - a.next_n + (r % a.next_n) + 1;
    const int64_t ldc = a.ld < 0x7fffffff ? a.ld : 0x7fffffff;
    lo = (int)min<int64_t>(max(lo, 0), ldc);
    hi = (int)min<int64_t>(max(hi, lo), ldc);
    hi = (int)min<int64_t>(hi, (int64_t)lo + a.max_width);
    const int n = hi - lo;
    const int k = a.k;
    int32_t *out = a.out + (int64_t)r * a.out_ld;
    const E *rowbase = (const E *)a.logits + (int64_t)r * a.ld;  // 16-B aligned

    if (n <= k) {
        for (int j = tid; j < k; j += NT) out[j] = j < n ? j : -1;
        return;
    }

    uint32_t prefix = 0, mask = 0, kk = (uint32_t)k;
    int first_pass = 0;  // radix digits already fixed: 0, or 1 after the streaming histogram
    int m = 0;           // entries in the candidate list (position order, positions relative to lo)
    bool in_list = true;
    bool ranged = false;  // the list's key range (max of key and of ~key) is known from the pack
    uint32_t rkmax = 0, rnkmin = 0;
    // After a sampled pass that holds, every wave keeps its region of the list
    // in registers (entry lane + 64 u in rk[u] / rp[u]) and the selection runs
    // there: no pack, and the placement by ballots over 64-entry chunks.
    constexpr int kRegs = Cfg::RCAP / kWave;
    uint32_t rk[kRegs];
    int32_t rp[kRegs];
    uint32_t rcnt = 0;  // entries of this wave's region (wave-uniform)
    bool regs = false;

    // this wave's share of the 16-B groups covering [lo, hi)
    const int gq0 = lo >> 2, gq1 = (hi + 3) >> 2;
    const int span = (gq1 - gq0 + NW - 1) / NW;
    const int wq0 = min(gq0 + wave * span, gq1), wq1 = min(wq0 + span, gq1);

    if (n <= CAP) {
        for (int i = tid; i < n; i += NT) {
            s_key[i] = order_key(elem(rowbase, lo + i));
            s_pos[i] = i;
        }
        m = n;
        __syncthreads();
    } else {
        constexpr int RCAP = Cfg::RCAP;
        bool exact = true;
        // (the word walk's positions stay below 2^31 when hi leaves two rounds of room)
        if (n >= kSampledMin && hi <= 0x7fffffff - 2 * kRound) {
        // sampled pass: the sample is the first half of each wave's first round
        // of the walk (up to 512 positions at the start of its span, 16 places
        // spread over the row). The round is loaded once: its top-digit
        // histogram picks the bucket, then the append starts from the same
        // registers.
        const int ps = max(4 * wq0, lo), pe = min(4 * wq1, hi);
        float x0[kWords];
        if (ps < pe) load_words(rowbase, ps, pe, x0);
        for (int b = tid; b < kBins; b += NT) s_hist[b] = 0;
        if (tid == 0) s_pick[0] = 0;  // bucket 0 (the whole row) if the sample runs short
        if (lane == 0) s_wcnt[wave] = (uint32_t)max(0, min(kSampleWords * kWave, pe - ps));
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kSampleWords; ++j)
            if (ps + j * kWave + lane < pe) atomicAdd(&s_hist[order_key(x0[j]) >> 21], 1u);
        uint32_t ns = 0;
        for (int w = 0; w < NW; ++w) ns += s_wcnt[w];
        __syncthreads();
        // the bucket of the t-th largest sampled key: 1.5 k scaled to the sample, + 16
        const uint32_t t = (uint32_t)((3ull * (uint64_t)k * ns) / (2ull * (uint64_t)n)) + 16;
        pick_bin_vec<NT, kBins / NT>(s_hist, t, s_wave, s_pick);
        const uint32_t sprefix = s_pick[0] << 21;
        // one pass: ordered append into the wave's region [wave * RCAP, +RCAP).
        // Above the key of -inf the bucket test is one float compare per
        // element; keys are formed only for the (few) candidates.
        uint32_t cnt = 0;
        const bool raw = sprefix >= 0x00800000u;  // the list holds float bits until the pack
        if (raw) {
            // Word walk over the wave's positions: for each word index the
            // ballot of the candidates gives every candidate its slot (the
            // count before it). Every lane stores, without a branch: a
            // non-candidate into a spare entry of its own (CAP + lane). A slot
            // past the region is clamped to its last entry: the count then
            // exceeds the region and the list is not used. Order keys are
            // formed when the regions are lifted into registers.
            const float tf = key_floor_float(sprefix);
            const uint32_t rbase = (uint32_t)wave * RCAP, rlast = rbase + RCAP - 1;
            wave_walk_words(rowbase, ps, pe, lo, x0, [&](int pl, float x, bool full) {
                const bool c = x >= tf && (full || pl < pe - lo);
                const uint64_t bm = __builtin_amdgcn_ballot_w64(c);
                const uint32_t at = __builtin_amdgcn_mbcnt_hi(
                    (uint32_t)(bm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bm, rbase + cnt));
                const uint32_t slot = c ? min(at, rlast) : (uint32_t)(CAP + lane);
                s_key[slot] = __float_as_uint(x);
                s_pos[slot] = pl;
                cnt = __builtin_amdgcn_readfirstlane(cnt + (uint32_t)__builtin_popcountll(bm));
            });
        } else {
            wave_walk(rowbase, lo, hi, wq0, wq1, [&](int p0, const uint32_t *key, const bool *ok) {
                uint32_t c = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) c += (ok[e] && key[e] >= sprefix) ? 1u : 0u;
                uint32_t pre, tot;
                wave_prefix4(c, pre, tot);
                uint32_t at = cnt + pre;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (ok[e] && key[e] >= sprefix) {
                        if (at < (uint32_t)RCAP) {
                            s_key[wave * RCAP + at] = key[e];
                            s_pos[wave * RCAP + at] = p0 + e - lo;
                        }
                        ++at;
                    }
                cnt += tot;
            });
        }
        if (lane == 0) s_wcnt[wave] = cnt;
        __syncthreads();
        uint32_t total = 0, over = 0;
        for (int w = 0; w < NW; ++w) {
            const uint32_t c = s_wcnt[w];
            total += c;
            over |= c > (uint32_t)RCAP;
        }
        if (!over && total >= (uint32_t)k) {
            // every wave lifts its region into registers (order keys formed here)
            uint32_t lmax = 0, lnmin = 0;
#pragma unroll
            for (int u = 0; u < kRegs; ++u) {
                const uint32_t i = lane + u * kWave;
                rk[u] = 0;
                rp[u] = 0;
                if (i < cnt) {
                    rk[u] = s_key[wave * RCAP + i];
                    if (raw) rk[u] = order_key(__uint_as_float(rk[u]));
                    rp[u] = s_pos[wave * RCAP + i];
                    lmax = max(lmax, rk[u]);
                    lnmin = max(lnmin, ~rk[u]);
                }
            }
            // the candidates' key range (read after the next barrier)
            lmax = wave_max_to_last(lmax);
            lnmin = wave_max_to_last(lnmin);
            if (lane == kWave - 1) {
                s_wave[wave] = lmax;
                s_wave[NW + wave] = lnmin;
            }
            rcnt = __builtin_amdgcn_readfirstlane(cnt);
            m = (int)total;  // all three digits are selected among the candidates
            ranged = true;
            regs = true;
        }
        __syncthreads();
        if (ranged) {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                rkmax = max(rkmax, s_wave[w]);
                rnkmin = max(rnkmin, s_wave[NW + w]);
            }
        }
        exact = over || total < (uint32_t)k;
        }  // sampled path
        if (exact) {
        // exact passes. pass 1: histogram of the top 11 bits
        for (int b = tid; b < kBins; b += NT) s_hist[b] = 0;
        __syncthreads();
        wave_walk(rowbase, lo, hi, wq0, wq1, [&](int, const uint32_t *key, const bool *ok) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (ok[e]) atomicAdd(&s_hist[key[e] >> 21], 1u);
        });
        __syncthreads();
        pick_bin_vec<NT, kBins / NT>(s_hist, kk, s_wave, s_pick);
        prefix = s_pick[0] << 21;
        mask = 0x7ffu << 21;
        kk -= s_pick[1];
        first_pass = 1;
        // pass 2: per-wave count of candidates (top digit >= the picked bin)
        uint32_t cnt = 0;
        wave_walk(rowbase, lo, hi, wq0, wq1, [&](int, const uint32_t *key, const bool *ok) {
            uint32_t c = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) c += (ok[e] && key[e] >= prefix) ? 1u : 0u;
            uint32_t pre, tot;
            wave_prefix4(c, pre, tot);
            cnt += tot;
        });
        if (lane == 0) s_wcnt[wave] = cnt;
        __syncthreads();
        uint32_t off = 0, total = 0;
        for (int w = 0; w < NW; ++w) {
            const uint32_t c = s_wcnt[w];
            if (w < wave) off += c;
            total += c;
        }
        if (total <= (uint32_t)CAP) {
            // pass 3: ordered append of the candidates
            wave_walk(rowbase, lo, hi, wq0, wq1, [&](int p0, const uint32_t *key, const bool *ok) {
                uint32_t c = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) c += (ok[e] && key[e] >= prefix) ? 1u : 0u;
                uint32_t pre, tot;
                wave_prefix4(c, pre, tot);
                uint32_t at = off + pre;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (ok[e] && key[e] >= prefix) {
                        s_key[at] = key[e];
                        s_pos[at] = p0 + e - lo;
                        ++at;
                    }
                off += tot;
            });
            m = (int)total;
        } else {
            in_list = false;
        }
        __syncthreads();
        }  // exact passes
    }

    if (regs) {
        // Radix digits over the registers, from the highest bit where the
        // candidates differ, until the picked bin is taken whole or holds at
        // most 64 keys (one wave sorts those); then the placement.
        const int nu = (int)((rcnt + kWave - 1) / kWave);  // register rows holding entries (uniform)
        auto rows_ = [nu]() {  // an opaque copy per loop: scalar tests, no lane masks kept alive
            int v = __builtin_amdgcn_readfirstlane(nu);
            asm volatile("" : "+s"(v));
            return v;
        };
        const uint32_t diff = rkmax ^ ~rnkmin;
        if (diff == 0) {
            prefix = rkmax;  // every candidate equal
            mask = 0xffffffffu;
        } else {
            int top = 31 - __builtin_clz(diff);
            mask = top == 31 ? 0u : ~((2u << top) - 1u);
            prefix = rkmax & mask;
#pragma unroll 1
            for (;;) {
                const int shift = max(top - 10, 0);
                const int nbins = 1 << (top - shift + 1);
                for (int b = tid; b < nbins; b += NT) s_hist[b] = 0;
                __syncthreads();
                const int nh = rows_();
#pragma unroll
                for (int u = 0; u < kRegs; ++u)
                    if (u < nh && lane + u * kWave < rcnt && (rk[u] & mask) == prefix)
                        atomicAdd(&s_hist[(rk[u] >> shift) & (nbins - 1)], 1u);
                __syncthreads();
                if (nbins == kBins)
                    pick_bin_vec<NT, kBins / NT>(s_hist, kk, s_wave, s_pick);
                else
                    pick_bin<NT>(s_hist, nbins, kk, s_wave, s_pick);
                const uint32_t cnt = s_hist[s_pick[0]];
                prefix |= s_pick[0] << shift;
                mask |= (uint32_t)(nbins - 1) << shift;
                kk -= s_pick[1];
                if (tid == 0) s_nsmall = 0;
                __syncthreads();
                if (cnt == kk || shift == 0) break;
                if (cnt <= (uint32_t)kWave) {
                    const int ng = rows_();
#pragma unroll
                    for (int u = 0; u < kRegs; ++u)
                        if (u < ng && lane + u * kWave < rcnt && (rk[u] & mask) == prefix)
                            s_small[atomicAdd(&s_nsmall, 1u)] = rk[u];
                    __syncthreads();
                    if (wave == 0) {
                        uint32_t v = (uint32_t)lane < cnt ? s_small[lane] : 0u;  // 0: below every key
#pragma unroll
                        for (int size = 2; size <= kWave; size <<= 1) {
#pragma unroll
                            for (int j = size >> 1; j > 0; j >>= 1) {
                                const uint32_t o = (uint32_t)lane_xor((int32_t)v, j);
                                const bool keep_max = ((lane & size) == 0) == ((lane & j) == 0);
                                v = keep_max ? max(v, o) : min(v, o);
                            }
                        }
                        const uint32_t t = (uint32_t)__builtin_amdgcn_readlane((int)v, (int)kk - 1);
                        const uint32_t above = (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(v > t));
                        if (lane == 0) {
                            s_pick[0] = t;
                            s_pick[1] = kk - above;
                        }
                    }
                    __syncthreads();
                    prefix = s_pick[0];
                    mask = 0xffffffffu;
                    kk = s_pick[1];
                    break;
                }
                top = shift - 1;
            }
        }
        // placement: chunk (wave, u) holds entries lane + 64 u of the wave's
        // region; chunks in (wave, u) order are in position order. Per chunk
        // the ballots of greater and equal keys give its counts, one block scan
        // gives each chunk its first slots, and mbcnt each lane's.
        const uint32_t T = prefix, need = kk;
        uint32_t *const s_base = s_hist;  // NW * kRegs packed (greater | equal << 16) counts
        uint32_t mine = 0;
        const int nc = rows_();
#pragma unroll
        for (int u = 0; u < kRegs; ++u) {
            if (u >= nc) continue;
            const bool v = lane + u * kWave < rcnt;
            const uint32_t key = rk[u] & mask;
            const uint32_t g = (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(v && key > T));
            const uint32_t e = (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(v && key == T));
            mine = lane == u ? (g | (e << 16)) : mine;
        }
        if (lane < kRegs) s_base[wave * kRegs + lane] = mine;
        __syncthreads();
        const uint32_t cv = tid < NW * kRegs ? s_base[tid] : 0u;
        uint32_t tot;
        const uint32_t excl = block_scan<NT>(cv, s_wave, &tot) - cv;
        if (tid < NW * kRegs) s_base[tid] = excl;
        __syncthreads();
        uint32_t T2 = __builtin_amdgcn_readfirstlane(T);
        asm volatile("" : "+s"(T2));  // the compares again, rather than 24 lane masks kept in SGPRs
        const int np = rows_();
#pragma unroll
        for (int u = 0; u < kRegs; ++u) {
            if (u >= np) continue;
            const uint32_t base = s_base[wave * kRegs + u];
            const bool v = lane + u * kWave < rcnt;
            const uint32_t key = rk[u] & mask;
            const bool gt = v && key > T2, eq = v && key == T2;
            const uint64_t gm = __builtin_amdgcn_ballot_w64(gt), em = __builtin_amdgcn_ballot_w64(eq);
            const uint32_t gb = (base & 0xffffu) +
                                __builtin_amdgcn_mbcnt_hi((uint32_t)(gm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)gm, 0u));
            const uint32_t eb = (base >> 16) +
                                __builtin_amdgcn_mbcnt_hi((uint32_t)(em >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)em, 0u));
            if (gt)
                out[gb + min(eb, need)] = rp[u];
            else if (eq && eb < need)
                out[gb + eb] = rp[u];
        }
        return;
    }

    // remaining radix digits. In the list, the live keys (those in the bin
    // picked so far) cluster: the digits start at the highest bit where they
    // differ, and the search stops once the picked bin is taken whole (then T
    // is a bin under mask, and keys compare under the mask). Over the row
    // (list overflow) the digits are 11, 11, 10 bits from the top.
    if (in_list) {
        uint32_t kmax = rkmax, nkmin = rnkmin;
        if (!ranged) {
            for (int i = tid; i < m; i += NT) {
                const uint32_t key = s_key[i];
                if ((key & mask) == prefix) {
                    kmax = max(kmax, key);
                    nkmin = max(nkmin, ~key);
                }
            }
            block_max2<NT>(kmax, nkmin, s_wave);
        }
        const uint32_t diff = kmax ^ ~nkmin;
        if (diff == 0) {
            prefix = kmax;  // every live key equal
            mask = 0xffffffffu;
        } else {
            int top = 31 - __builtin_clz(diff);
            mask = top == 31 ? 0u : ~((2u << top) - 1u);
            prefix = kmax & mask;
#pragma unroll 1
            for (;;) {
                const int shift = max(top - 10, 0);
                const int nbins = 1 << (top - shift + 1);
                for (int b = tid; b < nbins; b += NT) s_hist[b] = 0;
                __syncthreads();
                for (int i = tid; i < m; i += NT) {
                    const uint32_t key = s_key[i];
                    if ((key & mask) == prefix) atomicAdd(&s_hist[(key >> shift) & (nbins - 1)], 1u);
                }
                __syncthreads();
                if (nbins == kBins)
                    pick_bin_vec<NT, kBins / NT>(s_hist, kk, s_wave, s_pick);
                else
                    pick_bin<NT>(s_hist, nbins, kk, s_wave, s_pick);
                const uint32_t cnt = s_hist[s_pick[0]];
                prefix |= s_pick[0] << shift;
                mask |= (uint32_t)(nbins - 1) << shift;
                kk -= s_pick[1];
                if (tid == 0) s_nsmall = 0;
                __syncthreads();
                if (cnt == kk || shift == 0) break;
                if (cnt <= (uint32_t)kWave) {
                    // A bin of at most 64 keys: gather them and let one wave sort
                    // them (descending, bitonic) instead of more radix passes.
                    for (int i = tid; i < m; i += NT) {
                        const uint32_t key = s_key[i];
                        if ((key & mask) == prefix) s_small[atomicAdd(&s_nsmall, 1u)] = key;
                    }
                    __syncthreads();
                    if (wave == 0) {
                        uint32_t v = (uint32_t)lane < cnt ? s_small[lane] : 0u;  // 0: below every key
#pragma unroll
                        for (int size = 2; size <= kWave; size <<= 1) {
#pragma unroll
                            for (int j = size >> 1; j > 0; j >>= 1) {
                                const uint32_t o = (uint32_t)lane_xor((int32_t)v, j);
                                const bool keep_max = ((lane & size) == 0) == ((lane & j) == 0);
                                v = keep_max ? max(v, o) : min(v, o);
                            }
                        }
                        const uint32_t t = (uint32_t)__builtin_amdgcn_readlane((int)v, (int)kk - 1);
                        const uint32_t above = (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(v > t));
                        if (lane == 0) {
                            s_pick[0] = t;
                            s_pick[1] = kk - above;
                        }
                    }
                    __syncthreads();
                    prefix = s_pick[0];
                    mask = 0xffffffffu;
                    kk = s_pick[1];
                    break;
                }
                top = shift - 1;
            }
        }
    } else {
#pragma unroll 1
        for (int pass = first_pass; pass < 3; ++pass) {
            const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
            const int nbins = pass == 2 ? 1024 : 2048;
            for (int b = tid; b < kBins; b += NT) s_hist[b] = 0;
            __syncthreads();
            for (int i = lo + tid; i < hi; i += NT) {
                const uint32_t key = order_key(elem(rowbase, i));
                if ((key & mask) == prefix) atomicAdd(&s_hist[(key >> shift) & (nbins - 1)], 1u);
            }
            __syncthreads();
            if (nbins == kBins)
                    pick_bin_vec<NT, kBins / NT>(s_hist, kk, s_wave, s_pick);
                else
                    pick_bin<NT>(s_hist, nbins, kk, s_wave, s_pick);
            prefix |= s_pick[0] << shift;
            mask |= (uint32_t)(nbins - 1) << shift;
            kk -= s_pick[1];
            __syncthreads();
        }
    }
    const uint32_t T = prefix;  // the k-th key's bin under mask
    const uint32_t need = kk;   // keys in that bin that are taken (>= 1)
    const uint32_t n_gt = (uint32_t)k - need;

    // ordered compaction: slot = (# greater before) + min(# equal before, need)
    if (in_list) {
        const int per = (m + NT - 1) / NT;
        const int i0 = min(tid * per, m), i1 = min(i0 + per, m);
        uint32_t gt = 0, eq = 0;
        for (int i = i0; i < i1; ++i) {
            const uint32_t key = s_key[i] & mask;
            gt += key > T;
            eq += key == T;
        }
        uint32_t tot;
        const uint32_t packed = gt | (eq << 16);
        const uint32_t excl = block_scan<NT>(packed, s_wave, &tot) - packed;
        uint32_t gb = excl & 0xffffu, eb = excl >> 16;
        for (int i = i0; i < i1; ++i) {
            const uint32_t key = s_key[i] & mask;
            if (key > T) {
                out[gb + min(eb, need)] = s_pos[i];
                ++gb;
            } else if (key == T) {
                if (eb < need) out[gb + eb] = s_pos[i];
                ++eb;
            }
        }
    } else {
        uint32_t carry_gt = 0, carry_eq = 0;
#pragma unroll 1
        for (int base = 0; base < n; base += NT) {
            const int i = base + tid;
            uint32_t key = 0;
            const bool valid = i < n;
            if (valid) key = order_key(elem(rowbase, lo + i));
            const uint32_t gt = valid && key > T;
            const uint32_t eq = valid && key == T;
            uint32_t tot;
            const uint32_t packed = gt | (eq << 16);
            const uint32_t excl = block_scan<NT>(packed, s_wave, &tot) - packed;
            const uint32_t gt_before = carry_gt + (excl & 0xffffu);
            const uint32_t eq_before = carry_eq + (excl >> 16);
            if (gt || (eq && eq_before < need)) out[gt_before + min(eq_before, need)] = i;
            carry_gt += tot & 0xffffu;
            carry_eq += tot >> 16;
            if (carry_gt >= n_gt && carry_eq >= need) break;  // all k placed (uniform)
        }
    }
}

// order_key(f) + 1 (see select.h): -0 as +0, a NaN 1, every number at least
// 0x00800000 (the key of -inf plus one).
__device__ __forceinline__ uint32_t held_key(float f) {
    uint32_t u = __float_as_uint(f);
    u = u == 0x80000000u ? 0u : u;
    const uint32_t t = (uint32_t)((int32_t)u >> 31) | 0x80000000u;  // negative: all bits; else the sign
    return __builtin_isnan(f) ? 1u : (u ^ t) + 1u;
}

// Rows of at most 8192 columns (max_width <= 8192): each thread holds the keys
// of positions j * NT + tid (j < 32) in registers, loaded together, so the
// row costs one memory round trip. The kernel is bound by VALU issue (several
// rows share a CU), so the per-key work is kept small:
//  * A held key is the order key plus one, and 0 for a slot past the row's
//    end (the order key of -inf is 0x007fffff, so 1, a NaN, and 0 sit below
//    every number). Validity is then decided once, when the key is formed.
//  * Every pass histograms bins of 32-bit counters (8 KB of LDS). Empty slots
//    land in bin 0 of a pass whose fixed bits are all zero, and their count
//    is taken back out of that bin before it is searched.
//  * When the picked bin is taken whole (the usual end), the selected keys
//    are exactly those at or above its lower bound: one compare per key, whose
//    ballot gives both the 64-position chunk's count and each lane's slot.
//    Ties at the k-th key (a bin of equal keys only partly taken) take two
//    ballots per chunk, greater and equal, as before.
// Chunk (j, w) covers positions j * NT + 64 w + [0, 64); one block scan over
// the chunks' counts gives each chunk its first output slot, so selected
// positions go to consecutive slots in ascending order.
template <int NT, typename E>
__global__ __launch_bounds__(NT) void topk_small_kernel(TopkArgs a) {
    constexpr int NW = NT / kWave;
    constexpr int kMaxCols = kSmallMaxCols;
    constexpr int kPer = kMaxCols / NT;  // keys per thread
    constexpr int kChunks = kPer * NW;   // 64-position chunks of a full row
    static_assert(kChunks <= NT, "one chunk count per thread in the scan");
    static_assert(kPer <= kWave, "one chunk count per lane of a wave");
    __shared__ __attribute__((aligned(16))) uint32_t s_hist[kBins];
    __shared__ uint32_t s_base[kChunks];  // first output slot of each chunk (packed greater | equal << 16 on ties)
    __shared__ __attribute__((aligned(16))) uint32_t s_wave[NW];
    __shared__ uint32_t s_pick[2];
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int r = blockIdx.x;
    if (a.skip && a.skip[r]) return;
    int lo = a.ks ? a.ks[r] : 0;
    int hi;
    if (a.ks || a.next_n == 1)
        hi = a.ke[r];
    else
        hi = a.ke[r / a.next_n] - a.next_n + (r % a.next_n) + 1;
    const int64_t ldc = a.ld < 0x7fffffff ? a.ld : 0x7fffffff;
    lo = (int)min<int64_t>(max(lo, 0), ldc);
    hi = (int)min<int64_t>(max(hi, lo), ldc);
    hi = (int)min<int64_t>(hi, (int64_t)lo + min(a.max_width, kMaxCols));
    const int n = hi - lo;
    const int k = a.k;
    int32_t *out = a.out + (int64_t)r * a.out_ld;
    if (n <= k) {
        for (int j = tid; j < k; j += NT) out[j] = j < n ? j : -1;
        return;
    }
    const E *row = (const E *)a.logits + (int64_t)r * a.ld + lo;
    const int nj = (n + NT - 1) / NT;        // rounds j holding positions (uniform)
    // a fresh opaque copy of nj for each loop: the per-round tests are then
    // scalar compares in every loop, not 32 lane masks kept alive in SGPRs
    auto rounds = [nj]() {
        int v = nj;
        asm volatile("" : "+s"(v));
        return v;
    };
    const uint32_t empty = (uint32_t)(nj * NT - n);  // slots of those rounds past the row's end
    uint32_t key[kPer];
    {
        float x[kPer];
        const int nj0 = rounds();
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            if (j < nj0) x[j] = elem(row, min(j * NT + tid, n - 1));
        for (int b = tid; b < kBins; b += NT) s_hist[b] = 0;
        __syncthreads();
        const int nj1 = rounds();
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            key[j] = 0;
            if (j < nj1) {
                key[j] = tid < n - j * NT ? held_key(x[j]) : 0u;
                atomicAdd(&s_hist[key[j] >> 21], 1u);
            }
        }
        if (tid == 0 && empty) atomicSub(&s_hist[0], empty);
    }
    __syncthreads();
    uint32_t prefix = 0, mask = 0, kk = (uint32_t)k, cnt = 0;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const int nbins = pass == 2 ? 1024 : 2048;
        if (pass > 0) {
            for (int b = tid; b < nbins; b += NT) s_hist[b] = 0;
            __syncthreads();
            const int njp = rounds();
#pragma unroll
            for (int j = 0; j < kPer; ++j)
                if (j < njp && (key[j] & mask) == prefix) atomicAdd(&s_hist[(key[j] >> shift) & (nbins - 1)], 1u);
            if (tid == 0 && prefix == 0 && empty) atomicSub(&s_hist[0], empty);
            __syncthreads();
        }
        if (pass < 2)
            pick_bin_vec<NT, kBins / NT>(s_hist, kk, s_wave, s_pick);
        else
            pick_bin_vec<NT, kBins / 2 / NT>(s_hist, kk, s_wave, s_pick);
        cnt = s_hist[s_pick[0]];
        prefix |= s_pick[0] << shift;
        mask |= (uint32_t)(nbins - 1) << shift;
        kk -= s_pick[1];
        __syncthreads();
        if (cnt == kk) break;  // the picked bin is taken whole
    }
    const int nch = nj * NW;  // chunks holding positions
    if (cnt == kk) {
        // selected: key >= the picked bin's lower bound (at least 1: empty slots never)
        const uint32_t T = max(prefix, 1u);
        uint32_t mine = 0;  // lane j: this wave's count in round j
        int njl = rounds();
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            if (j >= njl) continue;
            const uint32_t c = (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(key[j] >= T));
            mine = lane == j ? c : mine;
        }
        if (lane < nj) s_base[lane * NW + wave] = mine;
        __syncthreads();
        const uint32_t v = tid < nch ? s_base[tid] : 0u;
        uint32_t tot;
        const uint32_t excl = block_scan<NT>(v, s_wave, &tot) - v;
        if (tid < nch) s_base[tid] = excl;
        __syncthreads();
        // recompute the compares rather than keep 32 lane masks in SGPRs across the scan
        uint32_t T2 = T;
        asm volatile("" : "+s"(T2));
        njl = rounds();
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            if (j >= njl) continue;
            const uint32_t base = s_base[j * NW + wave];
            const bool sel = key[j] >= T2;
            const uint64_t m = __builtin_amdgcn_ballot_w64(sel);
            const uint32_t slot =
                base + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            if (sel && slot < (uint32_t)k) out[slot] = j * NT + tid;  // (the counts give slot < k)
        }
        return;
    }
    // ties: every bit is fixed (mask is all ones), T >= 1, and `need` of the
    // keys equal to T are taken, in position order
    const uint32_t T = prefix;
    const uint32_t need = kk;
    uint32_t mine = 0;
    int njl = rounds();
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        if (j >= njl) continue;
        const uint32_t g = (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(key[j] > T));
        const uint32_t e = (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(key[j] == T));
        mine = lane == j ? (g | (e << 16)) : mine;
    }
    if (lane < nj) s_base[lane * NW + wave] = mine;
    __syncthreads();
    const uint32_t v = tid < nch ? s_base[tid] : 0u;
    uint32_t tot;
    const uint32_t excl = block_scan<NT>(v, s_wave, &tot) - v;
    if (tid < nch) s_base[tid] = excl;
    __syncthreads();
    uint32_t T2 = T;
    asm volatile("" : "+s"(T2));
    njl = rounds();
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        if (j >= njl) continue;
        const uint32_t base = s_base[j * NW + wave];
        const bool gt = key[j] > T2, eq = key[j] == T2;
        const uint64_t gm = __builtin_amdgcn_ballot_w64(gt), em = __builtin_amdgcn_ballot_w64(eq);
        const uint32_t gb = (base & 0xffffu) +
                            __builtin_amdgcn_mbcnt_hi((uint32_t)(gm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)gm, 0u));
        const uint32_t eb = (base >> 16) +
                            __builtin_amdgcn_mbcnt_hi((uint32_t)(em >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)em, 0u));
        if (gt)
            out[gb + min(eb, need)] = j * NT + tid;
        else if (eq && eb < need)
            out[gb + eb] = j * NT + tid;
    }
}

// Launch the top-k over num_rows rows (arguments validated by the caller).
template <typename E>
static void launch_topk_as(const TopkArgs &a, int num_rows, hipStream_t st) {
    if (a.max_width <= kSmallMaxCols)
        hipLaunchKernelGGL((topk_small_kernel<256, E>), dim3(num_rows), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((topk_kernel<1024, E>), dim3(num_rows), dim3(1024), 0, st, a);
}

int launch_topk(const TopkArgs &a, int num_rows, hipStream_t st) {
    if (a.bf16)
        launch_topk_as<uint16_t>(a, num_rows, st);
    else
        launch_topk_as<float>(a, num_rows, st);
    return hipGetLastError() == hipSuccess ? PML_OK : PML_ERR_HIP;
}

}  // namespace pml

extern "C" size_t top_k_per_row_workspace_size(int num_rows, int max_width, int k) {
    (void)num_rows;
    (void)max_width;
    (void)k;
    return 0;
}

static int top_k_rows(const void *logits, bool bf16, int num_rows, int64_t logits_ld, const int32_t *ks,
                      const int32_t *ke, int next_n, int k, int max_width, int32_t *out, int64_t out_ld,
                      void *stream) {
    if (num_rows < 0 || next_n < 1 || max_width < 0 || logits_ld < 0) return PML_ERR_SHAPE;
    if (k < 1 || k > PML_MAX_TOPK) return PML_ERR_K;
    if (ks && next_n != 1) return PML_ERR_UNSUPPORTED;
    if (!ks && next_n > 1 && num_rows % next_n != 0) return PML_ERR_SHAPE;
    if (num_rows == 0) return PML_OK;
    if (!logits || !ke || !out) return PML_ERR_NULL;
    if (out_ld < k) return PML_ERR_STRIDE;
    if (((uintptr_t)logits & 15) != 0) return PML_ERR_ALIGN;
    if (logits_ld % (bf16 ? 8 : 4) != 0) return PML_ERR_STRIDE;  // 16-byte rows
    pml::TopkArgs a{logits, logits_ld, ks, ke, next_n, k, max_width, out, out_ld, nullptr, bf16 ? 1 : 0};
    return pml::launch_topk(a, num_rows, (hipStream_t)stream);
}

extern "C" int top_k_per_row(const float *logits, int num_rows, int64_t logits_ld, const int32_t *ks,
                             const int32_t *ke, int next_n, int k, int max_width, int32_t *out,
                             int64_t out_ld, void *workspace, size_t workspace_bytes, void *stream) {
    (void)workspace;
    (void)workspace_bytes;
    return top_k_rows(logits, false, num_rows, logits_ld, ks, ke, next_n, k, max_width, out, out_ld, stream);
}

extern "C" int top_k_per_row_bf16(const uint16_t *logits, int num_rows, int64_t logits_ld, const int32_t *ks,
                                  const int32_t *ke, int next_n, int k, int max_width, int32_t *out,
                                  int64_t out_ld, void *workspace, size_t workspace_bytes, void *stream) {
    (void)workspace;
    (void)workspace_bytes;
    return top_k_rows(logits, true, num_rows, logits_ld, ks, ke, next_n, k, max_width, out, out_ld, stream);
}
