// Exact top-k over key tokens sharded across decode-context-parallel ranks
// ("vllm.model_executor.layers.sparse_attn_indexer", _merge_dcp_topk_global).
// Each rank scores only its share of a request's tokens and runs top_k_per_row
// on it; pack_dcp_topk_candidates turns that local top-k into (score, global
// token id) float32 pairs, the ranks all-gather the pairs along their leading
// dimension, and stable_topk_from_gathered_candidates keeps the k best of the
// world * k pairs per row. A token of the global top-k has fewer than k tokens
// ahead of it, so fewer than k on its own rank: it is in that rank's local
// top-k, and the merge equals the top-k over the whole row.
//
// Token placement: runs of `interleave` consecutive tokens are dealt to ranks
// 0, 1, ..., world - 1 in turn, so local position p of rank r is global token
// (p / interleave) * world * interleave + r * interleave + p % interleave.
//
// The merge runs one workgroup of 1024 threads per row:
//  * every thread loads up to P pairs (coalesced float2 loads with clamped
//    addresses, all in flight before the first use) into registers as
//    (order key, id);
//  * a three-pass radix select (11 / 11 / 10 key bits, LDS histogram) finds
//    the k-th largest key T; when more pairs hold T than the k slots left for
//    it, a second radix select over the 24-bit ids keeps the lowest ids;
//  * a pass stops the search early when the bin it picked is taken whole;
//  * the selected ids are compacted into LDS and put in ascending order by a
//    bitonic network run by four waves holding E = 4..16 consecutive entries
//    per lane: strides below E inside a lane's registers, strides inside a
//    wave by DPP / swizzle lane exchanges, the last few through LDS.
#include "select.h"
#include "fused.h"

namespace pml {

constexpr int kMergeThreads = 1024;
constexpr int kMergeWaves = kMergeThreads / kWave;
constexpr int kMergeMaxPairs = 32 * kMergeThreads;  // world * k per row
constexpr int kIdLimit = 1 << 24;                   // ids exact in float32

struct PackArgs {
    const float *logits;
    int64_t ld;
    const int32_t *row_starts;
    const int32_t *topk;
    int64_t topk_ld;
    int k, rank, world, interleave;
    float *packed;
};

__global__ __launch_bounds__(256) void pack_kernel(PackArgs a) {
    const int j = blockIdx.y * 256 + threadIdx.x;
    const int r = blockIdx.x;
    if (j >= a.k) return;
    const int64_t lo = a.row_starts ? min<int64_t>(max(a.row_starts[r], 0), a.ld) : 0;
    const int idx = a.topk[(int64_t)r * a.topk_ld + j];
    float2 o = make_float2(-__builtin_huge_valf(), -1.0f);
    if (idx >= 0 && lo + idx < a.ld) {
        o.x = a.logits[(int64_t)r * a.ld + lo + idx];
        const int64_t gid = (int64_t)(idx / a.interleave) * a.world * a.interleave +
                            (int64_t)a.rank * a.interleave + idx % a.interleave;
        o.y = (float)gid;
    }
    *reinterpret_cast<float2 *>(a.packed + ((int64_t)r * a.k + j) * 2) = o;
}

struct MergeArgs {
    const float *gathered;
    int world, rows, k;
    int32_t *out;
    int64_t out_ld;
};

// The k best of the pairs (key[i], id[i]) the workgroup holds (id < 0: no
// pair), P per thread: their ids in ascending order, then -1, into out_row[0, k).
template <int P, int E>
__device__ __forceinline__ void select_k_ids(const uint32_t (&key)[P], const int32_t (&id)[P], uint32_t nmine,
                                             int k, int32_t *out_row) {
    constexpr int NT = kMergeThreads;
    constexpr int NS = kSortThreads * E;  // sorted entries (>= k)
    __shared__ __attribute__((aligned(16))) uint32_t s_hist[2048];
    __shared__ int32_t s_ids[NS];
    __shared__ __attribute__((aligned(16))) uint32_t s_wave[kMergeWaves];
    __shared__ uint32_t s_pick[2];
    __shared__ uint32_t s_nsel;
    const int tid = threadIdx.x;
    if (tid == 0) s_nsel = 0;  // (published by the barriers of the first scan)
    uint32_t nvalid;
    block_scan<NT>(nmine, s_wave, &nvalid);

    // selection: the key under mask TM above T, or equal to T with id <= id_max
    uint32_t T = 0, TM = 0;
    int32_t id_max = kIdLimit;
    if (nvalid > (uint32_t)k) {
        uint32_t prefix = 0, mask = 0, kk = (uint32_t)k, cnt = 0;
        auto live = [&](int i) { return id[i] >= 0; };
        auto kf = [&](int i) { return key[i]; };
#pragma unroll 1
        for (int pass = 0; pass < 3; ++pass) {
            const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
            const int nbins = pass == 2 ? 1024 : 2048;
            cnt = radix_pass<kMergeThreads, P>(kf, live, prefix, mask, shift, nbins, kk, s_hist, s_wave, s_pick);
            prefix |= s_pick[0] << shift;
            mask |= (uint32_t)(nbins - 1) << shift;
            kk -= s_pick[1];
            if (cnt == kk) break;  // the picked bin is taken whole
        }
        T = prefix;
        TM = mask;
        if (cnt > kk) {
            // keep the kk lowest ids among key == T: select the largest of (2^24 - 1 - id)
            const uint32_t top = (uint32_t)kIdLimit - 1;
            auto tied = [&](int i) { return id[i] >= 0 && key[i] == T; };
            auto inv = [&](int i) { return top - (uint32_t)id[i]; };
            uint32_t p2 = 0, m2 = 0, k2 = kk;
#pragma unroll 1
            for (int pass = 0; pass < 3; ++pass) {
                const int shift = pass == 0 ? 13 : (pass == 1 ? 2 : 0);
                const int nbins = pass == 2 ? 4 : 2048;
                radix_pass<kMergeThreads, P>(inv, tied, p2, m2, shift, nbins, k2, s_hist, s_wave, s_pick);
                p2 |= s_pick[0] << shift;
                m2 |= (uint32_t)(nbins - 1) << shift;
                k2 -= s_pick[1];
            }
            id_max = (int32_t)(top - p2);
        }
    }

    // compaction into s_ids (any order, at most k entries): each wave takes a
    // contiguous run of slots and fills it in ballot order
    auto selected = [&](int i) {
        const uint32_t km = key[i] & TM;
        return id[i] >= 0 && (km > T || (km == T && id[i] <= id_max));
    };
    uint64_t sel[P];
    uint32_t wave_total = 0;
#pragma unroll
    for (int i = 0; i < P; ++i) {
        sel[i] = __ballot(selected(i));
        wave_total += (uint32_t)__popcll(sel[i]);
    }
    uint32_t slot = 0;
    if (lane_id() == 0) slot = atomicAdd(&s_nsel, wave_total);
    slot = __shfl(slot, 0, kWave);
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(sel[i] >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)sel[i], 0u));
        if (((sel[i] >> lane_id()) & 1) && slot + below < (uint32_t)k) s_ids[slot + below] = id[i];
        slot += (uint32_t)__popcll(sel[i]);
    }
    __syncthreads();
    const int m = min((int)s_nsel, k);
    for (int j = m + tid; j < NS; j += NT) s_ids[j] = 0x7fffffff;
    __syncthreads();

    int32_t x[E];
    bitonic_sort<E>(x, s_ids);
    if (tid < kSortThreads) {
        int32_t *out = out_row;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int j = tid * E + e;
            if (j < k) out[j] = j < m ? x[e] : -1;
        }
    }
}


template <int P, int E>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeArgs a) {
    constexpr int NT = kMergeThreads;
    const int tid = threadIdx.x;
    const int r = blockIdx.x;
    const int k = a.k;
    const int M = a.world * k;

    // pairs c = i * NT + tid: rank c / k, slot c % k
    float2 v[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int c = min(i * NT + tid, M - 1);
        const int w = c / k;
        const int j = c - w * k;
        v[i] = *reinterpret_cast<const float2 *>(a.gathered + (((int64_t)w * a.rows + r) * k + j) * 2);
    }
    uint32_t key[P];
    int32_t id[P];
    uint32_t nmine = 0;
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const bool ok = i * NT + tid < M && v[i].y >= 0.0f && v[i].y < (float)kIdLimit;
        key[i] = order_key(v[i].x);
        id[i] = ok ? (int32_t)v[i].y : -1;
        nmine += ok;
    }
    select_k_ids<P, E>(key, id, nmine, k, a.out + (int64_t)r * a.out_ld);
}

template <int E>
static void launch_merge(int P, const MergeArgs &a, hipStream_t st) {
    const dim3 g(a.rows), b(kMergeThreads);
    switch (P) {
        case 2: hipLaunchKernelGGL((merge_kernel<2, E>), g, b, 0, st, a); break;
        case 4: hipLaunchKernelGGL((merge_kernel<4, E>), g, b, 0, st, a); break;
        case 8: hipLaunchKernelGGL((merge_kernel<8, E>), g, b, 0, st, a); break;
        case 16: hipLaunchKernelGGL((merge_kernel<16, E>), g, b, 0, st, a); break;
        default: hipLaunchKernelGGL((merge_kernel<32, E>), g, b, 0, st, a); break;
    }
}

// Top-k from a row's candidates (the fused logits + top-k call): rows no
// wider than k take their columns in order; rows with k to cap candidates
// select among them (the candidates hold every column scoring at or above the
// row's threshold, so the k best of the row are among them); other rows are
// left to the full top-k (done[r] = 0).
//
// Block regions come in column order and each is filled in lane (column)
// order, so the candidates, read block after block, are in column order.
// Thread t takes candidates [P t, P t + P): a scan of the block counts gives
// each block's first candidate index, and the owner of each block marks its
// candidates' block in an LDS map. A radix select finds the k-th largest
// key, its first digit taken at the highest bit where the candidates' keys
// differ (they cluster just above the row's threshold, and a fixed top digit
// would send them all to a few bins). One scan of (larger, equal) counts then
// places every selected column, ascending, equal keys by lower column, with
// no sort.
template <int P>
__global__ __launch_bounds__(kMergeThreads) void cand_select_kernel(CandSelectArgs a) {
    constexpr int NT = kMergeThreads;
    constexpr int PB = kSelectMaxBlocks / NT;  // blocks per thread in the scan
    __shared__ int32_t s_off[kSelectMaxBlocks + 1];
    __shared__ uint16_t s_blk[P * NT];  // block of each candidate
    __shared__ __attribute__((aligned(16))) uint32_t s_hist[2048];
    __shared__ __attribute__((aligned(16))) uint32_t s_wave[2 * kMergeWaves];
    __shared__ uint32_t s_pick[2];
    const int tid = threadIdx.x;
    const int r = blockIdx.x;
    const int k = a.k;
    const int n = a.width[r];
    int32_t *out = a.out + (int64_t)r * a.out_ld;
    if (n <= k) {
        for (int j = tid; j < k; j += NT) out[j] = j < n ? j : -1;
        if (tid == 0) a.done[r] = 1;
        return;
    }
    const int nb = (n + a.bkv - 1) / a.bkv;
    if (nb > kSelectMaxBlocks) {
        if (tid == 0) a.done[r] = 0;
        return;
    }
    const int32_t *cnt = a.count + (int64_t)r * a.count_ld;
    int c[PB];
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < PB; ++j) {
        const int b = tid * PB + j;
        c[j] = b < nb ? cnt[b] : 0;
        mine += (uint32_t)c[j];
    }
    uint32_t total;
    uint32_t off = block_scan<NT>(mine, s_wave, &total) - mine;
    if (total < (uint32_t)k || total > (uint32_t)min(a.cap, P * NT)) {
        if (tid == 0) a.done[r] = 0;
        return;
    }
#pragma unroll
    for (int j = 0; j < PB; ++j) {
        const int b = tid * PB + j;
        if (b < nb) {
            s_off[b] = (int)off;
            for (int q = 0; q < c[j]; ++q) s_blk[off + q] = (uint16_t)b;
        }
        off += (uint32_t)c[j];
    }
    __syncthreads();
    // gather this thread's candidates [c0, c0 + P) (clamped into the list)
    const int c0 = tid * P;
    const float *row = a.cand + (int64_t)r * a.cand_ld * 2;
    int64_t addr[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int ci = min(c0 + i, (int)total - 1);
        const int blk = s_blk[ci];
        addr[i] = 2 * ((int64_t)blk * a.bkv + ci - s_off[blk]);
    }
    float2 v[P];
#pragma unroll
    for (int i = 0; i < P; ++i) v[i] = *reinterpret_cast<const float2 *>(row + addr[i]);
    uint32_t key[P];
    bool live[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        key[i] = order_key(v[i].x);
        live[i] = c0 + i < (int)total;
    }
    // k-th largest key: digits of up to 11 bits from the highest bit where the
    // live keys differ down (a pass stops early when its bin is taken whole)
    uint32_t kmax = 0, nkmin = 0;
#pragma unroll
    for (int i = 0; i < P; ++i)
        if (live[i]) {
            kmax = max(kmax, key[i]);
            nkmin = max(nkmin, ~key[i]);
        }
    block_max2<NT>(kmax, nkmin, s_wave);
    const uint32_t diff = kmax ^ ~nkmin;
    uint32_t kk = (uint32_t)k, prefix = kmax, mask = 0xffffffffu;
    if (diff != 0) {
        int top = 31 - __builtin_clz(diff);  // highest differing bit
        mask = top == 31 ? 0u : ~((2u << top) - 1u);
        prefix = kmax & mask;
        auto kf = [&](int i) { return key[i]; };
        auto lf = [&](int i) { return live[i]; };
#pragma unroll 1
        for (;;) {
            const int shift = max(top - 10, 0);
            const int nbins = 1 << (top - shift + 1);
            const uint32_t cntb = radix_pass<NT, P>(kf, lf, prefix, mask, shift, nbins, kk, s_hist, s_wave, s_pick);
            prefix |= s_pick[0] << shift;
            mask |= (uint32_t)(nbins - 1) << shift;
            kk -= s_pick[1];
            if (cntb == kk || shift == 0) break;
            top = shift - 1;
        }
    }
    // ordered placement: slot = (larger before) + min(equal before, kk)
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const uint32_t km = key[i] & mask;
        gt += live[i] && km > prefix;
        eq += live[i] && km == prefix;
    }
    uint32_t tot;
    const uint32_t packed = gt | (eq << 16);
    const uint32_t excl = block_scan<NT>(packed, s_wave, &tot) - packed;
    uint32_t gb = excl & 0xffffu, eb = excl >> 16;
#pragma unroll
    for (int i = 0; i < P; ++i) {
        if (!live[i]) continue;
        const uint32_t km = key[i] & mask;
        const int col = (int)v[i].y;
        if (km > prefix) {
            out[gb + min(eb, kk)] = col;
            ++gb;
        } else if (km == prefix) {
            if (eb < kk) out[gb + eb] = col;
            ++eb;
        }
    }
    if (tid == 0) a.done[r] = 1;
}

int launch_cand_select(const CandSelectArgs &a, int num_rows, hipStream_t st) {
    if (a.cap > 16 * kMergeThreads) return PML_ERR_SHAPE;
    const dim3 g(num_rows), b(kMergeThreads);
    if (a.cap <= 2 * kMergeThreads)
        hipLaunchKernelGGL(cand_select_kernel<2>, g, b, 0, st, a);
    else if (a.cap <= 4 * kMergeThreads)
        hipLaunchKernelGGL(cand_select_kernel<4>, g, b, 0, st, a);
    else if (a.cap <= 8 * kMergeThreads)
        hipLaunchKernelGGL(cand_select_kernel<8>, g, b, 0, st, a);
    else
        hipLaunchKernelGGL(cand_select_kernel<16>, g, b, 0, st, a);
    return hipGetLastError() == hipSuccess ? PML_OK : PML_ERR_HIP;
}

}  // namespace pml

extern "C" int pack_dcp_topk_candidates(const float *logits, int num_rows, int64_t logits_ld,
                                        const int32_t *row_starts, const int32_t *topk, int64_t topk_ld,
                                        int k, int rank, int world, int interleave, float *packed,
                                        void *stream) {
    if (num_rows < 0 || logits_ld < 0) return PML_ERR_SHAPE;
    if (k < 1 || k > PML_MAX_TOPK) return PML_ERR_K;
    if (world < 1 || rank < 0 || rank >= world || interleave < 1) return PML_ERR_SHAPE;
    if (logits_ld > 0) {
        const int64_t p = logits_ld - 1;  // largest local position that can be packed
        const int64_t gid = (p / interleave) * world * (int64_t)interleave + (int64_t)rank * interleave + p % interleave;
        if (gid >= pml::kIdLimit) return PML_ERR_SHAPE;
    }
    if (num_rows == 0) return PML_OK;
    if (!logits || !topk || !packed) return PML_ERR_NULL;
    if (topk_ld < k) return PML_ERR_STRIDE;
    if ((uintptr_t)packed % 8) return PML_ERR_ALIGN;
    pml::PackArgs a{logits, logits_ld, row_starts, topk, topk_ld, k, rank, world, interleave, packed};
    hipLaunchKernelGGL(pml::pack_kernel, dim3(num_rows, (k + 255) / 256), dim3(256), 0, (hipStream_t)stream, a);
    return hipGetLastError() == hipSuccess ? PML_OK : PML_ERR_HIP;
}

extern "C" int stable_topk_from_gathered_candidates(const float *gathered, int world, int num_rows, int k,
                                                    int32_t *out, int64_t out_ld, void *stream) {
    if (num_rows < 0 || world < 1) return PML_ERR_SHAPE;
    if (k < 1 || k > PML_MAX_TOPK) return PML_ERR_K;
    if ((int64_t)world * k > pml::kMergeMaxPairs) return PML_ERR_SHAPE;
    if (num_rows == 0) return PML_OK;
    if (!gathered || !out) return PML_ERR_NULL;
    if (out_ld < k) return PML_ERR_STRIDE;
    if ((uintptr_t)gathered % 8) return PML_ERR_ALIGN;
    const int pairs = world * k;
    int P = 2;
    while (P * pml::kMergeThreads < pairs) P <<= 1;
    pml::MergeArgs a{gathered, world, num_rows, k, out, out_ld};
    hipStream_t st = (hipStream_t)stream;
    if (k <= 4 * pml::kSortThreads)
        pml::launch_merge<4>(P, a, st);
    else if (k <= 8 * pml::kSortThreads)
        pml::launch_merge<8>(P, a, st);
    else
        pml::launch_merge<16>(P, a, st);
    return hipGetLastError() == hipSuccess ? PML_OK : PML_ERR_HIP;
}
