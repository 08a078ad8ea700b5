// top_k_per_row: the k largest logits of each row among its valid columns
// [lo, hi), returned as int32 positions relative to lo in ascending order and
// padded with -1 (the indexer's top-k selector; output preset to -1 and
// request-local positions as in the CPU decode path of the sparse_attn_indexer
// page). Selection order: larger value first, equal values by lower position.
//
// One workgroup per row:
//  1. Radix select on an order-preserving 32-bit key (NaN lowest, -0 == +0):
//     three histogram passes over digits of 11, 11 and 10 bits find the exact
//     key T of the k-th selected element and how many elements equal to T are
//     taken (the lowest-positioned ones).
//  2. One ordered compaction pass: a block-wide scan of (key > T, key == T)
//     gives each selected element its output slot, so positions come out
//     ascending without a sort; the pass stops once k elements are placed.
#include "pml_device.h"

namespace pml {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kBins = 2048;

__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN sorts below every number
    if (u == 0x80000000u) u = 0u;                    // -0 counts as +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive scan of one uint32 per thread over the whole workgroup; returns
// the inclusive prefix and writes the workgroup total to *total.
__device__ __forceinline__ uint32_t block_scan(uint32_t x, uint32_t *s_wave, uint32_t *total) {
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, kWave);
        if (lane >= o) x += y;
    }
    if (lane == kWave - 1) s_wave[wave] = x;
    __syncthreads();
    if (wave == 0) {
        uint32_t v = lane < kTopkWaves ? s_wave[lane] : 0u;
#pragma unroll
        for (int o = 1; o < kTopkWaves; o <<= 1) {
            const uint32_t y = __shfl_up(v, o, kWave);
            if (lane >= o) v += y;
        }
        if (lane < kTopkWaves) s_wave[kTopkWaves + lane] = v;  // inclusive wave prefix
    }
    __syncthreads();
    const uint32_t before = wave > 0 ? s_wave[kTopkWaves + wave - 1] : 0u;
    *total = s_wave[2 * kTopkWaves - 1];
    const uint32_t r = x + before;
    __syncthreads();  // s_wave is reused by the next call
    return r;
}

struct TopkArgs {
    const float *logits;
    int64_t ld;
    const int32_t *ks;
    const int32_t *ke;
    int next_n;
    int k;
    int max_width;
    int32_t *out;
    int64_t out_ld;
};

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
    __shared__ uint32_t s_hist[kBins];
    __shared__ uint32_t s_wave[2 * kTopkWaves];
    __shared__ uint32_t s_pick[2];

    const int tid = threadIdx.x;
    const int r = blockIdx.x;
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
    const float *row = a.logits + (int64_t)r * a.ld + lo;

    if (n <= k) {
        for (int j = tid; j < k; j += kTopkThreads) out[j] = j < n ? j : -1;
        return;
    }

    // 1. radix select of the k-th largest key
    uint32_t prefix = 0, mask = 0;
    uint32_t kk = (uint32_t)k;  // elements still to take inside the current prefix bucket
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const uint32_t nbins = pass == 2 ? 1024u : 2048u;
        for (int b = tid; b < kBins; b += kTopkThreads) s_hist[b] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += kTopkThreads) {
            const uint32_t key = order_key(row[i]);
            if ((key & mask) == prefix) atomicAdd(&s_hist[(key >> shift) & (nbins - 1)], 1u);
        }
        __syncthreads();
        // counts from the top bin down: thread t owns bins nbins-1-2t and nbins-2-2t
        const int b1 = (int)nbins - 1 - 2 * tid;
        const int b0 = b1 - 1;
        const uint32_t h1 = b1 >= 0 ? s_hist[b1] : 0u;
        const uint32_t h0 = b0 >= 0 ? s_hist[b0] : 0u;
        uint32_t tot;
        const uint32_t incl = block_scan(h1 + h0, s_wave, &tot);
        const uint32_t gt1 = incl - h1 - h0;  // elements in bins above b1
        if (b1 >= 0 && gt1 < kk && kk <= gt1 + h1) {
            s_pick[0] = (uint32_t)b1;
            s_pick[1] = gt1;
        }
        if (b0 >= 0 && gt1 + h1 < kk && kk <= gt1 + h1 + h0) {
            s_pick[0] = (uint32_t)b0;
            s_pick[1] = gt1 + h1;
        }
        __syncthreads();
        prefix |= s_pick[0] << shift;
        mask |= (nbins - 1) << shift;
        kk -= s_pick[1];
        __syncthreads();
    }
    const uint32_t T = prefix;
    const uint32_t need = kk;  // elements equal to T that are taken (1 <= need)
    const uint32_t n_gt = (uint32_t)k - need;

    // 2. ordered compaction
    uint32_t carry_gt = 0, carry_eq = 0;
#pragma unroll 1
    for (int base = 0; base < n; base += kTopkThreads) {
        const int i = base + tid;
        uint32_t key = 0;
        const bool valid = i < n;
        if (valid) key = order_key(row[i]);
        const uint32_t gt = valid && key > T;
        const uint32_t eq = valid && key == T;
        uint32_t tot;
        const uint32_t packed = gt | (eq << 16);
        const uint32_t incl = block_scan(packed, s_wave, &tot);
        const uint32_t excl = incl - packed;
        const uint32_t gt_before = carry_gt + (excl & 0xffffu);
        const uint32_t eq_before = carry_eq + (excl >> 16);
        if (gt || (eq && eq_before < need)) out[gt_before + min(eq_before, need)] = i;
        carry_gt += tot & 0xffffu;
        carry_eq += tot >> 16;
        if (carry_gt >= n_gt && carry_eq >= need) break;  // all k placed (uniform)
    }
}

}  // namespace pml

extern "C" size_t top_k_per_row_workspace_size(int num_rows, int max_width, int k) {
    (void)num_rows;
    (void)max_width;
    (void)k;
    return 0;
}

extern "C" int top_k_per_row(const float *logits, int num_rows, int64_t logits_ld, const int32_t *ks,
                             const int32_t *ke, int next_n, int k, int max_width, int32_t *out,
                             int64_t out_ld, void *workspace, size_t workspace_bytes, void *stream) {
    (void)workspace;
    (void)workspace_bytes;
    if (num_rows < 0 || next_n < 1 || max_width < 0 || logits_ld < 0) return PML_ERR_SHAPE;
    if (k < 1 || k > PML_MAX_TOPK) return PML_ERR_K;
    if (ks && next_n != 1) return PML_ERR_UNSUPPORTED;
    if (!ks && next_n > 1 && num_rows % next_n != 0) return PML_ERR_SHAPE;
    if (num_rows == 0) return PML_OK;
    if (!logits || !ke || !out) return PML_ERR_NULL;
    if (out_ld < k) return PML_ERR_STRIDE;
    pml::TopkArgs a{logits, logits_ld, ks, ke, next_n, k, max_width, out, out_ld};
    hipLaunchKernelGGL(pml::topk_kernel, dim3(num_rows), dim3(pml::kTopkThreads), 0, (hipStream_t)stream, a);
    return hipGetLastError() == hipSuccess ? PML_OK : PML_ERR_HIP;
}
