// as_fp32_logits: bf16 logits to fp32 over each row's valid span
// ("vllm.model_executor.layers.sparse_attn_indexer", as_fp32_logits: only the
// columns below the row's end are converted, the span the fp32 top-k reads,
// and the row stride of the logits is kept).
//
// A bf16 value is the upper half of the fp32 with the same sign, exponent and
// leading 7 mantissa bits, so the conversion is exact: shift the 16 bits up.
// The grid is rows x column chunks of 2048; each thread moves 8 columns (one
// 16-byte load, two 16-byte stores); chunks past a row's end exit at once.
#include "pml_device.h"

namespace pml {

constexpr int kUpThreads = 256;
constexpr int kUpCols = 8 * kUpThreads;

struct UpcastArgs {
    const uint16_t *in;
    int64_t in_ld;
    int cols;
    const int32_t *row_ends;
    float *out;
    int64_t out_ld;
};

__global__ __launch_bounds__(kUpThreads) void upcast_kernel(UpcastArgs a) {
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    const int r = blockIdx.x;
    const int end = min(max(a.row_ends[r], 0), a.cols);
    const int c = blockIdx.y * kUpCols + 8 * threadIdx.x;
    if (c >= end) return;
    const uint16_t *src = a.in + (int64_t)r * a.in_ld + c;
    float *dst = a.out + (int64_t)r * a.out_ld + c;
    if (c + 8 <= end) {
        const v4u h = *(const v4u *)src;
        v4u lo, hi;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            lo[2 * j] = h[j] << 16;
            lo[2 * j + 1] = h[j] & 0xffff0000u;
            hi[2 * j] = h[2 + j] << 16;
            hi[2 * j + 1] = h[2 + j] & 0xffff0000u;
        }
        *(v4u *)dst = lo;
        *(v4u *)(dst + 4) = hi;
    } else {
        for (int j = 0; c + j < end; ++j) dst[j] = __uint_as_float((uint32_t)src[j] << 16);
    }
}

}  // namespace pml

extern "C" int as_fp32_logits(const uint16_t *logits, int num_rows, int64_t logits_ld, int cols,
                              const int32_t *row_ends, float *out, int64_t out_ld, void *stream) {
    if (num_rows < 0 || cols < 0) return PML_ERR_SHAPE;
    if (num_rows == 0 || cols == 0) return PML_OK;
    if (!logits || !row_ends || !out) return PML_ERR_NULL;
    if (logits_ld < cols || out_ld < cols || logits_ld % 8 != 0 || out_ld % 4 != 0) return PML_ERR_STRIDE;
    if (((uintptr_t)logits & 15) != 0 || ((uintptr_t)out & 15) != 0) return PML_ERR_ALIGN;
    const int64_t chunks = ((int64_t)cols + pml::kUpCols - 1) / pml::kUpCols;
    if (chunks > 65535) return PML_ERR_SHAPE;
    pml::UpcastArgs a{logits, logits_ld, cols, row_ends, out, out_ld};
    const dim3 grid(num_rows, (unsigned)chunks);
    hipLaunchKernelGGL(pml::upcast_kernel, grid, dim3(pml::kUpThreads), 0, (hipStream_t)stream, a);
    return hipGetLastError() == hipSuccess ? PML_OK : PML_ERR_HIP;
}
