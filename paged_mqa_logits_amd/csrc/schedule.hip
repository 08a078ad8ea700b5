// paged_mqa_logits_metadata: split (row-piece, key-block) units over the
// persistent workgroups of the paged-logits kernel.
//
// The pages fix only that the schedule has one entry per persistent worker plus
// one and that a row slice needs its own ("vllm.model_executor.layers.
// sparse_attn_indexer", _varlen_decode_rows). Content (this library's): units
// are ordered by piece then block; a block of a piece with g rows costs
// kCostBase + g; worker c starts at the unit holding cost offset
// floor(c * T / W) of the total T and entry W is (num_rows, 0).
//
// One workgroup of 1024 threads walks the rows in chunks twice: first for the
// total cost, then for each piece's cost prefix, writing the entries of the
// workers whose start falls inside that piece.
#include "rows.h"

namespace pml {

constexpr int kSchedThreads = 1024;

template <typename T, typename Op>
__device__ T block_inclusive_scan(T x, T *s, Op op) {
    const int tid = threadIdx.x;
    s[tid] = x;
    __syncthreads();
    for (int off = 1; off < kSchedThreads; off <<= 1) {
        T y = tid >= off ? s[tid - off] : x;
        __syncthreads();
        if (tid >= off) {
            x = op(x, y);
            s[tid] = x;
        }
        __syncthreads();
    }
    return x;
}

__device__ __forceinline__ int rows_of_piece(const RowView &v, int r0) {
    int g = 1;
    while (g < kGMax && r0 + g < v.num_rows && v.same_group(r0 + g, r0)) ++g;
    return g;
}

// One walk over the rows. With write == false it returns the total cost; with
// write == true it writes the entries of workers starting inside each piece.
__device__ long long walk_rows(const RowView &v, int block_kv, int W, int32_t *sched, bool write,
                               long long total, int *s_int, long long *s_ll, int *s_run_carry,
                               long long *s_cost_carry) {
    const int tid = threadIdx.x;
    auto imax = [](int a, int b) { return a > b ? a : b; };
    auto ladd = [](long long a, long long b) { return a + b; };
    if (tid == 0) {
        *s_run_carry = 0;
        *s_cost_carry = 0;
    }
    __syncthreads();
    for (int base = 0; base < v.num_rows; base += kSchedThreads) {
        const int r = base + tid;
        const bool live = r < v.num_rows;
        int start_here = -1;
        if (live && (r == 0 || !v.same_group(r, r - 1))) start_here = r;
        int run = block_inclusive_scan(start_here, s_int, imax);
        run = imax(run, *s_run_carry);  // first row of the group holding r
        long long cost = 0;
        int g = 0;
        if (live && (r - run) % kGMax == 0) {  // r starts a piece
            g = rows_of_piece(v, r);
            int e = 0;
            for (int i = 0; i < g; ++i) e = imax(e, v.visible(r + i));
            cost = (long long)((e + block_kv - 1) / block_kv) * (kCostBase + g);
        }
        const long long incl = block_inclusive_scan(cost, s_ll, ladd);
        if (write && cost > 0) {
            const long long cum = *s_cost_carry + incl - cost;
            // workers c whose start offset floor(c*T/W) lies in [cum, cum + cost)
            long long c_lo = (cum * W + total - 1) / total;
            long long c_hi = ((cum + cost) * W + total - 1) / total - 1;
            if (c_hi > W - 1) c_hi = W - 1;
            for (long long c = c_lo; c <= c_hi; ++c) {
                const long long t = c * total / W;
                sched[2 * c] = r;
                sched[2 * c + 1] = (int)((t - cum) / (kCostBase + g));
            }
        }
        __syncthreads();
        if (tid == kSchedThreads - 1) {
            *s_run_carry = run;
            *s_cost_carry += incl;
        }
        __syncthreads();
    }
    return *s_cost_carry;
}

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(RowView v, int block_kv, int W,
                                                                  int32_t *sched) {
    __shared__ int s_int[kSchedThreads];
    __shared__ long long s_ll[kSchedThreads];
    __shared__ int s_run_carry;
    __shared__ long long s_cost_carry;
    const long long total = walk_rows(v, block_kv, W, sched, false, 0, s_int, s_ll, &s_run_carry,
                                      &s_cost_carry);
    __syncthreads();
    if (total == 0) {
        for (int c = threadIdx.x; c <= W; c += kSchedThreads) {
            sched[2 * c] = v.num_rows;
            sched[2 * c + 1] = 0;
        }
        return;
    }
    if (threadIdx.x == 0) {
        sched[2 * W] = v.num_rows;
        sched[2 * W + 1] = 0;
    }
    walk_rows(v, block_kv, W, sched, true, total, s_int, s_ll, &s_run_carry, &s_cost_carry);
}

}  // namespace pml

extern "C" int paged_mqa_logits_metadata(const int32_t *context_lens, int num_rows, int next_n,
                                         int context_lens_2d, const int32_t *indices,
                                         int block_kv, int num_CUs, int32_t *schedule,
                                         void *stream) {
    if (!schedule) return PML_ERR_NULL;
    if (num_rows < 0 || next_n < 1 || num_CUs < 1) return PML_ERR_SHAPE;
    if (num_rows > 0 && !context_lens) return PML_ERR_NULL;
    if (num_rows % next_n != 0) return PML_ERR_SHAPE;
    if (indices && next_n != 1) return PML_ERR_VARLEN_NEXT_N;
    if (block_kv != 32 && block_kv != 64) return PML_ERR_BLOCK_KV;
    pml::RowView v{context_lens, indices, context_lens_2d ? 1 : 0, next_n, num_rows};
    hipLaunchKernelGGL(pml::schedule_kernel, dim3(1), dim3(pml::kSchedThreads), 0,
                       (hipStream_t)stream, v, block_kv, num_CUs, schedule);
    return hipGetLastError() == hipSuccess ? PML_OK : PML_ERR_HIP;
}
