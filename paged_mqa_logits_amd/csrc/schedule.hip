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
// One workgroup of 1024 threads walks the rows in chunks of 1024: every
// thread loads its row's visible length and group-end flag into LDS (plus a
// halo of kGMax rows), a max-scan finds each row's group start, the thread of
// a piece's first row reads the piece's rows and extent from LDS, and a
// sum-scan of the piece costs gives each piece's offset; the thread of a
// piece then writes the entries of the workers whose start falls inside it.
// Up to 1024 rows take one walk; more take two (the total first).
#include "rows.h"

namespace pml {

constexpr int kSchedThreads = 1024;
constexpr int kSchedWaves = kSchedThreads / kWave;
constexpr int kHalo = kGMax;  // rows past a chunk that a piece starting in it may cover

// Block-wide inclusive scan: wave shuffles, then one pass over the wave totals.
template <typename T, typename Op>
__device__ __forceinline__ T block_scan_incl(T x, T *s_w, Op op, T ident) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const T y = __shfl_up(x, off, kWave);
        if (lane >= off) x = op(x, y);
    }
    if (lane == kWave - 1) s_w[wave] = x;
    __syncthreads();
    T pre = ident;
    for (int w = 0; w < wave; ++w) pre = op(pre, s_w[w]);
    __syncthreads();
    return op(pre, x);
}

struct SchedShared {
    int vis[kSchedThreads + kHalo];    // visible length of rows base + i
    int last[kSchedThreads + kHalo];   // row base + i ends its group (or is past the end)
    int wi[kSchedWaves];
    long long wl[kSchedWaves];
    int run_carry;
    long long cost_carry;
};

// Cost of the piece starting at row base + tid (0 if no piece starts there)
// and its row count, for the chunk of rows starting at base.
__device__ __forceinline__ long long chunk_cost(const RowView &v, int block_kv, int base, SchedShared &sh, int &g) {
    const int tid = threadIdx.x;
    const int n = v.num_rows;
    for (int i = tid; i < kSchedThreads + kHalo; i += kSchedThreads) {
        const int rr = base + i;
        int vis = 0, last = 1;
        if (rr < n) {
            vis = v.visible(rr);
            last = rr + 1 >= n || !v.same_group(rr + 1, rr);
        }
        sh.vis[i] = vis;
        sh.last[i] = last;
    }
    const int r = base + tid;
    const bool live = r < n;
    const int start_here = (live && (r == 0 || !v.same_group(r, r - 1))) ? r : -1;
    auto imax = [](int x, int y) { return x > y ? x : y; };
    int run = block_scan_incl(start_here, sh.wi, imax, -1);  // (its barriers publish vis / last)
    run = imax(run, sh.run_carry);                          // first row of the group holding r
    g = 0;
    long long cost = 0;
    if (live && (r - run) % kGMax == 0) {  // r starts a piece: rows up to its group's end, at most kGMax
        int e = 0;
        bool go = true;
#pragma unroll
        for (int i = 0; i < kGMax; ++i)
            if (go) {
                e = imax(e, sh.vis[tid + i]);
                g = i + 1;
                go = !sh.last[tid + i];
            }
        cost = (long long)((e + block_kv - 1) / block_kv) * (kCostBase + g);
    }
    __syncthreads();
    if (tid == kSchedThreads - 1) sh.run_carry = run;
    return cost;
}

// Entries of the workers whose start offset floor(c * T / W) falls inside
// [cum, cum + cost), the piece starting at row r with g rows.
__device__ __forceinline__ void write_entries(int32_t *sched, int W, long long total, long long cum, long long cost,
                                              int r, int g) {
    long long c = (cum * W + total - 1) / total;
    long long c_hi = ((cum + cost) * W + total - 1) / total - 1;
    if (c_hi > W - 1) c_hi = W - 1;
    if (c > c_hi) return;
    // t = floor(c * T / W), stepped without a division per entry
    const long long dq = total / W, dr = total % W;
    long long t = c * total / W, rem = c * total % W;
    for (; c <= c_hi; ++c) {
        sched[2 * c] = r;
        sched[2 * c + 1] = (int)((t - cum) / (kCostBase + g));
        t += dq;
        rem += dr;
        if (rem >= W) {
            rem -= W;
            ++t;
        }
    }
}

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(RowView v, int block_kv, int W, int32_t *sched) {
    __shared__ SchedShared sh;
    const int tid = threadIdx.x;
    const int n = v.num_rows;
    auto ladd = [](long long x, long long y) { return x + y; };
    if (tid == 0) {
        sh.run_carry = 0;
        sh.cost_carry = 0;
    }
    __syncthreads();
    if (n <= kSchedThreads) {
        // one chunk: costs, total and entries in a single walk
        int g;
        const long long cost = chunk_cost(v, block_kv, 0, sh, g);
        const long long incl = block_scan_incl(cost, sh.wl, ladd, 0LL);
        if (tid == kSchedThreads - 1) sh.cost_carry = incl;
        __syncthreads();
        const long long total = sh.cost_carry;
        if (total == 0) {
            for (int c = tid; c <= W; c += kSchedThreads) {
                sched[2 * c] = n;
                sched[2 * c + 1] = 0;
            }
            return;
        }
        if (tid == 0) {
            sched[2 * W] = n;
            sched[2 * W + 1] = 0;
        }
        if (cost > 0) write_entries(sched, W, total, incl - cost, cost, tid, g);
        return;
    }
    // several chunks: the total first, then the entries
    for (int base = 0; base < n; base += kSchedThreads) {
        int g;
        const long long cost = chunk_cost(v, block_kv, base, sh, g);
        const long long incl = block_scan_incl(cost, sh.wl, ladd, 0LL);
        if (tid == kSchedThreads - 1) sh.cost_carry += incl;
        __syncthreads();
    }
    const long long total = sh.cost_carry;
    __syncthreads();
    if (total == 0) {
        for (int c = tid; c <= W; c += kSchedThreads) {
            sched[2 * c] = n;
            sched[2 * c + 1] = 0;
        }
        return;
    }
    if (tid == 0) {
        sched[2 * W] = n;
        sched[2 * W + 1] = 0;
        sh.run_carry = 0;
        sh.cost_carry = 0;
    }
    __syncthreads();
    for (int base = 0; base < n; base += kSchedThreads) {
        int g;
        const long long cost = chunk_cost(v, block_kv, base, sh, g);
        const long long incl = block_scan_incl(cost, sh.wl, ladd, 0LL);
        const long long carry = sh.cost_carry;
        if (cost > 0) write_entries(sched, W, total, carry + incl - cost, cost, base + threadIdx.x, g);
        __syncthreads();
        if (tid == kSchedThreads - 1) sh.cost_carry = carry + incl;
        __syncthreads();
    }
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
