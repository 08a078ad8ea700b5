// paged_mqa_logits_metadata: split the (row-piece, key-block) units of the
// paged-logits call into one range per persistent workgroup.
//
// The pages fix that the schedule has one row per persistent worker plus one
// (a caller reads the worker count back as schedule.shape[0] - 1) and that a
// row slice needs its own ("vllm.model_executor.layers.sparse_attn_indexer",
// _varlen_decode_rows). Content (this library's): units are ordered by piece
// then block (a block is a step of max(block_kv, 64) tokens: a 32-token cache
// is scored two pages per step); a block of a piece with g rows costs
// kCostBase + g. The work is
// cut into W = num_CUs ranges: entry c is the unit holding cost offset
// floor(c * T / W) of the total T, as (first row of its piece, block offset),
// and entry W is (num_rows, 0). Logits workgroup c scores the units from
// entry c to entry c + 1. The logits call only reads the schedule, so one
// schedule serves any number of calls, at the same time too.
//
// One workgroup of 1024 threads walks the rows in tiles of 1024: every
// thread loads its row's visible length and group-end flag into LDS (plus a
// halo of kGMax rows), a max-scan finds each row's group start, the thread of
// a piece's first row reads the piece's rows and extent from LDS, and a
// sum-scan of the piece costs gives each piece's offset, and each entry that
// falls in the tile finds its piece by a binary search over those offsets.
// Up to 1024 rows take one walk; more take two (the total first). The walk is
// cheap next to the searches, so ceil(W / 1024) workgroups (at most 64) each
// walk all rows and write an equal share of the entries: about one search per
// thread.
#include "rows.h"

namespace pml {

constexpr int kSchedThreads = 1024;
constexpr int kSchedWaves = kSchedThreads / kWave;
constexpr int kHalo = kGMax;  // rows past a tile that a piece starting in it may cover
constexpr int kSchedMaxBlocks = 64;  // workgroups that share out the entries (each walks all rows)

// x of the lane the DPP control CTRL names (row shifts and row broadcasts),
// or ident where it names none or the row is outside ROWMASK.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ int dpp_from(int ident, int x) {
    return __builtin_amdgcn_update_dpp(ident, x, CTRL, ROWMASK, 0xf, false);
}
template <int CTRL, int ROWMASK>
__device__ __forceinline__ long long dpp_from(long long ident, long long x) {
    const int lo = dpp_from<CTRL, ROWMASK>((int)ident, (int)x);
    const int hi = dpp_from<CTRL, ROWMASK>((int)(ident >> 32), (int)(x >> 32));
    return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}

// Inclusive scan over the wave by DPP moves, no LDS traffic: shifts by 1, 2,
// 4, 8 lanes inside each row of 16, then row 0's and row 2's last lanes into
// rows 1 and 3, then lane 31 into rows 2 and 3.
template <typename T, typename Op>
__device__ __forceinline__ T wave_scan_dpp(T x, Op op, T ident) {
    x = op(x, dpp_from<0x111, 0xf>(ident, x));  // row_shr:1
    x = op(x, dpp_from<0x112, 0xf>(ident, x));  // row_shr:2
    x = op(x, dpp_from<0x114, 0xf>(ident, x));  // row_shr:4
    x = op(x, dpp_from<0x118, 0xf>(ident, x));  // row_shr:8
    x = op(x, dpp_from<0x142, 0xa>(ident, x));  // row_bcast:15
    x = op(x, dpp_from<0x143, 0xc>(ident, x));  // row_bcast:31
    return x;
}

// Block-wide inclusive scan: a DPP scan per wave, then one pass over the wave totals.
template <typename T, typename Op>
__device__ __forceinline__ T block_scan_incl(T x, T *s_w, Op op, T ident) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    x = wave_scan_dpp(x, op, ident);
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
    long long incl[kSchedThreads];     // cost of the pieces before row base + i + 1 (all tiles)
    int gs[kSchedThreads];             // rows of the piece starting at row base + i
    int wi[kSchedWaves];
    long long wl[kSchedWaves];
    int run_carry;
    long long cost_carry;
};

// Cost of the piece starting at row base + tid (0 if no piece starts there)
// and its row count, for the tile of rows starting at base.
__device__ __forceinline__ long long tile_cost(const RowView &v, int block_kv, int base, SchedShared &sh, int &g) {
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

// Start offset of chunk c: floor(c * T / C) = c * qC + floor(c * rC / C)
// with T = qC * C + rC, so no product passes 2^63 (c <= C <= 2^23). c * rC
// < C^2, so for C <= 46340 the quotient is a 32-bit division.
__device__ __forceinline__ long long chunk_start(long long c, long long qC, long long rC, int C) {
    const long long f = C <= 46340 ? (long long)((uint32_t)(c * rC) / (uint32_t)C) : c * rC / C;
    return c * qC + f;
}

// First chunk c whose start offset is at least x (0 <= x <= T): a double
// estimate of x * C / T, then exact steps (at most a couple).
__device__ __forceinline__ long long first_chunk_at(long long x, long long T, long long qC, long long rC, int C) {
    long long c = (long long)((double)x * (double)C / (double)T);
    c = c < 0 ? 0 : (c > C ? C : c);
    while (c > 0 && chunk_start(c - 1, qC, rC, C) >= x) --c;
    while (c < C && chunk_start(c, qC, rC, C) < x) ++c;
    return c;
}

// Entries of the chunks that start inside this tile, whose pieces cost
// [carry, carry + tile_total) of the total T. Chunk c starts at offset
// t = chunk_start(c); the piece holding t starts at the first row whose
// running cost sh.incl exceeds t (a binary search over the tile), and t's
// block is (t - that piece's start offset) / (kCostBase + g).
__device__ __forceinline__ void write_tile(int32_t *sched, int C, long long T, long long carry, long long tile_total,
                                           int base, int n_tile, const SchedShared &sh) {
    const long long qC = T / C, rC = T % C;
    const long long lo = first_chunk_at(carry, T, qC, rC, C);
    const long long hi = first_chunk_at(carry + tile_total, T, qC, rC, C);
    // the workgroups take consecutive equal shares of [lo, hi), so each writes whole lines
    const long long per = (hi - lo + gridDim.x - 1) / gridDim.x;
    const long long c0 = lo + per * blockIdx.x, c1 = c0 + per < hi ? c0 + per : hi;
    // (incl of the rows past the last live one equals the tile's total, which
    // no chunk start in the tile reaches)
    const int live = min(kSchedThreads, n_tile);
    for (long long c = c0 + threadIdx.x; c < c1; c += kSchedThreads) {
        const long long t = chunk_start(c, qC, rC, C);
        int l = 0, h = live - 1;
        while (l < h) {
            const int m = (l + h) >> 1;
            if (sh.incl[m] > t)
                h = m;
            else
                l = m + 1;
        }
        const long long start = l ? sh.incl[l - 1] : carry;
        sched[2 * c] = base + l;
        sched[2 * c + 1] = (int)((unsigned)(t - start) / (unsigned)(kCostBase + sh.gs[l]));  // < piece cost < 2^31
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
    const bool first = blockIdx.x == 0;
    __syncthreads();
    long long total;
    if (n <= kSchedThreads) {
        // one tile: costs, total and entries in a single walk
        int g;
        const long long cost = tile_cost(v, block_kv, 0, sh, g);
        const long long incl = block_scan_incl(cost, sh.wl, ladd, 0LL);
        sh.incl[tid] = incl;
        sh.gs[tid] = g;
        if (tid == kSchedThreads - 1) sh.cost_carry = incl;
        __syncthreads();
        total = sh.cost_carry;
        if (total > 0) {
            if (first && tid == 0) {
                sched[2 * W] = n;
                sched[2 * W + 1] = 0;
            }
            write_tile(sched, W, total, 0, total, 0, n, sh);
            return;
        }
    } else {
        // several tiles: the total first, then the entries
        for (int base = 0; base < n; base += kSchedThreads) {
            int g;
            const long long cost = tile_cost(v, block_kv, base, sh, g);
            const long long incl = block_scan_incl(cost, sh.wl, ladd, 0LL);
            if (tid == kSchedThreads - 1) sh.cost_carry += incl;
            __syncthreads();
        }
        total = sh.cost_carry;
        __syncthreads();
        if (total > 0) {
            if (tid == 0) {
                if (first) {
                    sched[2 * W] = n;
                    sched[2 * W + 1] = 0;
                }
                sh.run_carry = 0;
                sh.cost_carry = 0;
            }
            __syncthreads();
            for (int base = 0; base < n; base += kSchedThreads) {
                int g;
                const long long cost = tile_cost(v, block_kv, base, sh, g);
                const long long incl = block_scan_incl(cost, sh.wl, ladd, 0LL);
                const long long carry = sh.cost_carry;
                sh.incl[tid] = carry + incl;
                sh.gs[tid] = g;
                __syncthreads();
                const long long tile_total = sh.incl[kSchedThreads - 1] - carry;
                write_tile(sched, W, total, carry, tile_total, base, n - base, sh);
                __syncthreads();
                if (tid == kSchedThreads - 1) sh.cost_carry = carry + tile_total;
                __syncthreads();
            }
            return;
        }
    }
    // nothing to score: every entry is the end
    for (int c = blockIdx.x * kSchedThreads + tid; c <= W; c += gridDim.x * kSchedThreads) {
        sched[2 * c] = n;
        sched[2 * c + 1] = 0;
    }
}

}  // namespace pml

extern "C" int paged_mqa_logits_metadata(const int32_t *context_lens, int num_rows, int next_n,
                                         int context_lens_2d, const int32_t *indices,
                                         int block_kv, int num_CUs, int32_t *schedule,
                                         void *stream) {
    if (!schedule) return PML_ERR_NULL;
    if ((uintptr_t)schedule % 16) return PML_ERR_ALIGN;
    if (num_rows < 0 || next_n < 1 || num_CUs < 1) return PML_ERR_SHAPE;
    if (num_rows > 0 && !context_lens) return PML_ERR_NULL;
    if (num_rows % next_n != 0) return PML_ERR_SHAPE;
    if (indices && next_n != 1) return PML_ERR_VARLEN_NEXT_N;
    if (block_kv != 32 && block_kv != 64) return PML_ERR_BLOCK_KV;
    if (paged_mqa_logits_schedule_rows(num_CUs) < 0) return PML_ERR_SHAPE;
    pml::RowView v{context_lens, indices, context_lens_2d ? 1 : 0, next_n, num_rows};
    const int W = num_CUs;
    const int blocks = std::min((W + pml::kSchedThreads - 1) / pml::kSchedThreads, pml::kSchedMaxBlocks);
    // units are steps of max(block_kv, 64) tokens: a 32-token cache is scored two pages at a time
    hipLaunchKernelGGL(pml::schedule_kernel, dim3(blocks), dim3(pml::kSchedThreads), 0, (hipStream_t)stream, v,
                       pml::step_tokens(block_kv), W, schedule);
    return hipGetLastError() == hipSuccess ? PML_OK : PML_ERR_HIP;
}

extern "C" int paged_mqa_logits_schedule_rows(int num_CUs) {
    if (num_CUs < 1 || num_CUs > (1 << 20)) return -1;
    return num_CUs + 1;
}
