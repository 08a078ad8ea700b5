/*
 * CPU oracle for the paged MQA-logits path. TEST INFRASTRUCTURE ONLY: the
 * tests, the smoke check and the bench's CPU-baseline leg call it; the GPU
 * product path never does. It shares no code, header or table with the GPU
 * kernels.
 *
 * Plain C, one loop per definition, fp64 accumulation, OpenMP over output
 * cells. Every function states the passage it follows.
 *
 * Score (the indexer's MQA logit: the pages name it and pass its inputs, q,
 * the per-token key scale and the per-head weights, but never write it out;
 * this is the plain weighted-ReLU reading of those inputs, with no other
 * constants):
 *     logit[r, s] = sum_h w[r,h] * max(0, scale_k[s] * <q[r,h,:], k[s,:]>)
 * for visible key tokens s, and -inf for masked ones.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- number formats, written from their public definitions ------------ */

/* OCP 8-bit floating point, E4M3 "fn" variant: 1 sign, 4 exponent (bias 7),
 * 3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN;
 * there is no infinity (max 448). */
double pml_oracle_fp8_e4m3(uint8_t c)
{
    int s = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* OCP Microscaling v1.0 FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa
 * bit; exponent 0 is subnormal (m/2); no NaN or infinity (max 6). */
double pml_oracle_e2m1(uint8_t nib)
{
    int s = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

/* OCP Microscaling v1.0 E8M0 scale: 2^(e - 127); 0xFF is NaN. */
double pml_oracle_e8m0(uint8_t e)
{
    if (e == 0xFF)
        return NAN;
    return ldexp(1.0, (int)e - 127);
}

/* Decoded values of every code, filled from the three functions above. */
static double FP8[256], E2M1[16], E8M0[256];
static int tables_ready = 0;

static void init_tables(void)
{
    if (tables_ready)
        return;
    for (int c = 0; c < 256; ++c) {
        FP8[c] = pml_oracle_fp8_e4m3((uint8_t)c);
        E8M0[c] = pml_oracle_e8m0((uint8_t)c);
    }
    for (int c = 0; c < 16; ++c)
        E2M1[c] = pml_oracle_e2m1((uint8_t)c);
    tables_ready = 1;
}

static double fp32_le(const uint8_t *p)
{
    float f;
    memcpy(&f, p, 4); /* 4 little-endian bytes of an IEEE binary32 */
    return (double)f;
}

/* ---- paged key cache -------------------------------------------------- */

/* Dequantised key element k^[token at (page, slot), d].
 * fp8 page (sparse_attn_indexer page, _gather_workspace_shapes: per token D
 * fp8 values + a 4-byte fp32 scale): values region [block_kv][D] at offset 0,
 * scales region [block_kv] fp32 after it.
 * MXFP4 page (same function, MXFP4 branch, and kv_cache_as_quant_view: D/2
 * packed bytes + D/32 ue8m0 bytes per token): values region [block_kv][D/2]
 * (element 2i in the low nibble of byte i), then scales [block_kv][D/32]. */
static double key_elem(const uint8_t *page, int kv_format, int block_kv, int D, int slot, int d)
{
    if (kv_format == 0) {
        double code = FP8[page[(size_t)slot * D + d]];
        double scale = fp32_le(page + (size_t)block_kv * D + (size_t)slot * 4);
        return scale * code;
    } else {
        uint8_t byte = page[(size_t)slot * (D / 2) + d / 2];
        uint8_t nib = (d % 2 == 0) ? (byte & 15) : (byte >> 4);
        uint8_t e = page[(size_t)block_kv * (D / 2) + (size_t)slot * (D / 32) + d / 32];
        return E2M1[nib] * E8M0[e];
    }
}

/* Tokens that flattened row r sees (sparse_attn_indexer page, forward_cpu
 * decode branch: a 2-D seq_lens is [batch, next_n] per-row lengths; the
 * varlen decode rows each carry their own causal length). For a 1-D length
 * per batch entry with next_n > 1, row j of entry b sees len[b] - next_n + j + 1
 * tokens (its own position in the speculative window). */
static int64_t visible(const int32_t *lens, int lens_2d, int next_n, int r)
{
    int64_t v;
    if (lens_2d || next_n == 1)
        v = lens[r];
    else
        v = (int64_t)lens[r / next_n] - next_n + (r % next_n) + 1;
    return v < 0 ? 0 : v;
}

/* The visible length of every row [0, rows), by the rule above: the row's
 * last unmasked column plus one, so the bound a top-k over the row takes. */
void pml_oracle_visible_lengths(const int32_t *lens, int lens_2d, int next_n, int rows, int64_t *out)
{
    for (int r = 0; r < rows; ++r)
        out[r] = visible(lens, lens_2d, next_n, r);
}

/* Element d of head h of one query row. fp8 q (qsrow NULL): the e4m3 code.
 * fp4 q (the indexer's FP4 path passes q as a (values, scales) pair,
 * sparse_attn_indexer page, forward_cuda; the layout read here is the
 * library's: the MXFP4 key layout applied to q): values [H][D/2] packed e2m1,
 * element 2i in the low nibble of byte i, and scales [H][D/32] e8m0, one per
 * 32 consecutive elements. */
static double q_elem(const uint8_t *qrow, const uint8_t *qsrow, int D, int h, int d)
{
    if (!qsrow)
        return FP8[qrow[(size_t)h * D + d]];
    uint8_t byte = qrow[(size_t)h * (D / 2) + d / 2];
    uint8_t nib = (d % 2 == 0) ? (byte & 15) : (byte >> 4);
    return E2M1[nib] * E8M0[qsrow[(size_t)h * (D / 32) + d / 32]];
}

/* One score: sum_h w[h] * max(0, sum_d q^[h,d] * k^[s,d]). */
static double score_paged(const uint8_t *qrow, const uint8_t *qsrow, const float *wrow, int H, int D,
                          const uint8_t *page, int kv_format, int block_kv, int slot)
{
    double total = 0.0;
    for (int h = 0; h < H; ++h) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += q_elem(qrow, qsrow, D, h, d) *
                   key_elem(page, kv_format, block_kv, D, slot, d);
        total += (double)wrow[h] * (dot > 0.0 ? dot : 0.0);
    }
    return total;
}

/* Paged logits (fp8_fp4_paged_mqa_logits as called from _varlen_decode_rows,
 * and fp8_paged_mqa_logits_cpu in forward_cpu, which reads the cache through
 * the page table with an explicit page stride).
 *   q          fp8 e4m3 codes [rows][H][D]; with q_scale, packed e2m1
 *              [rows][H][D/2] and q_scale e8m0 [rows][H][D/32] (q_elem)
 *   w          float [rows][H]
 *   kv_cache   num_pages pages, page p at kv_cache + p * page_stride
 *   lens       int32 [rows] (next_n == 1), [rows/next_n] (1-D, next_n > 1)
 *              or [rows] read as [B][next_n] (lens_2d)
 *   block_table int32 [rows/next_n][bt_ld]; row r uses row r / next_n
 * Writes out[i][c - col_begin] for rows row_list[i] and columns
 * [col_begin, col_end): the score for c < visible(r), else -inf. Blocks that
 * are visible but whose table entry is outside [0, num_pages) give NaN. */
void pml_oracle_paged_logits(const uint8_t *q, const uint8_t *q_scale, int H, int D, const float *w,
                             const uint8_t *kv_cache, int kv_format, int block_kv,
                             int64_t page_stride, int64_t num_pages,
                             const int32_t *lens, int lens_2d, int next_n,
                             const int32_t *block_table, int64_t bt_ld,
                             const int32_t *row_list, int n_list,
                             int col_begin, int col_end, double *out)
{
    int ncol = col_end - col_begin;
    int64_t cells = (int64_t)n_list * ncol;
    init_tables();
#pragma omp parallel for schedule(dynamic, 256)
    for (int64_t cell = 0; cell < cells; ++cell) {
        int i = (int)(cell / ncol);
        int c = col_begin + (int)(cell % ncol);
        int r = row_list[i];
        double val;
        if (c >= visible(lens, lens_2d, next_n, r)) {
            val = -INFINITY;
        } else {
            int32_t page = block_table[(int64_t)(r / next_n) * bt_ld + c / block_kv];
            if (page < 0 || page >= num_pages)
                val = NAN;
            else
                val = score_paged(q_scale ? q + (size_t)r * H * (D / 2) : q + (size_t)r * H * D,
                                  q_scale ? q_scale + (size_t)r * H * (D / 32) : NULL, w + (size_t)r * H, H, D,
                                  kv_cache + (size_t)page * page_stride, kv_format,
                                  block_kv, c % block_kv);
        }
        out[cell] = val;
    }
}

/* Non-paged (ragged prefill) logits, mqa_logits: a dense [M][N] matrix whose
 * row r is scored on keys [ks[r], ke[r]) and -inf elsewhere (sparse_attn_indexer
 * page: forward_cpu prefill branch, lengths ke - ks; the dense M*N logits
 * tensor the chunking bounds).
 *   q fp8 codes [M][H][D]; k fp8 codes [N][D]; k_scale float [N]; w float [M][H]. */
void pml_oracle_ragged_logits(const uint8_t *q, int H, int D, const float *w,
                              const uint8_t *k, const float *k_scale, int N,
                              const int32_t *ks, const int32_t *ke,
                              const int32_t *row_list, int n_list,
                              int col_begin, int col_end, double *out)
{
    int ncol = col_end - col_begin;
    int64_t cells = (int64_t)n_list * ncol;
    init_tables();
#pragma omp parallel for schedule(dynamic, 256)
    for (int64_t cell = 0; cell < cells; ++cell) {
        int i = (int)(cell / ncol);
        int n = col_begin + (int)(cell % ncol);
        int r = row_list[i];
        double val = -INFINITY;
        if (n >= ks[r] && n < ke[r] && n < N) {
            double total = 0.0;
            for (int h = 0; h < H; ++h) {
                double dot = 0.0;
                for (int d = 0; d < D; ++d)
                    dot += FP8[q[((size_t)r * H + h) * D + d]] *
                           ((double)k_scale[n] * FP8[k[(size_t)n * D + d]]);
                total += (double)w[(size_t)r * H + h] * (dot > 0.0 ? dot : 0.0);
            }
            val = total;
        }
        out[cell] = val;
    }
}

/* ---- top-k per row ------------------------------------------------------ */

typedef struct {
    double v;
    int32_t i;
} cand_t;

/* Order: larger value first; equal values by lower index (a stable top-k).
 * -0.0 equals +0.0 under C's comparison. NaN sorts after every number. */
static int cand_cmp(const void *a, const void *b)
{
    const cand_t *x = (const cand_t *)a, *y = (const cand_t *)b;
    int xn = isnan(x->v), yn = isnan(y->v);
    if (xn != yn)
        return xn - yn;
    if (!xn && x->v > y->v)
        return -1;
    if (!xn && x->v < y->v)
        return 1;
    return (x->i > y->i) - (x->i < y->i);
}

static int idx_cmp(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/* top_k_per_row (the indexer's selector: k largest logits of each row among
 * its valid columns; int32 positions relative to the row start; -1 padding
 * when the row has fewer than k valid columns, as forward_cpu presets the
 * output to -1).
 *   scores  double [rows][ld]; row r's candidates are columns [ks[r], ke[r])
 *   out     int32 [rows][k]: the selected positions minus ks[r] in ascending
 *           order, then -1. */
void pml_oracle_topk(const double *scores, int rows, int64_t ld,
                     const int32_t *ks, const int32_t *ke, int k, int32_t *out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < rows; ++r) {
        /* Row bounds outside the row are clamped: the start to [0, ld], the
         * end to [start, ld]; positions count from the clamped start. The
         * pages only ever pass in-range bounds (forward_cpu reads
         * logits[r, ks:ke]); clamping is the reading that keeps every read
         * inside the row, and the pack below uses the same rule. */
        int64_t lo = ks ? ks[r] : 0;
        lo = lo < 0 ? 0 : (lo > ld ? ld : lo);
        int64_t hi = ke[r];
        hi = hi < lo ? lo : (hi > ld ? ld : hi);
        int n = (int)(hi - lo);
        cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (n > 0 ? n : 1));
        int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (k > 0 ? k : 1));
        for (int j = 0; j < n; ++j) {
            c[j].v = scores[(int64_t)r * ld + lo + j];
            c[j].i = j;
        }
        qsort(c, n, sizeof(cand_t), cand_cmp);
        int m = n < k ? n : k;
        for (int j = 0; j < m; ++j)
            sel[j] = c[j].i;
        qsort(sel, m, sizeof(int32_t), idx_cmp);
        for (int j = 0; j < k; ++j)
            out[(int64_t)r * k + j] = j < m ? sel[j] : -1;
        free(c);
        free(sel);
    }
}

int pml_oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the parallel loops above from now on (n >= 1). */
void pml_oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n < 1 ? 1 : n);
#else
    (void)n;
#endif
}

/* ---- exact merge of per-shard top-k candidates ---------------------------
 *
 * Decode context parallelism shards each request's key tokens over `world`
 * ranks. Every rank scores its shard, takes a local top-k, and ships
 * (score, global token id) pairs as float32; a stable top-k over all ranks'
 * candidates gives the global top-k ("vllm.model_executor.layers.
 * sparse_attn_indexer", _merge_dcp_topk_global). Nothing is lost: a token of
 * the global top-k has fewer than k tokens ahead of it overall, hence fewer
 * than k on its own rank, so it is in that rank's local top-k.
 *
 * Token placement (a reading: the pages name only the interleave size): runs
 * of `interleave` consecutive tokens go to ranks 0, 1, ..., world - 1 in turn,
 * so local position p of rank r holds global token
 *     (p / interleave) * world * interleave + r * interleave + p % interleave.
 */
int64_t pml_oracle_dcp_global_id(int64_t p, int rank, int world, int interleave)
{
    return (p / interleave) * (int64_t)world * interleave + (int64_t)rank * interleave + p % interleave;
}

/* Pack one rank's candidates (the page's pack step). For row r and slot j,
 * idx = topk[r * topk_ld + j] is a local position relative to the row's
 * start ks[r] (0 without ks; clamped to [0, ld]); it is a candidate when
 * 0 <= idx < ld - ks[r],
 * and then packed[r][j] = (logits[r][ks[r] + idx], global id of idx as a
 * float). Any other idx (the -1 padding) packs as (-inf, -1).
 *   packed  float [rows][k][2] */
void pml_oracle_dcp_pack(const float *logits, int rows, int64_t ld, const int32_t *ks,
                         const int32_t *topk, int64_t topk_ld, int k, int rank, int world,
                         int interleave, float *packed)
{
    for (int r = 0; r < rows; ++r) {
        int64_t lo = ks ? ks[r] : 0;
        lo = lo < 0 ? 0 : (lo > ld ? ld : lo); /* the top-k's bound rule: starts clamped to [0, ld] */
        for (int j = 0; j < k; ++j) {
            int64_t idx = topk[(int64_t)r * topk_ld + j];
            float *o = packed + ((int64_t)r * k + j) * 2;
            if (idx >= 0 && lo + idx < ld) {
                o[0] = logits[(int64_t)r * ld + lo + idx];
                o[1] = (float)pml_oracle_dcp_global_id(idx, rank, world, interleave);
            } else {
                o[0] = -INFINITY;
                o[1] = -1.0f;
            }
        }
    }
}

/* Stable top-k over the gathered candidates (the page's merge step).
 *   gathered  float [world][rows][k][2] (score, id), rank-major as the
 *             all-gather along dim 0 leaves it
 *   out       int32 [rows][k]
 * A pair is a candidate when its id field f satisfies 0 <= f < 2^24 (every
 * integer there is exact in float32); its id is f truncated to an integer.
 * Candidates are ordered as in pml_oracle_topk (larger score first, NaN after
 * every number, equal scores by lower id), the first k are kept, and row r
 * of out holds their ids in ascending order, then -1. */
void pml_oracle_dcp_merge(const float *gathered, int world, int rows, int k, int32_t *out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < rows; ++r) {
        int64_t cap = (int64_t)world * k;
        cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (cap > 0 ? cap : 1));
        int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (k > 0 ? k : 1));
        int n = 0;
        for (int w = 0; w < world; ++w)
            for (int j = 0; j < k; ++j) {
                const float *p = gathered + (((int64_t)w * rows + r) * k + j) * 2;
                if (p[1] >= 0.0f && p[1] < 16777216.0f) {
                    c[n].v = p[0];
                    c[n].i = (int32_t)p[1];
                    ++n;
                }
            }
        qsort(c, n, sizeof(cand_t), cand_cmp);
        int m = n < k ? n : k;
        for (int j = 0; j < m; ++j)
            sel[j] = c[j].i;
        qsort(sel, m, sizeof(int32_t), idx_cmp);
        for (int j = 0; j < k; ++j)
            out[(int64_t)r * k + j] = j < m ? sel[j] : -1;
        free(c);
        free(sel);
    }
}
