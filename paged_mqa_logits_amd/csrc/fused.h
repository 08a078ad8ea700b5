// Internal interfaces between the kernels of the fused logits + top-k call:
// the per-row top-k launcher (with a skip mask for rows already done) and the
// selection from a row's candidate list.
#pragma once
#include "pml_device.h"

namespace pml {

struct TopkArgs {
    const void *logits;  // fp32, or bf16 bits when bf16 is set
    int64_t ld;
    const int32_t *ks;
    const int32_t *ke;
    int next_n;
    int k;
    int max_width;
    int32_t *out;
    int64_t out_ld;
    const int32_t *skip;  // rows r with skip[r] != 0 are left as they are (NULL: none)
    int bf16;             // the logits are bf16 bits (uint16_t), not fp32
};

// Per-row top-k over the logits (top_k_per_row's kernels).
int launch_topk(const TopkArgs &a, int num_rows, hipStream_t st);

// Candidate capacity per row of the fused call: twice the count its threshold
// aims at.
constexpr int kCandPerK = 4;
constexpr int kSelectMaxBlocks = 4096;  // rows with more key blocks take the full top-k

// Top-k from each row's candidates: for every block b < ceil(width[r] /
// bkv) of row r, count[r][b] (score, column as a float) pairs at cand[r][b *
// bkv ...], that together hold every column of the row scoring at or above a
// threshold. Row r is done here when width[r] <= k (its columns in order) or
// k <= (candidates) <= cap (the k best, columns ascending); done[r] says which
// (1) or that the row needs the full top-k (0).
struct CandSelectArgs {
    const float *cand;
    const int32_t *count;
    const int32_t *width;
    int64_t count_ld, cand_ld;
    int bkv;
    int cap;
    int k;
    int32_t *out;
    int64_t out_ld;
    int32_t *done;
};
int launch_cand_select(const CandSelectArgs &a, int num_rows, hipStream_t st);

}  // namespace pml
