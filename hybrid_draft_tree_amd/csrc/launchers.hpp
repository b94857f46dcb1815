// Internal launch functions shared by the C-ABI layer (graft_api.hip) and the
// kernel translation units.  Arguments are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "graft.h"

namespace graft {

// ---- tree build (tree_kernels.hip) --------------------------------------------------
void launch_prune(int B, int Nd, int mode, const int32_t *parent, const int32_t *layer,
                  const float *score, const graft_prune_cfg &cfg, int32_t *stage, int32_t *n_keep,
                  uint8_t *keep, float *cum_out, hipStream_t s);

void launch_retrieve(int B, int V, int k, int mode, int slots, const int32_t *table,
                     const int32_t *root_tok, const int32_t *n_keep, const int32_t *d_tok, int Nd,
                     int tpl_size, const int32_t *tpl_parent, const int32_t *tpl_rank,
                     const int32_t *tpl_depth, int32_t *ret_tok, int32_t *ret_parent,
                     int32_t *n_ret, int r_out, hipStream_t s);

void launch_flatten(int B, int Nd, int T1, int layout, const int32_t *root_tok,
                    const int32_t *base_pos, const int32_t *d_tok, const int32_t *d_parent,
                    const uint8_t *keep, const int32_t *n_keep, const int32_t *ret_tok,
                    const int32_t *ret_parent, const int32_t *n_ret, int r_out, int32_t *tok,
                    int32_t *parent, int32_t *depth, int32_t *pos_id, uint64_t *anc,
                    hipStream_t s);

// ---- row-wise top-k (topk_kernels.hip) ----------------------------------------------
struct TopkPlan {
    int64_t n_rows = 0;
    int V = 0;
    int splits = 1;     // wave ranges per row
    int chunk = 0;      // elements per range (multiple of 8)
    size_t partial_bytes = 0;
    size_t stats_bytes = 0;
};

TopkPlan plan_topk(int64_t n_rows, int V, int dtype);

// Phase A: per-range top-8 candidates (and softmax statistics when want_prob).
// Phase B: merge per row into topk [n_rows, k] (+ probabilities).
void launch_topk(const TopkPlan &plan, int dtype, const void *logits, int k, int32_t *topk,
                 float *prob, void *ws, hipStream_t s);

// ---- verify / update (verify_kernels.hip) -------------------------------------------
void launch_accept(int B, int T1, int k, const int32_t *topk, const int32_t *tok,
                   const int32_t *parent, const int32_t *depth, int32_t *accept_len,
                   int32_t *accept_idx, int dmax, int32_t *bonus, int32_t *base_pos_io,
                   hipStream_t s);

void launch_update(int64_t n_rows, int V, int k, const int32_t *topk, const float *prob,
                   const int32_t *row_tok, int32_t *table, float *table_prob, hipStream_t s);

}  // namespace graft
