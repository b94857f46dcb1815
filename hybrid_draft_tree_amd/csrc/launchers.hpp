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

// ---- row-wise top-k + fused acceptance walk (topk_kernels.hip) ----------------------
struct TopkPlan {
    int64_t n_rows = 0;
    int V = 0;
    int splits = 1;     // wave ranges per row
    int chunk = 0;      // elements per range (multiple of 8)
    size_t partial_bytes = 0;
    size_t stats_bytes = 0;
    size_t off_stats = 0;     // workspace offsets
    size_t off_counters = 0;
    size_t ws_bytes = 0;      // bytes of workspace the kernel uses (zeroed counters inside)
};

TopkPlan plan_topk(int64_t n_rows, int V, int dtype);

struct TopkArgs {
    const void *logits;
    int64_t n_rows;
    int V, S, chunk;
    uint64_t *partials;
    float2 *stats;
    uint32_t *row_cnt;
    int k;
    int32_t *topk;
    float *prob;
};

struct VerifyArgs {
    int T1 = 0;
    const int32_t *tok = nullptr;
    const int32_t *parent = nullptr;
    const int32_t *depth = nullptr;
    int32_t *accept_len = nullptr;
    int32_t *accept_idx = nullptr;
    int dmax = 0;
    int32_t *bonus = nullptr;
    int32_t *base_pos_io = nullptr;
    uint32_t *req_cnt = nullptr;
};

// Row-wise top-k of logits [n_rows, V] into topk [n_rows, k] (+ probabilities);
// with `verify` the acceptance walk of every request (n_rows = B * verify->T1)
// runs in the same launch.  The workspace counters must be zero on entry and
// are zero again on exit.
void launch_topk(const TopkPlan &plan, int dtype, const void *logits, int k, int32_t *topk,
                 float *prob, void *ws, const VerifyArgs *verify, hipStream_t s);

// ---- matrix update (verify_kernels.hip) ---------------------------------------------
void launch_update(int64_t n_rows, int V, int k, const int32_t *topk, const float *prob,
                   const int32_t *row_tok, int32_t *table, float *table_prob, hipStream_t s);

}  // namespace graft
