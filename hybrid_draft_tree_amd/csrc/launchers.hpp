// Internal launch interface shared by the C-ABI layer (graft_api.hip) and the
// kernel translation units.  Arguments are validated by the caller; every
// struct is passed to its kernel by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "graft.h"

namespace graft {

// ---- tree build (tree_kernels.hip) --------------------------------------------------
struct PruneKernelArgs {
    int B, Nd, mode;
    const int32_t *parent, *layer;
    const float *score;
    graft_prune_cfg cfg;
    int32_t *stage, *n_keep;
    uint8_t *keep;
    float *cum_out;
};

struct CkptStatsArgs {
    int B, Nd;
    const int32_t *parent, *layer;
    const float *score;
    int32_t ckpt_layer[3], keep[3];
    float *out;  // [B, 3]
};

struct CalibArgs {
    int64_t n;
    const float *samples;  // [n, 3], NaN = not recorded
    float q[3];
    float *log_thr;        // [3]
};

struct RetrieveKernelArgs {
    int B, V, k, mode, slots;
    const int32_t *table, *root_tok, *n_keep, *d_tok;
    int Nd;
    int tpl_size;
    const int32_t *tpl_parent, *tpl_rank, *tpl_depth;
    int32_t *ret_tok, *ret_parent, *n_ret;
    int r_out;
};

struct FlattenKernelArgs {
    int B, Nd, T1, layout;
    const int32_t *root_tok, *base_pos, *d_tok, *d_parent;
    const uint8_t *keep;
    const int32_t *n_keep, *ret_tok, *ret_parent, *n_ret;
    int r_out;
    int32_t *tok, *parent, *depth, *pos_id;
    uint64_t *anc;
    uint8_t *row_src;  // nullable
};

struct BuildKernelArgs {
    int B, Nd, T1, mode, layout, slots, V, k;
    graft_prune_cfg cfg;
    int tpl_size;
    const int32_t *tpl_parent, *tpl_rank, *tpl_depth;
    const int32_t *table, *root_tok, *base_pos;
    const int32_t *d_parent, *d_layer;
    const float *d_score;
    const int32_t *d_tok;
    int32_t *stage, *n_keep;
    uint8_t *keep;
    float *cum_out;
    int32_t *ret_tok, *ret_parent, *n_ret;
    int r_out;
    int32_t *tok, *parent, *depth, *pos_id;
    uint64_t *anc;
    uint8_t *row_src;  // nullable
    int pre;           // TREE: ret_tok / ret_parent / n_ret already hold the whole template
};

void launch_prune(const PruneKernelArgs &a, hipStream_t s);
void launch_ckpt_stats(const CkptStatsArgs &a, hipStream_t s);
void launch_calibrate(const CalibArgs &a, hipStream_t s);
void launch_retrieve(const RetrieveKernelArgs &a, hipStream_t s);
void launch_flatten(const FlattenKernelArgs &a, hipStream_t s);
void launch_build(const BuildKernelArgs &a, hipStream_t s);

// ---- row-wise top-k + fused acceptance walk / matrix update (topk_kernels.hip) ------
// The first kCounterBytes of every top-k workspace hold, for rows below
// kTagRows, the rows' tagged completion words (launch counter << 32 | greedy
// token + 1) and the coordinators' launch counter per row.  Unlike the rest of
// the workspace these words are not cleared: each launch advances both counters
// of its rows by one, so a completion word is current iff its counter is the
// one the coordinator expects, and no coordinator has to wait for a row only to
// clear its word.  They sit at the same place whatever the launch's size, so
// calls of any size can share one workspace.
constexpr int64_t kTagRows = 16384;
constexpr size_t kCounterBytes = (size_t)kTagRows * (sizeof(uint64_t) + sizeof(uint32_t));

struct TopkPlan {
    int64_t n_rows = 0;
    int V = 0;
    int splits = 1;           // wavefronts per row (one workgroup per row), plain launches
    int dtype = 0;            // GRAFT_DTYPE_*
    size_t off_counters = 0;  // untagged completion words [n_rows] (after the kCounterBytes of tagged ones)
    size_t off_occ = 0;       // last holder per token [V], one spare word, hand-offs [n_rows]
    int groups = 1;           // workgroups per row (rows split when there are few of them)
    int loads = 2;            // 1 KB blocks per wave per batch (2 or 4)
    int merge_wave = 0;       // 1: a merge wavefront per row beside the `splits` streaming waves
    size_t off_cnt = 0;       // groups > 1: arrival counters [n_rows], slice results [n_rows, groups]
    size_t off_part = 0;
    size_t off_pstat = 0;
    size_t ws_bytes = 0;      // workspace bytes the kernel uses (zero between calls past kCounterBytes)
};

TopkPlan plan_topk(int64_t n_rows, int V, int dtype);
// Launches of merge-wave rows with the matrix update, at most kScanRows rows:
// each row finds whether it is its token's last holder by comparing its token
// with the later rows' tokens, which its merge wave loads into registers (at
// most 16 per lane) near its start and compares at its end, so no registration
// workgroup, hand-off word or atomic is needed.
constexpr int kScanRegs = 16;
constexpr int64_t kScanRows = 64 * kScanRegs + 1;
inline bool scans_holders(const TopkPlan &p) { return p.merge_wave && p.n_rows > 0 && p.n_rows <= kScanRows; }

// A verify launch of this plan tags its completion words with the per-row
// launch counters (at most kTagRows rows).
inline bool uses_launch_counters(const TopkPlan &p) { return p.n_rows > 0 && p.n_rows <= kTagRows; }
int coord_groups(const TopkPlan &plan, int B);  // coordinator workgroups of a verify launch of B requests

struct TopkArgs {
    const void *logits;
    int64_t n_rows;
    int V, S;
    int k;
    int32_t *topk;
    float *prob;   // nullable: softmax probability of each top-k id
    float *stats;  // nullable: per row (largest value, sum of exp(value - largest))
    // rows split over `groups` workgroups (groups > 1): per-row arrival counters,
    // each slice's top-8 (row ranks) and softmax statistics (largest value and
    // sum packed in one word), all in the workspace, zero between calls
    int groups;
    int loads;  // 1 KB blocks per wave per batch: selects the kernel instantiation
    int merge_wave;  // 1: S streaming wavefronts and a merge wavefront per row
    uint32_t *cnt;
    uint64_t *part;
    uint64_t *pstat;
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
    int32_t *done = nullptr;       // [n_rows] completion words (greedy token + 1), zero between calls
    // tagged completion words [kTagRows] (launch counter << 32 | greedy token + 1)
    // and the coordinators' launch counters [kTagRows], kept between calls; set
    // (instead of `done`) for launches of at most kTagRows rows
    uint64_t *tag_done = nullptr;
    uint32_t *tag_want = nullptr;
    // fused matrix update (table != nullptr)
    int32_t *table = nullptr;
    float *table_prob = nullptr;
    int32_t *last_occ = nullptr;   // [V] row+1 of the last row holding each token
    uint32_t *handoff = nullptr;   // [n_rows] row-done / registration-done hand-off
    int B = 0;
    int ncoord = 0;                // coordinator workgroups (one wavefront per request)
    int update_only = 0;           // no requests: the matrix update alone (one registration workgroup)
    int scan_holders = 0;          // rows find their token's last holder by scanning (no registration)
};

// Row-wise top-k of logits [n_rows, V] into topk [n_rows, k] (+ probabilities);
// with `verify` the acceptance walk of every request (n_rows = B * verify->T1)
// runs in the same launch, and with verify->table the matrix update too.  The
// workspace past its first kCounterBytes must be zero on entry and is zero
// again on exit; the first kCounterBytes (zero once) carry launch counters.
void launch_topk(const TopkPlan &plan, int dtype, const void *logits, int k, int32_t *topk,
                 float *prob, float *stats, void *ws, const VerifyArgs *verify, hipStream_t s);

// ---- matrix update (verify_kernels.hip) ---------------------------------------------
void launch_update(int64_t n_rows, int V, int k, const int32_t *topk, const float *prob,
                   const int32_t *row_tok, int32_t *table, float *table_prob, hipStream_t s);

// ---- zero fill of a device range, bytes a multiple of 16 (verify_kernels.hip) -------
void launch_zero(void *p, size_t bytes, hipStream_t s);

// ---- streaming read of n_rows rows of row_bytes (a multiple of 16) bytes, one XOR
// word per row into sink: the read ceiling of the verify launch's geometry ---------
void launch_stream_read(const void *data, int64_t n_rows, int64_t row_bytes, uint32_t *sink, hipStream_t s);

// ---- coverage gain (verify_kernels.hip) ---------------------------------------------
struct CoverageArgs {
    int B, T1, V, dtype;
    const void *logits;
    const int32_t *tok, *parent;
    const uint8_t *row_src;
    const float *row_stats;
    float *gain;
};
void launch_coverage(const CoverageArgs &a, hipStream_t s);

}  // namespace graft
