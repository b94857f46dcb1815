/*
 * graft.h -- C ABI of the Graft per-step hot path on AMD Instinct MI355X (gfx950).
 *
 * Graft ("精简草稿，增强检索：投机解码的混合树构建", arXiv 2605.20104) prunes a
 * speculative draft tree at confidence checkpoints, fills the freed
 * verification slots with tokens retrieved from a GPU-resident continuation
 * matrix (V rows x k successor ids), verifies the hybrid tree greedily against
 * the target and then writes the target's top-k at every verified position
 * back into the matrix.  Section numbers below refer to the Chinese news
 * write-up of the paper: section 二 ("three gears") describes every step,
 * section 四 the batched static-slot serving variant and long context,
 * section 七 the DFlash TAIL variant.
 *
 * Conventions (all entry points):
 *  - Array arguments are DEVICE pointers owned by the caller unless marked
 *    "host".  The library never allocates, frees or retains them.  Scratch
 *    comes from a caller workspace sized by graft_workspace_bytes(): it must
 *    be zero-filled once after allocation.  Its first GRAFT_WS_COUNTER_BYTES
 *    hold per-row launch counters that carry over from call to call (each
 *    verify call advances those of its rows); every call leaves the rest
 *    zero-filled again.  Zero-filling the whole workspace again between calls
 *    is always allowed (it resets the counters together).  Calls of any size
 *    may share one workspace; calls that share it must be ordered (same
 *    stream).
 *  - Work is enqueued asynchronously on `stream`; nothing is synchronised.
 *    Calls on different streams touching disjoint buffers are independent.
 *  - Return value: GRAFT_OK, or a negative status.  Arguments are validated
 *    on the host before anything is enqueued; on an error nothing is
 *    enqueued.  GRAFT_EDEVICE reports a launch failure (hipGetLastError).
 *  - Device-side data preconditions (token ids in [0, V), parents before
 *    children, log-probs finite) are the caller's; no NaN is handled.
 *    graft_check_draft / graft_check_tree test them on the device.
 *  - Row-major layouts throughout; "[B, T1]" means B*T1 contiguous elements.
 *  - The continuation matrix is int32 [V, k]; only graft_update_topk and
 *    graft_verify_update write it.
 */
#ifndef GRAFT_H
#define GRAFT_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GRAFT_OK 0
#define GRAFT_EINVAL (-1)       /* null/misaligned pointer, bad size or shape */
#define GRAFT_EUNSUPPORTED (-2) /* unknown dtype, mode or layout */
#define GRAFT_EDEVICE (-3)      /* the HIP runtime reported a launch error */
#define GRAFT_ESCRATCH (-4)     /* graft_verify_update_noalloc: sizes beyond its static scratch */

#define GRAFT_DTYPE_F32 0
#define GRAFT_DTYPE_BF16 1

#define GRAFT_MODE_TREE 0 /* autoregressive draft tree (section 二) */
#define GRAFT_MODE_TAIL 1 /* 16-token DFlash block, tail replaced (section 七) */

#define GRAFT_LAYOUT_COMPACT 0  /* root, kept draft nodes ascending, retrieval in template order */
#define GRAFT_LAYOUT_IN_PLACE 1 /* static slots: draft slot i -> row i+1, vacated rows take retrieval */
#define GRAFT_LAYOUT_CHAIN 2    /* TAIL: root, kept block prefix, retrieval chain */

/* row_src codes: where a flattened row comes from */
#define GRAFT_ROW_ROOT 0      /* row 0: the last committed token */
#define GRAFT_ROW_DRAFT 1     /* a kept draft node */
#define GRAFT_ROW_RETRIEVED 2 /* a node grafted from the continuation matrix */
#define GRAFT_ROW_EMPTY 3     /* a slot nothing was placed in (token -1) */

#define GRAFT_MAX_ROWS 64 /* rows per request (root + candidate slots); one wavefront */
#define GRAFT_MAX_K 8     /* successors per matrix row */
#define GRAFT_MAX_VOCAB 1000000 /* logits per row for the top-k calls (at most 16 wavefronts per row) */
#define GRAFT_MAX_BATCH (1 << 24) /* requests per call (a launch's thread count is 32-bit); larger B: EINVAL */
#define GRAFT_WS_COUNTER_BYTES 196608u /* leading workspace bytes kept between calls: per-row launch counters */

/* Prune configuration (host POD).  Section 二, gear 1: checkpoints at draft
 * depths 0, 1 and 5 compare the best cumulative path confidence with a
 * calibrated threshold; a prune there keeps 8, 24 or 40 draft nodes of the
 * 60-slot budget.  log_thr[s] = (float)ln(tau_s).  tail_thr: the TAIL
 * confidence cut (0.5 in section 七). */
typedef struct graft_prune_cfg {
    int32_t ckpt_layer[3]; /* draft layers of the checkpoints; layer 0 = the root's children */
    float log_thr[3];      /* fire when best cumulative log-confidence < log_thr[s] (+inf: always,
                              -inf: never -- a fixed draft/retrieval split, section 五's ablation) */
    int32_t keep[3];       /* draft nodes kept when checkpoint s fires */
    float tail_thr;        /* TAIL: keep the longest prefix with confidence >= tail_thr */
    int32_t node_mode;     /* TREE: nonzero = per-node variant (section 四's static slots): keep
                              every node with cumulative log-confidence >= node_log_thr instead of
                              the checkpoints; stage 4 when a node is cut, else 3 */
    float node_log_thr;
} graft_prune_cfg;

/* Retrieval template (host struct holding DEVICE arrays of `size` entries), in
 * a master order such as graft_template_master()'s or
 * graft_template_branching()'s; a budget of R retrieval slots uses entries
 * 0..min(R, size)-1.  parent[t] < t is a template index, -1 for the root. */
typedef struct graft_template {
    int32_t size;
    const int32_t *parent; /* device [size] */
    const int32_t *rank;   /* device [size]: successor rank in the parent's matrix row, < k */
    const int32_t *depth;  /* device [size]: 1 for children of the root */
} graft_template;

/* graft_prune_select -- section 二, gear 1 (TREE); section 七 (TAIL).
 * TREE: per request b, cum[i] = cum[parent[i]] + score[i] in fp32 (score =
 *   draft log-probability, root = 0).  Checkpoint s fires when layer
 *   ckpt_layer[s] is non-empty, layers <= ckpt_layer[s] hold at least keep[s]
 *   nodes, and the maximum cum over that layer is < log_thr[s]; the first s
 *   that fires is the stage (3 = none).  Kept: the keep[s] nodes of layers
 *   <= ckpt_layer[s] with the largest cum (ties -> lower index); stage 3 keeps
 *   all Nd nodes.
 * TAIL: score = block confidence; n_keep = the longest prefix with
 *   score >= tail_thr; stage = 0 when the block is cut, else 3.
 *   d_parent/d_layer are ignored and may be NULL.
 * d_parent, d_layer: int32 [B, Nd], parent[i] in [-1, i).  d_score: fp32 [B, Nd].
 * cfg: host.  Outputs: stage int32 [B], n_keep int32 [B], keep uint8 [B, Nd]
 * (1 = kept), cum_out fp32 [B, Nd] (nullable; TREE only).
 * Requires 1 <= Nd <= 64, B >= 0 (B == 0 enqueues nothing). */
int graft_prune_select(int B, int Nd, int mode, const int32_t *d_parent, const int32_t *d_layer,
                       const float *d_score, const graft_prune_cfg *cfg, int32_t *stage,
                       int32_t *n_keep, uint8_t *keep, float *cum_out, hipStream_t stream);

/* Optional input checks.  The other calls assume the data preconditions
 * below and never read out of bounds when they fail, but then compute
 * nothing meaningful.  These write, per request b, status[b] = the OR of the
 * flags of the conditions that fail (0 = all hold); status int32 [B], device.
 *
 * graft_check_draft (inputs of graft_prune_select / graft_build_hybrid_tree):
 *   GRAFT_BAD_TOKEN d_tok outside [0, V); GRAFT_BAD_SCORE a TREE log-
 *   probability that is NaN or > 0, or a TAIL confidence NaN or outside
 *   [0, 1]; TREE only: GRAFT_BAD_PARENT d_parent[i] outside [-1, i);
 *   GRAFT_BAD_LAYER d_layer[i] != d_layer[parent] + 1 (0 for root
 *   children).  TAIL ignores d_parent / d_layer (may be NULL).
 * graft_check_tree (the flattened tree given to graft_verify_accept /
 *   graft_verify_update): row 0 is the root (token in [0, V), parent -1,
 *   depth 0); a row f >= 1 is either empty (token -1, parent -1, depth 0) or
 *   has a token in [0, V), a parent row in [0, f) that is not empty, and
 *   depth = parent's depth + 1 (GRAFT_BAD_TOKEN / GRAFT_BAD_PARENT /
 *   GRAFT_BAD_DEPTH).
 * Requires 1 <= Nd, T1 <= 64, V >= 1. */
#define GRAFT_BAD_PARENT 1
#define GRAFT_BAD_LAYER 2
#define GRAFT_BAD_SCORE 4
#define GRAFT_BAD_TOKEN 8
#define GRAFT_BAD_DEPTH 16
int graft_check_draft(int B, int Nd, int mode, int V, const int32_t *d_parent, const int32_t *d_layer,
                      const float *d_score, const int32_t *d_tok, int32_t *status, hipStream_t stream);
int graft_check_tree(int B, int T1, int V, const int32_t *tok, const int32_t *parent, const int32_t *depth,
                     int32_t *status, hipStream_t stream);

/* Threshold calibration -- section 二, gear 1: the checkpoint thresholds are
 * set from the confidence the drafter shows at each checkpoint over a few
 * warm-up rounds.  The pages give no rule; the one here is a quantile.
 *
 * graft_checkpoint_stats: per request b and checkpoint s, out[b, s] = the
 *   largest cumulative log-confidence (cum as in graft_prune_select) on layer
 *   cfg->ckpt_layer[s], or NaN when that checkpoint is not reached (its layer
 *   is empty, or layers <= it hold fewer than cfg->keep[s] nodes).  All three
 *   are taken on the full tree, whether or not an earlier checkpoint would
 *   fire.  d_parent, d_layer int32 [B, Nd], d_score fp32 [B, Nd], out fp32
 *   [B, 3], all device; cfg host (only ckpt_layer and keep are read).
 *   Requires 1 <= Nd <= 64, B >= 0 (B == 0 enqueues nothing).
 *
 * graft_calibrate_thresholds: for each checkpoint s, log_thr[s] = the r-th
 *   smallest of the m non-NaN values in column s of samples, r = ceil(q[s] * m)
 *   computed in double (clamped to [1, m]), so the checkpoint fires
 *   (statistic < log_thr[s]) on fewer than a share q[s] of the samples;
 *   -inf (never fires) when q[s] == 0 or m == 0.  -0 and +0 count as one
 *   value (returned as +0).  samples fp32 [n, 3] device (rows of
 *   graft_checkpoint_stats outputs, NaN = not recorded); q host fp32 [3], each
 *   in [0, 1]; log_thr fp32 [3] device, ready for graft_prune_cfg.log_thr.
 *   0 <= n <= GRAFT_MAX_CALIB_SAMPLES.  One launch of 3 workgroups. */
#define GRAFT_MAX_CALIB_SAMPLES (1 << 26)
int graft_checkpoint_stats(int B, int Nd, const int32_t *d_parent, const int32_t *d_layer,
                           const float *d_score, const graft_prune_cfg *cfg, float *out,
                           hipStream_t stream);
int graft_calibrate_thresholds(int64_t n, const float *samples, const float *q, float *log_thr,
                               hipStream_t stream);

/* graft_template_master -- host only; section 二's stage-adaptive asymmetric
 * template and section 五's depth/width optimum (8, 8).  Writes the master
 * order into HOST arrays of capacity `cap`: the `width` children of the root
 * (rank j), then the rank-0 chain under rank 0 down to `depth`, then the other
 * chain nodes (rank j >= 1 continued by rank-0 successors to depth d >= 2) by
 * increasing j + d, ties by increasing j.  Budget R takes the first R entries,
 * so higher-ranked successors get longer chains.  Returns the node count
 * (min(cap, width*depth)) or GRAFT_EINVAL. */
int graft_template_master(int width, int depth, int cap, int32_t *parent, int32_t *rank,
                          int32_t *tdepth);

/* graft_template_branching -- host only; a branching form of section 二's
 * asymmetric template (better-ranked successors get more children and reach
 * deeper, after Token Recycling).  Nodes are rank paths (r_1..r_d), 1 <= d <=
 * depth, every r < width; cost = d*beta_den + beta_num*(r_1+..+r_d); the
 * master order is ascending (cost, d, ranks lexicographically), so beta =
 * beta_num/beta_den = 0 is breadth-first and a large beta approaches rank-0
 * chains.  Writes the first min(cap, all paths) nodes into HOST arrays and
 * returns their count, or GRAFT_EINVAL (width, depth >= 1, beta_num >= 0,
 * beta_den >= 1, cap >= 0).  With a matrix of k successors, width <= k. */
int graft_template_branching(int width, int depth, int beta_num, int beta_den, int cap, int32_t *parent,
                             int32_t *rank, int32_t *tdepth);

/* graft_retrieve_expand -- section 二, gear 2: one matrix row lookup per node,
 * GPU only.
 * TREE: R_b = min(slots - n_keep[b], tpl->size) retrieval nodes (a template
 *   smaller than the freed budget leaves the rest of it empty); node t reads
 *   ret_tok[t] = table[src][rank[t]] with src = root_tok[b] for root
 *   children, else ret_tok[parent[t]] (-1 below an out-of-range token or
 *   rank).  cfg (host) is used to check 0 <= slots - keep[s].  d_tok may be
 *   NULL.
 * TAIL: R_b = slots - n_keep[b]; a chain x <- table[x][0] of R_b steps from
 *   the last kept block token d_tok[b, n_keep-1] (root_tok[b] when n_keep is
 *   0); ret_parent[t] = t-1.  tpl and cfg may be NULL.
 * table int32 [V, k] (1 <= k <= 8); root_tok, n_keep int32 [B]; d_tok int32
 * [B, Nd].  Outputs: ret_tok, ret_parent int32 [B, r_out] (-1 beyond R_b),
 * n_ret int32 [B].  Requires r_out <= 64 and r_out >= the largest R_b.
 * TREE with n_keep == NULL: R_b = min(slots, tpl->size), the whole template
 * ahead of pruning (for graft_build_after_retrieval). */
int graft_retrieve_expand(int B, int V, int k, int mode, int slots, const int32_t *table,
                          const int32_t *root_tok, const int32_t *n_keep, const int32_t *d_tok,
                          int Nd, const graft_template *tpl, const graft_prune_cfg *cfg,
                          int32_t *ret_tok, int32_t *ret_parent, int32_t *n_ret, int r_out,
                          hipStream_t stream);

/* graft_build_tree_mask -- section 二, gear 3: flatten the hybrid tree into
 * one sequence, rebuild tree position ids and the attention mask.  Row 0 is
 * the root.  Layouts: GRAFT_LAYOUT_COMPACT, GRAFT_LAYOUT_IN_PLACE (section
 * 四: fixed slots per request, low-confidence draft slots replaced in place;
 * needs T1 == Nd + 1), GRAFT_LAYOUT_CHAIN (TAIL).  Every layout is
 * topological (parent row < child row).
 * Inputs: root_tok, base_pos int32 [B]; d_tok, d_parent int32 [B, Nd];
 * keep uint8 [B, Nd]; n_keep int32 [B]; ret_tok, ret_parent int32 [B, r_out];
 * n_ret int32 [B].  n_keep + n_ret <= T1 - 1 per request: rows nothing is
 * placed in are empty (token -1, parent -1, depth 0, mask = the row itself,
 * GRAFT_ROW_EMPTY).
 * Outputs [B, T1]: tok, parent (-1 at the root), depth, pos_id = base_pos +
 * depth (int32), anc (uint64: bit g set iff row g is an ancestor of the row or
 * the row itself), row_src (uint8, nullable: GRAFT_ROW_* of every row, the
 * input of graft_coverage_gain).  Requires 2 <= T1 <= 64, Nd <= 64,
 * r_out <= 64. */
int graft_build_tree_mask(int B, int Nd, int T1, int layout, const int32_t *root_tok,
                          const int32_t *base_pos, const int32_t *d_tok, const int32_t *d_parent,
                          const uint8_t *keep, const int32_t *n_keep, const int32_t *ret_tok,
                          const int32_t *ret_parent, const int32_t *n_ret, int r_out, int32_t *tok,
                          int32_t *parent, int32_t *depth, int32_t *pos_id, uint64_t *anc,
                          uint8_t *row_src, hipStream_t stream);

/* graft_verify_accept -- section 二, gear 3: strict greedy verification.
 * Row-wise top-k of logits [B, T1, V] (value descending, ties -> lower id,
 * -0 == +0; top-k of the softmax equals top-k of the logits), g = column 0.
 * A row is accepted iff every row on its path from the root (root excluded)
 * carries the token g of its parent row; the deepest accepted row wins, ties
 * -> lowest row.  Outputs: topk int32 [B, T1, k]; topk_prob fp32 [B, T1, k]
 * (nullable: softmax probability of each top-k id); accept_len int32 [B]
 * (candidate tokens accepted, root excluded); row_stats fp32 [B, T1, 2]
 * (nullable: per row the largest logit and the sum of exp(logit - largest),
 * the softmax normaliser, for graft_coverage_gain); accept_idx int32 [B, dmax]
 * (rows of the accepted path from depth 1, -1 padded); bonus int32 [B] (g at
 * the accepted row: the next root; `bonus` may alias the root buffer of the
 * next step); base_pos_io int32 [B] (nullable; += accept_len + 1).
 * tok, parent, depth: int32 [B, T1] from graft_build_tree_mask.  logits must
 * be 16-byte aligned.  ws: zero-filled device workspace (256-byte aligned) of
 * at least graft_workspace_bytes(B*T1, V, k, dtype) bytes.  One kernel launch:
 * one workgroup per row computes the top-k and publishes the row's greedy
 * token; a coordinating workgroup in the same launch runs each request's
 * acceptance walk as soon as all its rows are in.  accept_len[b] == -1 reports
 * a coordinator that gave up waiting (about a second; never in normal
 * operation): the outputs are then invalid and the workspace must be
 * zero-filled again.  Requires 1 <= T1 <= 64, 1 <= k <= 8, k <= V <= GRAFT_MAX_VOCAB,
 * dmax >= 0. */
int graft_verify_accept(int B, int T1, int V, int k, int dtype, const void *logits,
                        const int32_t *tok, const int32_t *parent, const int32_t *depth,
                        int32_t *topk, float *topk_prob, float *row_stats, int32_t *accept_len,
                        int32_t *accept_idx,
                        int dmax, int32_t *bonus, int32_t *base_pos_io, void *ws, size_t ws_bytes,
                        hipStream_t stream);

/* graft_update_topk -- section 二 gear 3 and section 六: online update of the
 * continuation matrix.  For every verified row P (accepted or rejected), in
 * increasing P, table[row_tok[P]] <- the row's top-k (the whole row is
 * overwritten); on a collision the highest P wins.  Either logits [n_rows, V]
 * (prompt ingest, section 四: the top-k is computed here) or topk_in int32
 * [n_rows, k] (the top-k graft_verify_accept already produced, so the logits
 * are read once per step) must be given; logits wins if both are.
 * table_prob fp32 [V, k] (nullable) receives the probabilities: from the
 * logits, or from prob_in fp32 [n_rows, k] (required then with topk_in).
 * row_tok int32 [n_rows].  topk_out int32 [n_rows, k] (nullable) receives the
 * top-k computed from `logits` (e.g. the last prompt row's greedy token is the
 * first decode root); ignored with topk_in.  ws as for graft_verify_accept
 * with n_rows rows.  With logits the update runs in the same launch as the
 * top-k (each row hands its result to the update as in graft_verify_update);
 * with topk_in it is a launch of its own.  Requires n_rows >= 0,
 * 1 <= k <= 8, k <= V <= GRAFT_MAX_VOCAB. */
int graft_update_topk(int64_t n_rows, int V, int k, int dtype, const void *logits,
                      const int32_t *topk_in, const float *prob_in, const int32_t *row_tok,
                      int32_t *table, float *table_prob, int32_t *topk_out, void *ws,
                      size_t ws_bytes, hipStream_t stream);

/* graft_build_hybrid_tree -- graft_prune_select, graft_retrieve_expand and
 * graft_build_tree_mask in one launch (one workgroup per request; the
 * retrieval chain runs in parallel with the pruning), with the same outputs
 * and the same preconditions.  Requires T1 == slots + 1; mode TREE pairs with
 * layout COMPACT or IN_PLACE, mode TAIL with layout CHAIN.  Section 二 (all
 * three gears); section 七 for TAIL; section 四 for the in-place layout. */
int graft_build_hybrid_tree(int B, int Nd, int T1, int mode, int layout, int slots,
                            const graft_prune_cfg *cfg, const graft_template *tpl, int V, int k,
                            const int32_t *table, const int32_t *root_tok, const int32_t *base_pos,
                            const int32_t *d_parent, const int32_t *d_layer, const float *d_score,
                            const int32_t *d_tok, int32_t *stage, int32_t *n_keep, uint8_t *keep,
                            float *cum_out, int32_t *ret_tok, int32_t *ret_parent, int32_t *n_ret,
                            int r_out, int32_t *tok, int32_t *parent, int32_t *depth, int32_t *pos_id,
                            uint64_t *anc, uint8_t *row_src, hipStream_t stream);

/* graft_build_after_retrieval -- graft_build_hybrid_tree with the retrieval
 * already done.  Section 二: retrieval depends only on the request's root
 * token and the matrix, so it can run while the drafter is still building the
 * tree, off the critical path.  ret_tok, ret_parent, n_ret (in/out) are as
 * graft_retrieve_expand writes them with n_keep == NULL: the whole template
 * from each root, computed before the draft exists, usually on another
 * stream that this call's stream waits for (an event).  This call prunes,
 * keeps the first R_b = min(slots - n_keep[b], n_ret[b]) retrieved nodes (the
 * template's master order makes every prefix a tree) and flattens, in one
 * launch; on return ret_tok / ret_parent hold -1 beyond R_b and n_ret[b] =
 * R_b, so every output equals graft_build_hybrid_tree's on the same inputs.
 * TREE only: layout COMPACT or IN_PLACE (a TAIL chain starts from the last
 * kept block token, known only after the prune -> GRAFT_EUNSUPPORTED).  Other
 * arguments and preconditions as graft_build_hybrid_tree. */
int graft_build_after_retrieval(int B, int Nd, int T1, int layout, int slots, const graft_prune_cfg *cfg,
                                const int32_t *root_tok, const int32_t *base_pos, const int32_t *d_parent,
                                const int32_t *d_layer, const float *d_score, const int32_t *d_tok,
                                int32_t *stage, int32_t *n_keep, uint8_t *keep, float *cum_out,
                                int32_t *ret_tok, int32_t *ret_parent, int32_t *n_ret, int r_out, int32_t *tok,
                                int32_t *parent, int32_t *depth, int32_t *pos_id, uint64_t *anc,
                                uint8_t *row_src, hipStream_t stream);

/* graft_verify_update -- graft_verify_accept followed by
 * graft_update_topk(row_tok = tok, topk_in = the top-k just computed) in one
 * launch: the logits are read once and the matrix is updated in the same
 * kernel (the coordinating workgroup registers every row's token first; each
 * row, once its top-k is known, writes it into the matrix row of its token if
 * it is the last holder of that token in the batch).  table int32 [V, k]
 * in/out; table_prob fp32 [V, k] (nullable; needs topk_prob).  Other
 * arguments and the accept_len == -1 report as for graft_verify_accept.
 * Section 二, gear 3; section 六 (online update). */
int graft_verify_update(int B, int T1, int V, int k, int dtype, const void *logits, const int32_t *tok,
                        const int32_t *parent, const int32_t *depth, int32_t *table, float *table_prob,
                        int32_t *topk, float *topk_prob, float *row_stats, int32_t *accept_len,
                        int32_t *accept_idx,
                        int dmax, int32_t *bonus, int32_t *base_pos_io, void *ws, size_t ws_bytes,
                        hipStream_t stream);

/* graft_verify_update_noalloc -- graft_verify_update without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * call allocates and frees nothing; its scratch is a static device array of
 * GRAFT_NOALLOC_SCRATCH_BYTES held by each GPU the library runs on until the
 * process ends (its address looked up once per device, on the device current
 * at the first call there).  Each call first clears the part it uses with a
 * fill kernel on `stream`, then runs the same launch as graft_verify_update.
 * All calls on one GPU share that array: calls that overlap on one GPU (other
 * streams, other host threads, without ordering between them) race and give
 * wrong results.  The scratch needed is the top-k launch's completion words,
 * one holder word per vocabulary entry and one hand-off word per row (plus
 * per-slice results when rows are split), about 4 * (V + 2 * B * T1) bytes:
 * sizes that need more than GRAFT_NOALLOC_SCRATCH_BYTES return
 * GRAFT_ESCRATCH and enqueue nothing (V = 151936 at B * T1 = 976 rows needs
 * about 0.6 MB).  Arguments, outputs and every other status are as for
 * graft_verify_update. */
#define GRAFT_NOALLOC_SCRATCH_BYTES (8u << 20)
int graft_verify_update_noalloc(int B, int T1, int V, int k, int dtype, const void *logits, const int32_t *tok,
                                const int32_t *parent, const int32_t *depth, int32_t *table, float *table_prob,
                                int32_t *topk, float *topk_prob, float *row_stats, int32_t *accept_len,
                                int32_t *accept_idx, int dmax, int32_t *bonus, int32_t *base_pos_io,
                                hipStream_t stream);

/* graft_coverage_gain -- section 三: what the grafted candidates add where
 * pruning cut.  For every row v of a request that has retrieved children, the
 * target's softmax probability (row v's logits) of the set of retrieved child
 * tokens that no kept draft child of v already carries (each token once, ids
 * outside [0, V) skipped), summed over v: gain fp32 [B].  Positive as soon as
 * one such token has nonzero probability; 0 when nothing was retrieved.
 * logits [B, T1, V] as verified; tok, parent, row_src [B, T1] from the build;
 * row_stats [B, T1, 2] from graft_verify_accept / graft_verify_update on the
 * same logits (so only the retrieved entries are read here).  One wavefront
 * per request, one launch.  Requires 1 <= T1 <= 64, V <= GRAFT_MAX_VOCAB. */
int graft_coverage_gain(int B, int T1, int V, int dtype, const void *logits, const int32_t *tok,
                        const int32_t *parent, const uint8_t *row_src, const float *row_stats,
                        float *gain, hipStream_t stream);

/* graft_stream_read -- a measurement aid, no part of the Graft step: the read
 * bandwidth the verify launch's geometry can reach on this device.  Reads
 * n_rows rows of row_bytes bytes (data, device, 16-byte aligned; row_bytes a
 * positive multiple of 16; rows contiguous) with one workgroup of four
 * wavefronts per row, 16-byte non-temporal loads in 1 KB blocks interleaved
 * over the wavefronts, two blocks per batch with the next batch in flight, and
 * writes the XOR of each row's 32-bit words to sink uint32 [n_rows] (so no load
 * is skipped, and the result can be checked).  One launch.  Requires
 * 0 <= n_rows <= 2^31 - 1; n_rows == 0 returns GRAFT_OK before any pointer is
 * looked at. */
int graft_stream_read(const void *data, int64_t n_rows, int64_t row_bytes, uint32_t *sink, hipStream_t stream);

/* Launch plan of the top-k launch of graft_verify_accept / graft_verify_update
 * (T1 = rows per request, n_rows = B * T1) or of graft_update_topk with logits
 * (T1 = 0: no requests; one registration workgroup unless holder_scan); host only, nothing is
 * enqueued.  A verify launch puts its coordinator workgroups (one wavefront
 * per request, at most GRAFT_MAX_COORD_GROUPS workgroups; each wavefront then
 * watches several requests in turn) ahead of the rows.  They wait for rows
 * that are dispatched after them, so their number is bounded whatever the
 * batch: GRAFT_MAX_COORD_GROUPS workgroups of at most 16 wavefronts take a
 * quarter of the chip's wavefront slots at most.  Returns GRAFT_OK, or
 * GRAFT_EINVAL for sizes the calls reject (out must be non-NULL; T1 in
 * [0, 64] dividing n_rows). */
#define GRAFT_MAX_COORD_GROUPS 128
typedef struct graft_plan {
    int32_t waves_per_group;  /* wavefronts per workgroup */
    int32_t groups_per_row;   /* workgroups per row (rows are cut into slices when few) */
    int32_t blocks_per_batch; /* 1 KB blocks each wavefront loads per batch */
    int32_t coord_groups;     /* coordinator (or registration) workgroups ahead of the rows */
    int64_t workgroups;       /* all workgroups of the launch */
    int32_t merge_wave;       /* 1: one wavefront of each row's workgroup merges, the others stream */
    int32_t launch_counters;  /* 1: the rows' completion words carry the workspace's per-row launch
                                 counters (verify launches of at most 16384 rows) */
    int32_t holder_scan;      /* 1: with the fused matrix update, each row finds whether it is its
                                 token's last holder by reading the later rows' tokens, with no
                                 registration workgroup (merge-wave launches of at most 1025 rows) */
} graft_plan;
int graft_launch_plan(int64_t n_rows, int V, int dtype, int T1, graft_plan *out);

/* Workspace bytes needed by graft_verify_accept / graft_verify_update /
 * graft_update_topk for n_rows rows of V logits (0 on invalid sizes).  Zero-fill it once after
 * allocating it; calls keep its first GRAFT_WS_COUNTER_BYTES as per-row launch counters and
 * leave the rest zero-filled.  Also 0 when n_rows rows do not fit one launch:
 * n_rows must be below 2^31 - 1, and (n_rows x workgroups per row + coordinator workgroups) x
 * wavefronts per workgroup x 64 threads below 2^32 (one wavefront per row from ~3000 rows on
 * at V <= 127 x 512 bf16, so up to ~67 million rows there; rows of larger V take more
 * wavefronts, up to 16 at V = 10^6).  Those three calls return GRAFT_EINVAL for such sizes:
 * split the rows over several calls. */
size_t graft_workspace_bytes(int64_t n_rows, int V, int k, int dtype);

/* Static description of a status code. */
const char *graft_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* GRAFT_H */
