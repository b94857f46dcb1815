/*
 * graft_oracle.c -- plain, slow CPU oracle for the Graft per-step path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no source,
 * header, table or helper with the HIP implementation.
 *
 * Source: "精简草稿，增强检索：投机解码的混合树构建" (arXiv 2605.20104), the
 * news write-up's section 二 ("three gears"): calibrated pruning at draft
 * checkpoints 0/1/5, the 8/52, 24/36, 40/20 slot splits, retrieval from a
 * GPU-resident continuation matrix through a stage-adaptive asymmetric
 * template, flatten + tree mask, strict greedy verification, and the online
 * matrix update at every verified position; section 七 for the DFlash TAIL
 * variant; section 四 (long context) for prompt ingest.
 *
 * Where the pages leave a step open, the reading taken is stated at that step.
 * Parity unpinned by the pages: the following readings are fixed by no worked
 * example, formula or table on the pages, so the tests pin them only through
 * invariants (budget split, superset and monotonicity of acceptance,
 * losslessness, closures) and through agreement with the GPU path -- which
 * draft nodes a prune keeps (top N by cumulative confidence among layers up
 * to the checkpoint, ties to the lower index); a checkpoint whose layer is
 * empty or too small is not reached; the static draft tree's layer sizes; the
 * rank-chain template and its master order; the flatten order of each layout;
 * static-slot replacement as the same stage logic; equally long accepted
 * paths resolved to the lowest row; the update overwriting whole rows for
 * every verified position, highest batch-wide position winning.
 * Every decision that floating point makes (stage, keep set, TAIL prefix) is
 * taken in fp32, the precision of the GPU kernels; top-k compares values as
 * reals (bf16/fp32 widened exactly to double); softmax probabilities are fp64.
 *
 * Plain loops throughout; the only parallelism is OpenMP over logit rows.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ODT_F32 0
#define ODT_BF16 1

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------- */
/* Gear 1: calibrated pruning (section 二).                                   */
/*                                                                           */
/* cum[i] = cum[parent] + logp[i] in fp32 (root contributes 0): the log of   */
/* the product of draft probabilities along the path.  Checkpoint s at draft */
/* layer c_s (layer 0 = the root's children) fires when the best cumulative  */
/* confidence on that layer is below log_thr[s] = (float) ln tau_s (taken   */
/* by the caller: tau 0 gives -inf, never fires; +inf always fires).         */
/* Checkpoints are taken in                                                  */
/* drafting order; the first that fires decides the stage.  Readings: a      */
/* checkpoint whose layer is empty, or whose layers 0..c_s hold fewer than   */
/* keep_s nodes, is not reached; the kept draft nodes are the keep_s nodes   */
/* of layers <= c_s with the highest cumulative confidence (ties -> lower    */
/* node index); with no prune every draft node is kept.                      */
/* ------------------------------------------------------------------------- */
/* node_tau > 0 selects the per-node variant instead of the checkpoints      */
/* (section 四's static slots, where draft nodes of low confidence give up   */
/* their slots):                                                             */
/* keep every node whose cumulative log-confidence is >= (float)ln node_tau, */
/* a set closed under ancestors since confidences only fall along a path;    */
/* stage 4 when a node was cut, else 3.                                      */
int oracle_prune_tree(int B, int Nd, const int32_t *parent, const int32_t *layer,
                      const float *logp, const int32_t *ckpt_layer, const float *log_thr,
                      const int32_t *keep_n, double node_tau, int32_t *stage, int32_t *n_keep,
                      uint8_t *keep, float *cum_out) {
    if (B < 0 || Nd <= 0) return -1;
    float *cum = (float *)malloc(sizeof(float) * (size_t)Nd);
    if (!cum) return -1;
    for (int b = 0; b < B; ++b) {
        const int32_t *par = parent + (size_t)b * Nd;
        const int32_t *lay = layer + (size_t)b * Nd;
        const float *lp = logp + (size_t)b * Nd;
        for (int i = 0; i < Nd; ++i) {
            if (par[i] >= i) {
                free(cum);
                return -1; /* nodes must come after their parents */
            }
            float base = (par[i] < 0) ? 0.0f : cum[par[i]];
            cum[i] = base + lp[i];
        }
        if (node_tau > 0.0) {
            float nthr = (float)log(node_tau);
            uint8_t *kp = keep + (size_t)b * Nd;
            int N = 0;
            for (int i = 0; i < Nd; ++i) {
                kp[i] = cum[i] >= nthr;
                N += kp[i];
            }
            stage[b] = N < Nd ? 4 : 3;
            n_keep[b] = N;
            if (cum_out)
                for (int i = 0; i < Nd; ++i) cum_out[(size_t)b * Nd + i] = cum[i];
            continue;
        }
        int st = 3;
        for (int s = 0; s < 3 && st == 3; ++s) {
            int c = ckpt_layer[s];
            int on_layer = 0, upto = 0;
            float best = -INFINITY;
            for (int i = 0; i < Nd; ++i) {
                if (lay[i] == c) {
                    on_layer++;
                    if (cum[i] > best) best = cum[i];
                }
                if (lay[i] <= c) upto++;
            }
            if (on_layer == 0 || upto < keep_n[s]) continue;
            if (best < log_thr[s]) st = s;
        }
        int N = (st < 3) ? keep_n[st] : Nd;
        int climit = (st < 3) ? ckpt_layer[st] : 0x7fffffff;
        uint8_t *kp = keep + (size_t)b * Nd;
        for (int i = 0; i < Nd; ++i) kp[i] = 0;
        /* select N times the best not-yet-kept eligible node */
        for (int r = 0; r < N; ++r) {
            int best_i = -1;
            for (int i = 0; i < Nd; ++i) {
                if (kp[i] || lay[i] > climit) continue;
                if (best_i < 0 || cum[i] > cum[best_i]) best_i = i; /* ties keep lower index */
            }
            if (best_i < 0) break;
            kp[best_i] = 1;
        }
        stage[b] = st;
        n_keep[b] = N;
        if (cum_out)
            for (int i = 0; i < Nd; ++i) cum_out[(size_t)b * Nd + i] = cum[i];
    }
    free(cum);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Threshold calibration (section 二: a few warm-up rounds show the spread of */
/* confidence at each checkpoint, and the thresholds are set from it; the    */
/* pages give no rule for turning that spread into a threshold).             */
/*                                                                           */
/* Readings.  The statistic recorded is the one a checkpoint compares: the   */
/* largest cumulative log-confidence on its layer, taken on the full warm-up */
/* draft tree for all three checkpoints (an earlier checkpoint firing does   */
/* not hide the later ones), NaN where the checkpoint is not reached (its    */
/* layer empty, or layers <= its layer holding fewer than keep_n[s] nodes).  */
/* The threshold of checkpoint s is the q_s-quantile of its recorded values: */
/* the r-th smallest of the m recorded values, r = ceil(q_s * m) in double   */
/* (at least 1), so that the checkpoint fires (value < threshold) on fewer   */
/* than a share q_s of the warm-up trees; q_s == 0, or nothing recorded,     */
/* gives -inf (never fires).                                                 */
int oracle_checkpoint_stats(int B, int Nd, const int32_t *parent, const int32_t *layer,
                            const float *logp, const int32_t *ckpt_layer, const int32_t *keep_n,
                            float *out) {
    if (B < 0 || Nd <= 0) return -1;
    float *cum = (float *)malloc(sizeof(float) * (size_t)Nd);
    if (!cum) return -1;
    for (int b = 0; b < B; ++b) {
        const int32_t *par = parent + (size_t)b * Nd;
        const int32_t *lay = layer + (size_t)b * Nd;
        const float *lp = logp + (size_t)b * Nd;
        for (int i = 0; i < Nd; ++i) {
            if (par[i] >= i) {
                free(cum);
                return -1;
            }
            cum[i] = ((par[i] < 0) ? 0.0f : cum[par[i]]) + lp[i];
        }
        for (int s = 0; s < 3; ++s) {
            int on_layer = 0, upto = 0;
            float best = -INFINITY;
            for (int i = 0; i < Nd; ++i) {
                if (lay[i] == ckpt_layer[s]) {
                    on_layer++;
                    if (cum[i] > best) best = cum[i];
                }
                if (lay[i] <= ckpt_layer[s]) upto++;
            }
            out[(size_t)b * 3 + s] = (on_layer == 0 || upto < keep_n[s]) ? NAN : best;
        }
    }
    free(cum);
    return 0;
}

static int cmp_float(const void *a, const void *b) {
    float x = *(const float *)a, y = *(const float *)b;
    return (x > y) - (x < y);
}

int oracle_calibrate(int64_t n, const float *samples, const float *q, float *log_thr) {
    if (n < 0) return -1;
    float *vals = (float *)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
    if (!vals) return -1;
    for (int s = 0; s < 3; ++s) {
        if (!(q[s] >= 0.0f && q[s] <= 1.0f)) {
            free(vals);
            return -1;
        }
        int64_t m = 0;
        for (int64_t i = 0; i < n; ++i) {
            float v = samples[(size_t)i * 3 + s];
            if (!isnan(v)) vals[m++] = v;
        }
        if (m == 0 || q[s] == 0.0f) {
            log_thr[s] = -INFINITY;
            continue;
        }
        qsort(vals, (size_t)m, sizeof(float), cmp_float);
        int64_t r = (int64_t)ceil((double)q[s] * (double)m);
        if (r < 1) r = 1;
        if (r > m) r = m;
        log_thr[s] = vals[r - 1];
    }
    free(vals);
    return 0;
}

/* TAIL (section 七): keep the longest prefix of the block whose confidence is */
/* >= thr (fp32 compare); the rest of the block is replaced by retrieval.    */
int oracle_prune_tail(int B, int L, const float *conf, float thr, int32_t *stage,
                      int32_t *n_keep, uint8_t *keep) {
    for (int b = 0; b < B; ++b) {
        int p = 0;
        while (p < L && conf[(size_t)b * L + p] >= thr) p++;
        n_keep[b] = p;
        stage[b] = (p < L) ? 0 : 3;
        for (int i = 0; i < L; ++i) keep[(size_t)b * L + i] = (uint8_t)(i < p);
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Gear 2: retrieval template (section 二, and the depth/width ablation).    */
/*                                                                           */
/* Reading of the asymmetric template: the root's W successors (ranks        */
/* 0..W-1) each head a chain of rank-0 successors.  Node (j, d) is the       */
/* rank-j root child continued d-1 times.  Master order: the W root          */
/* children, then the rank-0 chain down to depth D, then the other chain     */
/* nodes (j >= 1, d >= 2) by increasing d + j, ties by increasing j.  A      */
/* budget of R retrieval slots takes the first R nodes, so higher-ranked     */
/* successors get the longer chains.                                         */
/* ------------------------------------------------------------------------- */
int oracle_template(int W, int D, int Rmax, int32_t *parent, int32_t *rank, int32_t *depth) {
    int n = 0;
    /* index of node (j, d) in the order, -1 if not (yet) placed */
    int *at = (int *)malloc(sizeof(int) * (size_t)(W * (D + 1)));
    if (!at) return -1;
    for (int i = 0; i < W * (D + 1); ++i) at[i] = -1;
#define AT(j, d) at[(j) * (D + 1) + (d)]
#define PUT(j, d)                                                       \
    do {                                                                \
        if (n < Rmax) {                                                 \
            parent[n] = ((d) == 1) ? -1 : AT(j, (d) - 1);               \
            rank[n] = ((d) == 1) ? (j) : 0;                             \
            depth[n] = (d);                                             \
            AT(j, d) = n;                                               \
            n++;                                                        \
        }                                                               \
    } while (0)
    for (int j = 0; j < W; ++j) PUT(j, 1);
    for (int d = 2; d <= D; ++d) PUT(0, d);
    for (int key = 3; key <= (W - 1) + D; ++key)
        for (int j = 1; j < W; ++j) {
            int d = key - j;
            if (d >= 2 && d <= D) PUT(j, d);
        }
#undef PUT
#undef AT
    free(at);
    return n;
}

/* Retrieval: R_b = slots - n_keep[b] template nodes; node t reads the row of */
/* its template parent's token (the root token for root children) at its    */
/* rank: ret_tok[t] = M[src][rank_t].  ret_parent holds template indices.    */
int oracle_retrieve_tree(int B, int V, int k, const int32_t *table, const int32_t *root_tok,
                         const int32_t *n_keep, int slots, int Rtpl, const int32_t *tpl_parent,
                         const int32_t *tpl_rank, int Rmax_out, int32_t *ret_tok,
                         int32_t *ret_parent, int32_t *n_ret) {
    for (int b = 0; b < B; ++b) {
        /* the freed slots, as far as the template reaches (the rest stay empty) */
        int R = slots - n_keep[b];
        if (R > Rtpl) R = Rtpl;
        if (R < 0 || R > Rmax_out) return -1;
        int32_t *rt = ret_tok + (size_t)b * Rmax_out;
        int32_t *rp = ret_parent + (size_t)b * Rmax_out;
        for (int t = 0; t < Rmax_out; ++t) {
            rt[t] = -1;
            rp[t] = -1;
        }
        for (int t = 0; t < R; ++t) {
            int src = (tpl_parent[t] < 0) ? root_tok[b] : rt[tpl_parent[t]];
            if (src < 0 || src >= V) return -2;
            rt[t] = table[(size_t)src * k + tpl_rank[t]];
            rp[t] = tpl_parent[t];
        }
        n_ret[b] = R;
    }
    return 0;
}

/* Branching template (the asymmetric shape of section 二 gear 2, after Token  */
/* Recycling: better-ranked successors get more children and reach deeper).  */
/* Reading: a node is a path of ranks (r_1..r_d), 1 <= d <= D, each r < W;   */
/* its cost is d*den + num*(r_1+..+r_d) (beta = num/den >= 0 charges worse   */
/* ranks); the master order is ascending (cost, d, ranks lexicographic) and  */
/* a budget R takes its first R nodes.  A child costs more than its parent,  */
/* so every prefix is a tree.  Plain best-first expansion: the frontier is    */
/* scanned for its minimum each time.  Returns the number of nodes written.  */
#define OT_MAXD 64
typedef struct {
    long long cost;
    int d;
    int parent;           /* index in the order, -1 for root children */
    int path[OT_MAXD];
} ot_node;

static int ot_before(const ot_node *a, const ot_node *b) {
    if (a->cost != b->cost) return a->cost < b->cost;
    if (a->d != b->d) return a->d < b->d;
    for (int i = 0; i < a->d; ++i)
        if (a->path[i] != b->path[i]) return a->path[i] < b->path[i];
    return 0;
}

int oracle_template_branching(int W, int D, int num, int den, int Rmax, int32_t *parent,
                              int32_t *rank, int32_t *depth) {
    if (W < 1 || D < 1 || D > OT_MAXD || num < 0 || den < 1 || Rmax < 0) return -1;
    int cap = W + Rmax * W;
    ot_node *fr = (ot_node *)malloc(sizeof(ot_node) * (size_t)cap);
    if (!fr) return -1;
    int nf = 0, n = 0;
    for (int j = 0; j < W; ++j) {
        fr[nf].cost = (long long)den + (long long)num * j;
        fr[nf].d = 1;
        fr[nf].parent = -1;
        fr[nf].path[0] = j;
        nf++;
    }
    while (n < Rmax && nf > 0) {
        int best = 0;
        for (int i = 1; i < nf; ++i)
            if (ot_before(&fr[i], &fr[best])) best = i;
        ot_node cur = fr[best];
        fr[best] = fr[--nf];
        parent[n] = cur.parent;
        rank[n] = cur.path[cur.d - 1];
        depth[n] = cur.d;
        if (cur.d < D) {
            for (int j = 0; j < W && nf < cap; ++j) {
                ot_node c = cur;
                c.d = cur.d + 1;
                c.path[cur.d] = j;
                c.cost = cur.cost + den + (long long)num * j;
                c.parent = n;
                fr[nf++] = c;
            }
        }
        n++;
    }
    free(fr);
    return n;
}

/* TAIL retrieval: a chain of rank-0 successors x <- M[x][0], L - p steps long, */
/* starting from the last kept block token (the root when p = 0).            */
int oracle_retrieve_tail(int B, int V, int k, const int32_t *table, const int32_t *root_tok,
                         const int32_t *d_tok, const int32_t *n_keep, int L, int32_t *ret_tok,
                         int32_t *ret_parent, int32_t *n_ret) {
    for (int b = 0; b < B; ++b) {
        int p = n_keep[b];
        int x = (p == 0) ? root_tok[b] : d_tok[(size_t)b * L + p - 1];
        for (int t = 0; t < L; ++t) {
            ret_tok[(size_t)b * L + t] = -1;
            ret_parent[(size_t)b * L + t] = -1;
        }
        for (int t = 0; t < L - p; ++t) {
            if (x < 0 || x >= V) return -2;
            x = table[(size_t)x * k + 0];
            ret_tok[(size_t)b * L + t] = x;
            ret_parent[(size_t)b * L + t] = t - 1;
        }
        n_ret[b] = L - p;
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Gear 3a: flatten the hybrid tree, tree position ids and the ancestor mask */
/* (section 二).  Row 0 is the root (the last committed token).  Layouts:     */
/*   0 compact : kept draft nodes in increasing draft index, then retrieval   */
/*               nodes in template order;                                    */
/*   1 in-place: draft node i stays in row i+1 (static slots, section 四's   */
/*               batched serving); the vacated rows, in increasing order,    */
/*               take the retrieval nodes in template order;                 */
/*   2 chain   : TAIL: kept block prefix, then the retrieval chain.          */
/* depth[f] = depth[parent]+1; pos_id = base_pos + depth; anc[f] has bit g   */
/* set iff row g is an ancestor of row f or f itself (root included).        */
/* row_src (optional): where each row comes from -- 0 root, 1 kept draft     */
/* node, 2 retrieval node, 3 unfilled.  A row nothing is placed in (freed    */
/* slots beyond a small template) is empty: token -1, parent -1, depth 0,    */
/* its mask only itself.                                                     */
/* ------------------------------------------------------------------------- */
int oracle_flatten(int B, int Nd, int T1, int layout, const int32_t *root_tok,
                   const int32_t *base_pos, const int32_t *d_tok, const int32_t *d_parent,
                   const uint8_t *keep, const int32_t *n_keep, int Rmax, const int32_t *ret_tok,
                   const int32_t *ret_parent, const int32_t *n_ret, int32_t *tok, int32_t *parent,
                   int32_t *depth, int32_t *pos_id, uint64_t *anc, uint8_t *row_src) {
    if (T1 > 64) return -1;
    int *row_of_draft = (int *)malloc(sizeof(int) * (size_t)(Nd > 0 ? Nd : 1));
    int *row_of_ret = (int *)malloc(sizeof(int) * (size_t)(Rmax > 0 ? Rmax : 1));
    if (!row_of_draft || !row_of_ret) return -1;
    for (int b = 0; b < B; ++b) {
        int32_t *tk = tok + (size_t)b * T1;
        int32_t *pa = parent + (size_t)b * T1;
        const int32_t *dt = d_tok + (size_t)b * Nd;
        const int32_t *dp = d_parent + (size_t)b * Nd;
        const uint8_t *kp = keep + (size_t)b * Nd;
        const int32_t *rt = ret_tok + (size_t)b * Rmax;
        const int32_t *rp = ret_parent + (size_t)b * Rmax;
        int R = n_ret[b];
        uint8_t *sr = row_src ? row_src + (size_t)b * T1 : NULL;
        for (int f = 0; f < T1; ++f) {
            tk[f] = -1;
            pa[f] = -1;
            if (sr) sr[f] = 3;
        }
        tk[0] = root_tok[b];
        pa[0] = -1;
        if (sr) sr[0] = 0;
        int used = 1;
        if (layout == 0) {
            for (int i = 0; i < Nd; ++i) {
                row_of_draft[i] = -1;
                if (!kp[i]) continue;
                row_of_draft[i] = used;
                tk[used] = dt[i];
                pa[used] = (dp[i] < 0) ? 0 : row_of_draft[dp[i]];
                if (sr) sr[used] = 1;
                used++;
            }
            for (int t = 0; t < R; ++t) {
                row_of_ret[t] = used;
                tk[used] = rt[t];
                pa[used] = (rp[t] < 0) ? 0 : row_of_ret[rp[t]];
                if (sr) sr[used] = 2;
                used++;
            }
        } else if (layout == 1) {
            int t = 0;
            for (int i = 0; i < Nd; ++i) {
                int f = i + 1;
                if (kp[i]) {
                    tk[f] = dt[i];
                    pa[f] = (dp[i] < 0) ? 0 : dp[i] + 1;
                    if (sr) sr[f] = 1;
                } else {
                    if (t >= R) continue; /* freed slot the template does not reach: empty */
                    row_of_ret[t] = f;
                    tk[f] = rt[t];
                    pa[f] = (rp[t] < 0) ? 0 : row_of_ret[rp[t]];
                    if (sr) sr[f] = 2;
                    t++;
                }
            }
            if (t != R) return -3;
            used = Nd + 1;
        } else if (layout == 2) {
            int p = n_keep[b];
            for (int i = 0; i < p; ++i) {
                tk[used] = dt[i];
                pa[used] = used - 1;
                if (sr) sr[used] = 1;
                used++;
            }
            for (int t = 0; t < R; ++t) {
                tk[used] = rt[t];
                pa[used] = used - 1;
                if (sr) sr[used] = 2;
                used++;
            }
        } else {
            return -1;
        }
        if (used > T1) return -3; /* rows past `used` stay empty */
        for (int f = 0; f < T1; ++f) {
            int d = 0;
            uint64_t a = 0;
            for (int g = f; g >= 0; g = pa[g]) {
                a |= (uint64_t)1 << g;
                if (g != f) d++;
            }
            depth[(size_t)b * T1 + f] = d;
            pos_id[(size_t)b * T1 + f] = base_pos[b] + d;
            anc[(size_t)b * T1 + f] = a;
        }
    }
    free(row_of_draft);
    free(row_of_ret);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Row-wise top-k of the target's next-token scores (section 二, online       */
/* update; also the greedy token).  Order: value descending, ties by lower   */
/* token id; values compared as reals, so -0 == +0.  Top-k of the softmax is  */
/* top-k of the logits.  Definition by repeated selection: the j-th output   */
/* is the best element that ranks strictly after the (j-1)-th.               */
/* prob (nullable): fp64 softmax of the row at the selected ids.              */
/* ------------------------------------------------------------------------- */
static double elem(const void *row, int dtype, int i) {
    if (dtype == ODT_BF16) {
        uint32_t u = (uint32_t)((const uint16_t *)row)[i] << 16;
        float f;
        memcpy(&f, &u, 4);
        return (double)f;
    }
    return (double)((const float *)row)[i];
}

/* a ranks before b */
static int before(double va, int a, double vb, int b) {
    return (va > vb) || (va == vb && a < b);
}

int oracle_topk(int64_t n_rows, int V, int k, int dtype, const void *logits, int32_t *topk,
                double *prob) {
    if (k < 1 || k > V) return -1;
    size_t esz = (dtype == ODT_BF16) ? 2 : 4;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = 0; r < n_rows; ++r) {
        const void *row = (const char *)logits + (size_t)r * V * esz;
        int prev = -1;
        double vprev = 0.0;
        for (int j = 0; j < k; ++j) {
            int best = -1;
            double vbest = 0.0;
            for (int i = 0; i < V; ++i) {
                double v = elem(row, dtype, i);
                if (prev >= 0 && !before(vprev, prev, v, i)) continue;
                if (best < 0 || before(v, i, vbest, best)) {
                    best = i;
                    vbest = v;
                }
            }
            topk[r * k + j] = best;
            prev = best;
            vprev = vbest;
        }
        if (prob) {
            double m = -INFINITY;
            for (int i = 0; i < V; ++i) {
                double v = elem(row, dtype, i);
                if (v > m) m = v;
            }
            double s = 0.0;
            for (int i = 0; i < V; ++i) s += exp(elem(row, dtype, i) - m);
            for (int j = 0; j < k; ++j) prob[r * k + j] = exp(elem(row, dtype, topk[r * k + j]) - m) / s;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Gear 3b: strict greedy verification (section 二; lossless, Q&A).           */
/* Every root-to-node path is a candidate; it is accepted iff each edge      */
/* parent -> child has tok[child] == g[parent], g = the target's greedy token */
/* at the parent's row.  The longest accepted path wins; among equally long  */
/* ones the lowest final row (reading).  accept_len excludes the root;       */
/* bonus = g at the last accepted row; accept_idx lists the path's rows      */
/* from depth 1 down (-1 padded to Dmax).                                    */
/* ------------------------------------------------------------------------- */
int oracle_accept(int B, int T1, const int32_t *tok, const int32_t *parent, const int32_t *g,
                  int Dmax, int32_t *accept_len, int32_t *accept_idx, int32_t *bonus) {
    for (int b = 0; b < B; ++b) {
        const int32_t *tk = tok + (size_t)b * T1;
        const int32_t *pa = parent + (size_t)b * T1;
        const int32_t *gg = g + (size_t)b * T1;
        int best_f = 0, best_len = 0;
        for (int f = 0; f < T1; ++f) {
            int ok = 1, len = 0;
            for (int c = f; pa[c] >= 0; c = pa[c]) {
                if (tk[c] != gg[pa[c]]) ok = 0;
                len++;
            }
            if (ok && len > best_len) {
                best_len = len;
                best_f = f;
            }
        }
        accept_len[b] = best_len;
        bonus[b] = gg[best_f];
        for (int j = 0; j < Dmax; ++j) accept_idx[(size_t)b * Dmax + j] = -1;
        int c = best_f;
        for (int d = best_len; d >= 1; --d) {
            if (d - 1 < Dmax) accept_idx[(size_t)b * Dmax + d - 1] = c;
            c = pa[c];
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Online matrix update (section 二 gear 3, section 六): every verified row   */
/* P, accepted or rejected, overwrites the matrix row of its input token     */
/* with the target's top-k there.  Rows are applied in increasing P, so the  */
/* highest P wins a collision (reading).  table_prob (nullable) receives the */
/* probabilities in fp32.                                                    */
/* ------------------------------------------------------------------------- */
int oracle_update(int64_t n_rows, int V, int k, const int32_t *row_tok, const int32_t *topk,
                  int32_t *table, const double *prob, float *table_prob) {
    for (int64_t P = 0; P < n_rows; ++P) {
        int x = row_tok[P];
        if (x == -1) continue; /* an empty row (no candidate placed): nothing was verified */
        if (x < 0 || x >= V) return -2;
        for (int j = 0; j < k; ++j) {
            table[(size_t)x * k + j] = topk[P * k + j];
            if (prob && table_prob) table_prob[(size_t)x * k + j] = (float)prob[P * k + j];
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Softmax statistics of a row, fp64: stats[2r] = max value, stats[2r+1] =   */
/* sum over the row of exp(value - max).                                      */
/* ------------------------------------------------------------------------- */
int oracle_row_stats(int64_t n_rows, int V, int dtype, const void *logits, double *stats) {
    const size_t esz = dtype == ODT_BF16 ? 2 : 4;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        const void *row = (const char *)logits + (size_t)r * (size_t)V * esz;
        double m = -INFINITY;
        for (int i = 0; i < V; ++i) {
            double x = elem(row, dtype, i);
            if (x > m) m = x;
        }
        double sum = 0.0;
        for (int i = 0; i < V; ++i) sum += exp(elem(row, dtype, i) - m);
        stats[2 * r] = m;
        stats[2 * r + 1] = sum;
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Coverage gain (section 三): what the grafted candidates add where pruning  */
/* cut.  Reading: at every row v that has retrieval children, the target's   */
/* probability mass -- softmax of row v's logits, fp64 -- of the SET of      */
/* retrieval-child tokens of v that are not the token of a kept draft child */
/* of v (each token once); summed over the rows v of a request.  It is       */
/* positive as soon as one such token has nonzero probability.               */
/* tok, parent, row_src as produced by oracle_flatten; gain[B] fp64.         */
/* ------------------------------------------------------------------------- */
int oracle_coverage_gain(int B, int T1, int V, int dtype, const void *logits, const int32_t *tok,
                         const int32_t *parent, const uint8_t *row_src, double *gain) {
    const size_t esz = dtype == ODT_BF16 ? 2 : 4;
    int32_t *fresh = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T1 > 0 ? T1 : 1));
    if (!fresh) return -1;
    for (int b = 0; b < B; ++b) {
        const int32_t *tk = tok + (size_t)b * T1;
        const int32_t *pa = parent + (size_t)b * T1;
        const uint8_t *sr = row_src + (size_t)b * T1;
        double g = 0.0;
        for (int v = 0; v < T1; ++v) {
            int nf = 0;
            for (int c = 0; c < T1; ++c) {
                if (pa[c] != v || sr[c] != 2) continue;
                int x = tk[c];
                if (x < 0 || x >= V) continue;
                int seen = 0;
                for (int d = 0; d < T1; ++d)
                    if (pa[d] == v && sr[d] == 1 && tk[d] == x) seen = 1;
                for (int j = 0; j < nf; ++j)
                    if (fresh[j] == x) seen = 1;
                if (!seen) fresh[nf++] = x;
            }
            if (nf == 0) continue;
            const void *row = (const char *)logits + ((size_t)b * T1 + v) * (size_t)V * esz;
            double m = -INFINITY;
            for (int i = 0; i < V; ++i) {
                double x = elem(row, dtype, i);
                if (x > m) m = x;
            }
            double sum = 0.0;
            for (int i = 0; i < V; ++i) sum += exp(elem(row, dtype, i) - m);
            for (int j = 0; j < nf; ++j) g += exp(elem(row, dtype, fresh[j]) - m) / sum;
        }
        gain[b] = g;
    }
    free(fresh);
    return 0;
}
