// Tree-side kernels of the Graft step: prune-select (gear 1), retrieval
// expansion (gear 2) and flatten + tree position ids + ancestor mask (gear 3),
// as described in section 二 of the news write-up of arXiv 2605.20104, with
// the TAIL variant of section 七 and the static-slot layout of section 四.
//
// Each request is one wavefront: lanes are draft nodes, template nodes or
// flattened rows (all <= 64).  Cross-lane traffic uses shuffles and ballots;
// no LDS except the row-placement scatter of the flatten.
#include "device_utils.hpp"
#include "launchers.hpp"

namespace graft {
namespace {

constexpr int kReqPerBlock = 4;  // requests (wavefronts) per workgroup

// Depth below the root of every node, by pointer doubling over parent links
// (parent < 0 = child of the root, depth 1).  Lanes >= n report 0.
__device__ __forceinline__ int node_depth(int par, bool valid) {
    int lane = lane_id();
    int a = valid ? par : -1;
    int d = valid ? 1 : 0;
#pragma unroll
    for (int r = 0; r < 6; ++r) {
        int src = a >= 0 ? a : lane;
        int da = __shfl(d, src);
        int aa = __shfl(a, src);
        if (a >= 0) {
            d += da;
            a = aa;
        }
    }
    return d;
}

// ---------------------------------------------------------------------------------------
// Gear 1: prune-select.
__global__ __launch_bounds__(kWave *kReqPerBlock) void k_prune_tree(
    int B, int Nd, const int32_t *__restrict__ parent, const int32_t *__restrict__ layer,
    const float *__restrict__ score, graft_prune_cfg cfg, int32_t *__restrict__ stage_out,
    int32_t *__restrict__ n_keep_out, uint8_t *__restrict__ keep_out, float *__restrict__ cum_out) {
    const int lane = lane_id();
    const int b = blockIdx.x * kReqPerBlock + (threadIdx.x >> 6);
    if (b >= B) return;
    const bool valid = lane < Nd;
    const size_t o = (size_t)b * Nd + lane;
    const int par = valid ? parent[o] : -1;
    const int lay = valid ? layer[o] : 0x7fffffff;
    const float lp = valid ? score[o] : 0.0f;

    // cum[i] = cum[parent] + logp[i]: one fp32 add per node, level by level so the
    // parent's value is final when read (same association as the definition).
    const int dep = node_depth(par, valid);
    const int maxd = wave_max_i32(dep);
    float cum = 0.0f;
    for (int d = 1; d <= maxd; ++d) {
        float pc = __shfl(cum, par >= 0 ? par : lane);
        if (valid && dep == d) cum = (par >= 0 ? pc : 0.0f) + lp;
    }

    // Checkpoints in drafting order; the first that fires is the stage.
    int st = 3;
    for (int s = 0; s < 3; ++s) {
        const int c = cfg.ckpt_layer[s];
        const int on = __popcll(ballot(valid && lay == c));
        const int upto = __popcll(ballot(valid && lay <= c));
        const float best = wave_max_f32((valid && lay == c) ? cum : -INFINITY);
        if (on > 0 && upto >= cfg.keep[s] && best < cfg.log_thr[s]) {
            st = s;
            break;
        }
    }
    const int N = st < 3 ? cfg.keep[st] : Nd;
    const int climit = st < 3 ? cfg.ckpt_layer[st] : 0x7fffffff;
    const bool elig = valid && lay <= climit;
    const uint64_t emask = ballot(elig);

    // rank among eligible nodes by (cum desc, index asc)
    int rank = 0;
    for (int j = 0; j < Nd; ++j) {
        const float cj = __shfl(cum, j);
        const bool ej = (emask >> j) & 1ull;
        rank += (ej && (cj > cum || (cj == cum && j < lane))) ? 1 : 0;
    }
    const bool kept = elig && rank < N;
    if (valid) {
        keep_out[o] = kept ? 1 : 0;
        if (cum_out) cum_out[o] = cum;
    }
    if (lane == 0) {
        stage_out[b] = st;
        n_keep_out[b] = N;
    }
}

// TAIL (section 七): longest prefix of the block with confidence >= tail_thr.
__global__ __launch_bounds__(kWave *kReqPerBlock) void k_prune_tail(
    int B, int Nd, const float *__restrict__ conf, float thr, int32_t *__restrict__ stage_out,
    int32_t *__restrict__ n_keep_out, uint8_t *__restrict__ keep_out) {
    const int lane = lane_id();
    const int b = blockIdx.x * kReqPerBlock + (threadIdx.x >> 6);
    if (b >= B) return;
    const bool valid = lane < Nd;
    const float c = valid ? conf[(size_t)b * Nd + lane] : 1.0f;
    const uint64_t low = ballot(valid && !(c >= thr));
    const int p = low ? (__ffsll((unsigned long long)low) - 1) : Nd;
    if (valid) keep_out[(size_t)b * Nd + lane] = lane < p ? 1 : 0;
    if (lane == 0) {
        n_keep_out[b] = p;
        stage_out[b] = p < Nd ? 0 : 3;
    }
}

// ---------------------------------------------------------------------------------------
// Gear 2: retrieval from the continuation matrix.  Template node t (a lane) reads
// one entry of the row of its parent's token; depth levels are dependent gathers.
__global__ __launch_bounds__(kWave *kReqPerBlock) void k_retrieve_tree(
    int B, int V, int k, int slots, const int32_t *__restrict__ table,
    const int32_t *__restrict__ root_tok, const int32_t *__restrict__ n_keep, int tpl_size,
    const int32_t *__restrict__ tpl_parent, const int32_t *__restrict__ tpl_rank,
    const int32_t *__restrict__ tpl_depth, int32_t *__restrict__ ret_tok,
    int32_t *__restrict__ ret_parent, int32_t *__restrict__ n_ret, int r_out) {
    const int lane = lane_id();
    const int b = blockIdx.x * kReqPerBlock + (threadIdx.x >> 6);
    if (b >= B) return;
    int R = slots - n_keep[b];
    R = R < 0 ? 0 : (R > tpl_size ? tpl_size : R);
    const bool act = lane < R;
    const int tp = act ? tpl_parent[lane] : -1;
    const int tr = act ? tpl_rank[lane] : 0;
    const int td = act ? tpl_depth[lane] : 0;
    const int root = root_tok[b];
    const int maxd = wave_max_i32(td);
    int val = -1;
    for (int d = 1; d <= maxd; ++d) {
        const int pv = __shfl(val, tp >= 0 ? tp : lane);
        const int src = tp >= 0 ? pv : root;
        if (act && td == d)
            val = (src >= 0 && src < V && tr >= 0 && tr < k) ? table[(size_t)src * k + tr] : -1;
    }
    if (lane < r_out) {
        ret_tok[(size_t)b * r_out + lane] = act ? val : -1;
        ret_parent[(size_t)b * r_out + lane] = act ? tp : -1;
    }
    if (lane == 0) n_ret[b] = R;
}

// TAIL: chain of rank-0 successors from the last kept block token.
__global__ __launch_bounds__(kWave *kReqPerBlock) void k_retrieve_tail(
    int B, int V, int k, int slots, const int32_t *__restrict__ table,
    const int32_t *__restrict__ root_tok, const int32_t *__restrict__ n_keep,
    const int32_t *__restrict__ d_tok, int Nd, int32_t *__restrict__ ret_tok,
    int32_t *__restrict__ ret_parent, int32_t *__restrict__ n_ret, int r_out) {
    const int lane = lane_id();
    const int b = blockIdx.x * kReqPerBlock + (threadIdx.x >> 6);
    if (b >= B) return;
    const int p = min(max(n_keep[b], 0), Nd);
    int R = slots - p;
    R = R < 0 ? 0 : (R > r_out ? r_out : R);
    int x = (p <= 0) ? root_tok[b] : d_tok[(size_t)b * Nd + (p - 1)];
    // one lane walks the chain; the others fill padding
    int mine = -1;
    for (int t = 0; t < R; ++t) {
        int nx = -1;
        if (lane == 0) nx = (x >= 0 && x < V) ? table[(size_t)x * k] : -1;
        x = __shfl(nx, 0);
        if (lane == t) mine = x;
    }
    if (lane < r_out) {
        ret_tok[(size_t)b * r_out + lane] = lane < R ? mine : -1;
        ret_parent[(size_t)b * r_out + lane] = lane < R ? lane - 1 : -1;
    }
    if (lane == 0) n_ret[b] = R;
}

// ---------------------------------------------------------------------------------------
// Gear 3a: flatten + tree position ids + ancestor mask.  Source lanes (draft node
// i, retrieval node t) scatter their row into LDS; then lane f owns row f.
__global__ __launch_bounds__(kWave *kReqPerBlock) void k_flatten(
    int B, int Nd, int T1, int layout, const int32_t *__restrict__ root_tok,
    const int32_t *__restrict__ base_pos, const int32_t *__restrict__ d_tok,
    const int32_t *__restrict__ d_parent, const uint8_t *__restrict__ keep,
    const int32_t *__restrict__ n_keep, const int32_t *__restrict__ ret_tok,
    const int32_t *__restrict__ ret_parent, const int32_t *__restrict__ n_ret, int r_out,
    int32_t *__restrict__ tok_out, int32_t *__restrict__ par_out, int32_t *__restrict__ dep_out,
    int32_t *__restrict__ pos_out, uint64_t *__restrict__ anc_out) {
    __shared__ int s_tok[kReqPerBlock][kWave];
    __shared__ int s_par[kReqPerBlock][kWave];
    __shared__ int s_rowret[kReqPerBlock][kWave];
    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    const int b = blockIdx.x * kReqPerBlock + w;
    const bool live = b < B;
    int *stok = s_tok[w];
    int *spar = s_par[w];
    int *srr = s_rowret[w];
    stok[lane] = -1;
    spar[lane] = -1;
    srr[lane] = 0;
    __syncthreads();

    const int nk = live ? n_keep[b] : 0;
    const int R = live ? n_ret[b] : 0;
    const bool isd = live && lane < Nd;
    const int kp = isd ? keep[(size_t)b * Nd + lane] : 0;
    const int dt = isd ? d_tok[(size_t)b * Nd + lane] : -1;
    const int dp = (isd && layout != GRAFT_LAYOUT_CHAIN) ? d_parent[(size_t)b * Nd + lane] : -1;
    const bool isr = live && lane < R && lane < r_out;
    const int rt = isr ? ret_tok[(size_t)b * r_out + lane] : -1;
    const int rp = isr ? ret_parent[(size_t)b * r_out + lane] : -1;
    const uint64_t kmask = ballot(isd && kp);
    const uint64_t dmask = ballot(isd);

    if (layout == GRAFT_LAYOUT_COMPACT) {
        if (isd && kp) {
            const int row = 1 + lanes_below(kmask);
            const int prow =
                dp < 0 ? 0 : 1 + __popcll(kmask & ((dp >= 64) ? ~0ull : ((1ull << dp) - 1ull)));
            if (row < T1) {
                stok[row] = dt;
                spar[row] = prow;
            }
        }
        if (isr) {
            const int row = 1 + nk + lane;
            if (row < T1) {
                stok[row] = rt;
                spar[row] = rp < 0 ? 0 : 1 + nk + rp;
            }
        }
    } else if (layout == GRAFT_LAYOUT_IN_PLACE) {
        const uint64_t vmask = dmask & ~kmask;
        const bool vac = isd && !kp;
        const int r_i = lanes_below(vmask);  // which retrieval node fills this slot
        if (vac && r_i < kWave) srr[r_i] = lane + 1;
        __syncthreads();
        const int rt_i = __shfl(rt, r_i < kWave ? r_i : 0);
        const int rp_i = __shfl(rp, r_i < kWave ? r_i : 0);
        if (isd && lane + 1 < T1) {
            if (kp) {
                stok[lane + 1] = dt;
                spar[lane + 1] = dp < 0 ? 0 : dp + 1;
            } else if (r_i < R) {
                stok[lane + 1] = rt_i;
                spar[lane + 1] = (rp_i < 0 || rp_i >= kWave) ? 0 : srr[rp_i];
            }
        }
    } else {  // chain (TAIL)
        if (isd && lane < nk && lane + 1 < T1) {
            stok[lane + 1] = dt;
            spar[lane + 1] = lane;
        }
        if (isr) {
            const int row = 1 + nk + lane;
            if (row < T1) {
                stok[row] = rt;
                spar[row] = row - 1;
            }
        }
    }
    if (lane == 0 && live) {
        stok[0] = root_tok[b];
        spar[0] = -1;
    }
    __syncthreads();
    if (!live) return;

    const bool row_ok = lane < T1;
    const int t = row_ok ? stok[lane] : -1;
    const int p = row_ok ? spar[lane] : -1;
    // ancestor-or-self mask and depth by pointer doubling along parent links
    int a = (row_ok && lane > 0) ? p : -1;
    uint64_t A = row_ok ? ((1ull << lane) | (a >= 0 ? (1ull << a) : 0ull)) : 0ull;
    int D = a >= 0 ? 1 : 0;
#pragma unroll
    for (int r = 0; r < 6; ++r) {
        const int src = a >= 0 ? a : lane;
        const uint64_t Aa = shfl_u64(A, src);
        const int Da = __shfl(D, src);
        const int aa = __shfl(a, src);
        if (a >= 0) {
            A |= Aa;
            D += Da;
            a = aa;
        }
    }
    if (row_ok) {
        const size_t o = (size_t)b * T1 + lane;
        tok_out[o] = t;
        par_out[o] = lane == 0 ? -1 : p;
        dep_out[o] = D;
        pos_out[o] = base_pos[b] + D;
        anc_out[o] = A;
    }
}

}  // namespace

static inline int blocks_for(int B) { return (B + kReqPerBlock - 1) / kReqPerBlock; }

void launch_prune(int B, int Nd, int mode, const int32_t *parent, const int32_t *layer,
                  const float *score, const graft_prune_cfg &cfg, int32_t *stage, int32_t *n_keep,
                  uint8_t *keep, float *cum_out, hipStream_t s) {
    if (B <= 0) return;
    if (mode == GRAFT_MODE_TREE)
        hipLaunchKernelGGL(k_prune_tree, dim3(blocks_for(B)), dim3(kWave * kReqPerBlock), 0, s, B, Nd,
                           parent, layer, score, cfg, stage, n_keep, keep, cum_out);
    else
        hipLaunchKernelGGL(k_prune_tail, dim3(blocks_for(B)), dim3(kWave * kReqPerBlock), 0, s, B, Nd,
                           score, cfg.tail_thr, stage, n_keep, keep);
}

void launch_retrieve(int B, int V, int k, int mode, int slots, const int32_t *table,
                     const int32_t *root_tok, const int32_t *n_keep, const int32_t *d_tok, int Nd,
                     int tpl_size, const int32_t *tpl_parent, const int32_t *tpl_rank,
                     const int32_t *tpl_depth, int32_t *ret_tok, int32_t *ret_parent,
                     int32_t *n_ret, int r_out, hipStream_t s) {
    if (B <= 0) return;
    if (mode == GRAFT_MODE_TREE)
        hipLaunchKernelGGL(k_retrieve_tree, dim3(blocks_for(B)), dim3(kWave * kReqPerBlock), 0, s, B,
                           V, k, slots, table, root_tok, n_keep, tpl_size, tpl_parent, tpl_rank,
                           tpl_depth, ret_tok, ret_parent, n_ret, r_out);
    else
        hipLaunchKernelGGL(k_retrieve_tail, dim3(blocks_for(B)), dim3(kWave * kReqPerBlock), 0, s, B,
                           V, k, slots, table, root_tok, n_keep, d_tok, Nd, ret_tok, ret_parent,
                           n_ret, r_out);
}

void launch_flatten(int B, int Nd, int T1, int layout, const int32_t *root_tok,
                    const int32_t *base_pos, const int32_t *d_tok, const int32_t *d_parent,
                    const uint8_t *keep, const int32_t *n_keep, const int32_t *ret_tok,
                    const int32_t *ret_parent, const int32_t *n_ret, int r_out, int32_t *tok,
                    int32_t *parent, int32_t *depth, int32_t *pos_id, uint64_t *anc,
                    hipStream_t s) {
    if (B <= 0) return;
    hipLaunchKernelGGL(k_flatten, dim3(blocks_for(B)), dim3(kWave * kReqPerBlock), 0, s, B, Nd, T1,
                       layout, root_tok, base_pos, d_tok, d_parent, keep, n_keep, ret_tok,
                       ret_parent, n_ret, r_out, tok, parent, depth, pos_id, anc);
}

}  // namespace graft
