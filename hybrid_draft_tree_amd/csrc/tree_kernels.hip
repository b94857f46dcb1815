// Tree-side kernels of the Graft step: prune-select (gear 1), retrieval
// expansion (gear 2) and flatten + tree position ids + ancestor mask (gear 3),
// as described in section 二 of the news write-up of arXiv 2605.20104, with
// the TAIL variant of section 七 and the static-slot layout of section 四.
//
// Each step of a request runs in one wavefront (lanes are draft nodes, template
// nodes or flattened rows, all <= 64) as a device function.  The standalone
// kernels behind graft_prune_select / graft_retrieve_expand /
// graft_build_tree_mask run one function each; k_build_tree runs all three in
// one launch with one workgroup per request, the retrieval chain (dependent
// gathers, latency-bound) in one wavefront while the other prunes.
#include "device_utils.hpp"
#include "launchers.hpp"

namespace graft {
namespace {

constexpr int kReqPerBlock = 4;  // requests (wavefronts) per workgroup, standalone kernels

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct PruneOut {
    int stage;   // uniform
    int N;       // uniform: kept draft nodes
    bool kept;   // this lane's node
    float cum;   // this lane's cumulative log-confidence
};

// Gear 1 (TREE): cum[i] = cum[parent] + logp[i] in fp32, level by level so the
// parent's value is final when read (the association of the definition);
// checkpoints in drafting order, the first that fires is the stage; keep the
// N nodes of layers <= c_s with the largest cum (ties -> lower index).
__device__ __forceinline__ float cum_levels(bool valid, int par, float lp) {
    const int lane = lane_id();
    // one level per pass: a node is done once its parent is (root children
    // first).  The done set is a wave-uniform lane mask, so a node tests its
    // parent's bit without a shuffle; lane masks are combined as scalars.
    const uint64_t vmask = ballot(valid);
    const uint64_t cmask = ballot(par >= 0) & vmask;  // nodes below another node
    uint64_t done = vmask & ~cmask;
    float cum = (valid && par < 0) ? 0.0f + lp : 0.0f;
    const int src = (par >= 0 ? par : lane) & (kWave - 1);
    while (done != vmask) {
        const float pc = __shfl(cum, src);
        const uint64_t newly = ballot(((done >> src) & 1ull) != 0ull) & cmask & ~done;
        if (!newly) break;  // a parent link that never resolves (bad input)
        if ((newly >> lane) & 1ull) cum = pc + lp;
        done |= newly;
    }
    return cum;
}

__device__ __forceinline__ PruneOut prune_tree_wave(bool valid, int par, int lay, float lp, int Nd,
                                                   const graft_prune_cfg &cfg) {
    const float cum = cum_levels(valid, par, lp);
    // order-preserving integer keys (-0 == +0): integer max and compares
    const int key = f32_key(__float_as_uint(cum));
    if (cfg.node_mode) {
        // per-node variant: every node at or above the threshold (closed under
        // ancestors: confidences only fall along a path)
        const bool kept = valid && key >= f32_key(__float_as_uint(cfg.node_log_thr));
        const int N = __popcll(ballot(kept));
        return {N < __popcll(ballot(valid)) ? 4 : 3, N, kept, cum};
    }
    // the three checkpoints are evaluated independently (their wave reductions
    // overlap); the first in drafting order that fires is the stage
    const uint64_t vmask = ballot(valid);
    int on[3], upto[3], best[3];
#pragma unroll
    for (int s = 0; s < 3; ++s) {
        const int c = cfg.ckpt_layer[s];
        on[s] = __popcll(ballot(lay == c) & vmask);
        upto[s] = __popcll(ballot(lay <= c) & vmask);
        best[s] = wave_max_i32((valid && lay == c) ? key : INT_MIN);
    }
    int st = 3;
#pragma unroll
    for (int s = 2; s >= 0; --s)
        if (on[s] > 0 && upto[s] >= cfg.keep[s] && best[s] < f32_key(__float_as_uint(cfg.log_thr[s]))) st = s;
    const int N = st < 3 ? cfg.keep[st] : Nd;
    const int climit = st < 3 ? cfg.ckpt_layer[st] : 0x7fffffff;
    const uint64_t emask = ballot(lay <= climit) & vmask;  // eligible nodes
    const bool elig = (emask >> lane_id()) & 1ull;
    // T = the N-th largest key among the eligible nodes (bitwise search on the
    // unsigned image of the key; each step is one compare and a scalar count);
    // keep every node above T and, of the nodes at T, the lowest-indexed ones
    // up to N
    const uint32_t u = (uint32_t)key ^ 0x80000000u;
    uint32_t T = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = T | (1u << bit);
        if (__popcll(ballot(u >= cand) & emask) >= N) T = cand;
    }
    const uint64_t gt = ballot(u > T) & emask;
    const uint64_t eq = ballot(u == T) & emask;
    const int need = N - __popcll(gt);
    const bool kept = elig && (u > T || (u == T && lanes_below(eq) < need));
    return {st, N, kept, cum};
}

// TAIL (section 七): the longest prefix of the block with confidence >= thr.
__device__ __forceinline__ PruneOut prune_tail_wave(bool valid, float conf, int Nd, float thr) {
    const int lane = lane_id();
    const uint64_t low = ballot(valid && !(conf >= thr));
    const int p = low ? (__ffsll((unsigned long long)low) - 1) : Nd;
    return {p < Nd ? 0 : 3, p, lane < p, 0.0f};
}

// Gear 2 (TREE): template node t (lane t < R) reads one entry of the matrix row
// of its parent's token (the root's for root children); depth levels are
// dependent gathers.  Returns the node's token (-1 for lanes >= R, and for a
// node below an out-of-range token or rank).
//
// Level by level, each node reading its parent's token across lanes: any depth.
__device__ __forceinline__ int retrieve_tree_levels(int R, int tp, int tr, int td, int root,
                                                    const int32_t *__restrict__ table, int V, int k) {
    const int lane = lane_id();
    const bool act = lane < R;
    const int maxd = wave_max_i32(act ? td : 0);
    int val = -1;
    for (int d = 1; d <= maxd; ++d) {
        const int pv = __shfl(val, tp >= 0 ? tp : lane);
        const int src = tp >= 0 ? pv : root;
        if (act && td == d)
            val = (src >= 0 && src < V && tr >= 0 && tr < k) ? table[(size_t)src * k + tr] : -1;
    }
    return act ? val : -1;
}

constexpr int kPathLevels = 21;  // 3-bit ranks in a 64-bit path code

// Same result with no cross-lane step between the dependent gathers: every
// node walks its own path from the root (nodes sharing a prefix read the same
// matrix entries).  The ranks along the path are packed 3 bits per depth by
// pointer doubling over the template's parent links before the first gather.
// Needs depth <= kPathLevels (ranks < 8 always hold: k <= 8).
__device__ __forceinline__ int retrieve_tree_wave(int R, int tp, int tr, int td, int root,
                                                  const int32_t *__restrict__ table, int V, int k) {
    const int lane = lane_id();
    const bool act = lane < R;
    const int maxd = wave_max_i32(act ? td : 0);
    if (maxd > kPathLevels) return retrieve_tree_levels(R, tp, tr, td, root, table, V, k);
    // depth 1 reads the root's row: load all of it now, so the first gather
    // overlaps the path-code doubling below
    const int rrow = (root >= 0 && root < V && lane < k) ? table[(size_t)root * k + lane] : -1;
    const bool own_ok = tr >= 0 && tr < k && td >= 1;
    // bit 63 (above the 21 levels of 3-bit ranks) flags a path with a rank out of range
    constexpr uint64_t kBad = 1ull << 63;
    uint64_t P = act ? (own_ok ? ((uint64_t)tr << (3 * (td - 1))) : kBad) : 0ull;
    int a = act ? tp : -1;
    for (int r = 0; r < 6; ++r) {
        if (!ballot(a >= 0)) break;  // every path complete (depth <= 2^r)
        const int src = a >= 0 ? a : lane;
        const uint64_t Pa = shfl_u64(P, src);
        const int aa = __shfl(a, src);
        if (a >= 0) {
            P |= Pa;
            a = aa;
        }
    }
    const bool bad = (P & kBad) != 0ull;
    // the path's rank at depth 1 is a valid rank or 0 (a path with a rank out of
    // range carries only the bad flag), so it indexes the loaded root row
    int x = __shfl(rrow, (int)(P & 7ull));
    for (int d = 2; d <= maxd; ++d) {
        if (act && d <= td) {
            const int r = (int)((P >> (3 * (d - 1))) & 7ull);
            x = (x >= 0 && x < V) ? table[(size_t)x * k + r] : -1;
        }
    }
    return (act && !bad) ? x : -1;
}

// TAIL: chain of rank-0 successors x <- M[x][0], R steps from x0; lane t gets
// the t-th chain token.
__device__ __forceinline__ int retrieve_tail_wave(int R, int x0, const int32_t *__restrict__ table,
                                                  int V, int k) {
    const int lane = lane_id();
    int x = x0, mine = -1;
    for (int t = 0; t < R; ++t) {
        int nx = -1;
        if (lane == 0) nx = (x >= 0 && x < V) ? table[(size_t)x * k] : -1;
        x = readlane_i32(nx, 0);
        if (lane == t) mine = x;
    }
    return mine;
}

struct FlatIn {
    // per lane, as draft node i = lane
    bool isd;
    int kp, dt, dp;
    // per lane, as retrieval node t = lane
    bool isr;
    int rt, rp;
    // uniform
    int nk, R, root, base;
};

// Gear 3a: rows of the flattened hybrid tree.  Source lanes scatter their row
// into the wave's LDS slices (stok/spar/srr: 64 ints each); lane f then owns
// row f: token, parent row, depth and ancestor-or-self mask (pointer doubling).
// spar holds (parent row + 1) | (row source << 8), so an unfilled row reads as
// parent -1, source GRAFT_ROW_EMPTY.  The structure does not depend on the
// retrieved tokens: with `srowtpl` (an LDS slice) the template node held by each
// row (or -1) is recorded there and the tokens of those rows are left for the
// caller to store.  src_out (nullable) receives the row sources.
__device__ __forceinline__ int flat_link(int prow, int src) { return (prow + 1) | (src << 8); }

__device__ __forceinline__ void flatten_wave(int layout, int T1, const FlatIn &in, int *stok,
                                             int *spar, int *srr, int *srowtpl, int32_t *tok_out,
                                             int32_t *par_out, int32_t *dep_out, int32_t *pos_out,
                                             uint64_t *anc_out, uint8_t *src_out) {
    const int lane = lane_id();
    stok[lane] = -1;
    spar[lane] = flat_link(-1, GRAFT_ROW_EMPTY);
    srr[lane] = 0;
    if (srowtpl) srowtpl[lane] = -1;
    wave_sync_lds();
    const uint64_t kmask = ballot(in.isd && in.kp);
    const uint64_t dmask = ballot(in.isd);
    const int nk = in.nk;
    if (layout == GRAFT_LAYOUT_COMPACT) {
        if (in.isd && in.kp) {
            const int row = 1 + lanes_below(kmask);
            const int dp = in.dp;
            const int prow = dp < 0 ? 0 : 1 + __popcll(kmask & ((dp >= 64) ? ~0ull : ((1ull << dp) - 1ull)));
            if (row < T1) {
                stok[row] = in.dt;
                spar[row] = flat_link(prow, GRAFT_ROW_DRAFT);
            }
        }
        if (in.isr) {
            const int row = 1 + nk + lane;
            if (row < T1) {
                stok[row] = in.rt;
                spar[row] = flat_link(in.rp < 0 ? 0 : 1 + nk + in.rp, GRAFT_ROW_RETRIEVED);
                if (srowtpl) srowtpl[row] = lane;
            }
        }
    } else if (layout == GRAFT_LAYOUT_IN_PLACE) {
        const uint64_t vmask = dmask & ~kmask;
        const bool vac = in.isd && !in.kp;
        const int r_i = lanes_below(vmask);  // which retrieval node fills this slot
        if (vac && r_i < kWave) srr[r_i] = lane + 1;
        wave_sync_lds();
        const int rt_i = __shfl(in.rt, r_i < kWave ? r_i : 0);
        const int rp_i = __shfl(in.rp, r_i < kWave ? r_i : 0);
        if (in.isd && lane + 1 < T1) {
            if (in.kp) {
                stok[lane + 1] = in.dt;
                spar[lane + 1] = flat_link(in.dp < 0 ? 0 : in.dp + 1, GRAFT_ROW_DRAFT);
            } else if (r_i < in.R) {
                stok[lane + 1] = rt_i;
                spar[lane + 1] = flat_link((rp_i < 0 || rp_i >= kWave) ? 0 : srr[rp_i], GRAFT_ROW_RETRIEVED);
                if (srowtpl) srowtpl[lane + 1] = r_i;
            }
        }
    } else {  // chain (TAIL)
        if (in.isd && lane < nk && lane + 1 < T1) {
            stok[lane + 1] = in.dt;
            spar[lane + 1] = flat_link(lane, GRAFT_ROW_DRAFT);
        }
        if (in.isr) {
            const int row = 1 + nk + lane;
            if (row < T1) {
                stok[row] = in.rt;
                spar[row] = flat_link(row - 1, GRAFT_ROW_RETRIEVED);
                if (srowtpl) srowtpl[row] = lane;
            }
        }
    }
    if (lane == 0) {
        stok[0] = in.root;
        spar[0] = flat_link(-1, GRAFT_ROW_ROOT);
    }
    wave_sync_lds();
    const bool row_ok = lane < T1;
    const int t = row_ok ? stok[lane] : -1;
    const int link = row_ok ? spar[lane] : flat_link(-1, GRAFT_ROW_EMPTY);
    const int p = (link & 0xff) - 1;
    int a = (row_ok && lane > 0) ? p : -1;
    uint64_t A = row_ok ? ((1ull << lane) | (a >= 0 ? (1ull << a) : 0ull)) : 0ull;
    for (int r = 0; r < 6; ++r) {
        if (!ballot(a >= 0)) break;  // every row's chain has reached the root
        const int src = a >= 0 ? a : lane;
        const uint64_t Aa = shfl_u64(A, src);
        const int aa = __shfl(a, src);
        if (a >= 0) {
            A |= Aa;
            a = aa;
        }
    }
    const int D = __popcll(A) - 1;  // ancestors of the row (root: 0)
    if (row_ok) {
        if (!srowtpl || srowtpl[lane] < 0) tok_out[lane] = t;
        par_out[lane] = lane == 0 ? -1 : p;
        dep_out[lane] = D;
        pos_out[lane] = in.base + D;
        anc_out[lane] = A;
        if (src_out) src_out[lane] = (uint8_t)(link >> 8);
    }
}

// ---------------------------------------------------------------------------------------
// Standalone kernels (one wavefront per request).

__global__ __launch_bounds__(kWave *kReqPerBlock) void k_prune(PruneKernelArgs a) {
    const int lane = lane_id();
    const int b = blockIdx.x * kReqPerBlock + (threadIdx.x >> 6);
    if (b >= a.B) return;
    const bool valid = lane < a.Nd;
    const size_t o = (size_t)b * a.Nd + lane;
    PruneOut r;
    if (a.mode == GRAFT_MODE_TREE) {
        const int par = valid ? a.parent[o] : -1;
        const int lay = valid ? a.layer[o] : 0x7fffffff;
        const float lp = valid ? a.score[o] : 0.0f;
        r = prune_tree_wave(valid, par, lay, lp, a.Nd, a.cfg);
        if (valid && a.cum_out) a.cum_out[o] = r.cum;
    } else {
        const float c = valid ? a.score[o] : 1.0f;
        r = prune_tail_wave(valid, c, a.Nd, a.cfg.tail_thr);
    }
    if (valid) a.keep[o] = r.kept ? 1 : 0;
    if (lane == 0) {
        a.stage[b] = r.stage;
        a.n_keep[b] = r.N;
    }
}

// Warm-up statistic of every checkpoint (the value its test compares): the
// largest cumulative log-confidence on its layer, NaN where the checkpoint is
// not reached; all three are taken on the full tree.
__global__ __launch_bounds__(kWave *kReqPerBlock) void k_ckpt_stats(CkptStatsArgs a) {
    const int lane = lane_id();
    const int b = blockIdx.x * kReqPerBlock + (threadIdx.x >> 6);
    if (b >= a.B) return;
    const bool valid = lane < a.Nd;
    const size_t o = (size_t)b * a.Nd + lane;
    const int par = valid ? a.parent[o] : -1;
    const int lay = valid ? a.layer[o] : 0x7fffffff;
    const float lp = valid ? a.score[o] : 0.0f;
    const int key = f32_key(__float_as_uint(cum_levels(valid, par, lp)));
    float mine = 0.0f;
#pragma unroll
    for (int s = 0; s < 3; ++s) {
        const int c = a.ckpt_layer[s];
        const int on = __popcll(ballot(valid && lay == c));
        const int upto = __popcll(ballot(valid && lay <= c));
        const int best = wave_max_i32((valid && lay == c) ? key : INT_MIN);
        if (lane == s) mine = (on > 0 && upto >= a.keep[s]) ? key_to_f32(best) : __int_as_float(0x7fc00000);
    }
    if (lane < 3) a.out[(size_t)b * 3 + lane] = mine;
}

constexpr int kCalibThreads = 256;

// Number of recorded (non-NaN) samples of column s whose order-preserving
// unsigned key u has (u & mask) == want; block-wide, every thread gets it.
__device__ int calib_count(const float *__restrict__ x, int64_t n, int s, uint32_t mask, uint32_t want,
                           int *s_cnt) {
    int c = 0;
    for (int64_t i = threadIdx.x; i < n; i += kCalibThreads) {
        const float v = x[i * 3 + s];
        if (v == v) {
            const uint32_t u = (uint32_t)f32_key(__float_as_uint(v)) ^ 0x80000000u;
            c += (u & mask) == want ? 1 : 0;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
    __syncthreads();  // every thread has read the previous total
    if (threadIdx.x == 0) *s_cnt = 0;
    __syncthreads();
    if (lane_id() == 0) atomicAdd(s_cnt, c);
    __syncthreads();
    return *s_cnt;
}

// Threshold of checkpoint s = blockIdx.x: the r-th smallest recorded sample,
// r = ceil(q * m) (m recorded), found bit by bit on the unsigned key image
// (32 block-wide counts); -inf when q == 0 or nothing was recorded.
__global__ __launch_bounds__(kCalibThreads) void k_calibrate(CalibArgs a) {
    __shared__ int s_cnt;
    const int s = blockIdx.x;
    const float q = a.q[s];
    const int64_t m = calib_count(a.samples, a.n, s, 0u, 0u, &s_cnt);
    if (q == 0.0f || m == 0) {
        if (threadIdx.x == 0) a.log_thr[s] = -__builtin_huge_valf();
        return;
    }
    int64_t r = (int64_t)ceil((double)q * (double)m);
    r = r < 1 ? 1 : (r > m ? m : r);
    uint32_t T = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t mask = ~0u << bit;
        const int64_t c0 = calib_count(a.samples, a.n, s, mask, T, &s_cnt);
        if (r > c0) {
            r -= c0;
            T |= 1u << bit;
        }
    }
    if (threadIdx.x == 0) a.log_thr[s] = key_to_f32((int32_t)(T ^ 0x80000000u));
}

__global__ __launch_bounds__(kWave *kReqPerBlock) void k_retrieve(RetrieveKernelArgs a) {
    const int lane = lane_id();
    const int b = blockIdx.x * kReqPerBlock + (threadIdx.x >> 6);
    if (b >= a.B) return;
    int R, val, rp;
    if (a.mode == GRAFT_MODE_TREE) {
        // no n_keep: the whole template, ahead of pruning
        R = min(max(a.slots - (a.n_keep ? a.n_keep[b] : 0), 0), a.tpl_size);
        const bool act = lane < R;
        const int tp = act ? a.tpl_parent[lane] : -1;
        const int tr = act ? a.tpl_rank[lane] : 0;
        const int td = act ? a.tpl_depth[lane] : 0;
        val = retrieve_tree_wave(R, tp, tr, td, a.root_tok[b], a.table, a.V, a.k);
        rp = act ? tp : -1;
    } else {
        const int p = min(max(a.n_keep[b], 0), a.Nd);
        R = min(max(a.slots - p, 0), a.r_out);
        const int x0 = (p <= 0) ? a.root_tok[b] : a.d_tok[(size_t)b * a.Nd + (p - 1)];
        val = retrieve_tail_wave(R, x0, a.table, a.V, a.k);
        rp = lane < R ? lane - 1 : -1;
    }
    if (lane < a.r_out) {
        a.ret_tok[(size_t)b * a.r_out + lane] = lane < R ? val : -1;
        a.ret_parent[(size_t)b * a.r_out + lane] = lane < R ? rp : -1;
    }
    if (lane == 0) a.n_ret[b] = R;
}

__global__ __launch_bounds__(kWave *kReqPerBlock) void k_flatten(FlattenKernelArgs a) {
    __shared__ int s_tok[kReqPerBlock][kWave];
    __shared__ int s_par[kReqPerBlock][kWave];
    __shared__ int s_rowret[kReqPerBlock][kWave];
    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    const int b = blockIdx.x * kReqPerBlock + w;
    if (b >= a.B) return;
    FlatIn in;
    in.nk = a.n_keep[b];
    in.R = a.n_ret[b];
    in.root = a.root_tok[b];
    in.base = a.base_pos[b];
    in.isd = lane < a.Nd;
    in.kp = in.isd ? a.keep[(size_t)b * a.Nd + lane] : 0;
    in.dt = in.isd ? a.d_tok[(size_t)b * a.Nd + lane] : -1;
    in.dp = (in.isd && a.layout != GRAFT_LAYOUT_CHAIN) ? a.d_parent[(size_t)b * a.Nd + lane] : -1;
    in.isr = lane < in.R && lane < a.r_out;
    in.rt = in.isr ? a.ret_tok[(size_t)b * a.r_out + lane] : -1;
    in.rp = in.isr ? a.ret_parent[(size_t)b * a.r_out + lane] : -1;
    const size_t o = (size_t)b * a.T1;
    flatten_wave(a.layout, a.T1, in, s_tok[w], s_par[w], s_rowret[w], nullptr, a.tok + o, a.parent + o,
                 a.depth + o, a.pos_id + o, a.anc + o, a.row_src ? a.row_src + o : nullptr);
}

// ---------------------------------------------------------------------------------------
// Fused build: one workgroup (2 wavefronts) per request.  TREE: wave 0 expands
// the whole template from the root while wave 1 prunes; after one barrier wave
// 0 keeps the first R = slots - n_keep template nodes and flattens.  TAIL:
// both waves take the prefix; wave 0 walks the chain (from the last kept block
// token) while wave 1 flattens, then wave 0 stores the chain's tokens.
__global__ __launch_bounds__(2 * kWave) void k_build_tree(BuildKernelArgs a) {
    __shared__ int s_misc[1];
    __shared__ int s_tok[kWave], s_par[kWave], s_rowret[kWave], s_rowtpl[kWave];
    const int lane = lane_id();
    const int wv = threadIdx.x >> 6;
    const int b = blockIdx.x;
    const size_t od = (size_t)b * a.Nd + lane;
    const bool isd = lane < a.Nd;
    const int root = a.root_tok[b];

    if (a.mode == GRAFT_MODE_TREE) {
        // pre: the retrieval was done ahead (whole template, n_ret[b] nodes in
        // ret_tok / ret_parent); read before anything is written
        const int tsz = a.pre ? min(max(a.n_ret[b], 0), a.r_out) : a.tpl_size;
        const bool act = lane < tsz;
        const size_t orr = (size_t)b * a.r_out + lane;
        const int tp = act ? (a.pre ? a.ret_parent[orr] : a.tpl_parent[lane]) : -1;
        int val = -1;
        if (a.pre) {
            if (wv == 0 && act) val = a.ret_tok[orr];
            __syncthreads();
        }
        if (wv == 0) {
            if (!a.pre) {
                // wave 0: the whole template from the root (the budget R is not known yet)
                const int tr = act ? a.tpl_rank[lane] : 0;
                const int td = act ? a.tpl_depth[lane] : 0;
                val = retrieve_tree_wave(a.tpl_size, tp, tr, td, root, a.table, a.V, a.k);
            }
        } else {
            // wave 1: prune, then the whole tree structure, which does not depend on
            // the retrieved tokens (rows, parents, depths, positions, masks, draft
            // and root tokens); the retrieval rows are recorded in s_rowtpl
            const int par = isd ? a.d_parent[od] : -1;
            const int lay = isd ? a.d_layer[od] : 0x7fffffff;
            const float lp = isd ? a.d_score[od] : 0.0f;
            const int dt = isd ? a.d_tok[od] : -1;
            const int base = a.base_pos[b];
            const PruneOut r = prune_tree_wave(isd, par, lay, lp, a.Nd, a.cfg);
            if (isd) {
                a.keep[od] = r.kept ? 1 : 0;
                if (a.cum_out) a.cum_out[od] = r.cum;
            }
            const int nk = r.N;
            const int R = min(max(a.slots - nk, 0), tsz);
            const bool isr = lane < R;
            FlatIn in;
            in.isd = isd;
            in.kp = r.kept ? 1 : 0;
            in.dt = dt;
            in.dp = par;
            in.isr = isr;
            in.rt = -1;
            in.rp = isr ? tp : -1;
            in.nk = nk;
            in.R = R;
            in.root = root;
            in.base = base;
            if (lane < a.r_out) a.ret_parent[(size_t)b * a.r_out + lane] = isr ? tp : -1;
            if (lane == 0) {
                a.stage[b] = r.stage;
                a.n_keep[b] = nk;
                a.n_ret[b] = R;
                s_misc[0] = R;
            }
            const size_t o = (size_t)b * a.T1;
            flatten_wave(a.layout, a.T1, in, s_tok, s_par, s_rowret, s_rowtpl, a.tok + o, a.parent + o,
                         a.depth + o, a.pos_id + o, a.anc + o, a.row_src ? a.row_src + o : nullptr);
        }
        __syncthreads();
        if (wv != 0) return;
        // wave 0: the first R retrieved tokens, into ret_tok and the rows holding them
        const int R = s_misc[0];
        if (lane < a.r_out) a.ret_tok[(size_t)b * a.r_out + lane] = lane < R ? val : -1;
        const int tn = lane < a.T1 ? s_rowtpl[lane] : -1;
        const int tv = __shfl(val, tn >= 0 ? tn : lane);
        if (tn >= 0) a.tok[(size_t)b * a.T1 + lane] = tv;
    } else {
        // TAIL: both waves take the prefix (one ballot); wave 0 follows the
        // retrieval chain (dependent gathers) while wave 1 flattens the rows,
        // whose structure does not depend on the retrieved tokens
        const float c = isd ? a.d_score[od] : 1.0f;
        const PruneOut r = prune_tail_wave(isd, c, a.Nd, a.cfg.tail_thr);
        const int p = r.N;
        const int dt = isd ? a.d_tok[od] : -1;
        const int R = min(max(a.slots - p, 0), a.r_out);
        int val = -1;
        if (wv == 0) {
            const int x0 = p <= 0 ? root : readlane_i32(dt, p - 1);
            val = retrieve_tail_wave(R, x0, a.table, a.V, a.k);
            if (lane < a.r_out) a.ret_tok[(size_t)b * a.r_out + lane] = lane < R ? val : -1;
        } else {
            if (isd) a.keep[od] = r.kept ? 1 : 0;
            FlatIn in;
            in.isd = isd;
            in.kp = r.kept ? 1 : 0;
            in.dt = dt;
            in.dp = -1;
            in.isr = lane < R;
            in.rt = -1;
            in.rp = lane < R ? lane - 1 : -1;
            in.nk = p;
            in.R = R;
            in.root = root;
            in.base = a.base_pos[b];
            if (lane < a.r_out) a.ret_parent[(size_t)b * a.r_out + lane] = in.rp;
            if (lane == 0) {
                a.stage[b] = r.stage;
                a.n_keep[b] = p;
                a.n_ret[b] = R;
            }
            const size_t o = (size_t)b * a.T1;
            flatten_wave(GRAFT_LAYOUT_CHAIN, a.T1, in, s_tok, s_par, s_rowret, s_rowtpl, a.tok + o, a.parent + o,
                         a.depth + o, a.pos_id + o, a.anc + o, a.row_src ? a.row_src + o : nullptr);
        }
        __syncthreads();
        if (wv != 0) return;
        // wave 0: the retrieved tokens into the rows that hold them
        const int tn = lane < a.T1 ? s_rowtpl[lane] : -1;
        const int tv = __shfl(val, tn >= 0 ? tn : lane);
        if (tn >= 0) a.tok[(size_t)b * a.T1 + lane] = tv;
    }
}

}  // namespace

static inline int blocks_for(int B) { return (B + kReqPerBlock - 1) / kReqPerBlock; }

void launch_prune(const PruneKernelArgs &a, hipStream_t s) {
    if (a.B <= 0) return;
    hipLaunchKernelGGL(k_prune, dim3(blocks_for(a.B)), dim3(kWave * kReqPerBlock), 0, s, a);
}

void launch_ckpt_stats(const CkptStatsArgs &a, hipStream_t s) {
    if (a.B <= 0) return;
    hipLaunchKernelGGL(k_ckpt_stats, dim3(blocks_for(a.B)), dim3(kWave * kReqPerBlock), 0, s, a);
}

void launch_calibrate(const CalibArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(k_calibrate, dim3(3), dim3(kCalibThreads), 0, s, a);
}

void launch_retrieve(const RetrieveKernelArgs &a, hipStream_t s) {
    if (a.B <= 0) return;
    hipLaunchKernelGGL(k_retrieve, dim3(blocks_for(a.B)), dim3(kWave * kReqPerBlock), 0, s, a);
}

void launch_flatten(const FlattenKernelArgs &a, hipStream_t s) {
    if (a.B <= 0) return;
    hipLaunchKernelGGL(k_flatten, dim3(blocks_for(a.B)), dim3(kWave * kReqPerBlock), 0, s, a);
}

void launch_build(const BuildKernelArgs &a, hipStream_t s) {
    if (a.B <= 0) return;
    hipLaunchKernelGGL(k_build_tree, dim3(a.B), dim3(2 * kWave), 0, s, a);
}

}  // namespace graft
