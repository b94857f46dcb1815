// C ABI of the Graft per-step path (declared in include/graft.h): host-side
// argument validation, workspace planning and kernel launches.  No call
// allocates, frees or keeps state; every launch is asynchronous on the
// caller's stream.
#include <algorithm>
#include <mutex>
#include <vector>

#include "graft.h"
#include "launchers.hpp"

using namespace graft;

namespace {

inline bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

inline int launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? GRAFT_OK : GRAFT_EDEVICE;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// workspace: [the top-k launch's words (completion words, last holder per
// token, hand-offs; with split rows: arrival counters and slice results) |
// top-k rows | top-k probabilities] -- the last two for graft_update_topk
struct WsLayout {
    TopkPlan plan;
    size_t off_topk = 0, off_prob = 0, total = 0;
    bool fits = false;  // the launch's size is within what one launch can hold
};

WsLayout ws_layout(int64_t n_rows, int V, int k, int dtype) {
    WsLayout L;
    if (n_rows < 0 || n_rows >= INT32_MAX) return L;  // row positions are kept as P + 1 in 32 bits
    L.plan = plan_topk(n_rows, V, dtype);
    L.off_topk = align256(L.plan.ws_bytes);
    L.off_prob = L.off_topk + align256((size_t)n_rows * k * sizeof(int32_t));
    L.total = L.off_prob + align256((size_t)n_rows * k * sizeof(float));
    // the launch's thread count is 32-bit: (row slices + coordinators, at most
    // GRAFT_MAX_COORD_GROUPS and never more than the rows) x wavefronts per slice x 64 lanes
    const int64_t units = n_rows * L.plan.groups + std::min<int64_t>(n_rows, GRAFT_MAX_COORD_GROUPS);
    L.fits = units * (L.plan.splits + L.plan.merge_wave) * 64 <= (int64_t)UINT32_MAX;
    return L;
}

bool dtype_ok(int dtype) { return dtype == GRAFT_DTYPE_F32 || dtype == GRAFT_DTYPE_BF16; }

}  // namespace

// Scratch of graft_verify_update_noalloc: the top-k launch's completion words,
// holder words and hand-offs.  One copy per GPU the library runs on, kept until
// the process ends.  Host code never uses this name as an address (on the host
// it is only a stand-in for the symbol): the device address comes from
// scratch_ptr().
static __device__ __align__(256) unsigned char scratch[GRAFT_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device
// with that device current and kept; nullptr if the lookup fails.
void *scratch_ptr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_dev[dev] = p;
    }
    return g_scratch_dev[dev];
}

// graft_verify_update with a caller workspace, or (static_scratch) with the
// library's per-GPU scratch, cleared by a fill kernel on `stream` first.
int verify_update_impl(int B, int T1, int V, int k, int dtype, const void *logits, const int32_t *tok,
                       const int32_t *parent, const int32_t *depth, int32_t *table, float *table_prob,
                       int32_t *topk, float *topk_prob, float *row_stats, int32_t *accept_len,
                       int32_t *accept_idx, int dmax, int32_t *bonus, int32_t *base_pos_io, void *ws,
                       size_t ws_bytes, bool static_scratch, hipStream_t stream) {
    if (!dtype_ok(dtype)) return GRAFT_EUNSUPPORTED;
    if (B < 0 || B > GRAFT_MAX_BATCH || T1 < 1 || T1 > GRAFT_MAX_ROWS || V < 1 || V > GRAFT_MAX_VOCAB || k < 1 ||
        k > GRAFT_MAX_K || k > V || dmax < 0)
        return GRAFT_EINVAL;
    if (B == 0) return GRAFT_OK;
    if (!logits || !tok || !parent || !depth || !table || !topk || !accept_len || !bonus ||
        (dmax > 0 && !accept_idx) || (!static_scratch && !ws) || (table_prob && !topk_prob))
        return GRAFT_EINVAL;
    if (!aligned(logits, 16) || !aligned(row_stats, 8)) return GRAFT_EINVAL;
    const int64_t n_rows = (int64_t)B * T1;
    const WsLayout L = ws_layout(n_rows, V, k, dtype);
    if (!L.fits) return GRAFT_EINVAL;
    if (static_scratch) {
        if (L.plan.ws_bytes > (size_t)GRAFT_NOALLOC_SCRATCH_BYTES) return GRAFT_ESCRATCH;
        ws = scratch_ptr();
        if (!ws) {
            (void)hipGetLastError();
            return GRAFT_EDEVICE;
        }
        launch_zero(ws, L.plan.ws_bytes, stream);
    } else if (!aligned(ws, 256) || ws_bytes < L.total) {
        return GRAFT_EINVAL;
    }
    VerifyArgs v;
    v.T1 = T1;
    v.tok = tok;
    v.parent = parent;
    v.depth = depth;
    v.accept_len = accept_len;
    v.accept_idx = accept_idx;
    v.dmax = dmax;
    v.bonus = bonus;
    v.base_pos_io = base_pos_io;
    v.table = table;
    v.table_prob = table_prob;
    launch_topk(L.plan, dtype, logits, k, topk, topk_prob, row_stats, ws, &v, stream);
    return launch_status();
}

}  // namespace

extern "C" {

const char *graft_status_string(int status) {
    switch (status) {
        case GRAFT_OK: return "ok";
        case GRAFT_EINVAL: return "invalid argument (null or misaligned pointer, bad size or shape)";
        case GRAFT_EUNSUPPORTED: return "unsupported dtype, mode or layout";
        case GRAFT_EDEVICE: return "HIP launch error";
        case GRAFT_ESCRATCH: return "sizes need more than the static scratch of graft_verify_update_noalloc";
        default: return "unknown status";
    }
}

int graft_launch_plan(int64_t n_rows, int V, int dtype, int T1, graft_plan *out) {
    if (!out || n_rows < 0 || V <= 0 || V > GRAFT_MAX_VOCAB || !dtype_ok(dtype) || T1 < 0 || T1 > GRAFT_MAX_ROWS)
        return GRAFT_EINVAL;
    if (T1 > 0 && n_rows % T1 != 0) return GRAFT_EINVAL;
    const WsLayout L = ws_layout(n_rows, V, 1, dtype);
    if (!L.fits) return GRAFT_EINVAL;
    const int B = T1 > 0 ? (int)std::min<int64_t>(n_rows / T1, INT32_MAX) : 0;
    out->waves_per_group = L.plan.splits + L.plan.merge_wave;
    out->groups_per_row = L.plan.groups;
    out->blocks_per_batch = L.plan.loads;
    out->coord_groups = n_rows == 0 ? 0 : (T1 > 0 ? coord_groups(L.plan, B) : (scans_holders(L.plan) ? 0 : 1));
    out->workgroups = n_rows == 0 ? 0 : n_rows * L.plan.groups + out->coord_groups;
    out->merge_wave = L.plan.merge_wave;
    out->launch_counters = (T1 > 0 && uses_launch_counters(L.plan)) ? 1 : 0;
    out->holder_scan = scans_holders(L.plan) ? 1 : 0;
    return GRAFT_OK;
}

size_t graft_workspace_bytes(int64_t n_rows, int V, int k, int dtype) {
    if (n_rows < 0 || V <= 0 || V > GRAFT_MAX_VOCAB || k < 1 || k > GRAFT_MAX_K || k > V || !dtype_ok(dtype))
        return 0;
    const WsLayout L = ws_layout(n_rows, V, k, dtype);
    return L.fits ? L.total : 0;
}

int graft_prune_select(int B, int Nd, int mode, const int32_t *d_parent, const int32_t *d_layer,
                       const float *d_score, const graft_prune_cfg *cfg, int32_t *stage,
                       int32_t *n_keep, uint8_t *keep, float *cum_out, hipStream_t stream) {
    if (mode != GRAFT_MODE_TREE && mode != GRAFT_MODE_TAIL) return GRAFT_EUNSUPPORTED;
    if (B < 0 || B > GRAFT_MAX_BATCH || Nd < 1 || Nd > GRAFT_MAX_ROWS || !cfg) return GRAFT_EINVAL;
    if (B == 0) return GRAFT_OK;
    if (!d_score || !stage || !n_keep || !keep) return GRAFT_EINVAL;
    if (mode == GRAFT_MODE_TREE) {
        if (!d_parent || !d_layer) return GRAFT_EINVAL;
        for (int s = 0; s < 3; ++s)
            if (cfg->keep[s] < 0 || cfg->keep[s] > Nd) return GRAFT_EINVAL;
    }
    PruneKernelArgs a{B, Nd, mode, d_parent, d_layer, d_score, *cfg, stage, n_keep, keep,
                      mode == GRAFT_MODE_TREE ? cum_out : nullptr};
    launch_prune(a, stream);
    return launch_status();
}

int graft_checkpoint_stats(int B, int Nd, const int32_t *d_parent, const int32_t *d_layer,
                           const float *d_score, const graft_prune_cfg *cfg, float *out,
                           hipStream_t stream) {
    if (B < 0 || B > GRAFT_MAX_BATCH || Nd < 1 || Nd > GRAFT_MAX_ROWS || !cfg) return GRAFT_EINVAL;
    if (B == 0) return GRAFT_OK;
    if (!d_parent || !d_layer || !d_score || !out) return GRAFT_EINVAL;
    CkptStatsArgs a{B, Nd, d_parent, d_layer, d_score, {}, {}, out};
    for (int s = 0; s < 3; ++s) {
        a.ckpt_layer[s] = cfg->ckpt_layer[s];
        a.keep[s] = cfg->keep[s];
    }
    launch_ckpt_stats(a, stream);
    return launch_status();
}

int graft_calibrate_thresholds(int64_t n, const float *samples, const float *q, float *log_thr,
                               hipStream_t stream) {
    if (n < 0 || n > GRAFT_MAX_CALIB_SAMPLES || !q || !log_thr || (n > 0 && !samples)) return GRAFT_EINVAL;
    CalibArgs a{n, samples, {q[0], q[1], q[2]}, log_thr};
    for (int s = 0; s < 3; ++s)
        if (!(q[s] >= 0.0f && q[s] <= 1.0f)) return GRAFT_EINVAL;  // NaN fails too
    launch_calibrate(a, stream);
    return launch_status();
}

int graft_template_master(int width, int depth, int cap, int32_t *parent, int32_t *rank,
                          int32_t *tdepth) {
    if (width < 1 || depth < 1 || cap < 0 || !parent || !rank || !tdepth) return GRAFT_EINVAL;
    // Enumerate (rank j, depth d) chain nodes and order them: root children, the
    // rank-0 chain, then the rest by (j + d, j).
    struct Node {
        int j, d, cls, key;
    };
    std::vector<Node> nodes;
    for (int j = 0; j < width; ++j)
        for (int d = 1; d <= depth; ++d) {
            int cls = d == 1 ? 0 : (j == 0 ? 1 : 2);
            nodes.push_back({j, d, cls, cls == 0 ? j : (cls == 1 ? d : (j + d) * 1024 + j)});
        }
    std::stable_sort(nodes.begin(), nodes.end(), [](const Node &a, const Node &b) {
        return a.cls != b.cls ? a.cls < b.cls : a.key < b.key;
    });
    const int n = std::min<int>(cap, (int)nodes.size());
    std::vector<int> where((size_t)width * (depth + 1), -1);
    for (int t = 0; t < n; ++t) where[(size_t)nodes[t].j * (depth + 1) + nodes[t].d] = t;
    for (int t = 0; t < n; ++t) {
        const Node &x = nodes[t];
        parent[t] = x.d == 1 ? -1 : where[(size_t)x.j * (depth + 1) + x.d - 1];
        rank[t] = x.d == 1 ? x.j : 0;
        tdepth[t] = x.d;
    }
    return n;
}

int graft_template_branching(int width, int depth, int beta_num, int beta_den, int cap, int32_t *parent,
                             int32_t *rank, int32_t *tdepth) {
    if (width < 1 || depth < 1 || beta_num < 0 || beta_den < 1 || cap < 0 || !parent || !rank || !tdepth)
        return GRAFT_EINVAL;
    // Best-first over rank paths with a binary heap keyed (cost, depth, ranks),
    // cost = depth*den + num*sum(ranks): a popped node is the next in the order.
    struct Cand {
        long long cost;
        std::vector<int> path;
        int parent;
    };
    auto later = [](const Cand &a, const Cand &b) {  // heap order: a after b
        if (a.cost != b.cost) return a.cost > b.cost;
        if (a.path.size() != b.path.size()) return a.path.size() > b.path.size();
        return a.path > b.path;
    };
    std::vector<Cand> heap;
    for (int j = 0; j < width; ++j) heap.push_back({(long long)beta_den + (long long)beta_num * j, {j}, -1});
    std::make_heap(heap.begin(), heap.end(), later);
    int n = 0;
    while (n < cap && !heap.empty()) {
        std::pop_heap(heap.begin(), heap.end(), later);
        Cand c = std::move(heap.back());
        heap.pop_back();
        parent[n] = c.parent;
        rank[n] = c.path.back();
        tdepth[n] = (int)c.path.size();
        if ((int)c.path.size() < depth) {
            for (int j = 0; j < width; ++j) {
                Cand ch{c.cost + beta_den + (long long)beta_num * j, c.path, n};
                ch.path.push_back(j);
                heap.push_back(std::move(ch));
                std::push_heap(heap.begin(), heap.end(), later);
            }
        }
        ++n;
    }
    return n;
}

int graft_retrieve_expand(int B, int V, int k, int mode, int slots, const int32_t *table,
                          const int32_t *root_tok, const int32_t *n_keep, const int32_t *d_tok,
                          int Nd, const graft_template *tpl, const graft_prune_cfg *cfg,
                          int32_t *ret_tok, int32_t *ret_parent, int32_t *n_ret, int r_out,
                          hipStream_t stream) {
    if (mode != GRAFT_MODE_TREE && mode != GRAFT_MODE_TAIL) return GRAFT_EUNSUPPORTED;
    if (B < 0 || B > GRAFT_MAX_BATCH || V < 1 || k < 1 || k > GRAFT_MAX_K || slots < 0 || r_out < 1 ||
        r_out > GRAFT_MAX_ROWS)
        return GRAFT_EINVAL;
    if (B == 0) return GRAFT_OK;
    if (!table || !root_tok || !ret_tok || !ret_parent || !n_ret) return GRAFT_EINVAL;
    if (!n_keep && mode != GRAFT_MODE_TREE) return GRAFT_EINVAL;
    int tsize = 0;
    const int32_t *tp = nullptr, *tr = nullptr, *td = nullptr;
    if (mode == GRAFT_MODE_TREE) {
        if (!tpl || !cfg || tpl->size < 0 || tpl->size > GRAFT_MAX_ROWS) return GRAFT_EINVAL;
        if (tpl->size > 0 && (!tpl->parent || !tpl->rank || !tpl->depth)) return GRAFT_EINVAL;
        if (r_out < tpl->size) return GRAFT_EINVAL;
        for (int s = 0; s < 3; ++s)
            if (slots - cfg->keep[s] < 0) return GRAFT_EINVAL;
        tsize = tpl->size;
        tp = tpl->parent;
        tr = tpl->rank;
        td = tpl->depth;
    } else {
        if (!d_tok || Nd < 1 || Nd > GRAFT_MAX_ROWS || slots > r_out) return GRAFT_EINVAL;
    }
    RetrieveKernelArgs a{B, V, k, mode, slots, table, root_tok, n_keep, d_tok, Nd, tsize, tp, tr, td,
                         ret_tok, ret_parent, n_ret, r_out};
    launch_retrieve(a, stream);
    return launch_status();
}

int graft_build_tree_mask(int B, int Nd, int T1, int layout, const int32_t *root_tok,
                          const int32_t *base_pos, const int32_t *d_tok, const int32_t *d_parent,
                          const uint8_t *keep, const int32_t *n_keep, const int32_t *ret_tok,
                          const int32_t *ret_parent, const int32_t *n_ret, int r_out, int32_t *tok,
                          int32_t *parent, int32_t *depth, int32_t *pos_id, uint64_t *anc,
                          uint8_t *row_src, hipStream_t stream) {
    if (layout != GRAFT_LAYOUT_COMPACT && layout != GRAFT_LAYOUT_IN_PLACE &&
        layout != GRAFT_LAYOUT_CHAIN)
        return GRAFT_EUNSUPPORTED;
    if (B < 0 || B > GRAFT_MAX_BATCH || Nd < 1 || Nd > GRAFT_MAX_ROWS || T1 < 2 || T1 > GRAFT_MAX_ROWS || r_out < 1 ||
        r_out > GRAFT_MAX_ROWS)
        return GRAFT_EINVAL;
    if (layout == GRAFT_LAYOUT_IN_PLACE && T1 != Nd + 1) return GRAFT_EINVAL;
    if (B == 0) return GRAFT_OK;
    if (!root_tok || !base_pos || !d_tok || !keep || !n_keep || !ret_tok || !ret_parent || !n_ret ||
        !tok || !parent || !depth || !pos_id || !anc)
        return GRAFT_EINVAL;
    if (layout != GRAFT_LAYOUT_CHAIN && !d_parent) return GRAFT_EINVAL;
    if (!aligned(anc, 8)) return GRAFT_EINVAL;
    FlattenKernelArgs a{B, Nd, T1, layout, root_tok, base_pos, d_tok, d_parent, keep, n_keep, ret_tok,
                        ret_parent, n_ret, r_out, tok, parent, depth, pos_id, anc, row_src};
    launch_flatten(a, stream);
    return launch_status();
}

namespace {

int build_tree(int B, int Nd, int T1, int mode, int layout, int slots, const graft_prune_cfg *cfg,
               const graft_template *tpl, int V, int k, const int32_t *table, const int32_t *root_tok,
               const int32_t *base_pos, const int32_t *d_parent, const int32_t *d_layer, const float *d_score,
               const int32_t *d_tok, int32_t *stage, int32_t *n_keep, uint8_t *keep, float *cum_out,
               int32_t *ret_tok, int32_t *ret_parent, int32_t *n_ret, int r_out, int32_t *tok, int32_t *parent,
               int32_t *depth, int32_t *pos_id, uint64_t *anc, uint8_t *row_src, bool pre, hipStream_t stream) {
    if (mode != GRAFT_MODE_TREE && mode != GRAFT_MODE_TAIL) return GRAFT_EUNSUPPORTED;
    if (layout != GRAFT_LAYOUT_COMPACT && layout != GRAFT_LAYOUT_IN_PLACE && layout != GRAFT_LAYOUT_CHAIN)
        return GRAFT_EUNSUPPORTED;
    if ((mode == GRAFT_MODE_TAIL) != (layout == GRAFT_LAYOUT_CHAIN)) return GRAFT_EUNSUPPORTED;
    if (B < 0 || B > GRAFT_MAX_BATCH || Nd < 1 || Nd > GRAFT_MAX_ROWS || T1 < 2 || T1 > GRAFT_MAX_ROWS || r_out < 1 ||
        r_out > GRAFT_MAX_ROWS || V < 1 || k < 1 || k > GRAFT_MAX_K || slots < 0 || !cfg)
        return GRAFT_EINVAL;
    if (T1 != slots + 1) return GRAFT_EINVAL;
    if (layout == GRAFT_LAYOUT_IN_PLACE && T1 != Nd + 1) return GRAFT_EINVAL;
    if (B == 0) return GRAFT_OK;
    if ((!pre && !table) || !root_tok || !base_pos || !d_score || !d_tok || !stage || !n_keep || !keep ||
        !ret_tok || !ret_parent || !n_ret || !tok || !parent || !depth || !pos_id || !anc)
        return GRAFT_EINVAL;
    if (!aligned(anc, 8)) return GRAFT_EINVAL;
    BuildKernelArgs a{};
    if (pre) {
        if (!d_parent || !d_layer) return GRAFT_EINVAL;
        for (int s = 0; s < 3; ++s)
            if (cfg->keep[s] < 0 || cfg->keep[s] > Nd || slots - cfg->keep[s] < 0) return GRAFT_EINVAL;
        a.pre = 1;
    } else if (mode == GRAFT_MODE_TREE) {
        if (!d_parent || !d_layer || !tpl || tpl->size < 0 || tpl->size > GRAFT_MAX_ROWS) return GRAFT_EINVAL;
        if (tpl->size > 0 && (!tpl->parent || !tpl->rank || !tpl->depth)) return GRAFT_EINVAL;
        if (r_out < tpl->size) return GRAFT_EINVAL;
        for (int s = 0; s < 3; ++s)
            if (cfg->keep[s] < 0 || cfg->keep[s] > Nd || slots - cfg->keep[s] < 0) return GRAFT_EINVAL;
        a.tpl_size = tpl->size;
        a.tpl_parent = tpl->parent;
        a.tpl_rank = tpl->rank;
        a.tpl_depth = tpl->depth;
    } else {
        if (slots > r_out || slots > Nd) return GRAFT_EINVAL;
    }
    a.B = B;
    a.Nd = Nd;
    a.T1 = T1;
    a.mode = mode;
    a.layout = layout;
    a.slots = slots;
    a.V = V;
    a.k = k;
    a.cfg = *cfg;
    a.table = table;
    a.root_tok = root_tok;
    a.base_pos = base_pos;
    a.d_parent = d_parent;
    a.d_layer = d_layer;
    a.d_score = d_score;
    a.d_tok = d_tok;
    a.stage = stage;
    a.n_keep = n_keep;
    a.keep = keep;
    a.cum_out = mode == GRAFT_MODE_TREE ? cum_out : nullptr;
    a.ret_tok = ret_tok;
    a.ret_parent = ret_parent;
    a.n_ret = n_ret;
    a.r_out = r_out;
    a.tok = tok;
    a.parent = parent;
    a.depth = depth;
    a.pos_id = pos_id;
    a.anc = anc;
    a.row_src = row_src;
    launch_build(a, stream);
    return launch_status();
}

}  // namespace

int graft_build_hybrid_tree(int B, int Nd, int T1, int mode, int layout, int slots,
                            const graft_prune_cfg *cfg, const graft_template *tpl, int V, int k,
                            const int32_t *table, const int32_t *root_tok, const int32_t *base_pos,
                            const int32_t *d_parent, const int32_t *d_layer, const float *d_score,
                            const int32_t *d_tok, int32_t *stage, int32_t *n_keep, uint8_t *keep,
                            float *cum_out, int32_t *ret_tok, int32_t *ret_parent, int32_t *n_ret,
                            int r_out, int32_t *tok, int32_t *parent, int32_t *depth, int32_t *pos_id,
                            uint64_t *anc, uint8_t *row_src, hipStream_t stream) {
    return build_tree(B, Nd, T1, mode, layout, slots, cfg, tpl, V, k, table, root_tok, base_pos, d_parent,
                      d_layer, d_score, d_tok, stage, n_keep, keep, cum_out, ret_tok, ret_parent, n_ret, r_out,
                      tok, parent, depth, pos_id, anc, row_src, false, stream);
}

int graft_build_after_retrieval(int B, int Nd, int T1, int layout, int slots, const graft_prune_cfg *cfg,
                                const int32_t *root_tok, const int32_t *base_pos, const int32_t *d_parent,
                                const int32_t *d_layer, const float *d_score, const int32_t *d_tok,
                                int32_t *stage, int32_t *n_keep, uint8_t *keep, float *cum_out,
                                int32_t *ret_tok, int32_t *ret_parent, int32_t *n_ret, int r_out, int32_t *tok,
                                int32_t *parent, int32_t *depth, int32_t *pos_id, uint64_t *anc,
                                uint8_t *row_src, hipStream_t stream) {
    if (layout == GRAFT_LAYOUT_CHAIN) return GRAFT_EUNSUPPORTED;  // TAIL retrieval follows the prune
    // the table and vocabulary are not read: the retrieval is done
    return build_tree(B, Nd, T1, GRAFT_MODE_TREE, layout, slots, cfg, nullptr, 1, 1, nullptr, root_tok,
                      base_pos, d_parent, d_layer, d_score, d_tok, stage, n_keep, keep, cum_out, ret_tok,
                      ret_parent, n_ret, r_out, tok, parent, depth, pos_id, anc, row_src, true, stream);
}

int graft_verify_update(int B, int T1, int V, int k, int dtype, const void *logits, const int32_t *tok,
                        const int32_t *parent, const int32_t *depth, int32_t *table, float *table_prob,
                        int32_t *topk, float *topk_prob, float *row_stats, int32_t *accept_len,
                        int32_t *accept_idx, int dmax, int32_t *bonus, int32_t *base_pos_io, void *ws,
                        size_t ws_bytes, hipStream_t stream) {
    return verify_update_impl(B, T1, V, k, dtype, logits, tok, parent, depth, table, table_prob, topk, topk_prob,
                              row_stats, accept_len, accept_idx, dmax, bonus, base_pos_io, ws, ws_bytes, false,
                              stream);
}

int graft_verify_update_noalloc(int B, int T1, int V, int k, int dtype, const void *logits, const int32_t *tok,
                                const int32_t *parent, const int32_t *depth, int32_t *table, float *table_prob,
                                int32_t *topk, float *topk_prob, float *row_stats, int32_t *accept_len,
                                int32_t *accept_idx, int dmax, int32_t *bonus, int32_t *base_pos_io,
                                hipStream_t stream) {
    return verify_update_impl(B, T1, V, k, dtype, logits, tok, parent, depth, table, table_prob, topk, topk_prob,
                              row_stats, accept_len, accept_idx, dmax, bonus, base_pos_io, nullptr, 0, true,
                              stream);
}

int graft_verify_accept(int B, int T1, int V, int k, int dtype, const void *logits,
                        const int32_t *tok, const int32_t *parent, const int32_t *depth,
                        int32_t *topk, float *topk_prob, float *row_stats, int32_t *accept_len,
                        int32_t *accept_idx, int dmax, int32_t *bonus, int32_t *base_pos_io, void *ws,
                        size_t ws_bytes, hipStream_t stream) {
    if (!dtype_ok(dtype)) return GRAFT_EUNSUPPORTED;
    if (B < 0 || B > GRAFT_MAX_BATCH || T1 < 1 || T1 > GRAFT_MAX_ROWS || V < 1 || V > GRAFT_MAX_VOCAB || k < 1 || k > GRAFT_MAX_K ||
        k > V || dmax < 0)
        return GRAFT_EINVAL;
    if (B == 0) return GRAFT_OK;
    if (!logits || !tok || !parent || !depth || !topk || !accept_len || !bonus ||
        (dmax > 0 && !accept_idx) || !ws)
        return GRAFT_EINVAL;
    if (!aligned(logits, 16) || !aligned(ws, 256) || !aligned(row_stats, 8)) return GRAFT_EINVAL;
    const int64_t n_rows = (int64_t)B * T1;
    const WsLayout L = ws_layout(n_rows, V, k, dtype);
    if (!L.fits || ws_bytes < L.total) return GRAFT_EINVAL;
    VerifyArgs v;
    v.T1 = T1;
    v.tok = tok;
    v.parent = parent;
    v.depth = depth;
    v.accept_len = accept_len;
    v.accept_idx = accept_idx;
    v.dmax = dmax;
    v.bonus = bonus;
    v.base_pos_io = base_pos_io;
    launch_topk(L.plan, dtype, logits, k, topk, topk_prob, row_stats, ws, &v, stream);
    return launch_status();
}

int graft_update_topk(int64_t n_rows, int V, int k, int dtype, const void *logits,
                      const int32_t *topk_in, const float *prob_in, const int32_t *row_tok,
                      int32_t *table, float *table_prob, int32_t *topk_out, void *ws,
                      size_t ws_bytes, hipStream_t stream) {
    if (!dtype_ok(dtype)) return GRAFT_EUNSUPPORTED;
    if (n_rows < 0 || V < 1 || V > GRAFT_MAX_VOCAB || k < 1 || k > GRAFT_MAX_K || k > V) return GRAFT_EINVAL;
    if (n_rows == 0) return GRAFT_OK;
    if (!row_tok || !table || (!logits && !topk_in)) return GRAFT_EINVAL;
    const int32_t *tk = topk_in;
    const float *pr = prob_in;
    if (logits) {
        if (!ws || !aligned(logits, 16) || !aligned(ws, 256)) return GRAFT_EINVAL;
        const WsLayout L = ws_layout(n_rows, V, k, dtype);
        if (!L.fits || ws_bytes < L.total) return GRAFT_EINVAL;
        int32_t *tk_ws = topk_out ? topk_out : (int32_t *)((char *)ws + L.off_topk);
        float *pr_ws = table_prob ? (float *)((char *)ws + L.off_prob) : nullptr;
        // top-k and the matrix update in one launch: the registration workgroup
        // and the per-row hand-off of graft_verify_update, without requests
        VerifyArgs v{};
        v.tok = row_tok;
        v.table = table;
        v.table_prob = table_prob;
        v.update_only = 1;
        launch_topk(L.plan, dtype, logits, k, tk_ws, pr_ws, nullptr, ws, &v, stream);
        return launch_status();
    } else if (table_prob && !prob_in) {
        return GRAFT_EINVAL;
    }
    launch_update(n_rows, V, k, tk, table_prob ? pr : nullptr, row_tok, table, table_prob, stream);
    return launch_status();
}

int graft_coverage_gain(int B, int T1, int V, int dtype, const void *logits, const int32_t *tok,
                        const int32_t *parent, const uint8_t *row_src, const float *row_stats,
                        float *gain, hipStream_t stream) {
    if (!dtype_ok(dtype)) return GRAFT_EUNSUPPORTED;
    if (B < 0 || B > GRAFT_MAX_BATCH || T1 < 1 || T1 > GRAFT_MAX_ROWS || V < 1 || V > GRAFT_MAX_VOCAB) return GRAFT_EINVAL;
    if (B == 0) return GRAFT_OK;
    if (!logits || !tok || !parent || !row_src || !row_stats || !gain) return GRAFT_EINVAL;
    if (!aligned(row_stats, 8)) return GRAFT_EINVAL;
    CoverageArgs a{B, T1, V, dtype, logits, tok, parent, row_src, row_stats, gain};
    launch_coverage(a, stream);
    return launch_status();
}

int graft_stream_read(const void *data, int64_t n_rows, int64_t row_bytes, uint32_t *sink, hipStream_t stream) {
    if (n_rows < 0 || n_rows > INT32_MAX || row_bytes <= 0 || row_bytes % 16 != 0) return GRAFT_EINVAL;
    if (n_rows == 0) return GRAFT_OK;
    if (!data || !sink || !aligned(data, 16)) return GRAFT_EINVAL;
    launch_stream_read(data, n_rows, row_bytes, sink, stream);
    return launch_status();
}

}  // extern "C"
