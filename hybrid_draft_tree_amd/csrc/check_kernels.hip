// Optional checks of the data preconditions the Graft calls assume (the
// draft tree of section 二's gear 1, the flattened hybrid tree that gear 3
// verifies).  The other kernels never read out of bounds on bad values, but
// their results are then meaningless; these report which condition failed,
// one status word of flag bits per request, so a caller can stop before
// using them.  One wavefront per request, lanes are nodes or rows.
#include "device_utils.hpp"
#include "graft.h"

namespace {

constexpr int kReq = 4;  // requests (wavefronts) per workgroup

// OR of a small flag word over the wavefront (one ballot per flag bit).
__device__ __forceinline__ int wave_or_flags(int f) {
    int all = 0;
#pragma unroll
    for (int bit = 0; bit < 5; ++bit)
        if (graft::ballot((f >> bit) & 1)) all |= 1 << bit;
    return all;
}

__global__ __launch_bounds__(graft::kWave *kReq) void k_check_draft(int B, int Nd, int mode, int V,
                                                             const int32_t *__restrict__ parent,
                                                             const int32_t *__restrict__ layer,
                                                             const float *__restrict__ score,
                                                             const int32_t *__restrict__ tok, int32_t *status) {
    using namespace graft;
    const int lane = lane_id();
    const int b = blockIdx.x * kReq + (threadIdx.x >> 6);
    if (b >= B) return;
    const bool node = lane < Nd;
    const size_t o = (size_t)b * Nd + lane;
    int bad = 0;
    if (node) {
        const float sc = score[o];
        const int t = tok[o];
        if (t < 0 || t >= V) bad |= GRAFT_BAD_TOKEN;
        if (mode == GRAFT_MODE_TREE) {
            if (!(sc <= 0.0f)) bad |= GRAFT_BAD_SCORE;  // NaN fails too
        } else {
            if (!(sc >= 0.0f && sc <= 1.0f)) bad |= GRAFT_BAD_SCORE;
        }
    }
    if (mode == GRAFT_MODE_TREE) {
        const int p = node ? parent[o] : -1;
        const int ly = node ? layer[o] : 0;
        const bool p_ok = p >= -1 && p < lane;
        if (node && !p_ok) bad |= GRAFT_BAD_PARENT;
        // the parent's layer, read across lanes (only for in-range parents)
        const int pl = __shfl(ly, (p_ok && p >= 0) ? p : lane);
        if (node && p_ok && ly != (p < 0 ? 0 : pl + 1)) bad |= GRAFT_BAD_LAYER;
    }
    const int all = wave_or_flags(bad);
    if (lane == 0) status[b] = all;
}

__global__ __launch_bounds__(graft::kWave *kReq) void k_check_tree(int B, int T1, int V, const int32_t *__restrict__ tok,
                                                            const int32_t *__restrict__ parent,
                                                            const int32_t *__restrict__ depth, int32_t *status) {
    using namespace graft;
    const int lane = lane_id();
    const int b = blockIdx.x * kReq + (threadIdx.x >> 6);
    if (b >= B) return;
    const bool row = lane < T1;
    const size_t o = (size_t)b * T1 + lane;
    const int t = row ? tok[o] : 0;
    const int p = row ? parent[o] : -1;
    const int d = row ? depth[o] : 0;
    const bool empty = lane > 0 && t == -1;  // an unfilled slot: token -1, parent -1, depth 0
    int bad = 0;
    if (row) {
        if (empty) {
            if (p != -1) bad |= GRAFT_BAD_PARENT;
            if (d != 0) bad |= GRAFT_BAD_DEPTH;
        } else {
            if (t < 0 || t >= V) bad |= GRAFT_BAD_TOKEN;
            if (lane == 0 ? p != -1 : (p < 0 || p >= lane)) bad |= GRAFT_BAD_PARENT;
        }
    }
    const bool p_ok = !empty && (lane == 0 ? p == -1 : (p >= 0 && p < lane));
    const int pd = __shfl(d, (p_ok && p >= 0) ? p : lane);
    const int pt = __shfl(t, (p_ok && p >= 0) ? p : lane);
    if (row && p_ok && d != (lane == 0 ? 0 : pd + 1)) bad |= GRAFT_BAD_DEPTH;
    if (row && p_ok && lane > 0 && pt == -1) bad |= GRAFT_BAD_PARENT;  // a child of an empty slot
    const int all = wave_or_flags(bad);
    if (lane == 0) status[b] = all;
}

inline int launch_status() { return hipGetLastError() == hipSuccess ? GRAFT_OK : GRAFT_EDEVICE; }

}  // namespace

extern "C" {

int graft_check_draft(int B, int Nd, int mode, int V, const int32_t *d_parent, const int32_t *d_layer,
                      const float *d_score, const int32_t *d_tok, int32_t *status, hipStream_t stream) {
    if (mode != GRAFT_MODE_TREE && mode != GRAFT_MODE_TAIL) return GRAFT_EUNSUPPORTED;
    if (B < 0 || B > GRAFT_MAX_BATCH || Nd < 1 || Nd > GRAFT_MAX_ROWS || V < 1) return GRAFT_EINVAL;
    if (B == 0) return GRAFT_OK;
    if (!d_score || !d_tok || !status || (mode == GRAFT_MODE_TREE && (!d_parent || !d_layer))) return GRAFT_EINVAL;
    hipLaunchKernelGGL(k_check_draft, dim3((B + kReq - 1) / kReq), dim3(graft::kWave * kReq), 0, stream, B, Nd,
                       mode, V, d_parent, d_layer, d_score, d_tok, status);
    return launch_status();
}

int graft_check_tree(int B, int T1, int V, const int32_t *tok, const int32_t *parent, const int32_t *depth,
                     int32_t *status, hipStream_t stream) {
    if (B < 0 || B > GRAFT_MAX_BATCH || T1 < 1 || T1 > GRAFT_MAX_ROWS || V < 1) return GRAFT_EINVAL;
    if (B == 0) return GRAFT_OK;
    if (!tok || !parent || !depth || !status) return GRAFT_EINVAL;
    hipLaunchKernelGGL(k_check_tree, dim3((B + kReq - 1) / kReq), dim3(graft::kWave * kReq), 0, stream, B, T1, V,
                       tok, parent, depth, status);
    return launch_status();
}

}  // extern "C"
