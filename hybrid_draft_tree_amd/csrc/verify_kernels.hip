// Verification-side kernels of the Graft step (section 二, gear 3 of the news
// write-up of arXiv 2605.20104): the strict greedy acceptance walk over the
// flattened hybrid tree, and the online update of the continuation matrix with
// the target's top-k at every verified position.
#include "device_utils.hpp"
#include "launchers.hpp"

namespace graft {
namespace {

constexpr int kReqPerBlock = 4;

// One wavefront per request; lane f is flattened row f.
__global__ __launch_bounds__(kWave *kReqPerBlock) void k_accept(
    int B, int T1, int k, const int32_t *__restrict__ topk, const int32_t *__restrict__ tok,
    const int32_t *__restrict__ parent, const int32_t *__restrict__ depth,
    int32_t *__restrict__ accept_len, int32_t *__restrict__ accept_idx, int dmax,
    int32_t *__restrict__ bonus, int32_t *__restrict__ base_pos_io) {
    __shared__ int s_path[kReqPerBlock][kWave];
    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    const int b = blockIdx.x * kReqPerBlock + w;
    const bool live = b < B;
    const bool row = live && lane < T1;
    const size_t o = (size_t)b * T1 + lane;
    const int g = row ? topk[o * k] : -1;
    const int t = row ? tok[o] : -1;
    const int p = (row && lane > 0) ? parent[o] : -1;
    const int d = row ? depth[o] : 0;
    int *sp = s_path[w];
    sp[lane] = -1;

    // edge check: the row's token equals the greedy token at its parent row
    const int gp = __shfl(g, p >= 0 ? p : lane);
    bool ok = row && (lane == 0 || (p >= 0 && t == gp));
    // accepted iff every edge on the path to the root is correct, and the
    // ancestor-or-self mask of the row: both by pointer doubling
    int a = p;
    uint64_t A = row ? ((1ull << lane) | (a >= 0 ? (1ull << a) : 0ull)) : 0ull;
#pragma unroll
    for (int r = 0; r < 6; ++r) {
        const int src = a >= 0 ? a : lane;
        const int oka = __shfl((int)ok, src);
        const uint64_t Aa = shfl_u64(A, src);
        const int aa = __shfl(a, src);
        if (a >= 0) {
            ok = ok && oka;
            A |= Aa;
            a = aa;
        }
    }
    // deepest accepted row, ties -> lowest row
    const int key = ok ? (d << 8) | (255 - lane) : -1;
    const int best = wave_max_i32(key);
    const int fstar = 255 - (best & 255);
    const int len = best >> 8;
    const uint64_t path = shfl_u64(A, fstar);
    const int gstar = __shfl(g, fstar);
    __syncthreads();
    if (live && lane > 0 && ((path >> lane) & 1ull) && d >= 1 && d <= kWave) sp[d - 1] = lane;
    __syncthreads();
    if (!live) return;
    for (int j = lane; j < dmax; j += kWave)
        accept_idx[(size_t)b * dmax + j] = (j < len && j < kWave) ? sp[j] : -1;
    if (lane == 0) {
        accept_len[b] = len;
        bonus[b] = gstar;
        if (base_pos_io) base_pos_io[b] += len + 1;
    }
}

// Matrix update: one workgroup; rows in blocks of kHashRows, each resolved with
// an LDS hash table keyed by token that keeps the highest row index (atomic
// max, so the outcome does not depend on arrival order).  Blocks are applied in
// order, so later rows overwrite earlier ones as a sequential pass would.
constexpr int kUpdThreads = 1024;
constexpr int kHashRows = 4096;
constexpr int kHashSlots = 8192;
constexpr int kRowsPerThread = kHashRows / kUpdThreads;

__device__ __forceinline__ uint32_t hash_slot(int x) {
    return ((uint32_t)x * 2654435761u) >> (32 - 13);
}

__global__ __launch_bounds__(kUpdThreads) void k_update(int64_t n_rows, int V, int k,
                                                        const int32_t *__restrict__ topk,
                                                        const float *__restrict__ prob,
                                                        const int32_t *__restrict__ row_tok,
                                                        int32_t *__restrict__ table,
                                                        float *__restrict__ table_prob) {
    __shared__ int s_key[kHashSlots];
    __shared__ int s_max[kHashSlots];
    for (int64_t blk = 0; blk < n_rows; blk += kHashRows) {
        const int nb = (int)min((int64_t)kHashRows, n_rows - blk);
        for (int i = threadIdx.x; i < kHashSlots; i += kUpdThreads) {
            s_key[i] = -1;
            s_max[i] = -1;
        }
        __syncthreads();
        int slot[kRowsPerThread];
        int tokv[kRowsPerThread];
#pragma unroll
        for (int r = 0; r < kRowsPerThread; ++r) {
            const int P = threadIdx.x + r * kUpdThreads;
            slot[r] = -1;
            tokv[r] = -1;
            const int x = P < nb ? row_tok[blk + P] : -1;
            if (x >= 0 && x < V) {  // out-of-range tokens are skipped
                tokv[r] = x;
                uint32_t h = hash_slot(x);
                for (;;) {
                    const int old = atomicCAS(&s_key[h], -1, x);
                    if (old == -1 || old == x) break;
                    h = (h + 1) & (kHashSlots - 1);
                }
                atomicMax(&s_max[h], P);
                slot[r] = (int)h;
            }
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < kRowsPerThread; ++r) {
            const int P = threadIdx.x + r * kUpdThreads;
            if (slot[r] >= 0 && s_max[slot[r]] == P) {
                const int64_t src = blk + P;
                const size_t dst = (size_t)tokv[r] * k;
                for (int j = 0; j < k; ++j) table[dst + j] = topk[src * k + j];
                if (table_prob)
                    for (int j = 0; j < k; ++j) table_prob[dst + j] = prob[src * k + j];
            }
        }
        __threadfence();
        __syncthreads();
    }
}

}  // namespace

void launch_accept(int B, int T1, int k, const int32_t *topk, const int32_t *tok,
                   const int32_t *parent, const int32_t *depth, int32_t *accept_len,
                   int32_t *accept_idx, int dmax, int32_t *bonus, int32_t *base_pos_io,
                   hipStream_t s) {
    if (B <= 0) return;
    hipLaunchKernelGGL(k_accept, dim3((B + kReqPerBlock - 1) / kReqPerBlock),
                       dim3(kWave * kReqPerBlock), 0, s, B, T1, k, topk, tok, parent, depth,
                       accept_len, accept_idx, dmax, bonus, base_pos_io);
}

void launch_update(int64_t n_rows, int V, int k, const int32_t *topk, const float *prob,
                   const int32_t *row_tok, int32_t *table, float *table_prob, hipStream_t s) {
    if (n_rows <= 0) return;
    hipLaunchKernelGGL(k_update, dim3(1), dim3(kUpdThreads), 0, s, n_rows, V, k, topk, prob, row_tok,
                       table, table_prob);
}

}  // namespace graft
