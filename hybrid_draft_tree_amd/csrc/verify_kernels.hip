// Online update of the continuation matrix (section 二, gear 3 of the news
// write-up of arXiv 2605.20104): the target's top-k at every verified position,
// accepted or rejected, overwrites the row of that position's input token.  The
// acceptance walk lives in the top-k kernel's epilogue (topk_kernels.hip).
#include "device_utils.hpp"
#include "launchers.hpp"

namespace graft {
namespace {

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
        // the next block may overwrite the same rows: order this block's stores first
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
}

}  // namespace

void launch_update(int64_t n_rows, int V, int k, const int32_t *topk, const float *prob,
                   const int32_t *row_tok, int32_t *table, float *table_prob, hipStream_t s) {
    if (n_rows <= 0) return;
    hipLaunchKernelGGL(k_update, dim3(1), dim3(kUpdThreads), 0, s, n_rows, V, k, topk, prob, row_tok,
                       table, table_prob);
}

}  // namespace graft
