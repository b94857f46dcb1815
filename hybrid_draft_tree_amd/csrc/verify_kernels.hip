// Online update of the continuation matrix (section 二, gear 3 of the news
// write-up of arXiv 2605.20104): the target's top-k at every verified position,
// accepted or rejected, overwrites the row of that position's input token (this
// kernel serves the prompt ingest and the separate-call path; the fused verify
// launch updates the matrix itself, topk_kernels.hip).  Also the coverage-gain
// diagnostic of section 三.
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

// Coverage gain (section 三 of the news write-up): for each request (one
// wavefront, lane c = row c), the retrieved rows whose token is new under their
// parent row v -- no kept draft sibling carries it, no earlier retrieved sibling
// either -- add the target's softmax probability of that token at row v, from
// the row's logit and its softmax statistics (largest value, normaliser).
constexpr int kCovReqPerBlock = 4;

__global__ __launch_bounds__(kWave *kCovReqPerBlock) void k_coverage(CoverageArgs a) {
    const int lane = lane_id();
    const int b = blockIdx.x * kCovReqPerBlock + (int)(threadIdx.x >> 6);
    if (b >= a.B) return;
    const int T1 = a.T1;
    const bool row = lane < T1;
    const size_t o = (size_t)b * T1 + lane;
    const int src = row ? (int)a.row_src[o] : GRAFT_ROW_EMPTY;
    const int t = row ? a.tok[o] : -1;
    const int v = row ? a.parent[o] : -1;
    const bool ret = src == GRAFT_ROW_RETRIEVED && v >= 0 && v < T1 && t >= 0 && t < a.V;
    bool dup = false;
    for (int d = 0; d < T1; ++d) {
        const int sd = readlane_i32(src, d);
        const int td = readlane_i32(t, d);
        const int vd = readlane_i32(v, d);
        dup |= vd == v && td == t &&
               (sd == GRAFT_ROW_DRAFT || (sd == GRAFT_ROW_RETRIEVED && d < lane));
    }
    float p = 0.0f;
    if (ret && !dup) {
        const size_t r = (size_t)b * T1 + v;
        const float2 st = *(const float2 *)&a.row_stats[2 * r];
        const size_t i = r * (size_t)a.V + t;
        const float x = a.dtype == GRAFT_DTYPE_BF16
                            ? __uint_as_float((uint32_t)((const uint16_t *)a.logits)[i] << 16)
                            : ((const float *)a.logits)[i];
        p = expf(x - st.x) / st.y;
    }
    const float g = wave_sum_f32(p);
    if (lane == 0) a.gain[b] = g;
}

// Zero fill of a scratch range with 16-byte vector stores (a kernel rather
// than a memset node, so the clear can sit inside a captured graph).
constexpr int kZeroThreads = 256;
constexpr int64_t kZeroMaxBlocks = 1024;

__global__ __launch_bounds__(kZeroThreads) void k_zero(uint4 *__restrict__ p, int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * kZeroThreads;
    for (int64_t i = (int64_t)blockIdx.x * kZeroThreads + threadIdx.x; i < n16; i += stride)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Streaming-read ceiling (a measurement aid, no part of the Graft step): one
// workgroup of kStreamWaves wavefronts per row, the verify launch's geometry.
// Wavefront w reads the row's 1 KB blocks w, w + kStreamWaves, ... with 16-byte
// non-temporal loads, two blocks per batch with the next batch in flight, and
// folds every 32-bit word into an XOR so that no load can be dropped; the row's
// XOR goes to sink[row].  Loads past the row's last 16-byte group are skipped.
constexpr int kStreamWaves = 4;

__device__ __forceinline__ uint4 stream_load(const uint4 *p, int64_t g, int64_t groups) {
    if (g >= groups) return make_uint4(0u, 0u, 0u, 0u);
    typedef int int4v __attribute__((ext_vector_type(4)));
    const int4v v = __builtin_nontemporal_load((const int4v *)(p + g));
    return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}

__global__ __launch_bounds__(kWave *kStreamWaves) void k_stream_read(const uint4 *__restrict__ data, int64_t groups,
                                                                      uint32_t *__restrict__ sink) {
    __shared__ uint32_t s_x[kStreamWaves];
    const int lane = lane_id();
    const int wv = (int)(threadIdx.x / kWave);
    const uint4 *p = data + (int64_t)blockIdx.x * groups;
    const int64_t nblk = (groups + kWave - 1) / kWave;
    constexpr int64_t kStep = kStreamWaves;
    int64_t b = wv;
    uint4 c0 = stream_load(p, b * kWave + lane, groups);
    uint4 c1 = stream_load(p, (b + kStep) * kWave + lane, groups);
    uint32_t x = 0;
    for (; b < nblk; b += 2 * kStep) {
        const uint4 n0 = stream_load(p, (b + 2 * kStep) * kWave + lane, groups);
        const uint4 n1 = stream_load(p, (b + 3 * kStep) * kWave + lane, groups);
        x ^= c0.x ^ c0.y ^ c0.z ^ c0.w ^ c1.x ^ c1.y ^ c1.z ^ c1.w;
        c0 = n0;
        c1 = n1;
    }
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o);
    if (lane == 0) s_x[wv] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
#pragma unroll
        for (int w = 0; w < kStreamWaves; ++w) r ^= s_x[w];
        sink[blockIdx.x] = r;
    }
}

}  // namespace

void launch_stream_read(const void *data, int64_t n_rows, int64_t row_bytes, uint32_t *sink, hipStream_t s) {
    if (n_rows <= 0) return;
    hipLaunchKernelGGL(k_stream_read, dim3((unsigned)n_rows), dim3(kWave * kStreamWaves), 0, s, (const uint4 *)data,
                       row_bytes / 16, sink);
}

void launch_zero(void *p, size_t bytes, hipStream_t s) {
    const int64_t n16 = (int64_t)(bytes / 16);
    if (n16 <= 0) return;
    int64_t blocks = (n16 + kZeroThreads - 1) / kZeroThreads;
    blocks = blocks < kZeroMaxBlocks ? blocks : kZeroMaxBlocks;
    hipLaunchKernelGGL(k_zero, dim3((unsigned)blocks), dim3(kZeroThreads), 0, s, (uint4 *)p, n16);
}

void launch_coverage(const CoverageArgs &a, hipStream_t s) {
    if (a.B <= 0) return;
    const int blocks = (a.B + kCovReqPerBlock - 1) / kCovReqPerBlock;
    hipLaunchKernelGGL(k_coverage, dim3(blocks), dim3(kWave * kCovReqPerBlock), 0, s, a);
}

void launch_update(int64_t n_rows, int V, int k, const int32_t *topk, const float *prob,
                   const int32_t *row_tok, int32_t *table, float *table_prob, hipStream_t s) {
    if (n_rows <= 0) return;
    hipLaunchKernelGGL(k_update, dim3(1), dim3(kUpdThreads), 0, s, n_rows, V, k, topk, prob, row_tok,
                       table, table_prob);
}

}  // namespace graft
