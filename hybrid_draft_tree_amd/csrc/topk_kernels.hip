// Row-wise top-k of vocab-wide target logits: the step that moves almost every
// byte of a Graft step (section 二, gear 3: the target's top-k at every verified
// position feeds both the greedy check and the matrix update).
//
// Order: value descending, ties -> lower id, -0 == +0.  The kernel is an HBM
// stream: no MFMA (nothing is a contraction).
//
// Phase A: each wavefront owns a contiguous range of one row and streams it
//   with 16-byte loads (8 bf16 or 4 fp32 per lane, U loads in flight).  A
//   wave-uniform threshold -- the key of the wave's current 8th-best value --
//   filters groups with a few packed integer ops; the rare groups that pass
//   are compacted into LDS with a ballot, and merged into the wave's exact
//   top-8 (8 rounds of wave-wide max) when 64 are pending.  The range's top-8
//   goes to the workspace as 64-bit (value, id) ranks.
// Phase B: one wavefront per row merges the ranges' candidates into the final
//   top-k (and combines online-softmax statistics for probabilities).
#include "device_utils.hpp"
#include "launchers.hpp"

namespace graft {
namespace {

constexpr int kWavesPerBlockA = 4;
constexpr int kLoadsInFlight = 4;  // U: 16-byte loads per lane per batch
constexpr int kCap = kWave * (kLoadsInFlight + 1);
constexpr int kTop = 8;

typedef short short2v __attribute__((ext_vector_type(2)));
typedef int int4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ short2v as_s2(uint32_t x) { return __builtin_bit_cast(short2v, x); }
__device__ __forceinline__ uint32_t as_u32(short2v x) { return __builtin_bit_cast(uint32_t, x); }

template <bool NT>
__device__ __forceinline__ uint4 load16(const uint4 *p) {
    if constexpr (NT) {
        int4v v = __builtin_nontemporal_load((const int4v *)p);
        return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
    } else {
        return *p;
    }
}

// ---- element traits ---------------------------------------------------------------------
// A wave-local rank packs (value key, local offset) so that unsigned max is the
// ranking order; 0 marks "no candidate".
struct Bf16Traits {
    using Rank = uint32_t;
    static constexpr int kPerGroup = 8;
    static constexpr int kMaxRange = 65536;  // offsets fit 16 bits
    __device__ static uint32_t elem(const uint4 &d, int e) {
        const uint32_t w = e < 2 ? d.x : e < 4 ? d.y : e < 6 ? d.z : d.w;
        return (e & 1) ? (w >> 16) : (w & 0xffffu);
    }
    __device__ static uint32_t load_scalar(const void *row, int i) {
        return ((const uint16_t *)row)[i];
    }
    __device__ static int32_t key(uint32_t raw) { return bf16_key(raw); }
    __device__ static float value(uint32_t raw) { return __uint_as_float(raw << 16); }
    __device__ static Rank make(uint32_t raw, int off) {
        return ((uint32_t)(bf16_key(raw) + 0x8000) << 16) | (0xffffu - (uint32_t)off);
    }
    __device__ static int32_t rank_key(Rank r) { return (int32_t)(r >> 16) - 0x8000; }
    __device__ static uint64_t to_row_rank(Rank r, int col0) {
        const int off = (int)(0xffffu - (r & 0xffffu));
        return rank64(rank_key(r) * 65536, (uint32_t)(col0 + off));
    }
    // Superset filter: does any element of the group have key >= thr?
    __device__ static bool group_pass(const uint4 &d, int thr) {
        if (thr >= 1) {
            // keys >= thr >= 1 are positive values, whose raw bits order as int16
            short2v m = __builtin_elementwise_max(__builtin_elementwise_max(as_s2(d.x), as_s2(d.y)),
                                                  __builtin_elementwise_max(as_s2(d.z), as_s2(d.w)));
            const short t = (short)(thr - 1);
            const short2v T = {t, t};
            return as_u32(__builtin_elementwise_max(m, T)) != as_u32(T);
        }
        bool p = false;
#pragma unroll
        for (int e = 0; e < 8; ++e) p |= bf16_key(elem(d, e)) >= thr;
        return p;
    }
};

struct F32Traits {
    using Rank = uint64_t;
    static constexpr int kPerGroup = 4;
    static constexpr int kMaxRange = 65536 * 4;  // group index fits 16 bits
    __device__ static uint32_t elem(const uint4 &d, int e) {
        return e == 0 ? d.x : e == 1 ? d.y : e == 2 ? d.z : d.w;
    }
    __device__ static uint32_t load_scalar(const void *row, int i) {
        return ((const uint32_t *)row)[i];
    }
    __device__ static int32_t key(uint32_t raw) { return f32_key(raw); }
    __device__ static float value(uint32_t raw) { return __uint_as_float(raw); }
    __device__ static Rank make(uint32_t raw, int off) { return rank64(f32_key(raw), (uint32_t)off); }
    __device__ static int32_t rank_key(Rank r) { return rank64_key(r); }
    __device__ static uint64_t to_row_rank(Rank r, int col0) {
        return rank64(rank64_key(r), (uint32_t)col0 + rank64_id(r));
    }
    __device__ static bool group_pass(const uint4 &d, int thr) {
        if (thr >= 1) {
            const int m = max(max((int)d.x, (int)d.y), max((int)d.z, (int)d.w));
            return m >= thr;
        }
        return f32_key(d.x) >= thr || f32_key(d.y) >= thr || f32_key(d.z) >= thr ||
               f32_key(d.w) >= thr;
    }
};

template <typename Rank>
__device__ __forceinline__ Rank wave_max_rank(Rank v) {
    if constexpr (sizeof(Rank) == 4)
        return wave_max_u32(v);
    else
        return wave_max_u64(v);
}

// Merge the lanes' candidate ranks c[0..N-1] (0 = none) into the wave's exact
// top-8, held as `top` in lanes 0..7 (descending).  Returns the new 8th best.
template <typename Rank, int N>
__device__ __forceinline__ Rank merge_top8(Rank (&c)[N], Rank &top) {
    const int lane = lane_id();
    Rank extra = lane < kTop ? top : (Rank)0;
    Rank newtop = 0, kth = 0;
#pragma unroll
    for (int j = 0; j < kTop; ++j) {
        Rank lm = extra;
#pragma unroll
        for (int e = 0; e < N; ++e) lm = c[e] > lm ? c[e] : lm;
        const Rank M = wave_max_rank<Rank>(lm);
        if (lane == j) newtop = M;
        kth = M;
        if (extra == M) extra = 0;
#pragma unroll
        for (int e = 0; e < N; ++e)
            if (c[e] == M) c[e] = 0;
    }
    top = newtop;
    return kth;
}

struct SoftStats {
    float m = -INFINITY;
    float s = 0.0f;
    __device__ void add(float v) {
        if (v > m) {
            s = (m == -INFINITY) ? 0.0f : s * __expf(m - v);
            m = v;
        }
        s += __expf(v - m);
    }
};

template <typename TR, bool PROB, bool NT>
__global__ __launch_bounds__(kWave *kWavesPerBlockA) void k_topk_phase_a(
    const void *__restrict__ logits, int64_t n_rows, int V, int S, int chunk,
    uint64_t *__restrict__ partials, float2 *__restrict__ stats) {
    using Rank = typename TR::Rank;
    constexpr int EPG = TR::kPerGroup;
    constexpr int ESZ = 16 / EPG;
    __shared__ uint4 s_data[kWavesPerBlockA][kCap];
    __shared__ uint16_t s_gidx[kWavesPerBlockA][kCap];

    const int lane = lane_id();
    const int wv = threadIdx.x >> 6;
    const int64_t w = (int64_t)blockIdx.x * kWavesPerBlockA + wv;
    if (w >= n_rows * S) return;
    const int64_t row = w / S;
    const int split = (int)(w - row * S);
    const int c0 = split * chunk;
    const int c1 = min(V, c0 + chunk);
    const char *rowp = (const char *)logits + (size_t)row * (size_t)V * ESZ;

    // head (until 16-byte alignment), body (16-byte groups), tail
    const uintptr_t a_addr = (uintptr_t)(rowp + (size_t)c0 * ESZ);
    int head = (int)(((16u - (uint32_t)(a_addr & 15u)) & 15u) / ESZ);
    head = min(head, c1 - c0);
    const int a0 = c0 + head;
    const int ng = (c1 - a0) / EPG;
    const int a1 = a0 + ng * EPG;
    const int ntail = c1 - a1;

    Rank top = 0;   // lanes 0..7: the wave's top-8, descending
    Rank kth = 0;   // the 8th best (uniform); 0 while fewer than 8 candidates
    int thr = INT_MIN;
    SoftStats st;

    {  // head and tail elements: at most EPG-1 each
        Rank c[1] = {0};
        uint32_t raw = 0;
        bool have = false;
        int off = 0;
        if (lane < head) {
            off = lane;
            have = true;
        } else if (lane >= 16 && lane - 16 < ntail) {
            off = (a1 - c0) + (lane - 16);
            have = true;
        }
        if (have) {
            raw = TR::load_scalar(rowp, c0 + off);
            c[0] = TR::make(raw, off);
            if constexpr (PROB) st.add(TR::value(raw));
        }
        if (ballot(have)) {
            kth = merge_top8<Rank, 1>(c, top);
            thr = kth ? TR::rank_key(kth) : INT_MIN;
        }
    }

    const uint4 *vp = (const uint4 *)(rowp + (size_t)a0 * ESZ);
    uint4 *sd = s_data[wv];
    uint16_t *sg = s_gidx[wv];
    int count = 0;

    auto process = [&]() {
        for (int base = 0; base < count; base += kWave) {
            const int gi = base + lane;
            Rank c[EPG];
            bool any = false;
            if (gi < count) {
                const uint4 d = sd[gi];
                const int goff = head + (int)sg[gi] * EPG;
#pragma unroll
                for (int e = 0; e < EPG; ++e) {
                    const Rank r = TR::make(TR::elem(d, e), goff + e);
                    c[e] = r > kth ? r : (Rank)0;
                    any |= c[e] != 0;
                }
            } else {
#pragma unroll
                for (int e = 0; e < EPG; ++e) c[e] = 0;
            }
            if (ballot(any)) kth = merge_top8<Rank, EPG>(c, top);
        }
        count = 0;
        thr = kth ? TR::rank_key(kth) : INT_MIN;
    };

    for (int g0 = 0; g0 < ng; g0 += kWave * kLoadsInFlight) {
        uint4 d[kLoadsInFlight];
#pragma unroll
        for (int u = 0; u < kLoadsInFlight; ++u) {
            const int gi = g0 + u * kWave + lane;
            if (gi < ng)
                d[u] = load16<NT>(vp + gi);
            else
                d[u] = make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < kLoadsInFlight; ++u) {
            const int gi = g0 + u * kWave + lane;
            const bool inb = gi < ng;
            if constexpr (PROB) {
                if (inb) {
#pragma unroll
                    for (int e = 0; e < EPG; ++e) st.add(TR::value(TR::elem(d[u], e)));
                }
            }
            const bool pass = inb && (thr == INT_MIN || TR::group_pass(d[u], thr));
            const uint64_t bal = ballot(pass);
            if (bal) {
                if (pass) {
                    const int pos = count + lanes_below(bal);
                    sd[pos] = d[u];
                    sg[pos] = (uint16_t)gi;
                }
                count += __popcll(bal);
            }
        }
        if (count > kCap - kWave * kLoadsInFlight) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            process();
        }
    }
    if (count) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        process();
    }

    if (lane < kTop) partials[w * kTop + lane] = top ? TR::to_row_rank(top, c0) : 0ull;
    if constexpr (PROB) {
        const float M = wave_max_f32(st.m);
        const float s = (st.m == -INFINITY) ? 0.0f : st.s * __expf(st.m - M);
        const float Ssum = wave_sum_f32(s);
        if (lane == 0) stats[w] = make_float2(M, Ssum);
    }
}

// Phase B: one wavefront per row.
constexpr int kRowsPerBlockB = 4;
constexpr int kMaxPerLaneB = 4;  // S * 8 <= 256 candidates per row

__global__ __launch_bounds__(kWave *kRowsPerBlockB) void k_topk_phase_b(
    const uint64_t *__restrict__ partials, const float2 *__restrict__ stats, int64_t n_rows, int S,
    int k, int32_t *__restrict__ topk, float *__restrict__ prob) {
    const int lane = lane_id();
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlockB + (threadIdx.x >> 6);
    if (row >= n_rows) return;
    const int n = S * kTop;
    uint64_t c[kMaxPerLaneB];
#pragma unroll
    for (int i = 0; i < kMaxPerLaneB; ++i) {
        const int j = i * kWave + lane;
        c[i] = j < n ? partials[row * n + j] : 0ull;
    }
    uint64_t top = 0;
    merge_top8<uint64_t, kMaxPerLaneB>(c, top);
    if (lane < k) topk[row * k + lane] = top ? (int32_t)rank64_id(top) : -1;
    if (prob) {
        const float2 sv = lane < S ? stats[row * S + lane] : make_float2(-INFINITY, 0.0f);
        const float M = wave_max_f32(sv.x);
        const float s = (sv.x == -INFINITY) ? 0.0f : sv.y * __expf(sv.x - M);
        const float Ssum = wave_sum_f32(s);
        if (lane < k) {
            const float x = key_to_f32(rank64_key(top));
            prob[row * k + lane] = top ? __expf(x - M) / Ssum : 0.0f;
        }
    }
}

template <typename TR>
void launch_phase_a(bool want_prob, const TopkPlan &p, const void *logits, uint64_t *partials,
                    float2 *stats, hipStream_t s) {
    const int64_t waves = p.n_rows * p.splits;
    const dim3 grid((unsigned)((waves + kWavesPerBlockA - 1) / kWavesPerBlockA));
    const dim3 block(kWave * kWavesPerBlockA);
    if (want_prob)
        hipLaunchKernelGGL((k_topk_phase_a<TR, true, true>), grid, block, 0, s, logits, p.n_rows, p.V,
                           p.splits, p.chunk, partials, stats);
    else
        hipLaunchKernelGGL((k_topk_phase_a<TR, false, true>), grid, block, 0, s, logits, p.n_rows,
                           p.V, p.splits, p.chunk, partials, stats);
}

}  // namespace

TopkPlan plan_topk(int64_t n_rows, int V, int dtype) {
    TopkPlan p;
    p.n_rows = n_rows;
    p.V = V;
    const int max_range = dtype == GRAFT_DTYPE_BF16 ? Bf16Traits::kMaxRange : F32Traits::kMaxRange;
    // Enough ranges to fill 256 CUs x 16 waves, each range >= 4096 elements,
    // and at most 32 ranges per row (phase B holds 8 candidates per range).
    const int64_t target_waves = 256 * 16;
    int S = (int)((target_waves + n_rows - 1) / (n_rows > 0 ? n_rows : 1));
    S = S < 1 ? 1 : S;
    const int by_len = (V + 4095) / 4096;
    if (S > by_len) S = by_len;
    const int min_s = (V + max_range - 1) / max_range;
    if (S < min_s) S = min_s;
    if (S > 32) S = 32;
    int chunk = (V + S - 1) / S;
    chunk = (chunk + 7) / 8 * 8;
    S = (V + chunk - 1) / chunk;
    p.splits = S;
    p.chunk = chunk;
    p.partial_bytes = (size_t)n_rows * S * kTop * sizeof(uint64_t);
    p.stats_bytes = (size_t)n_rows * S * sizeof(float2);
    return p;
}

void launch_topk(const TopkPlan &p, int dtype, const void *logits, int k, int32_t *topk,
                 float *prob, void *ws, hipStream_t s) {
    if (p.n_rows <= 0) return;
    uint64_t *partials = (uint64_t *)ws;
    float2 *stats = (float2 *)((char *)ws + ((p.partial_bytes + 255) / 256) * 256);
    if (dtype == GRAFT_DTYPE_BF16)
        launch_phase_a<Bf16Traits>(prob != nullptr, p, logits, partials, stats, s);
    else
        launch_phase_a<F32Traits>(prob != nullptr, p, logits, partials, stats, s);
    const dim3 gridb((unsigned)((p.n_rows + kRowsPerBlockB - 1) / kRowsPerBlockB));
    hipLaunchKernelGGL(k_topk_phase_b, gridb, dim3(kWave * kRowsPerBlockB), 0, s, partials, stats,
                       p.n_rows, p.splits, k, topk, prob);
}

}  // namespace graft
