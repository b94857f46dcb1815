// Row-wise top-k of vocab-wide target logits: the step that moves almost every
// byte of a Graft step (section 二, gear 3: the target's top-k at every verified
// position feeds both the greedy check and the matrix update).
//
// Order: value descending, ties -> lower id, -0 == +0.  The kernel is an HBM
// stream: no MFMA (nothing is a contraction).
//
// Each wavefront owns a contiguous range of one row and streams it
//   with 16-byte loads (8 bf16 or 4 fp32 per lane, U loads in flight).  A
//   wave-uniform threshold -- the key of the wave's current 8th-best value --
//   filters groups with a few packed integer ops; the rare groups that pass
//   are compacted into LDS with a ballot, and merged into the wave's exact
//   top-8 (8 rounds of wave-wide max) when 64 are pending.  The range's top-8
//   goes to the workspace as 64-bit (value, id) ranks.
// Epilogue: the last range of a row to finish merges the ranges' candidates
//   into the final top-k (and combines online-softmax statistics); with the
//   acceptance walk fused, the last row of a request to be merged runs the
//   walk for that request.  One launch per call.
#include "device_utils.hpp"
#include "launchers.hpp"

namespace graft {
namespace {

constexpr int kWavesPerBlockA = 4;
constexpr int kLoadsInFlight = 2;  // U: 16-byte loads per lane per batch
template <int U>
constexpr int kCapOf = kWave * (U + 1);  // pending groups per wave
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
    // Largest raw bit pattern of the group read as int16 (equals the largest key
    // whenever that is positive).
    __device__ static int raw_max(const uint4 &d) {
        const short2v m = __builtin_elementwise_max(
            __builtin_elementwise_max(as_s2(d.x), as_s2(d.y)), __builtin_elementwise_max(as_s2(d.z), as_s2(d.w)));
        return max((int)m.x, (int)m.y);
    }
    static constexpr int kRawMin = -32768;
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
    __device__ static int raw_max(const uint4 &d) {
        return max(max((int)d.x, (int)d.y), max((int)d.z, (int)d.w));
    }
    static constexpr int kRawMin = INT_MIN;
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

// Same result as merge_top8, cheaper when few candidates are live: if they fit
// one per lane next to the current top-8, compact them through the wave's LDS
// scratch (64 entries) and extract the 8 largest with one value per lane.
template <typename Rank, int N>
__device__ __forceinline__ Rank merge_top8_compact(Rank (&c)[N], Rank &top, Rank *scratch) {
    const int lane = lane_id();
    uint64_t bal[N];
    int total = 0;
#pragma unroll
    for (int e = 0; e < N; ++e) {
        bal[e] = ballot(c[e] != 0);
        total += __popcll(bal[e]);
    }
    if (total + kTop > kWave) return merge_top8<Rank, N>(c, top);
    int base = 0;
#pragma unroll
    for (int e = 0; e < N; ++e) {
        if (c[e] != 0) scratch[base + lanes_below(bal[e])] = c[e];
        base += __popcll(bal[e]);
    }
    if (lane < kTop) scratch[total + lane] = top;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    Rank v = lane < total + kTop ? scratch[lane] : (Rank)0;
    __builtin_amdgcn_wave_barrier();
    Rank newtop = 0, kth = 0;
#pragma unroll
    for (int j = 0; j < kTop; ++j) {
        const Rank M = wave_max_rank<Rank>(v);
        if (lane == j) newtop = M;
        kth = M;
        if (v == M) v = 0;
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

// Merge the ranges' candidates of one row into its final top-k (+ softmax
// probabilities), one wavefront.
constexpr int kMaxPerLaneB = 4;  // S * 8 <= 256 candidates per row

__device__ __forceinline__ void merge_row(const TopkArgs &a, int64_t row) {
    const int lane = lane_id();
    const int n = a.S * kTop;
    uint64_t c[kMaxPerLaneB];
#pragma unroll
    for (int i = 0; i < kMaxPerLaneB; ++i) {
        const int j = i * kWave + lane;
        c[i] = j < n ? ld_agent(&a.partials[row * n + j]) : 0ull;
    }
    uint64_t top = 0;
    merge_top8<uint64_t, kMaxPerLaneB>(c, top);
    if (lane < a.k) st_agent(&a.topk[row * a.k + lane], top ? (int32_t)rank64_id(top) : -1);
    if (a.prob) {
        float2 sv = make_float2(-INFINITY, 0.0f);
        if (lane < a.S) {
            const uint64_t u = ld_agent(&a.stats[row * a.S + lane]);
            sv = make_float2(__uint_as_float((uint32_t)u), __uint_as_float((uint32_t)(u >> 32)));
        }
        const float M = wave_max_f32(sv.x);
        const float s = (sv.x == -INFINITY) ? 0.0f : sv.y * __expf(sv.x - M);
        const float Ssum = wave_sum_f32(s);
        if (lane < a.k) {
            const float x = key_to_f32(rank64_key(top));
            const float pj = top ? __expf(x - M) / Ssum : 0.0f;
            st_agent((int32_t *)&a.prob[row * a.k + lane], __float_as_int(pj));
        }
    }
}

// Strict greedy acceptance walk of request b (section 二, gear 3), one wavefront;
// lane f is flattened row f.  A row is accepted iff every row on its path from
// the root carries the greedy token of its parent row; the deepest accepted row
// wins, ties -> lowest row.
__device__ __forceinline__ void accept_walk(const VerifyArgs &v, int k, int32_t *topk, int b) {
    const int lane = lane_id();
    const int T1 = v.T1;
    const bool row = lane < T1;
    const size_t o = (size_t)b * T1 + lane;
    const int g = row ? ld_agent(&topk[o * k]) : -1;
    const int t = row ? v.tok[o] : -1;
    const int p = (row && lane > 0) ? v.parent[o] : -1;
    const int d = row ? v.depth[o] : 0;
    const int gp = __shfl(g, p >= 0 ? p : lane);
    bool ok = row && (lane == 0 || (p >= 0 && t == gp));
    // AND of the edge checks along the path and the ancestor-or-self mask, by
    // pointer doubling over parent links
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
    const int key = ok ? (d << 8) | (255 - lane) : -1;
    const int best = wave_max_i32(key);
    const int fstar = 255 - (best & 255);
    const int len = best >> 8;
    const uint64_t path = shfl_u64(A, fstar);
    const int gstar = __shfl(g, fstar);
    // the path's rows have depths 1..len: row at depth d goes to slot d-1
    if (row && lane > 0 && ((path >> lane) & 1ull) && d >= 1 && d <= v.dmax)
        v.accept_idx[(size_t)b * v.dmax + d - 1] = lane;
    for (int j = lane; j < v.dmax; j += kWave)
        if (j >= len) v.accept_idx[(size_t)b * v.dmax + j] = -1;
    if (lane == 0) {
        v.accept_len[b] = len;
        v.bonus[b] = gstar;
        if (v.base_pos_io) v.base_pos_io[b] += len + 1;
    }
}

// Matrix update for the rows of request b (one wavefront, lane f = row b*T1+f):
// a row writes its top-k into the matrix row of its token iff it is the last
// row of the whole batch holding that token (highest row wins), then clears
// that token's registration.  Called once every row is registered and the
// request's rows are merged.
__device__ __forceinline__ void update_request(const VerifyArgs &v, int V, int k, int32_t *topk,
                                               const float *prob, int b) {
    const int lane = lane_id();
    if (lane >= v.T1) return;
    const int64_t P = (int64_t)b * v.T1 + lane;
    const int t = v.tok[P];
    if (t < 0 || t >= V) return;
    if (ld_agent(&v.last_occ[t]) != (int32_t)(P + 1)) return;
    for (int j = 0; j < k; ++j) v.table[(size_t)t * k + j] = ld_agent(&topk[P * k + j]);
    if (v.table_prob)
        for (int j = 0; j < k; ++j)
            v.table_prob[(size_t)t * k + j] = __int_as_float(ld_agent((const int32_t *)&prob[P * k + j]));
    st_agent(&v.last_occ[t], 0);
}

// Hand-off between "request b accepted" and "every row registered": the second
// of the two arrivals runs request b's update.  Returns true for the second.
__device__ __forceinline__ bool handoff_second(const VerifyArgs &v, int b) {
    uint32_t prev = 0;
    if (lane_id() == 0) prev = count_in(&v.handoff[b]);
    prev = (uint32_t)readlane_i32((int)prev, 0);
    return prev == 1u;
}

template <typename TR, bool PROB, bool ACCEPT, bool NT, int U = kLoadsInFlight>
__global__ __launch_bounds__(kWave *kWavesPerBlockA) void k_topk_rows(TopkArgs a, VerifyArgs v) {
    using Rank = typename TR::Rank;
    constexpr int EPG = TR::kPerGroup;
    constexpr int ESZ = 16 / EPG;
    __shared__ uint4 s_data[kWavesPerBlockA][kCapOf<U>];
    __shared__ uint16_t s_gidx[kWavesPerBlockA][kCapOf<U>];
    __shared__ Rank s_merge[kWavesPerBlockA][kWave];

    const int lane = lane_id();
    const int wv = threadIdx.x >> 6;
    int64_t wg = blockIdx.x;
    if constexpr (ACCEPT) {
        if (v.table) {
            // Workgroup 0 registers every row as a holder of its token (highest
            // row wins the matrix row), then completes each request's hand-off.
            // Kept off the streaming waves: no contended counter on their path.
            if (blockIdx.x == 0) {
                for (int64_t P = (int64_t)wv * kWave + lane; P < a.n_rows; P += kWave * kWavesPerBlockA) {
                    const int t = v.tok[P];
                    if (t >= 0 && t < a.V)
                        __hip_atomic_fetch_max(&v.last_occ[t], (int32_t)(P + 1), __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                }
                publish();
                __syncthreads();
                if (wv != 0) return;
                for (int b0 = 0; b0 < v.B; b0 += kWave) {
                    const int b = b0 + lane;
                    uint32_t old = 0;
                    if (b < v.B) old = count_in(&v.handoff[b]);
                    uint64_t second = ballot(b < v.B && old == 1u);
                    while (second) {
                        const int j = __ffsll((unsigned long long)second) - 1;
                        second &= second - 1;
                        after_count();
                        update_request(v, a.V, a.k, a.topk, a.prob, b0 + j);
                        if (lane == 0) st_agent(&v.handoff[b0 + j], 0u);
                    }
                }
                return;
            }
            wg -= 1;
        }
    }
    const int64_t w = wg * kWavesPerBlockA + wv;
    const int S = a.S;
    Rank *scratch = s_merge[wv];
    if (w >= a.n_rows * S) return;
    const int64_t row = w / S;
    const int split = (int)(w - row * S);
    const int c0 = split * a.chunk;
    const int c1 = min(a.V, c0 + a.chunk);
    const char *rowp = (const char *)a.logits + (size_t)row * (size_t)a.V * ESZ;

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
            const uint32_t raw = TR::load_scalar(rowp, c0 + off);
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
            if (ballot(any)) kth = merge_top8_compact<Rank, EPG>(c, top, scratch);
        }
        count = 0;
        thr = kth ? TR::rank_key(kth) : INT_MIN;
    };

    // Software-pipelined stream: the next batch's loads are in flight while the
    // current batch is filtered.  Loads are never predicated (indices past the
    // range are clamped to its last group and the data ignored), so the
    // compiler's wait counts only the older batch.
    auto issue = [&](uint4 (&d)[U], int g0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int gi = min(g0 + u * kWave + lane, ng - 1);
            d[u] = load16<NT>(vp + gi);
        }
    };
    auto filter = [&](const uint4 (&d)[U], int g0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
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
        if (count > kCapOf<U> - kWave * U) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            process();
        }
    };

    if (ng > 0) {
        uint4 cur[U], nxt[U];
        issue(cur, 0);
        {
            // Seed the threshold: the 8th largest lane maximum of the first batch is a
            // lower bound of the range's 8th best key when it is positive (8 distinct
            // elements reach it), so the first batch is filtered like the rest.
            int m = TR::kRawMin;
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (u * kWave + lane < ng) m = max(m, TR::raw_max(cur[u]));
            int m8 = TR::kRawMin;
#pragma unroll
            for (int j = 0; j < kTop; ++j) {
                m8 = wave_max_i32(m);
                const uint64_t own = ballot(m == m8);
                if (lane == __ffsll((unsigned long long)own) - 1) m = TR::kRawMin;
            }
            if (m8 >= 1 && m8 > thr) thr = m8;
        }
        int g0 = 0;
        for (; g0 + kWave * U < ng; g0 += kWave * U) {
            issue(nxt, g0 + kWave * U);
            filter(cur, g0);
#pragma unroll
            for (int u = 0; u < U; ++u) cur[u] = nxt[u];
        }
        filter(cur, g0);
    }
    if (count) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        process();
    }

    // Publish this range's candidates.  The last range of a row to finish
    // (device-scope counter) merges the row; with ACCEPT, the last row of a
    // request to be merged runs that request's acceptance walk.  Counters are
    // reset by the wave that consumed them, so the workspace is left zeroed.
    if (lane < kTop) st_agent(&a.partials[w * kTop + lane], top ? TR::to_row_rank(top, c0) : 0ull);
    if constexpr (PROB) {
        const float M = wave_max_f32(st.m);
        const float s = (st.m == -INFINITY) ? 0.0f : st.s * __expf(st.m - M);
        const float Ssum = wave_sum_f32(s);
        if (lane == 0)
            st_agent(&a.stats[w], ((uint64_t)__float_as_uint(Ssum) << 32) | __float_as_uint(M));
    }
    publish();
    uint32_t prev = 0;
    if (lane == 0) prev = count_in(&a.row_cnt[row]);
    prev = (uint32_t)readlane_i32((int)prev, 0);
    if (prev != (uint32_t)(S - 1)) return;
    after_count();
    merge_row(a, row);
    if (lane == 0) st_agent(&a.row_cnt[row], 0u);
    if constexpr (ACCEPT) {
        const int b = (int)(row / v.T1);
        publish();
        uint32_t prev_r = 0;
        if (lane == 0) prev_r = count_in(&v.req_cnt[b]);
        prev_r = (uint32_t)readlane_i32((int)prev_r, 0);
        if (prev_r != (uint32_t)(v.T1 - 1)) return;
        after_count();
        accept_walk(v, a.k, a.topk, b);
        if (lane == 0) st_agent(&v.req_cnt[b], 0u);
        if (v.table) {
            publish();
            if (handoff_second(v, b)) {
                after_count();
                update_request(v, a.V, a.k, a.topk, a.prob, b);
                if (lane == 0) st_agent(&v.handoff[b], 0u);
            }
        }
    }
}

template <typename TR>
void launch_rows(const TopkArgs &a, const VerifyArgs *v, hipStream_t s) {
    const int64_t waves = a.n_rows * a.S;
    const int extra = (v && v->table) ? 1 : 0;  // the registration workgroup
    const dim3 grid((unsigned)((waves + kWavesPerBlockA - 1) / kWavesPerBlockA + extra));
    const dim3 block(kWave * kWavesPerBlockA);
    const VerifyArgs vv = v ? *v : VerifyArgs{};
    const bool prob = a.prob != nullptr;
    if (v) {
        if (prob)
            hipLaunchKernelGGL((k_topk_rows<TR, true, true, true>), grid, block, 0, s, a, vv);
        else
            hipLaunchKernelGGL((k_topk_rows<TR, false, true, true>), grid, block, 0, s, a, vv);
    } else {
        if (prob)
            hipLaunchKernelGGL((k_topk_rows<TR, true, false, true>), grid, block, 0, s, a, vv);
        else
            hipLaunchKernelGGL((k_topk_rows<TR, false, false, true>), grid, block, 0, s, a, vv);
    }
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
    // workspace: [partials | stats | row counters, request counters |
    //             last occurrence per token [V], (unused word), hand-offs [n_rows]]
    p.off_stats = (p.partial_bytes + 255) / 256 * 256;
    p.off_counters = p.off_stats + (p.stats_bytes + 255) / 256 * 256;
    p.off_occ = p.off_counters + ((size_t)n_rows * 2 * sizeof(uint32_t) + 255) / 256 * 256;
    p.ws_bytes = p.off_occ + ((size_t)(V + 1 + n_rows) * sizeof(uint32_t) + 255) / 256 * 256;
    return p;
}

void launch_topk(const TopkPlan &p, int dtype, const void *logits, int k, int32_t *topk,
                 float *prob, void *ws, const VerifyArgs *verify, hipStream_t s) {
    if (p.n_rows <= 0) return;
    TopkArgs a;
    a.logits = logits;
    a.n_rows = p.n_rows;
    a.V = p.V;
    a.S = p.splits;
    a.chunk = p.chunk;
    a.partials = (uint64_t *)ws;
    a.stats = (uint64_t *)((char *)ws + p.off_stats);
    a.row_cnt = (uint32_t *)((char *)ws + p.off_counters);
    a.k = k;
    a.topk = topk;
    a.prob = prob;
    VerifyArgs v;
    if (verify) {
        v = *verify;
        v.req_cnt = a.row_cnt + p.n_rows;
        v.last_occ = (int32_t *)((char *)ws + p.off_occ);
        v.handoff = (uint32_t *)(v.last_occ + p.V + 1);
        v.B = (int)(p.n_rows / (v.T1 > 0 ? v.T1 : 1));
    }
    if (dtype == GRAFT_DTYPE_BF16)
        launch_rows<Bf16Traits>(a, verify ? &v : nullptr, s);
    else
        launch_rows<F32Traits>(a, verify ? &v : nullptr, s);
}

}  // namespace graft
