// Row-wise top-k of vocab-wide target logits: the step that moves almost every
// byte of a Graft step (section 二, gear 3: the target's top-k at every verified
// position feeds both the greedy check and the matrix update).
//
// Order: value descending, ties -> lower id, -0 == +0.  The kernel is an HBM
// stream: no MFMA (nothing is a contraction).
//
// One workgroup per row, S wavefronts (with few rows, G workgroups per row,
//   each on a slice of whole blocks).  The row is cut into 1 KB blocks (64
//   lanes x 16 bytes = 8 bf16 or 4 fp32 per lane); wavefront j reads blocks
//   j, j+S, j+2S, ... so that the S waves of a row sweep it together (a
//   contiguous front per row keeps HBM pages open), U blocks per batch (2 or
//   4, chosen per launch) with the next batch issued before the current one is
//   filtered.  A wave-uniform threshold -- the key of the wave's current
//   8th-best value -- filters each 16-byte group with a few packed integer
//   ops; the rare groups that pass are compacted into LDS with a ballot and
//   merged into the wave's exact top-8 when 64 are pending (their elements
//   below the threshold dropped; a few inserted one by one, more by DPP wave
//   maxima).
// Epilogue: the S waves meet at one barrier; wave 0 ranks their candidates
//   by counting over LDS broadcasts
//   (and combines their softmax statistics) into the row's top-k; with G > 1
//   the row's last slice to arrive merges the slices' results.  The row then
//   publishes its greedy token in a completion word, which coordinator
//   wavefronts (one per request, in front of the rows) watch to run the
//   acceptance walk, and hands its top-k to the matrix update, which a
//   registration workgroup has prepared.  One launch per call.
#include "device_utils.hpp"
#include "launchers.hpp"

namespace graft {
namespace {

// U = 1 KB blocks per wave per batch (a template parameter: 2 or 4, chosen per
// launch); each wave keeps up to kWave * (U + 1) pending groups
constexpr int kMaxLdsPerGroup = 65536;  // dynamic LDS a workgroup may take
constexpr int kTop = 8;
constexpr int kMaxWavesPerRow = 16;
constexpr int kHeadPad = 8;  // local offsets below this are the row's unaligned head
constexpr uint64_t kSpinTicks = 100000000ull;  // coordinator gives up after ~1 s (100 MHz clock)
constexpr uint64_t kEmptyRank = 1ull;  // a slice's empty top-8 entry (no real row rank has a zero high word)

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
    __device__ static uint32_t local_off(Rank r) { return 0xffffu - (r & 0xffffu); }
    // fp32 key of the value (the row ranks' key) and back to the filter's bf16 key
    __device__ static int32_t row_key(uint32_t raw) { return bf16_key(raw) * 65536; }
    __device__ static int32_t filter_key(int32_t rk) { return rk / 65536; }
    // Largest raw bit pattern of the group read as int16 (equals the largest key
    // whenever that is positive).
    __device__ static int raw_max(const uint4 &d) {
        const short2v m = __builtin_elementwise_max(
            __builtin_elementwise_max(as_s2(d.x), as_s2(d.y)), __builtin_elementwise_max(as_s2(d.z), as_s2(d.w)));
        return max((int)m.x, (int)m.y);
    }
    static constexpr int kRawMin = -32768;
    // For a threshold thr >= 1: (thr-1) in both 16-bit halves, and the packed test
    // "some element's raw bits, read as int16, exceed thr-1" -- exactly "some key
    // >= thr", since keys >= 1 are positive values, whose bits order as int16.
    __device__ static uint32_t splat_below(int thr) {
        const uint32_t t = (uint32_t)(thr - 1) & 0xffffu;
        return t | (t << 16);
    }
    __device__ static bool pass_positive(const uint4 &d, uint32_t t2) {
        const short2v m = __builtin_elementwise_max(
            __builtin_elementwise_max(as_s2(d.x), as_s2(d.y)), __builtin_elementwise_max(as_s2(d.z), as_s2(d.w)));
        return as_u32(__builtin_elementwise_max(m, as_s2(t2))) != t2;
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
    __device__ static uint32_t local_off(Rank r) { return rank64_id(r); }
    __device__ static int32_t row_key(uint32_t raw) { return f32_key(raw); }
    __device__ static int32_t filter_key(int32_t rk) { return rk; }
    __device__ static int raw_max(const uint4 &d) {
        return max(max((int)d.x, (int)d.y), max((int)d.z, (int)d.w));
    }
    static constexpr int kRawMin = INT_MIN;
    __device__ static uint32_t splat_below(int thr) { return (uint32_t)thr; }
    __device__ static bool pass_positive(const uint4 &d, uint32_t t) {
        return max(max((int)d.x, (int)d.y), max((int)d.z, (int)d.w)) >= (int)t;
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

// Same result as merge_top8, by counting: the live candidates and the current
// top-8 are compacted into the wave's LDS scratch (64 entries), each counts the
// entries above it over LDS broadcasts (ranks are distinct), and the 8 best are
// written to scratch[0..7] at their rank and read back.  A wave's LDS accesses
// complete in order, so the scratch is rewritten only after every read.
template <typename Rank, int N>
__device__ __forceinline__ Rank merge_top8_count(Rank (&c)[N], Rank &top, Rank *scratch) {
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
    const int n = total + kTop;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const Rank x = lane < n ? scratch[lane] : (Rank)0;
    int above = 0;
    for (int j = 0; j < n; ++j) above += scratch[j] > x ? 1 : 0;
    if (lane < kTop) scratch[lane] = 0;
    if (x != 0 && above < kTop) scratch[above] = x;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    top = lane < kTop ? scratch[lane] : (Rank)0;
    __builtin_amdgcn_wave_barrier();
    if constexpr (sizeof(Rank) == 4) {
        return (Rank)__builtin_amdgcn_readlane((int)top, kTop - 1);
    } else {
        const uint32_t kl = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)top, kTop - 1);
        const uint32_t kh = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(top >> 32), kTop - 1);
        return ((uint64_t)kh << 32) | kl;
    }
}

// Few candidates: insert them one by one into the top-8 held in lanes 0..7
// (row ranks, descending, zero = empty).  A candidate's place is the number of
// entries above it (one ballot); the entries below it move down one lane (a
// DPP shift within the first row of 16 lanes).  Candidates at or below the
// 8th best are skipped.  Returns the new 8th best (0 while fewer than 8).
__device__ __forceinline__ uint64_t dpp_shr1_u64(uint64_t v) {
    const int l = (int)(uint32_t)v, h = (int)(uint32_t)(v >> 32);
    constexpr int kRowShr1 = 0x111;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(l, l, kRowShr1, 0xf, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(h, h, kRowShr1, 0xf, 0xf, false);
    return ((uint64_t)hi << 32) | lo;
}

template <int N>
__device__ __forceinline__ uint64_t insert_top8(const uint64_t (&c)[N], uint64_t &top, uint64_t kth) {
    const int lane = lane_id();
#pragma unroll
    for (int e = 0; e < N; ++e) {
        uint64_t bal = ballot(c[e] > kth);
        while (bal) {
            const int src = __ffsll((unsigned long long)bal) - 1;
            bal &= bal - 1ull;
            const uint32_t xl = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)c[e], src);
            const uint32_t xh = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(c[e] >> 32), src);
            const uint64_t x = ((uint64_t)xh << 32) | xl;
            if (x <= kth) continue;
            const int pos = __popcll(ballot(lane < kTop && top > x));
            const uint64_t left = dpp_shr1_u64(top);
            if (lane < kTop && lane > pos) top = left;
            if (lane == pos) top = x;
            const uint32_t kl = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)top, kTop - 1);
            const uint32_t kh = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(top >> 32), kTop - 1);
            kth = ((uint64_t)kh << 32) | kl;
        }
    }
    return kth;
}

// insert_top8 for the 32-bit wave-local ranks of bf16 rows.
template <int N>
__device__ __forceinline__ uint32_t insert_top8_u32(const uint32_t (&c)[N], uint32_t &top, uint32_t kth) {
    const int lane = lane_id();
#pragma unroll
    for (int e = 0; e < N; ++e) {
        uint64_t bal = ballot(c[e] > kth);
        while (bal) {
            const int src = __ffsll((unsigned long long)bal) - 1;
            bal &= bal - 1ull;
            const uint32_t x = (uint32_t)__builtin_amdgcn_readlane((int)c[e], src);
            if (x <= kth) continue;
            const int pos = __popcll(ballot(lane < kTop && top > x));
            const uint32_t left = (uint32_t)__builtin_amdgcn_update_dpp((int)top, (int)top, 0x111, 0xf, 0xf, false);
            if (lane < kTop && lane > pos) top = left;
            if (lane == pos) top = x;
            kth = (uint32_t)__builtin_amdgcn_readlane((int)top, kTop - 1);
        }
    }
    return kth;
}

// A row wave's pending candidates c (0 = none, else above kth) into its top-8:
// up to kPendingInsert live ones are inserted one by one, up to a wavefront's
// worth are compacted and ranked, more take the full merge.  Returns the new
// 8th best.
constexpr int kPendingInsert = 8;
template <typename Rank, int N>
__device__ __forceinline__ Rank merge_pending(Rank (&c)[N], Rank &top, Rank kth, Rank *scratch) {
    int total = 0;
#pragma unroll
    for (int e = 0; e < N; ++e) total += __popcll(ballot(c[e] != 0));
    if (total == 0) return kth;
    if (total <= kPendingInsert) {
        if constexpr (sizeof(Rank) == 4)
            return insert_top8_u32<N>(c, top, kth);
        else
            return insert_top8<N>(c, top, kth);
    }
    // 64-bit ranks (fp32 rows) rank faster by counting than by eight 64-bit DPP
    // wave maxima (61 rows of 32000 fp32: 10.22 -> 9.37 us); for 32-bit ranks
    // the two measured alike
    if constexpr (sizeof(Rank) == 8)
        return merge_top8_count<Rank, N>(c, top, scratch);
    else
        return merge_top8_compact<Rank, N>(c, top, scratch);
}

// Per-lane online softmax statistics: running maximum m and sum of exp(x - m).
// Values arrive in batches: one rescale when a batch raises the maximum, then
// one subtract, exponential and add per value (no per-value branch).  While
// the maximum is still -inf every value so far is -inf and adds nothing.
struct SoftStats {
    float m = -INFINITY;
    float s = 0.0f;
    template <int N>
    __device__ __forceinline__ void add_batch(const float (&x)[N]) {
        float mb = x[0];
#pragma unroll
        for (int i = 1; i < N; ++i) mb = fmaxf(mb, x[i]);
        if (mb > m) {
            s = (m == -INFINITY) ? 0.0f : s * __expf(m - mb);
            m = mb;
        }
        if (m != -INFINITY) {
#pragma unroll
            for (int i = 0; i < N; ++i) s += __expf(x[i] - m);
        }
    }
    __device__ __forceinline__ void add(float v) {
        const float x[1] = {v};
        add_batch<1>(x);
    }
};

// A slice's softmax statistics (largest value, sum of exp(value - largest)) in
// one word: never zero (a finite largest value contributes at least 1 to the
// sum, and -inf has nonzero bits).
__device__ __forceinline__ uint64_t pack_stats(float m, float s) {
    return ((uint64_t)__float_as_uint(m) << 32) | __float_as_uint(s);
}

template <typename TR, int U>
__device__ __forceinline__ void add_groups(SoftStats &st, const uint4 (&d)[U]) {
    constexpr int EPG = TR::kPerGroup;
    float x[U * EPG];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < EPG; ++e) x[u * EPG + e] = TR::value(TR::elem(d[u], e));
    st.add_batch<U * EPG>(x);
}

// Ancestor-or-self mask of flattened row `lane` (p = parent row, -1 for the
// root and for lanes that are not rows), by pointer doubling over the parent
// links.  Depends on the tree alone, so coordinators compute it while they wait
// for the rows.
__device__ __forceinline__ uint64_t ancestor_mask(bool row, int p) {
    const int lane = lane_id();
    int a = p;
    uint64_t A = row ? ((1ull << lane) | (a >= 0 ? (1ull << a) : 0ull)) : 0ull;
    for (int r = 0; r < 6; ++r) {
        if (!ballot(a >= 0)) break;  // every chain has reached the root
        const int src = a >= 0 ? a : lane;
        const uint64_t Aa = shfl_u64(A, src);
        const int aa = __shfl(a, src);
        if (a >= 0) {
            A |= Aa;
            a = aa;
        }
    }
    return A;
}

// Strict greedy acceptance walk of request b (section 二, gear 3), one wavefront;
// lane f is flattened row f with its greedy token g, token t, parent row p (-1
// for the root and non-rows), depth d and ancestor-or-self mask A; base is the
// request's position base (read before the rows were waited for).  A row is
// accepted iff every row on its path from the root carries the greedy token of
// its parent row, i.e. iff its mask holds no row whose edge check fails; the
// deepest accepted row wins, ties -> lowest row.
__device__ __forceinline__ void accept_walk(const VerifyArgs &v, int b, int g, int t, int p, int d, uint64_t A,
                                            int base) {
    const int lane = lane_id();
    const int T1 = v.T1;
    const bool row = lane < T1;
    const int gp = __shfl(g, p >= 0 ? p : lane);
    const uint64_t E = ballot(row && (lane == 0 || (p >= 0 && t == gp)));  // edges that hold
    const bool ok = row && (A & ~E) == 0ull;
    const int key = ok ? (d << 8) | (255 - lane) : -1;
    const int best = wave_max_i32(key);
    const int fstar = 255 - (best & 255);  // uniform (the root is always accepted)
    const int len = best >> 8;
    const uint64_t path = ((uint64_t)(uint32_t)readlane_i32((int)(uint32_t)(A >> 32), fstar) << 32) |
                          (uint32_t)readlane_i32((int)(uint32_t)A, fstar);
    const int gstar = readlane_i32(g, fstar);
    // the path's rows have depths 1..len: row at depth d goes to slot d-1
    if (row && lane > 0 && ((path >> lane) & 1ull) && d >= 1 && d <= v.dmax)
        v.accept_idx[(size_t)b * v.dmax + d - 1] = lane;
    for (int j = lane; j < v.dmax; j += kWave)
        if (j >= len) v.accept_idx[(size_t)b * v.dmax + j] = -1;
    if (lane == 0) {
        v.accept_len[b] = len;
        v.bonus[b] = gstar;
        if (v.base_pos_io) v.base_pos_io[b] = base + len + 1;
    }
}

// Matrix update (section 三): a row writes its top-k into the matrix row of its
// token iff it is the last row of the whole batch holding that token (highest
// row wins), then clears that token's registration.  Runs once every row of the
// batch is registered; each row is updated by whichever of {the row's own
// workgroup, the registration workgroup} arrives second at the row's hand-off
// word, so neither waits for the other.

// One row from registers (one wavefront): lanes j < k hold the row's j-th id
// and probability.  t is the row's token (valid, uniform).  occ_read: the
// token's holder word if the row already read it (nonzero, uniform), else 0
// and it is read here (only then does this wait for memory).
__device__ __forceinline__ void update_row_regs(const VerifyArgs &v, int k, int64_t P, int t, int32_t id,
                                                float pj, bool with_prob, int occ_read) {
    const int lane = lane_id();
    int occ = occ_read;
    if (occ == 0) {
        int x = 0;
        if (lane == 0) x = ld_agent(&v.last_occ[t]);
        occ = readlane_i32(x, 0);
    }
    if (occ != (int32_t)(P + 1)) return;
    if (lane < k) {
        v.table[(size_t)t * k + lane] = id;
        if (v.table_prob && with_prob) v.table_prob[(size_t)t * k + lane] = pj;
    }
    if (lane == 0) st_agent(&v.last_occ[t], 0);
}

// One row from the published top-k (one thread; the rare case of a row that
// finished before the registration did).
__device__ __forceinline__ void update_row_mem(const VerifyArgs &v, int k, const int32_t *topk,
                                               const float *prob, int64_t P, int t) {
    if (ld_agent(&v.last_occ[t]) != (int32_t)(P + 1)) return;
    for (int j = 0; j < k; ++j) v.table[(size_t)t * k + j] = ld_agent(&topk[P * k + j]);
    if (v.table_prob && prob)
        for (int j = 0; j < k; ++j)
            v.table_prob[(size_t)t * k + j] = __int_as_float(ld_agent((const int32_t *)&prob[P * k + j]));
    st_agent(&v.last_occ[t], 0);
}

// Registration (fused update only): every row with a valid token
// records itself as a holder of that token (atomic max of row+1); once all are
// in, the workgroup arrives at every such row's hand-off word and updates the
// rows that arrived first.
__device__ __forceinline__ void register_rows(const TopkArgs &a, const VerifyArgs &v) {
    constexpr int kR = 4;  // hand-off arrivals in flight per thread
    const int nth = blockDim.x;
    for (int64_t P = threadIdx.x; P < a.n_rows; P += nth) {
        const int t = v.tok[P];
        if (t >= 0 && t < a.V)
            __hip_atomic_fetch_max(&v.last_occ[t], (int32_t)(P + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    publish();
    __syncthreads();
    for (int64_t P0 = threadIdx.x; P0 < a.n_rows; P0 += (int64_t)kR * nth) {
        uint32_t old[kR];
        int tk[kR];
#pragma unroll
        for (int u = 0; u < kR; ++u) {
            const int64_t P = P0 + (int64_t)u * nth;
            tk[u] = P < a.n_rows ? v.tok[P] : -1;
            old[u] = (tk[u] >= 0 && tk[u] < a.V) ? count_in(&v.handoff[P]) : 0u;
        }
#pragma unroll
        for (int u = 0; u < kR; ++u) {
            if (old[u] == 1u) {
                const int64_t P = P0 + (int64_t)u * nth;
                after_count();
                update_row_mem(v, a.k, a.topk, a.prob, P, tk[u]);
                st_agent(&v.handoff[P], 0u);
            }
        }
    }
}

// Coordinators (the first v.ncoord workgroups of a verify launch, one wavefront
// per request up to a fixed number of workgroups; nothing waits on them, so
// they cannot hold up the rows).  The first one registers the rows' tokens for
// the fused update.  Row P publishes (greedy token + 1) into done[P], zero
// meaning "not yet"; wavefront w watches requests w, w + N, w + 2N, ... (N =
// coordinator wavefronts) in turn, in the order their rows are dispatched (one
// load per unfinished row per poll, no atomics), clearing each word as soon as
// it has been read.  The walk does not wait for every row: its outcome is
// fixed once each row is either cut off by a known failed edge on its path
// (an ancestor-or-self whose parent's greedy token is in and differs from its
// token) or accepted with its own greedy token in, which for most requests is
// long before their last row ends; the wave then only keeps clearing words.
// With tagged completion words (v.tag_done) nothing is cleared: a word is the
// row's for this launch iff its launch counter is the one the coordinator
// expects for that row (its own counter, advanced once per launch), so the
// wave is done with the walk.  A watch that exceeds kSpinTicks reports
// accept_len = -1 for that request and moves on.
__device__ __forceinline__ void coordinate(const TopkArgs &a, const VerifyArgs &v, int cw) {
    if (cw == 0 && v.table && !v.scan_holders) register_rows(a, v);
    const int lane = lane_id();
    const int S = blockDim.x >> 6;
    const int T1 = v.T1;
    const bool row = lane < T1;
    for (int b = cw * S + (int)(threadIdx.x >> 6); b < v.B; b += v.ncoord * S) {
        const size_t o = (size_t)b * T1 + lane;
        int t = -1, p = -1, d = 0, g = 1;
        if (row) {
            t = v.tok[o];
            p = v.parent[o];
            d = v.depth[o];
            g = 0;
        }
        if (!row || lane == 0) p = -1;
        const uint64_t A = ancestor_mask(row, p);
        const int base = v.base_pos_io ? v.base_pos_io[b] : 0;  // only this wave writes it
        const bool tagged = v.tag_done != nullptr;
        uint32_t want = 0;  // tagged: the launch counter of this launch's words
        if (tagged && row) {
            want = v.tag_want[o] + 1u;  // only this wave touches the row's counter
            v.tag_want[o] = want;
        }
        const uint64_t t0 = wall_clock64();
        bool walked = false;
        while (true) {
            if (g == 0) {
                if (tagged) {
                    const uint64_t w = ld_agent(&v.tag_done[o]);
                    if ((uint32_t)(w >> 32) == want) g = (int)(uint32_t)w;
                } else {
                    g = ld_agent(&v.done[o]);
                    if (g != 0) st_agent(&v.done[o], 0);  // the row writes it once per launch
                }
            }
            if (!walked) {
                const int gp = __shfl(g, p >= 0 ? p : lane);     // parent's greedy token + 1, 0 = not in
                const bool known = lane == 0 || gp != 0;          // the edge into this row can be checked
                const bool holds = lane == 0 || (gp != 0 && t == gp - 1);
                const uint64_t cut = ballot(row && known && !holds);
                const uint64_t held = ballot(row && holds);
                const bool fixed = !row || (A & cut) != 0ull || ((A & ~held) == 0ull && g != 0);
                if (!ballot(!fixed)) {
                    // rows not in yet are all cut off: their greedy tokens are not used
                    accept_walk(v, b, g - 1, t, p, d, A, base);
                    walked = true;
                    if (tagged) break;
                }
            }
            if (walked && !ballot(g == 0)) break;
            if (wall_clock64() - t0 > kSpinTicks) {
                if (lane == 0) v.accept_len[b] = -1;
                break;
            }
        }
    }
}

// A row's result, from one wavefront whose lanes 0..7 hold the row's top-8
// row ranks (descending; zero where the row has fewer elements): the top-k ids
// (and softmax probabilities), the completion word the coordinators watch, and
// the hand-off to the matrix update.  Uniform (scalar) arguments, so that no
// wait for an earlier load falls after this row's stores (a wait on the vector
// memory counter also waits for the stores issued before it): row_tok, the
// row's token (-1 without an update); handoff_seen, the row's hand-off word as
// read earlier (1 = the registration had arrived, so the fast path applies),
// else 0; occ, the token's holder word read after handoff_seen showed 1, else 0;
// tag, this launch's counter for the row's tagged completion word (with
// v.tag_done).
template <bool PROB, bool ACCEPT>
__device__ __forceinline__ void finish_row(const TopkArgs &a, const VerifyArgs &v, int64_t row, uint64_t rtop,
                                           float rowM, float rowS, int row_tok, int handoff_seen, int occ,
                                           uint32_t tag = 0) {
    const int lane = lane_id();
    const int32_t my_id = rtop ? (int32_t)rank64_id(rtop) : -1;  // lanes j < k: the row's j-th id
    float my_p = 0.0f;
    if (lane < a.k) st_agent(&a.topk[row * a.k + lane], my_id);
    if (PROB) {
        if (a.stats && lane == 0) *(float2 *)&a.stats[row * 2] = make_float2(rowM, rowS);
        if (a.prob && lane < a.k) {
            const float x = key_to_f32(rank64_key(rtop));
            my_p = rtop ? __expf(x - rowM) / rowS : 0.0f;
            st_agent((int32_t *)&a.prob[row * a.k + lane], __float_as_int(my_p));
        }
    }
    if constexpr (ACCEPT) {
        // Completion word for the coordinator: greedy token + 1 (lane 0 holds it),
        // tagged with the launch counter or plain.
        if (v.B > 0 && lane == 0) {
            if (v.tag_done)
                st_agent(&v.tag_done[row], ((uint64_t)tag << 32) | (uint32_t)(my_id + 1));
            else
                st_agent(&v.done[row], my_id + 1);
        }
        // Fused update: hand the row to the update.  Fast path: the registration
        // already arrived (it finishes long before the rows do); otherwise the
        // second arrival at the row's hand-off word updates the row.
        const int t = v.table ? row_tok : -1;
        if (t >= 0 && t < a.V && v.scan_holders) {
            // occ: 1 iff no later row of the launch holds this row's token
            if (occ == 1 && lane < a.k) {
                v.table[(size_t)t * a.k + lane] = my_id;
                if (v.table_prob && a.prob) v.table_prob[(size_t)t * a.k + lane] = my_p;
            }
        } else if (t >= 0 && t < a.V) {
            const bool fast = handoff_seen == 1;
            bool mine = fast;
            if (!mine) {
                publish();
                uint32_t o = 0;
                if (lane == 0) o = count_in(&v.handoff[row]);
                mine = readlane_i32((int)o, 0) == 1;
            }
            if (mine) {
                // the holder word read after the hand-off showed the registration
                // needs no further ordering (an acquire here would also wait for
                // this row's stores above); otherwise order the read that follows
                if (!fast || occ == 0) after_count();
                update_row_regs(v, a.k, row, t, my_id, my_p, a.prob != nullptr, occ);
                if (lane == 0) st_agent(&v.handoff[row], 0u);
            }
        }
    }
}

// ---- rows with long streams: S streaming wavefronts and one merge wavefront ----------
// The S streaming waves of a row only filter: each 16-byte group with an
// element at or above the current threshold (the larger of the wave's own seed
// and the row threshold the merge wave publishes in LDS) goes into the wave's
// ring in LDS (one producer, one consumer, no atomics: entries are written,
// then the producer's count).  The merge wave drains the rings into the row's
// exact top-8 (64-bit row ranks: value key, inverted element id), publishes
// the new threshold, and when every streaming wave has raised its flag and the
// rings are empty, finishes the row itself.  A streaming wave never stops
// issuing loads to merge, and no cross-wave selection is left at the row's end.
template <int U>
struct MwSmem {
    static constexpr int kRing = kWave * U;  // pending groups per streaming wave: one full batch
    // control block: counts [16] @0 (entries written, kRingDone once the
    // wave is done), consumed [16] @64, threshold @128; softmax statistics
    // float2 [16] @256; merge scratch u64 [64] @512
    static constexpr size_t kCtrl = 1024;
    static size_t bytes(int S) { return kCtrl + (size_t)S * kRing * (sizeof(uint4) + sizeof(uint32_t)); }
};

// Control words in LDS: relaxed workgroup-scope atomics, so each access is one
// LDS instruction (a volatile access through a generic pointer would become a
// flat access, which also waits for the wave's loads in flight).
__device__ __forceinline__ uint32_t lds_ld(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_st(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// LDS ordering: one wavefront's LDS accesses are performed in program order,
// so a consumer that sees a count written after the entries sees the entries.
// The compiler is kept from moving memory accesses across these points.
__device__ __forceinline__ void lds_order() { __asm__ volatile("" ::: "memory"); }
__device__ __forceinline__ void lds_drain() {
    lds_order();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS accesses have completed
    lds_order();
}

constexpr uint64_t kHandoffTicks = 500;     // the merge wave reads the row's hand-off word ~5 us in
constexpr uint32_t kRingDone = 0x80000000u;  // a ring's count word: the streaming wave is done
constexpr uint32_t kMaxIdlePolls = 1u << 25; // ~2 s of 64-cycle sleeps: a stuck row gives up (never in normal operation)
constexpr int kInsertMax = 8;  // candidates inserted one by one; more take the wave merge (4-8 measured best)

template <typename TR, bool PROB, bool ACCEPT, int U>
__global__ __launch_bounds__(1024) void k_topk_mw(TopkArgs a, VerifyArgs v) {
    using SM = MwSmem<U>;
    constexpr int kRing = SM::kRing;
    constexpr int EPG = TR::kPerGroup;
    constexpr int ESZ = 16 / EPG;
    constexpr int BLK = kWave * EPG;  // elements per 1 KB block
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t *s_cnt = (uint32_t *)smem;
    uint32_t *s_rd = s_cnt + 16;
    uint32_t *s_thr = s_cnt + 32;  // int32 filter key as its bits
    float2 *s_stat = (float2 *)(smem + 256);
    uint64_t *s_scr = (uint64_t *)(smem + 512);

    const int lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = (int)(blockDim.x >> 6) - 1;  // streaming waves; wave S merges
    int64_t row = blockIdx.x;
    if constexpr (ACCEPT) {
        if (row < v.ncoord) {
            coordinate(a, v, (int)row);
            return;
        }
        row -= v.ncoord;
    }
    if (row >= a.n_rows) return;
    uint4 *ring_d = (uint4 *)(smem + SM::kCtrl);
    uint32_t *ring_g = (uint32_t *)(smem + SM::kCtrl + (size_t)S * kRing * sizeof(uint4));

    const int V = a.V;
    const char *rowp = (const char *)a.logits + (size_t)row * (size_t)V * ESZ;
    // head (until 16-byte alignment), body of 16-byte groups in 1 KB blocks, tail
    int head = (int)(((16u - (uint32_t)((uintptr_t)rowp & 15u)) & 15u) / ESZ);
    head = min(head, V);
    const int ng = (V - head) / EPG;
    const int ntail = V - head - ng * EPG;
    const int nblk = (ng + kWave - 1) / kWave;
    const uint4 *vp = (const uint4 *)(rowp + (size_t)head * ESZ);

    if (wv < S) {
        // ---------------- streaming wave ----------------
        uint4 *rd_ring = ring_d + (size_t)wv * kRing;
        uint32_t *rg_ring = ring_g + (size_t)wv * kRing;
        const int kcount = nblk > wv ? (nblk - wv + S - 1) / S : 0;  // blocks of this wave
        const int nfull = ng / kWave;                                 // complete blocks of the row
        const int kfull = nfull > wv ? (nfull - wv + S - 1) / S : 0;
        int seed = INT_MIN;          // the wave's own lower bound of the row's 8th best key
        uint32_t wr = 0, seen = 0;   // entries written; entries the merge wave had taken when last read
        SoftStats st;
        auto push = [&](const uint4 (&d)[U], const bool (&pass)[U], int kq0) __attribute__((always_inline)) {
            uint64_t bal[U];
            uint32_t n = 0;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                bal[u] = ballot(pass[u]);
                n += (uint32_t)__popcll(bal[u]);
            }
            if (n == 0) return;
            if (wr + n - seen > (uint32_t)kRing) {
                // wait for room (only when candidates pile up, e.g. rising rows)
                const uint64_t t0 = wall_clock64();
                while (true) {
                    seen = __builtin_amdgcn_readfirstlane(lds_ld(&s_rd[wv]));
                    if (wr + n - seen <= (uint32_t)kRing || wall_clock64() - t0 > kSpinTicks) break;
                    __builtin_amdgcn_s_sleep(1);
                }
            }
            uint32_t base = wr;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (pass[u]) {
                    const uint32_t slot = (base + (uint32_t)lanes_below(bal[u])) & (uint32_t)(kRing - 1);
                    rd_ring[slot] = d[u];
                    rg_ring[slot] = (uint32_t)(head + (wv + (kq0 + u) * S) * BLK + lane * EPG);
                }
                base += (uint32_t)__popcll(bal[u]);
            }
            wr += n;
            lds_drain();
            if (lane == 0) lds_st(&s_cnt[wv], wr);
            lds_order();
        };
        auto cur_thr = [&]() __attribute__((always_inline)) {
            return max(seed, __builtin_amdgcn_readfirstlane((int)lds_ld(s_thr)));
        };
        auto filter_full = [&](const uint4 (&d)[U], int kq) __attribute__((always_inline)) {
            if constexpr (PROB) add_groups<TR, U>(st, d);
            const int t = cur_thr();
            bool pass[U];
            if (t >= 1) {
                const uint32_t t2 = TR::splat_below(t);
#pragma unroll
                for (int u = 0; u < U; ++u) pass[u] = TR::pass_positive(d[u], t2);
            } else if (t == INT_MIN) {
#pragma unroll
                for (int u = 0; u < U; ++u) pass[u] = true;
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u) pass[u] = TR::group_pass(d[u], t);
            }
            push(d, pass, kq);
        };
        auto issue_full = [&](uint4 (&d)[U], int kk) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < U; ++u) d[u] = load16<true>(vp + (size_t)(wv + (kk + u) * S) * kWave + lane);
        };
        auto load_rem = [&](uint4 (&d)[U], int k0) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int gi = min((wv + (k0 + u) * S) * kWave + lane, ng - 1);
                d[u] = load16<true>(vp + gi);
            }
        };
        auto filter_rem = [&](const uint4 (&d)[U], int k0) __attribute__((always_inline)) {
            const int t = cur_thr();
            bool pass[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool inb = (k0 + u < kcount) && ((wv + (k0 + u) * S) * kWave + lane < ng);
                if constexpr (PROB) {
                    if (inb) {
                        const uint4 one[1] = {d[u]};
                        add_groups<TR, 1>(st, one);
                    }
                }
                pass[u] = inb && (t == INT_MIN || TR::group_pass(d[u], t));
            }
            push(d, pass, k0);
        };
        uint4 cur[U], nxt[U];
        if (kfull >= U) issue_full(cur, 0);
        // the merge wave has initialised the control block (a plain barrier: a
        // workgroup fence would wait for the batch just issued)
        lds_order();
        __builtin_amdgcn_s_barrier();
        lds_order();
        int kk = 0;
        if (kfull >= U) {
            {
                // Seed: the 8th largest lane maximum of the first batch is a lower
                // bound of the row's 8th best key when positive (8 distinct
                // elements reach it).
                int m = TR::kRawMin;
#pragma unroll
                for (int u = 0; u < U; ++u) m = max(m, TR::raw_max(cur[u]));
                int m8 = TR::kRawMin;
#pragma unroll
                for (int j = 0; j < kTop; ++j) {
                    m8 = wave_max_i32(m);
                    const uint64_t own = ballot(m == m8);
                    if (lane == __ffsll((unsigned long long)own) - 1) m = TR::kRawMin;
                }
                if (m8 >= 1) seed = __builtin_amdgcn_readfirstlane(m8);
            }
            for (; kk + 2 * U <= kfull; kk += U) {
                issue_full(nxt, kk + U);
                filter_full(cur, kk);
#pragma unroll
                for (int u = 0; u < U; ++u) cur[u] = nxt[u];
            }
            const bool rem = kk + U < kcount;
            if (rem) load_rem(nxt, kk + U);
            filter_full(cur, kk);
            kk += U;
            if (rem) {
                filter_rem(nxt, kk);
                kk += U;
            }
        }
        for (; kk < kcount; kk += U) {
            uint4 d[U];
            load_rem(d, kk);
            filter_rem(d, kk);
        }
        if constexpr (PROB) {
            const float M = wave_max_f32(st.m);
            const float s = (st.m == -INFINITY) ? 0.0f : st.s * __expf(st.m - M);
            const float Ssum = wave_sum_f32(s);
            if (lane == 0) s_stat[wv] = make_float2(M, Ssum);
        }
        lds_drain();
        if (lane == 0) lds_st(&s_cnt[wv], wr | kRingDone);
        return;
    }

    // ---------------- merge wave ----------------
    // head and tail elements (at most EPG-1 each), loaded before the barrier
    bool have = false;
    int hidx = 0;
    uint32_t hraw = 0;
    if (lane < head) {
        hidx = lane;
        have = true;
    } else if (lane >= 16 && lane - 16 < ntail) {
        hidx = head + ng * EPG + (lane - 16);
        have = true;
    }
    if (have) hraw = TR::load_scalar(rowp, hidx);
    if (lane < 32) lds_st(&s_cnt[lane], 0u);  // counts, consumed
    if (lane == 32) lds_st(s_thr, (uint32_t)INT_MIN);
    int row_tok = -1;
    uint64_t tag_old = 0;  // the row's tagged completion word from the last launch
    int later_tok[kScanRegs];  // scan mode: tokens of rows row+1+lane+64i, -1 past the launch
#pragma unroll
    for (int i = 0; i < kScanRegs; ++i) later_tok[i] = -1;
    if constexpr (ACCEPT) {
        if (v.table) row_tok = v.tok[row];
        if (v.tag_done && lane == 0) tag_old = ld_agent(&v.tag_done[row]);
    }
    lds_drain();
    __builtin_amdgcn_s_barrier();
    lds_order();

    uint64_t top = 0;  // lanes 0..7: the row's top-8 so far, descending
    uint64_t kth = 0;  // the 8th best (uniform); 0 while fewer than 8
    SoftStats st;
    {
        uint64_t c[1] = {have ? rank64(TR::row_key(hraw), (uint32_t)hidx) : 0ull};
        if constexpr (PROB) {
            if (have) st.add(TR::value(hraw));
        }
        if (ballot(have)) kth = merge_top8<uint64_t, 1>(c, top);
    }
    int thr_pub = INT_MIN;
    if (kth) {
        thr_pub = TR::filter_key(rank64_key(kth));
        if (lane == 0) lds_st(s_thr, (uint32_t)thr_pub);
    }
    if constexpr (ACCEPT) {
        // scan mode: the later rows' tokens, loaded now (after the head and tail
        // elements are used, so nothing waits for them before the row's end)
        if (v.scan_holders) {
#pragma unroll
            for (int i = 0; i < kScanRegs; ++i) {
                const int64_t q = row + 1 + lane + (int64_t)kWave * i;
                if (q < a.n_rows) later_tok[i] = v.tok[q];
            }
        }
    }
    uint32_t taken = 0;  // lane w < S: entries of ring w taken so far
    int hs = 0, occ = 0;
    bool hs_read = false, occ_read = false;
    uint32_t idle = 0, iter = 0;  // idle polls; loop passes
    // scan mode: the row's token (uniform), compared with the later rows' at the end
    int scan_tok = -1;
    if constexpr (ACCEPT) {
        if (v.scan_holders) scan_tok = __builtin_amdgcn_readfirstlane(row_tok);
    }
    const uint64_t t_start = wall_clock64();
    uint64_t hs_at = kHandoffTicks;  // when the hand-off word is (next) read
    while (true) {
        const uint32_t cw = lane < S ? lds_ld(&s_cnt[lane]) : kRingDone;  // count and done bit in one word
        const bool fl = (cw & kRingDone) != 0u;
        const uint32_t av = lane < S ? (cw & ~kRingDone) - taken : 0u;
        if constexpr (ACCEPT) {
            // the row's hand-off word some microseconds in (the registration is
            // done within the launch's first microseconds), then the token's
            // holder word; the clock is read on every 8th pass
            if (v.table && !v.scan_holders && !occ_read && (++iter & 7u) == 0u) {
                const uint64_t dt = wall_clock64() - t_start;
                if (!hs_read && dt > hs_at) {
                    hs = ld_agent((const int32_t *)&v.handoff[row]);
                    hs_read = true;
                } else if (hs_read && dt > hs_at + kHandoffTicks) {
                    if (__builtin_amdgcn_readfirstlane(hs) == 1) {
                        occ_read = true;
                        if (row_tok >= 0 && row_tok < V) {
                            after_count();
                            occ = ld_agent(&v.last_occ[row_tok]);
                        }
                    } else {
                        // the registration has not reached this row yet: read again later
                        hs_read = false;
                        hs_at = dt + kHandoffTicks;
                    }
                }
            }
        }
        if (!ballot(av != 0u)) {
            if (!ballot(!fl)) break;                 // every streaming wave is done and its ring is empty
            if (++idle > kMaxIdlePolls) break;       // never in normal operation
            __builtin_amdgcn_s_sleep(1);
            continue;
        }
        // lane i takes the i-th pending entry, rings in order, 64 at most
        int my_w = -1;
        uint32_t my_j = 0, tk = 0;
        int got = 0;
        for (int w = 0; w < S && got < kWave; ++w) {
            const int aw = __builtin_amdgcn_readlane((int)av, w);
            if (aw == 0) continue;
            const int t = min(aw, kWave - got);
            const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)taken, w);
            if (lane >= got && lane < got + t) {
                my_w = w;
                my_j = r0 + (uint32_t)(lane - got);
            }
            if (lane == w) tk = (uint32_t)t;
            got += t;
        }
        uint4 d = make_uint4(0u, 0u, 0u, 0u);
        uint32_t g0 = 0;
        if (my_w >= 0) {
            const uint32_t slot = (uint32_t)my_w * kRing + (my_j & (uint32_t)(kRing - 1));
            d = ring_d[slot];
            g0 = ring_g[slot];
        }
        // the slots are handed back at once: this wave's LDS accesses are
        // performed in order, so the reads above complete before the producer
        // can see the new count and overwrite them
        lds_order();
        taken += tk;
        if (lane < S && tk) lds_st(&s_rd[lane], taken);
        lds_order();
        // an entry that passed an older threshold may hold nothing above the
        // current one: only the others are ranked
        const bool live = my_w >= 0 && (thr_pub == INT_MIN || TR::group_pass(d, thr_pub));
        uint64_t c[EPG];
        bool any = false;
#pragma unroll
        for (int e = 0; e < EPG; ++e) {
            const uint64_t r = rank64(TR::row_key(TR::elem(d, e)), g0 + (uint32_t)e);
            c[e] = live && r > kth ? r : 0ull;
            any |= c[e] != 0ull;
        }
        if (ballot(any)) {
            int ncand = 0;
#pragma unroll
            for (int e = 0; e < EPG; ++e) ncand += __popcll(ballot(c[e] != 0ull));
            kth = ncand <= kInsertMax ? insert_top8<EPG>(c, top, kth) : merge_top8_compact<uint64_t, EPG>(c, top, s_scr);
            const int nt = kth ? TR::filter_key(rank64_key(kth)) : INT_MIN;
            if (nt > thr_pub) {
                thr_pub = nt;
                if (lane == 0) lds_st(s_thr, (uint32_t)nt);
            }
        }
    }
    int handoff_seen = 0, occ_val = 0;
    if constexpr (ACCEPT) {
        if (v.scan_holders) {
            // the last holder: no later row of the launch holds the row's token
            bool hit = false;
#pragma unroll
            for (int i = 0; i < kScanRegs; ++i) hit |= later_tok[i] == scan_tok;
            occ_val = (scan_tok >= 0 && scan_tok < V && !ballot(hit)) ? 1 : 0;
        } else if (v.table) {
            if (!hs_read) hs = ld_agent((const int32_t *)&v.handoff[row]);
            handoff_seen = __builtin_amdgcn_readfirstlane(hs);
            if (handoff_seen == 1 && row_tok >= 0 && row_tok < V) {
                if (!occ_read) {
                    after_count();
                    occ = ld_agent(&v.last_occ[row_tok]);
                }
                occ_val = __builtin_amdgcn_readfirstlane(occ);
            }
        }
    }
    row_tok = __builtin_amdgcn_readfirstlane(row_tok);
    float rowM = -INFINITY, rowS = 0.0f;
    if constexpr (PROB) {
        // the streaming waves' statistics and the merge wave's own (head and tail)
        const float ownM = wave_max_f32(st.m);
        const float ownS = wave_sum_f32((st.m == -INFINITY) ? 0.0f : st.s * __expf(st.m - ownM));
        lds_order();
        float m = -INFINITY, ss = 0.0f;
        if (lane < S) {
            const float2 sv = s_stat[lane];
            m = sv.x;
            ss = sv.y;
        } else if (lane == S) {
            m = ownM;
            ss = ownS;
        }
        rowM = wave_max_f32(m);
        rowS = wave_sum_f32((m == -INFINITY) ? 0.0f : ss * __expf(m - rowM));
    }
    uint32_t tag = 0;
    if constexpr (ACCEPT) tag = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(tag_old >> 32)) + 1u;
    finish_row<PROB, ACCEPT>(a, v, row, top, rowM, rowS, row_tok, handoff_seen, occ_val, tag);
}

// Dynamic LDS layout of a row's workgroup (S waves, U blocks per batch).
template <typename Rank, int U>
struct RowSmem {
    static constexpr int kCap = kWave * (U + 1);                // pending groups per wave
    static constexpr size_t kData = sizeof(uint4) * kCap;      // pending groups
    static constexpr size_t kMerge = sizeof(Rank) * kWave;     // compaction scratch
    static constexpr size_t kGidx = sizeof(uint16_t) * kCap;   // pending group indices
    static constexpr size_t kPerWave = kData + kMerge + kGidx;
    // row tail: the waves' top-8 (S*kTop u64, at least one wavefront's worth), the
    // row's top-8 (u64), softmax statistics (float2)
    __host__ __device__ static size_t cand_entries(int S) { return (size_t)(S * kTop > kWave ? S * kTop : kWave); }
    static size_t bytes(int S) {
        return (size_t)S * kPerWave + (cand_entries(S) + kTop) * sizeof(uint64_t) +
               (size_t)S * sizeof(float2) + 16;
    }
};

template <typename TR, bool PROB, bool ACCEPT, bool NT, bool SPLIT, int U>
__global__ __launch_bounds__(kWave *kMaxWavesPerRow) void k_topk_rows(TopkArgs a, VerifyArgs v) {
    using Rank = typename TR::Rank;
    using SM = RowSmem<Rank, U>;
    constexpr int kCap = SM::kCap;
    constexpr int EPG = TR::kPerGroup;
    constexpr int ESZ = 16 / EPG;
    constexpr int BLK = kWave * EPG;  // elements per 1 KB block
    extern __shared__ __align__(16) unsigned char smem[];

    const int lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int S = blockDim.x >> 6;
    int64_t unit = blockIdx.x;
    if constexpr (ACCEPT) {
        if (unit < v.ncoord) {
            coordinate(a, v, (int)unit);
            return;
        }
        unit -= v.ncoord;
    }
    // SPLIT: the row is cut into G slices of whole blocks, one per workgroup
    const int G = SPLIT ? a.groups : 1;
    const int64_t row = SPLIT ? unit / G : unit;
    const int g = SPLIT ? (int)(unit - row * G) : 0;
    if (row >= a.n_rows) return;

    uint4 *sd = (uint4 *)(smem + (size_t)wv * SM::kData);
    Rank *scratch = (Rank *)(smem + (size_t)S * SM::kData + (size_t)wv * SM::kMerge);
    uint16_t *sg = (uint16_t *)(smem + (size_t)S * (SM::kData + SM::kMerge) + (size_t)wv * SM::kGidx);
    uint64_t *s_cand = (uint64_t *)(smem + (size_t)S * SM::kPerWave);
    uint64_t *s_top = s_cand + SM::cand_entries(S);
    float2 *s_stat = (float2 *)(s_top + kTop);

    const int V = a.V;
    const char *rowp = (const char *)a.logits + (size_t)row * (size_t)V * ESZ;
    // head (until 16-byte alignment), body of 16-byte groups in 1 KB blocks, tail
    int head = (int)(((16u - (uint32_t)((uintptr_t)rowp & 15u)) & 15u) / ESZ);
    head = min(head, V);
    const int ng_row = (V - head) / EPG;
    const int ntail = V - head - ng_row * EPG;
    const int nblk_row = (ng_row + kWave - 1) / kWave;
    const int blk0 = SPLIT ? (int)((int64_t)g * nblk_row / G) : 0;  // this slice's blocks [blk0, blk1)
    const int blk1 = SPLIT ? (int)((int64_t)(g + 1) * nblk_row / G) : nblk_row;
    const int ng = SPLIT ? min(ng_row, blk1 * kWave) - blk0 * kWave : ng_row;  // groups of the slice
    const int nblk = blk1 - blk0;
    const int kcount = nblk > wv ? (nblk - wv + S - 1) / S : 0;  // blocks of this wave
    const uint4 *vp = (const uint4 *)(rowp + (size_t)head * ESZ) + (size_t)blk0 * kWave;

    // Local offsets (monotone in the element id for this wave): head elements
    // 0..head-1 (wave 0), body kHeadPad + k*BLK + lane*EPG + e for the wave's
    // k-th block, tail after the wave's body (wave 0).
    auto global_id = [&](uint32_t off) __attribute__((always_inline)) -> uint32_t {
        if (off < (uint32_t)kHeadPad) return off;
        const uint32_t q = off - kHeadPad;
        if (q < (uint32_t)kcount * BLK) return head + (blk0 + wv + (q / BLK) * S) * BLK + q % BLK;
        return head + ng_row * EPG + (q - (uint32_t)kcount * BLK);
    };

    // the row's token for the matrix update and its tagged completion word from
    // the last launch, loaded now and used at the row's end (with split rows,
    // by the slice that finishes the row: its own load came before its store)
    int row_tok = -1;
    uint64_t tag_old = 0;
    if constexpr (ACCEPT) {
        if (wv == 0 && v.table) row_tok = v.tok[row];
        if (wv == 0 && lane == 0 && v.tag_done) tag_old = ld_agent(&v.tag_done[row]);
    }
    Rank top = 0;   // lanes 0..7: the wave's top-8, descending
    Rank kth = 0;   // the 8th best (uniform); 0 while fewer than 8 candidates
    int thr = INT_MIN;
    SoftStats st;

    if (wv == 0 && g == 0) {  // head and tail elements: at most EPG-1 each
        Rank c[1] = {0};
        bool have = false;
        int off = 0, idx = 0;
        if (lane < head) {
            off = lane;
            idx = lane;
            have = true;
        } else if (lane >= 16 && lane - 16 < ntail) {
            off = kHeadPad + kcount * BLK + (lane - 16);
            idx = head + ng_row * EPG + (lane - 16);
            have = true;
        }
        if (have) {
            const uint32_t raw = TR::load_scalar(rowp, idx);
            c[0] = TR::make(raw, off);
            if constexpr (PROB) st.add(TR::value(raw));
        }
        if (ballot(have)) {
            kth = merge_top8<Rank, 1>(c, top);
            thr = __builtin_amdgcn_readfirstlane(kth ? TR::rank_key(kth) : INT_MIN);
        }
    }

    int count = 0;
    auto set_thr = [&](int t) __attribute__((always_inline)) { thr = __builtin_amdgcn_readfirstlane(t); };
    auto process = [&]() __attribute__((always_inline)) {
        // candidates: above the 8th best so far and at or above the threshold,
        // a lower bound of the wave's 8th best key (its seed or an earlier merge)
        const int tq = thr;
        for (int base = 0; base < count; base += kWave) {
            const int gi = base + lane;
            Rank c[EPG];
            if (gi < count) {
                const uint4 d = sd[gi];
                const int goff = kHeadPad + (int)sg[gi] * EPG;
#pragma unroll
                for (int e = 0; e < EPG; ++e) {
                    const Rank r = TR::make(TR::elem(d, e), goff + e);
                    c[e] = (r > kth && TR::rank_key(r) >= tq) ? r : (Rank)0;
                }
            } else {
#pragma unroll
                for (int e = 0; e < EPG; ++e) c[e] = 0;
            }
            kth = merge_pending<Rank, EPG>(c, top, kth, scratch);
        }
        count = 0;
        set_thr(kth ? TR::rank_key(kth) : INT_MIN);
    };
    // Append the groups that pass (one per lane at most) to the pending buffer.
    auto append = [&](const uint4 &d, bool pass, int kq) __attribute__((always_inline)) {
        const uint64_t bal = ballot(pass);
        if (bal) {
            if (pass) {
                const int pos = count + lanes_below(bal);
                sd[pos] = d;
                sg[pos] = (uint16_t)(kq * kWave + lane);
            }
            count += __popcll(bal);
        }
    };
    auto maybe_process = [&]() __attribute__((always_inline)) {
        if (__builtin_amdgcn_readfirstlane(count) > kCap - kWave * U) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            process();
        }
    };

    // Steady state: this wave's complete blocks, U per batch, the next batch in
    // flight.  Block (wv + k*S) starts at group (wv + k*S)*64: a wave-uniform
    // base plus the lane, no per-lane bounds checks.
    const int nfull = ng / kWave;  // complete 1 KB blocks of the row
    const int kfull = nfull > wv ? (nfull - wv + S - 1) / S : 0;
    auto issue_full = [&](uint4 (&d)[U], int kk) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) d[u] = load16<NT>(vp + (size_t)(wv + (kk + u) * S) * kWave + lane);
    };
    auto filter_full = [&](const uint4 (&d)[U], int kk) __attribute__((always_inline)) {
        if constexpr (PROB) add_groups<TR, U>(st, d);
        const int thr_u = __builtin_amdgcn_readfirstlane(thr);
        if (thr_u >= 1) {
            const uint32_t t2 = TR::splat_below(thr_u);
#pragma unroll
            for (int u = 0; u < U; ++u) append(d[u], TR::pass_positive(d[u], t2), kk + u);
        } else if (thr_u == INT_MIN) {
#pragma unroll
            for (int u = 0; u < U; ++u) append(d[u], true, kk + u);
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) append(d[u], TR::group_pass(d[u], thr), kk + u);
        }
        maybe_process();
    };

    // the wave's last blocks (fewer than U complete ones and the row's partial
    // last block if this wave owns it), with bounds checks: loaded by load_rem,
    // filtered by filter_rem
    auto load_rem = [&](uint4 (&d)[U], int k0) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int gi = min((wv + (k0 + u) * S) * kWave + lane, ng - 1);
            d[u] = load16<NT>(vp + gi);
        }
    };
    auto filter_rem = [&](const uint4 (&d)[U], int k0) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool inb = (k0 + u < kcount) && ((wv + (k0 + u) * S) * kWave + lane < ng);
            if constexpr (PROB) {
                if (inb) {
                    const uint4 one[1] = {d[u]};
                    add_groups<TR, 1>(st, one);
                }
            }
            append(d[u], inb && (thr == INT_MIN || TR::group_pass(d[u], thr)), k0 + u);
        }
        maybe_process();
    };
    int kk = 0;
    if (kfull >= U) {
        uint4 cur[U], nxt[U];
        issue_full(cur, 0);
        {
            // Seed the threshold: the 8th largest lane maximum of the first batch is a
            // lower bound of the wave's 8th best key when it is positive (8 distinct
            // elements reach it), so the first batch is filtered like the rest.
            int m = TR::kRawMin;
#pragma unroll
            for (int u = 0; u < U; ++u) m = max(m, TR::raw_max(cur[u]));
            int m8 = TR::kRawMin;
#pragma unroll
            for (int j = 0; j < kTop; ++j) {
                m8 = wave_max_i32(m);
                const uint64_t own = ballot(m == m8);
                if (lane == __ffsll((unsigned long long)own) - 1) m = TR::kRawMin;
            }
            if (m8 >= 1 && m8 > thr) set_thr(m8);
        }
        for (; kk + 2 * U <= kfull; kk += U) {
            issue_full(nxt, kk + U);
            filter_full(cur, kk);
#pragma unroll
            for (int u = 0; u < U; ++u) cur[u] = nxt[u];
        }
        // unsplit rows: the last blocks are loaded while the last full batch is
        // filtered (measured: -0.15 us per launch at 976 rows; split rows, whose
        // waves stream few blocks, were 0.1 us slower with it)
        const bool rem = !SPLIT && kk + U < kcount;
        if (rem) load_rem(nxt, kk + U);
        filter_full(cur, kk);
        kk += U;
        if (rem) {
            filter_rem(nxt, kk);
            kk += U;
        }
    }
    for (; kk < kcount; kk += U) {
        uint4 d[U];
        load_rem(d, kk);
        filter_rem(d, kk);
    }
    // the row's hand-off word, read before the final merges: once it shows the
    // registration (1) it keeps that value until this row clears it
    int handoff_seen = 0;
    if constexpr (ACCEPT) {
        if (wv == 0 && lane == 0 && v.table) handoff_seen = ld_agent((const int32_t *)&v.handoff[row]);
    }
    if (count) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        process();
    }

    // The row's S waves meet: each publishes its exact top-8 (row ranks); wave 0
    // ranks the S x 8 entries by counting, for each, the entries above it.
    constexpr int kScale = sizeof(Rank) == 4 ? 65536 : 1;  // wave key -> fp32 key
    if (lane < kTop) {
        uint64_t r = 0;
        if (top) r = rank64(TR::rank_key(top) * kScale, global_id(TR::local_off(top)));
        s_cand[wv * kTop + lane] = r;
    }
    if constexpr (PROB) {
        const float M = wave_max_f32(st.m);
        const float s = (st.m == -INFINITY) ? 0.0f : st.s * __expf(st.m - M);
        const float Ssum = wave_sum_f32(s);
        if (lane == 0) s_stat[wv] = make_float2(M, Ssum);
    }
    __syncthreads();
    if (wv != 0) return;
    // Unsplit rows: once the hand-off word has shown the registration, the row's
    // holder word is final (the registration published its maxima before it
    // arrived), so it is read now, under the row selection, instead of after it.
    int occ_read = 0;
    if constexpr (ACCEPT && !SPLIT) {
        if (v.table && lane == 0 && handoff_seen == 1 && row_tok >= 0 && row_tok < a.V) {
            after_count();
            occ_read = ld_agent(&v.last_occ[row_tok]);
        }
    }
    uint64_t rtop = 0;  // lanes 0..7: the row's top-8 (row ranks), descending
    {
        // each entry's rank is the number of entries above it (row ranks are
        // distinct, zeros mark empty slots), counted over LDS broadcasts; up to
        // two entries per lane
        const int nent = S * kTop;
        const uint64_t x0 = lane < nent ? s_cand[lane] : 0ull;
        int a0 = 0, a1 = 0;
        if (nent <= kWave) {
            for (int j = 0; j < nent; ++j) a0 += s_cand[j] > x0 ? 1 : 0;
        } else {
            const uint64_t x1 = lane + kWave < nent ? s_cand[lane + kWave] : 0ull;
            for (int j = 0; j < nent; ++j) {
                const uint64_t y = s_cand[j];
                a0 += y > x0 ? 1 : 0;
                a1 += y > x1 ? 1 : 0;
            }
            if (lane < kTop) s_top[lane] = 0ull;
            if (x1 != 0ull && a1 < kTop) s_top[a1] = x1;
        }
        if (nent <= kWave && lane < kTop) s_top[lane] = 0ull;
        if (x0 != 0ull && a0 < kTop) s_top[a0] = x0;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        rtop = lane < kTop ? s_top[lane] : 0ull;
    }
    // the workgroup's softmax statistics (largest value, sum of exp(x - largest))
    float rowM = -INFINITY, rowS = 0.0f;
    if constexpr (PROB) {
        const float2 sv = lane < S ? s_stat[lane] : make_float2(-INFINITY, 0.0f);
        rowM = wave_max_f32(sv.x);
        const float s = (sv.x == -INFINITY) ? 0.0f : sv.y * __expf(sv.x - rowM);
        rowS = wave_sum_f32(s);
    }
    if constexpr (SPLIT) {
        // Store this slice's top-8 and statistics and arrive at the row's counter
        // at once, without waiting for the stores: the row's last slice to arrive
        // merges the G results and goes on as the row's finisher, clearing what it
        // read.  Every stored word is nonzero (an empty entry is stored as
        // kEmptyRank; the packed statistics never read zero), so the finisher
        // reads another slice's words again until none is zero (a store still on
        // its way); its own come from registers.  A wait beyond kSpinTicks gives
        // up: the row then reports no ids.
        const size_t pb = (size_t)row * G * kTop;
        const size_t ps = (size_t)row * G;
        if (lane < kTop) st_agent(&a.part[pb + (size_t)g * kTop + lane], rtop ? rtop : kEmptyRank);
        if (PROB && lane == 0) st_agent(&a.pstat[ps + g], pack_stats(rowM, rowS));
        uint32_t old = 0;
        if (lane == 0) old = __hip_atomic_fetch_add(&a.cnt[row], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((int)readlane_i32((int)old, 0) != G - 1) return;
        after_count();
        // the finisher reads the token's holder word now, beside the slices'
        // results, once its hand-off word has shown the registration (as above)
        if constexpr (ACCEPT) {
            if (v.table && lane == 0 && handoff_seen == 1 && row_tok >= 0 && row_tok < a.V)
                occ_read = ld_agent(&v.last_occ[row_tok]);
        }
        const int n = G * kTop;  // <= 64: one entry per lane
        const bool own = lane >= g * kTop && lane < (g + 1) * kTop;
        const bool other = lane < n && !own;
        const bool other_st = PROB && lane < G && lane != g;
        const uint64_t mine = shfl_u64(rtop, own ? lane - g * kTop : 0);
        uint64_t x = own ? (mine ? mine : kEmptyRank) : 0ull;
        uint64_t sv = 0ull;
        const uint64_t t0 = wall_clock64();
        bool ok = true;
        while (true) {
            if (other && x == 0ull) x = ld_agent(&a.part[pb + lane]);
            if (other_st && sv == 0ull) sv = ld_agent(&a.pstat[ps + lane]);
            if (!ballot((other && x == 0ull) || (other_st && sv == 0ull))) break;
            if (wall_clock64() - t0 > kSpinTicks) {
                ok = false;
                break;
            }
        }
        if (x == kEmptyRank) x = 0ull;
        // rank over LDS broadcasts (the row's candidate area is this wave's now)
        if (lane < n) s_cand[lane] = x;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        int above = 0;
        for (int j = 0; j < n; ++j) above += s_cand[j] > x ? 1 : 0;
        if (lane < kTop) s_top[lane] = 0ull;
        if (x != 0ull && above < kTop) s_top[above] = x;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        rtop = (lane < kTop && ballot(!ok) == 0ull) ? s_top[lane] : 0ull;
        // clear what was read: the other slices' words by the lanes that read
        // them, this slice's own by the lanes that stored them
        if (other) st_agent(&a.part[pb + lane], 0ull);
        if (lane < kTop) st_agent(&a.part[pb + (size_t)g * kTop + lane], 0ull);
        if constexpr (PROB) {
            if (lane == 0) st_agent(&a.pstat[ps + g], 0ull);
            float m = -INFINITY, ss = 0.0f;
            if (lane == g) {
                m = rowM;
                ss = rowS;
            } else if (other_st) {
                m = __uint_as_float((uint32_t)(sv >> 32));
                ss = __uint_as_float((uint32_t)sv);
                st_agent(&a.pstat[ps + lane], 0ull);
            }
            rowM = wave_max_f32(m);
            rowS = wave_sum_f32((m == -INFINITY) ? 0.0f : ss * __expf(m - rowM));
        }
        if (lane == 0) st_agent(&a.cnt[row], 0u);
    }
    const int tok_u = __builtin_amdgcn_readfirstlane(row_tok);
    const int hs_u = readlane_i32(handoff_seen, 0);
    const int occ_u = readlane_i32(occ_read, 0);
    const uint32_t tag_u = (uint32_t)readlane_i32((int)(uint32_t)(tag_old >> 32), 0) + 1u;
    finish_row<PROB, ACCEPT>(a, v, row, rtop, rowM, rowS, tok_u, hs_u, occ_u, tag_u);
}

template <typename TR, bool PROB, bool ACCEPT, int U>
void launch_rows_u(const TopkArgs &a, const VerifyArgs &vv, dim3 grid, dim3 block, hipStream_t s) {
    if (a.merge_wave) {
        hipLaunchKernelGGL((k_topk_mw<TR, PROB, ACCEPT, U>), grid, block, MwSmem<U>::bytes(a.S), s, a, vv);
        return;
    }
    const size_t lds = RowSmem<typename TR::Rank, U>::bytes(a.S);
    if (a.groups > 1)
        hipLaunchKernelGGL((k_topk_rows<TR, PROB, ACCEPT, true, true, U>), grid, block, lds, s, a, vv);
    else
        hipLaunchKernelGGL((k_topk_rows<TR, PROB, ACCEPT, true, false, U>), grid, block, lds, s, a, vv);
}

template <typename TR, bool PROB, bool ACCEPT>
void launch_rows_as(const TopkArgs &a, const VerifyArgs &vv, dim3 grid, dim3 block, hipStream_t s) {
    // four blocks per batch where the plan asks for them and the LDS allows;
    // merge-wave rows with softmax statistics always take four (an exponential
    // per element: 976 x 151936 with statistics 55.8 us with four, 68.6 with two)
    const size_t lds4 = a.merge_wave ? MwSmem<4>::bytes(a.S) : RowSmem<typename TR::Rank, 4>::bytes(a.S);
    if ((a.loads == 4 || (PROB && a.merge_wave)) && lds4 <= (size_t)kMaxLdsPerGroup)
        launch_rows_u<TR, PROB, ACCEPT, 4>(a, vv, grid, block, s);
    else
        launch_rows_u<TR, PROB, ACCEPT, 2>(a, vv, grid, block, s);
}

template <typename TR>
void launch_rows(const TopkArgs &a, const VerifyArgs *v, hipStream_t s) {
    const int extra = v ? v->ncoord : 0;  // the coordinator workgroups
    const dim3 grid((unsigned)(a.n_rows * a.groups + extra));
    const dim3 block(kWave * (a.S + a.merge_wave));
    const VerifyArgs vv = v ? *v : VerifyArgs{};
    const bool prob = a.prob != nullptr || a.stats != nullptr;  // softmax statistics wanted
    if (v) {
        if (prob)
            launch_rows_as<TR, true, true>(a, vv, grid, block, s);
        else
            launch_rows_as<TR, false, true>(a, vv, grid, block, s);
    } else {
        if (prob)
            launch_rows_as<TR, true, false>(a, vv, grid, block, s);
        else
            launch_rows_as<TR, false, false>(a, vv, grid, block, s);
    }
}

}  // namespace

// S waves per row: about target_waves over the chip, at most 16 per row, and
// few enough blocks per wave that local offsets fit: bf16 ranks hold 16-bit
// offsets (127 blocks of 512 elements per wave), fp32 ranks 32-bit ones,
// where the 16-bit pending-group index allows 1023 blocks of 256.
static int waves_per_row(int64_t n_rows, int V, int dtype, int64_t target_waves, int groups) {
    const int epg = dtype == GRAFT_DTYPE_BF16 ? 8 : 4;
    const int64_t nblk = (((int64_t)V / epg + kWave - 1) / kWave + groups - 1) / groups;  // blocks per slice
    const int64_t units = (n_rows > 0 ? n_rows : 1) * groups;
    int64_t S = (target_waves + units - 1) / units;
    S = S < 1 ? 1 : (S > kMaxWavesPerRow ? kMaxWavesPerRow : S);
    const int64_t per_wave = dtype == GRAFT_DTYPE_BF16 ? 127 : 1023;
    const int64_t smin = (nblk + per_wave - 1) / per_wave;
    if (S < smin) S = smin;
    if (S > nblk && nblk > 0) S = nblk;
    if (S < 1) S = 1;
    return (int)S;
}

// About 2928 waves (11-12 per CU: at 976 rows 3 per row with four blocks per
// batch beat 4 per row with two by 0.4 us per step; 3 per row with two blocks,
// and 5 or 6 per row, were slower).  Launches with softmax statistics take the
// same plan (58.1 us at 976 rows, against 58.5-58.8 us for 5 per row with two
// blocks, the best plan with two).
constexpr int64_t kTargetWaves = 2928;

// Rows are split over several workgroups when there are too few of them to
// spread over the chip (fewer than 512): about 1024 workgroups in all, at most
// 4 per row, each slice at least 8 blocks, and about 1920 waves in all (fewer,
// longer waves than the unsplit launch: measured over 61-, 244- and 272-row
// launches, 4 slices x 1920 waves beat 8 slices x 3840 by 2-3 us at 61 rows and
// 1 us at 244 rows, and 2 or 3 slices, 960 or 2880 waves did worse overall).
constexpr int64_t kSplitBelowRows = 512, kSplitTargetUnits = 1024;
constexpr int kMaxGroups = 4;
constexpr int64_t kSplitTargetWaves = 1920;

// Blocks per batch (measured): four for one workgroup per row (a 2048-row
// ingest chunk: 109 -> 101 us; 976 rows at 3 waves per row: see kTargetWaves)
// and for split rows whose waves stream at least 6 blocks each (TAIL 272 rows:
// 26.1 -> 23.9 us; 244 rows: 1.8 us off the step; 61 rows of 128256 bf16, ~7.8
// blocks per wave: 11.27 -> 10.98 us); two for split rows with only a few
// blocks per wave (61 rows: 3.4 us slower with four at V=32000 fp32).
constexpr int64_t kDeepBatchMinBlocks = 6;
static int loads_for(int64_t n_rows, int V, int dtype, int groups, int S) {
    if (n_rows >= kSplitBelowRows) return 4;
    const int epg = dtype == GRAFT_DTYPE_BF16 ? 8 : 4;
    const int64_t nblk = (((int64_t)V / epg + kWave - 1) / kWave + groups - 1) / groups;  // blocks per slice
    return nblk / (S > 0 ? S : 1) >= kDeepBatchMinBlocks ? 4 : 2;
}

// Rows stay whole below kSplitBelowRows too when one workgroup per row puts at
// most one workgroup on each of the chip's 256 CUs and the per-row wave cap
// still reaches kTargetWaves (183-256 rows).  Measured: 244 rows whole take 0.45
// us off the step; 272 rows whole (16 CUs with two rows, finishing last) cost
// 2.8 us, so they stay split.
constexpr int64_t kCUs = 256;
constexpr int kFewRowWaves = 8;
constexpr int64_t kTwoRowsMin = 436;  // about 0.85 x two rows on every CU
constexpr int64_t kSliceBlocksFor8 = 68, kSliceWavesMax = 4096;
static int groups_per_row(int64_t n_rows, int V, int dtype) {
    if (n_rows <= 0 || n_rows >= kSplitBelowRows) return 1;
    if (n_rows <= kCUs && (kTargetWaves + n_rows - 1) / n_rows <= kMaxWavesPerRow) return 1;
    const int epg = dtype == GRAFT_DTYPE_BF16 ? 8 : 4;
    const int64_t nblk = ((int64_t)V / epg + kWave - 1) / kWave;
    int64_t G = (kSplitTargetUnits + n_rows - 1) / n_rows;
    G = G > kMaxGroups ? kMaxGroups : G;
    G = G > nblk / 8 ? nblk / 8 : G;
    return G < 1 ? 1 : (int)G;
}

// One workgroup per row with long streams gets a merge wavefront beside its
// streaming waves: at least kMwMinBlocks 1 KB blocks per streaming wave, and
// at most kMwMaxStreams of them (measured: 244 rows of 12 streaming waves took
// 35 us with one merge wave against 20 us without; 976 rows of 3, 48.4 against
// 48.9 us; a 2048-row prompt chunk of 3, 98.6 against 100.3 us).
constexpr int64_t kMwMinBlocks = 16;
constexpr int kMwMaxStreams = 4;
constexpr int64_t kMwDeepBatchRows = 1536;
static int merge_wave_for(int V, int dtype, int groups, int S) {
    if (groups != 1 || S > kMwMaxStreams) return 0;
    const int epg = dtype == GRAFT_DTYPE_BF16 ? 8 : 4;
    const int64_t nblk = ((int64_t)V / epg + kWave - 1) / kWave;
    return nblk / S >= kMwMinBlocks ? 1 : 0;
}

// Coordinator workgroups of a verify launch: one wavefront per request, at
// most GRAFT_MAX_COORD_GROUPS workgroups (each wavefront then watches every
// (groups x S)-th request in turn).  The coordinators are dispatched ahead of
// the rows and wait for them, so they must never fill the chip: 128
// workgroups of at most 16 wavefronts and 64 KB of LDS take at most a quarter
// of its wavefront slots and half the LDS of 128 CUs, whatever the batch.
int coord_groups(const TopkPlan &p, int B) {
    const int w = p.splits + p.merge_wave;  // wavefronts per workgroup
    const int64_t want = ((int64_t)B + w - 1) / w;
    return (int)(want < GRAFT_MAX_COORD_GROUPS ? want : GRAFT_MAX_COORD_GROUPS);
}

static_assert(kCounterBytes == GRAFT_WS_COUNTER_BYTES, "the header states the counter region's size");
static_assert(kCounterBytes % 256 == 0, "the regions after the counters stay 256-byte aligned");

TopkPlan plan_topk(int64_t n_rows, int V, int dtype) {
    TopkPlan p;
    p.n_rows = n_rows;
    p.V = V;
    p.dtype = dtype;
    p.groups = groups_per_row(n_rows, V, dtype);
    p.splits = waves_per_row(n_rows, V, dtype, p.groups > 1 ? kSplitTargetWaves : kTargetWaves, p.groups);
    // whole rows at one workgroup per CU (183-256 rows) stream best with 8 waves
    // of four blocks per batch (244 rows x 151936 bf16: 17.7 us against 18.8 with
    // 12 waves of two, 18.1 with 6 and 18.9 with 10 of four; 183 rows: 16.2
    // against 18.3 us), and so do whole rows at two workgroups on nearly every CU
    // (436-511 rows; 448 rows: 27.7 against 29.3 us in slices, 476: 28.9 against
    // 30.1, 488: 29.4 against 30.4; at 427 rows the two tie and below that the
    // CUs holding a second row finish last: 305 rows 24.5 against 22.6 us),
    // where 8 waves keep within the per-wave block cap
    {
        const int epg = dtype == GRAFT_DTYPE_BF16 ? 8 : 4;
        const int64_t nblk = ((int64_t)V / epg + kWave - 1) / kWave;
        const int64_t per_wave = dtype == GRAFT_DTYPE_BF16 ? 127 : 1023;
        const bool fits = (nblk + kFewRowWaves - 1) / kFewRowWaves <= per_wave;
        if (fits && p.groups == 1 && n_rows <= kCUs && p.splits > kFewRowWaves) p.splits = kFewRowWaves;
        if (fits && p.groups > 1 && n_rows >= kTwoRowsMin && n_rows < kSplitBelowRows) {
            p.groups = 1;
            p.splits = kFewRowWaves;
        }
    }
    // split bf16 rows: 8 waves per slice while every slice still holds at least
    // 68 blocks and the launch stays within 4096 waves (122 rows: 13.76 against
    // 14.14 us at V=151936, 13.26 against 13.65 at 140000, 14.43 against 15.52 at
    // 180000; with fewer blocks the wave target's 4 waves do better: 12.38 against
    // 12.68 us at 128256, 10.38 against 11.65 at 64000).  fp32 rows keep the wave
    // target (122 rows of 151936: 19.53 against 19.30 us with 8 waves)
    if (dtype == GRAFT_DTYPE_BF16 && p.groups > 1 && p.splits < kFewRowWaves) {
        const int epg = dtype == GRAFT_DTYPE_BF16 ? 8 : 4;
        const int64_t nblk = ((int64_t)V / epg + kWave - 1) / kWave;
        const int64_t per_slice = (nblk + p.groups - 1) / p.groups;
        if (per_slice >= kSliceBlocksFor8 && n_rows * p.groups * kFewRowWaves <= kSliceWavesMax) p.splits = kFewRowWaves;
    }
    p.loads = loads_for(n_rows, V, dtype, p.groups, p.splits);
    p.merge_wave = merge_wave_for(V, dtype, p.groups, p.splits);
    // streaming waves that never stop to merge do best with two blocks per batch
    // while every row's workgroup is resident at once (976 x 151936: 47.98 against
    // 48.31 us with four; 2 or 4 streaming waves with two blocks, 57.1 and 48.6
    // us); more rows keep four (2048-row prompt chunk: 98.0 us against 108.7)
    if (p.merge_wave && n_rows < kMwDeepBatchRows) p.loads = 2;
    // four blocks per batch only where that workgroup's LDS stays within the cap
    // (the 244-row launch's 12 waves take two: 71 KB with four; with a 160 KB
    // cap four measured no faster there)
    if (p.loads == 4 && !p.merge_wave) {
        const size_t lds4 = dtype == GRAFT_DTYPE_BF16 ? RowSmem<uint32_t, 4>::bytes(p.splits)
                                                      : RowSmem<uint64_t, 4>::bytes(p.splits);
        if (lds4 > (size_t)kMaxLdsPerGroup) p.loads = 2;
    }
    // workspace: [tagged completion words [kTagRows], launch counters [kTagRows] |
    //             completion words [n_rows] | last holder per token [V], spare,
    //             hand-offs [n_rows]]
    p.off_counters = kCounterBytes;
    p.off_occ = p.off_counters + ((size_t)n_rows * sizeof(int32_t) + 255) / 256 * 256;
    p.ws_bytes = p.off_occ + ((size_t)(V + 1 + n_rows) * sizeof(uint32_t) + 255) / 256 * 256;
    if (p.groups > 1) {  // [arrival counters [n_rows] | slice top-8s [n_rows, G, 8] | slice statistics]
        const size_t nr = (size_t)n_rows, G = (size_t)p.groups;
        p.off_cnt = p.ws_bytes;
        p.off_part = p.off_cnt + (nr * sizeof(uint32_t) + 255) / 256 * 256;
        p.off_pstat = p.off_part + (nr * G * kTop * sizeof(uint64_t) + 255) / 256 * 256;
        p.ws_bytes = p.off_pstat + (nr * G * sizeof(uint64_t) + 255) / 256 * 256;
    }
    return p;
}

void launch_topk(const TopkPlan &p, int dtype, const void *logits, int k, int32_t *topk,
                 float *prob, float *stats, void *ws, const VerifyArgs *verify, hipStream_t s) {
    if (p.n_rows <= 0) return;
    TopkArgs a;
    a.logits = logits;
    a.n_rows = p.n_rows;
    a.V = p.V;
    a.S = p.splits;
    a.groups = p.groups;
    a.loads = p.loads;
    a.merge_wave = p.merge_wave;
    a.cnt = p.groups > 1 ? (uint32_t *)((char *)ws + p.off_cnt) : nullptr;
    a.part = p.groups > 1 ? (uint64_t *)((char *)ws + p.off_part) : nullptr;
    a.pstat = p.groups > 1 ? (uint64_t *)((char *)ws + p.off_pstat) : nullptr;
    a.k = k;
    a.topk = topk;
    a.prob = prob;
    a.stats = stats;
    VerifyArgs v;
    if (verify) {
        v = *verify;
        v.done = (int32_t *)((char *)ws + p.off_counters);
        v.last_occ = (int32_t *)((char *)ws + p.off_occ);
        v.handoff = (uint32_t *)(v.last_occ + p.V + 1);
        v.scan_holders = (v.table && scans_holders(p)) ? 1 : 0;
        if (v.update_only) {
            v.B = 0;
            v.ncoord = v.scan_holders ? 0 : 1;  // the registration, unless the rows scan
        } else {
            v.B = (int)(p.n_rows / (v.T1 > 0 ? v.T1 : 1));
            v.ncoord = coord_groups(p, v.B);
            if (uses_launch_counters(p)) {
                v.tag_done = (uint64_t *)ws;
                v.tag_want = (uint32_t *)((char *)ws + (size_t)kTagRows * sizeof(uint64_t));
            }
        }
    }
    if (dtype == GRAFT_DTYPE_BF16)
        launch_rows<Bf16Traits>(a, verify ? &v : nullptr, s);
    else
        launch_rows<F32Traits>(a, verify ? &v : nullptr, s);
}

}  // namespace graft
