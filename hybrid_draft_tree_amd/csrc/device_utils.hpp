// Wavefront (64-lane) helpers and order-preserving keys for the Graft kernels.
// gfx950 only: every kernel here is written for wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <climits>

namespace graft {

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63u); }

// Number of set bits of `mask` below this lane (prefix count for compaction).
__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Wave-wide reductions through DPP row operations (no LDS crossbar): pairs, quads,
// half-rows, rows, then rows 0+1 and 2+3 via row broadcasts; lane 63 ends up with
// the full result, read back as a wave-uniform value.  The mirror steps pair each
// lane with a distinct partner, so the sequence is valid for max and for sum.
// Lanes a step leaves out (row mask) take `id`; with the operation's identity
// there the compiler folds each step into one DPP-modified ALU instruction.
#define GRAFT_DPP_ID(id, v, ctrl, rmask) __builtin_amdgcn_update_dpp((id), (v), (ctrl), (rmask), 0xf, false)
#define GRAFT_DPP(v, ctrl, rmask) GRAFT_DPP_ID((v), (v), (ctrl), (rmask))
constexpr int kDppXor1 = 0xb1;      // quad_perm(1,0,3,2)
constexpr int kDppXor2 = 0x4e;      // quad_perm(2,3,0,1)
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppBcast15 = 0x142;
constexpr int kDppBcast31 = 0x143;

template <typename Op>
__device__ __forceinline__ int dpp_reduce_i32(int v, Op op) {
    v = op(v, GRAFT_DPP(v, kDppXor1, 0xf));
    v = op(v, GRAFT_DPP(v, kDppXor2, 0xf));
    v = op(v, GRAFT_DPP(v, kDppHalfMirror, 0xf));
    v = op(v, GRAFT_DPP(v, kDppMirror, 0xf));
    v = op(v, GRAFT_DPP(v, kDppBcast15, 0xa));
    v = op(v, GRAFT_DPP(v, kDppBcast31, 0xc));
    return __builtin_amdgcn_readlane(v, 63);
}

// Same with the operation's identity for the left-out lanes (integer max).
template <typename Op>
__device__ __forceinline__ int dpp_reduce_id_i32(int v, int id, Op op) {
    v = op(v, GRAFT_DPP_ID(id, v, kDppXor1, 0xf));
    v = op(v, GRAFT_DPP_ID(id, v, kDppXor2, 0xf));
    v = op(v, GRAFT_DPP_ID(id, v, kDppHalfMirror, 0xf));
    v = op(v, GRAFT_DPP_ID(id, v, kDppMirror, 0xf));
    v = op(v, GRAFT_DPP_ID(id, v, kDppBcast15, 0xa));
    v = op(v, GRAFT_DPP_ID(id, v, kDppBcast31, 0xc));
    return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    return (uint32_t)dpp_reduce_id_i32((int)v, 0, [](int a, int b) { return (int)max((uint32_t)a, (uint32_t)b); });
}

__device__ __forceinline__ int wave_max_i32(int v) {
    return dpp_reduce_id_i32(v, INT_MIN, [](int a, int b) { return max(a, b); });
}

__device__ __forceinline__ float wave_max_f32(float v) {
    return __int_as_float(dpp_reduce_i32(__float_as_int(v), [](int a, int b) {
        return __float_as_int(fmaxf(__int_as_float(a), __int_as_float(b)));
    }));
}

__device__ __forceinline__ float wave_sum_f32(float v) {
    return __int_as_float(dpp_reduce_i32(__float_as_int(v), [](int a, int b) {
        return __float_as_int(__int_as_float(a) + __int_as_float(b));
    }));
}

template <int CTRL, int RMASK>
__device__ __forceinline__ uint64_t max_u64_dpp(uint64_t v) {
    const int l = (int)(uint32_t)v, h = (int)(uint32_t)(v >> 32);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(l, l, CTRL, RMASK, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(h, h, CTRL, RMASK, 0xf, false);
    const uint64_t w = ((uint64_t)hi << 32) | lo;
    return v > w ? v : w;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = max_u64_dpp<kDppXor1, 0xf>(v);
    v = max_u64_dpp<kDppXor2, 0xf>(v);
    v = max_u64_dpp<kDppHalfMirror, 0xf>(v);
    v = max_u64_dpp<kDppMirror, 0xf>(v);
    v = max_u64_dpp<kDppBcast15, 0xa>(v);
    v = max_u64_dpp<kDppBcast31, 0xc>(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
    return (uint64_t)__shfl((long long)v, src);
}

// Order-preserving signed key of an IEEE fp32 bit pattern: the two's complement
// of the sign-magnitude value, so signed integer order is numeric order and
// -0 and +0 share the key 0.  NaN is outside the contract.
__device__ __forceinline__ int32_t f32_key(uint32_t bits) {
    int32_t mag = (int32_t)(bits & 0x7fffffffu);
    return (bits & 0x80000000u) ? -mag : mag;
}

// Same for a bf16 bit pattern (low 16 bits of h); range [-32767, 32767].
__device__ __forceinline__ int32_t bf16_key(uint32_t h) {
    int32_t mag = (int32_t)(h & 0x7fffu);
    return (h & 0x8000u) ? -mag : mag;
}

// Inverse of f32_key for a non-NaN key: the fp32 value.
__device__ __forceinline__ float key_to_f32(int32_t key) {
    uint32_t bits = key >= 0 ? (uint32_t)key : (0x80000000u | (uint32_t)(-key));
    return __uint_as_float(bits);
}

// Row-level ranking key: value (fp32 key, descending) then id (ascending) in one
// unsigned 64-bit word; larger ranks first.  0 never occurs for a real element.
__device__ __forceinline__ uint64_t rank64(int32_t fkey, uint32_t id) {
    return ((uint64_t)((uint32_t)fkey ^ 0x80000000u) << 32) | (uint64_t)(0xffffffffu - id);
}
__device__ __forceinline__ uint32_t rank64_id(uint64_t r) { return 0xffffffffu - (uint32_t)r; }
__device__ __forceinline__ int32_t rank64_key(uint64_t r) {
    return (int32_t)((uint32_t)(r >> 32) ^ 0x80000000u);
}

// ---- cross-workgroup hand-off without cache maintenance ---------------------------
// Data handed from one wavefront to another inside a launch (possibly on another
// XCD, whose L2 is not coherent with ours) is written and read with agent-scope
// relaxed atomics: the stores write through to the device coherence point and
// the loads do not hit stale lines.  publish() waits until this wave's earlier
// stores have completed, so a completion counter bumped afterwards is only seen
// once the data is visible.  This replaces a device-scope fence, which on this
// chip writes back and invalidates the whole L2.
__device__ __forceinline__ void st_agent(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(int32_t *p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_agent(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_agent(const int32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void publish() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
}
__device__ __forceinline__ uint32_t count_in(uint32_t *ctr) {
    return __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void after_count() {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Broadcast lane `j` (wave-uniform) of a 32-bit value.
__device__ __forceinline__ int readlane_i32(int v, int j) { return __builtin_amdgcn_readlane(v, j); }
__device__ __forceinline__ float readlane_f32(float v, int j) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j));
}

}  // namespace graft
