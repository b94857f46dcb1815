// Wavefront (64-lane) helpers and order-preserving keys for the Graft kernels.
// gfx950 only: every kernel here is written for wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace graft {

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63u); }

// Number of set bits of `mask` below this lane (prefix count for compaction).
__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
    return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        uint64_t w = (uint64_t)__shfl_xor((long long)v, o);
        v = v > w ? v : w;
    }
    return v;
}

__device__ __forceinline__ int wave_max_i32(int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
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

}  // namespace graft
