// Device helpers shared by the decode kernels (the one-layer kernel and the
// persistent multi-layer kernel): matrix-vector products on packed 4-bit
// words, wave sums, and the {epoch, value} words workgroups hand over through
// memory.  Internal to libbitmoe.
#pragma once

#include "common.h"

namespace bitmoe {
namespace dec {

// workspace control word (uint32 index) set to nonzero when a device-side wait
// of a decode kernel gave up; shared by every decode kernel
constexpr int kCtlError = 255;

// float16 pairs of 8 activations in the order the exponent trick produces codes
struct Pairs8 {
    half2_t a04, a15, a26, a37;
};

__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t mask, uint32_t magic) {
    // (w & mask) | magic in one VALU op; gfx950 allows one scalar operand, so the
    // magic constant sits in a VGPR
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(mask), "v"(magic));
    return r;
}

// accumulate one packed word (8 codes) against its 8 activations
__device__ __forceinline__ void dot_word(uint32_t w, const Pairs8& p, float& acc_lo, float& acc_hi) {
    const uint32_t w8 = w >> 8;
    acc_lo = __builtin_amdgcn_fdot2(as_half2(and_or(w, 0x000F000Fu, 0x64006400u)), p.a04, acc_lo, false);
    acc_hi = __builtin_amdgcn_fdot2(as_half2(and_or(w, 0x00F000F0u, 0x54005400u)), p.a15, acc_hi, false);
    acc_lo = __builtin_amdgcn_fdot2(as_half2(and_or(w8, 0x000F000Fu, 0x64006400u)), p.a26, acc_lo, false);
    acc_hi = __builtin_amdgcn_fdot2(as_half2(and_or(w8, 0x00F000F0u, 0x54005400u)), p.a37, acc_hi, false);
}

__device__ __forceinline__ Pairs8 pairs_of(const uint4& v) {
    Pairs8 p;
    p.a04 = as_half2(v.x);
    p.a15 = as_half2(v.y);
    p.a26 = as_half2(v.z);
    p.a37 = as_half2(v.w);
    return p;
}

// 8 bf16 activations -> float16 pairs in nibble order; adds the low/high sums
__device__ __forceinline__ Pairs8 pairs_from_bf16(const uint4& raw, float& lo, float& hi) {
    const uint16_t* b = reinterpret_cast<const uint16_t*>(&raw);
    _Float16 h[8];
#pragma unroll
    for (int i = 0; i < 8; i++) h[i] = (_Float16)bf16_to_f32(b[i]);
    lo += (float)h[0] + (float)h[4] + (float)h[2] + (float)h[6];
    hi += (float)h[1] + (float)h[5] + (float)h[3] + (float)h[7];
    Pairs8 p;
    p.a04 = half2_t{h[0], h[4]};
    p.a15 = half2_t{h[1], h[5]};
    p.a26 = half2_t{h[2], h[6]};
    p.a37 = half2_t{h[3], h[7]};
    return p;
}

template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// sum over aligned groups of n consecutive lanes (n a power of two <= 64); every
// lane of a group receives the group's total
__device__ __forceinline__ float group_sum(float v, int n) {
    if (n >= 2) v += dpp<0xB1>(v);    // quad_perm 1,0,3,2
    if (n >= 4) v += dpp<0x4E>(v);    // quad_perm 2,3,0,1
    if (n >= 8) v += dpp<0x141>(v);   // row_half_mirror
    if (n >= 16) v += dpp<0x140>(v);  // row_mirror
    if (n >= 32) v += __shfl_xor(v, 16);
    if (n >= 64) v += __shfl_xor(v, 32);
    return v;
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// {epoch, value} words and plain values crossing workgroups: agent-scope
// accesses bypass the per-XCD L2, so no write-back or invalidate is needed
__device__ __forceinline__ void publish(unsigned long long* p, unsigned epoch, uint32_t bits) {
    __hip_atomic_store(p, ((unsigned long long)epoch << 32) | bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long peek(const unsigned long long* p) {
    return __hip_atomic_load(const_cast<unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void flag_error(unsigned* ctl) {
    __hip_atomic_store(ctl + kCtlError, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


}  // namespace dec
}  // namespace bitmoe
