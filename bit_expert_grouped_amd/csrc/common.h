// Internal helpers of the gfx950 MoE kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bitmoe {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr int kGroup = 64;      // quantisation group (input columns per scale/bias)
constexpr int kMaxE = 256;
constexpr int kMaxTopK = 8;

// Order of the eight 4-bit codes of one packed word inside the float16 vector
// that dequantisation produces: element e holds code kNibbleOf[e].  The low and
// high nibble of each byte pair come out of one 32-bit mask each, so the
// activation operand is stored with its 8-column blocks in the same order.
//   element: 0 1 2 3 4 5 6 7
//   nibble : 0 4 1 5 2 6 3 7
__host__ __device__ constexpr int nibble_of(int e) { return (e >> 1) + 4 * (e & 1); }
// position inside an 8-block at which column c (0..7) is stored
__host__ __device__ constexpr int slot_of_column(int c) { return 2 * (c & 3) + (c >> 2); }

__device__ __forceinline__ half2_t as_half2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t as_u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Affine 4-bit dequantisation of one packed word into float16, in the element
// order given by nibble_of().  Codes become exact float16 integers through the
// exponent trick: OR-ing a code into the mantissa of 1024.0 (0x6400, unit 1)
// yields 1024+q; OR-ing the high nibble of a byte (already scaled by 16) into
// the mantissa of 64.0 (0x5400, unit 1/16) yields 64+q.  One packed subtract
// recovers q exactly and one packed fma gives scale*q + bias, rounded once.
__device__ __forceinline__ half8_t dequant_word(uint32_t w, half2_t s, half2_t b) {
    const half2_t k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
    const half2_t k64 = {(_Float16)64.0f, (_Float16)64.0f};
    uint32_t w8 = w >> 8;
    half2_t q04 = as_half2((w & 0x000F000Fu) | 0x64006400u) - k1024;   // codes 0, 4
    half2_t q15 = as_half2((w & 0x00F000F0u) | 0x54005400u) - k64;     // codes 1, 5
    half2_t q26 = as_half2((w8 & 0x000F000Fu) | 0x64006400u) - k1024;  // codes 2, 6
    half2_t q37 = as_half2((w8 & 0x00F000F0u) | 0x54005400u) - k64;    // codes 3, 7
    half2_t r0 = __builtin_elementwise_fma(q04, s, b);
    half2_t r1 = __builtin_elementwise_fma(q15, s, b);
    half2_t r2 = __builtin_elementwise_fma(q26, s, b);
    half2_t r3 = __builtin_elementwise_fma(q37, s, b);
    half8_t out = {r0.x, r0.y, r1.x, r1.y, r2.x, r2.y, r3.x, r3.y};
    return out;
}

// scale/bias element as float, for either storage type
template <typename SB> __device__ __forceinline__ float sb_to_f32(SB v);
template <> __device__ __forceinline__ float sb_to_f32<uint16_t>(uint16_t v) { return bf16_to_f32(v); }
template <> __device__ __forceinline__ float sb_to_f32<float>(float v) { return v; }

__device__ __forceinline__ half2_t splat_half2(float v) {
    _Float16 h = (_Float16)v;
    half2_t r = {h, h};
    return r;
}

__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

template <int kCtrl>
__device__ __forceinline__ void argmax_dpp_step(float& bv, int& bi) {
    const float ov = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(bv), kCtrl, 0xF, 0xF, false));
    const int oi = __builtin_amdgcn_mov_dpp(bi, kCtrl, 0xF, 0xF, false);
    if (ranks_before(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
    }
}

// Wave-wide arg-max of (value desc, index asc): DPP butterflies inside each row
// of 16 lanes (quad xor 1, quad xor 2, half-row mirror, row mirror), then the four
// row winners through readlane.  Every lane receives the winner.
__device__ __forceinline__ void wave_argmax(float& bv, int& bi) {
    argmax_dpp_step<0xB1>(bv, bi);   // quad_perm 1,0,3,2
    argmax_dpp_step<0x4E>(bv, bi);   // quad_perm 2,3,0,1
    argmax_dpp_step<0x141>(bv, bi);  // row_half_mirror
    argmax_dpp_step<0x140>(bv, bi);  // row_mirror
    float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 0));
    int i = __builtin_amdgcn_readlane(bi, 0);
#pragma unroll
    for (int r = 1; r < 4; r++) {
        const float rv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 16 * r));
        const int ri = __builtin_amdgcn_readlane(bi, 16 * r);
        if (ranks_before(rv, ri, v, i)) {
            v = rv;
            i = ri;
        }
    }
    bv = v;
    bi = i;
}

// Top-k of one token's logits by one wave: k rounds of a wave-wide arg-max on
// (logit desc, expert index asc), then the softmax of the kept logits (equal to
// the softmax over all E renormalised over the kept ones).  `logit(e)` returns
// the logit of expert e < E.  Lane j < k receives rank j: idx_j and w_j.
template <typename LogitFn>
__device__ __forceinline__ void wave_topk(LogitFn logit, int E, int top_k, int lane, int* idx_j, float* w_j) {
    float v[kMaxE / kWave];
    int id[kMaxE / kWave];
#pragma unroll
    for (int i = 0; i < kMaxE / kWave; i++) {
        id[i] = lane + kWave * i;
        v[i] = id[i] < E ? logit(id[i]) : -INFINITY;
        if (id[i] >= E) id[i] = 0x7fffffff;
    }
    float kept_v[kMaxTopK];
    int kept_i[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; j++) {
        if (j >= top_k) break;
        float bv = v[0];
        int bi = id[0];
#pragma unroll
        for (int i = 1; i < kMaxE / kWave; i++) {
            if (ranks_before(v[i], id[i], bv, bi)) {
                bv = v[i];
                bi = id[i];
            }
        }
        wave_argmax(bv, bi);
        kept_v[j] = bv;
        kept_i[j] = bi;
#pragma unroll
        for (int i = 0; i < kMaxE / kWave; i++) {
            if (id[i] == bi) v[i] = -INFINITY, id[i] = 0x7fffffff;
        }
    }
    float z = 0.0f, wj = 0.0f;
    int ij = 0;
#pragma unroll
    for (int j = 0; j < kMaxTopK; j++) {
        if (j >= top_k) break;
        const float p = expf(kept_v[j] - kept_v[0]);
        z += p;
        if (j == lane) {
            wj = p;
            ij = kept_i[j];
        }
    }
    *idx_j = ij;
    *w_j = wj / z;
}

}  // namespace bitmoe
