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

// 8 codes of an 8-bit router row (two words, low byte first) restored to the
// bf16 weights a dense router would hold: nearest-even bf16 of the float32
// fused multiply-add scale * code + bias
__device__ __forceinline__ uint4 restore_q8x8(uint2 w, float s, float b) {
    uint32_t r[8];
#pragma unroll
    for (int k = 0; k < 8; k++) {
        const uint32_t code = ((k < 4 ? w.x : w.y) >> (8 * (k % 4))) & 0xFFu;
        const uint32_t u = __float_as_uint(__builtin_fmaf(s, (float)code, b));
        r[k] = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    }
    return make_uint4(r[0] | (r[1] << 16), r[2] | (r[3] << 16), r[4] | (r[5] << 16), r[6] | (r[7] << 16));
}

__device__ __forceinline__ half2_t splat_half2(float v) {
    _Float16 h = (_Float16)v;
    half2_t r = {h, h};
    return r;
}

// Order-preserving unsigned key of a finite float: a larger float gives a
// larger key.  -0 is taken as +0 (they compare equal).  Key 0 is below every
// finite float's key.
__device__ __forceinline__ uint32_t order_key(float v) {
    const uint32_t u = v == 0.0f ? 0u : __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// max with the value of the lane that DPP control kCtrl selects (every lane
// has one for the controls used here; bound_ctrl lets the move fold into the max)
template <int kCtrl>
__device__ __forceinline__ uint32_t max_dpp(uint32_t v) {
    return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, 0xF, 0xF, true));
}

// Largest v over the wave, as a wave-uniform value: DPP butterflies inside each
// row of 16 lanes, then the four row results through readlane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max_dpp<0xB1>(v);   // quad_perm 1,0,3,2
    v = max_dpp<0x4E>(v);   // quad_perm 2,3,0,1
    v = max_dpp<0x141>(v);  // row_half_mirror
    v = max_dpp<0x140>(v);  // row_mirror
    const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
    const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
    return max(max(a, b), max(c, d));
}

// Top-k of one token's logits held by one wave: lane l holds the logits of
// experts l, l + 64, l + 128, l + 192 in held[0..3] (entries of experts >= E are
// ignored).  Rank order is (logit desc, expert index asc).  Each of the k
// rounds takes the wave-wide largest order key; the ballots of key == max, in
// held order then lane order, give the lowest expert index holding it, whose
// key is then cleared.  Then the softmax of the kept logits (equal to the
// softmax over all E renormalised over the kept ones), summed in rank order.
// Lane j < k receives rank j: idx_j and w_j.
__device__ __forceinline__ void wave_topk_held(const float (&held)[kMaxE / kWave], int E, int top_k, int lane,
                                               int* idx_j, float* w_j) {
    constexpr int kPer = kMaxE / kWave;
    uint32_t key[kPer];
#pragma unroll
    for (int i = 0; i < kPer; i++) key[i] = lane + kWave * i < E ? order_key(held[i]) : 0u;
    uint32_t kept_key = 0;  // lane j: key of rank j
    int kept_idx = 0;       // lane j: expert of rank j
#pragma unroll
    for (int j = 0; j < kMaxTopK; j++) {
        if (j >= top_k) break;
        uint32_t lm = key[0];
#pragma unroll
        for (int i = 1; i < kPer; i++) lm = max(lm, key[i]);
        const uint32_t m = wave_max_u32(lm);
        int win_i = kPer - 1;
        uint64_t win_mask = 0;
#pragma unroll
        for (int i = kPer - 1; i >= 0; i--) {
            const uint64_t b = __ballot(key[i] == m);
            if (b) {
                win_i = i;
                win_mask = b;
            }
        }
        const int win_lane = (int)__builtin_ctzll(win_mask);
#pragma unroll
        for (int i = 0; i < kPer; i++)
            if (i == win_i && lane == win_lane) key[i] = 0u;
        if (lane == j) {
            kept_key = m;
            kept_idx = win_lane + kWave * win_i;
        }
    }
    const float top = key_float(__builtin_amdgcn_readlane(kept_key, 0));
    const float p = expf(key_float(kept_key) - top);
    float z = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxTopK; j++) {
        if (j >= top_k) break;
        z += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), j));
    }
    *idx_j = lane < top_k ? kept_idx : 0;
    *w_j = lane < top_k ? p / z : 0.0f;
}

// The same for logits read through `logit(e)` (expert e < E).
template <typename LogitFn>
__device__ __forceinline__ void wave_topk(LogitFn logit, int E, int top_k, int lane, int* idx_j, float* w_j) {
    float held[kMaxE / kWave];
#pragma unroll
    for (int i = 0; i < kMaxE / kWave; i++) {
        const int e = lane + kWave * i;
        held[i] = e < E ? logit(e) : -INFINITY;
    }
    wave_topk_held(held, E, top_k, lane, idx_j, w_j);
}

}  // namespace bitmoe
