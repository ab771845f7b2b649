// Router + top-k kernel for gfx950.
//
// Pages: every token scores all experts and keeps 8 (aimanavo.com page, section
// "Qwen3.6's 256 experts and two layer types make the MLX-Lily gap"); routing
// stays on the GPU (same page, section "Lily does not treat prefill and decode as
// the same job").
//
// One workgroup = 32 tokens x all E (<= 256) experts.  The logits are a bf16
// MFMA product (32x32x16, exact bf16 products, float32 accumulation): wave w
// owns experts [64w, 64w+64) as two 32-column tiles.  Both operands stream
// straight from global memory (x rows are shared by the four waves through the
// vector L1).  The 32x256 float32 logit tile then goes through LDS and each wave
// ranks 8 of the tokens: k rounds of a wave-wide arg-max (ties -> lower index),
// then the softmax of the kept logits.
//
// The fused variant used by the whole-layer call also
//   - writes the float16 copy of x (8-column blocks in dequantisation order)
//     that the expert kernels read, and
//   - clears the float32 output rows that the down kernel accumulates into.
#include "common.h"
#include "kernels.h"

namespace bitmoe {

namespace {

constexpr int kRouterTokens = 32;

template <bool kFused>
__global__ __launch_bounds__(256) void router_kernel(const uint16_t* __restrict__ x,
                                                     const uint16_t* __restrict__ wr,
                                                     const float* __restrict__ logit_bias, int T,
                                                     int H, int E, int top_k,
                                                     int32_t* __restrict__ topk_idx,
                                                     float* __restrict__ topk_w,
                                                     _Float16* __restrict__ x16,
                                                     float* __restrict__ out_clear) {
    __shared__ float logits[kRouterTokens][kMaxE + 1];

    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int t0 = blockIdx.x * kRouterTokens;
    const int row = lane % 32;
    const int half = lane / 32;

    // ---- logits: [32 tokens] x [64 experts of this wave] ----
    const int ebase = wave * 64;
    if (ebase < E) {
        const int ta = min(t0 + row, T - 1);
        const uint4* arow = reinterpret_cast<const uint4*>(x + (size_t)ta * H);
        const int e0 = min(ebase + row, E - 1);
        const int e1 = min(ebase + 32 + row, E - 1);
        const uint4* b0 = reinterpret_cast<const uint4*>(wr + (size_t)e0 * H);
        const uint4* b1 = reinterpret_cast<const uint4*>(wr + (size_t)e1 * H);
        floatx16 acc0 = {0}, acc1 = {0};
        const int nk = H / 16;
#pragma unroll 8
        for (int kk = 0; kk < nk; kk++) {
            const int c = 2 * kk + half;  // 16-byte chunk: columns [8c, 8c+8)
            uint4 a = arow[c];
            uint4 v0 = b0[c];
            uint4 v1 = b1[c];
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                           __builtin_bit_cast(bf16x8_t, v0), acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                           __builtin_bit_cast(bf16x8_t, v1), acc1, 0, 0, 0);
        }
        // C layout of 32x32 MFMA: lane holds column (lane%32), rows 8i + 4*(lane/32) + j
        const int ec0 = ebase + row, ec1 = ebase + 32 + row;
        const float bias0 = (logit_bias && ec0 < E) ? logit_bias[ec0] : 0.0f;
        const float bias1 = (logit_bias && ec1 < E) ? logit_bias[ec1] : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; i++) {
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int r = 8 * i + 4 * half + j;
                logits[r][ec0] = ec0 < E ? acc0[4 * i + j] + bias0 : -INFINITY;
                logits[r][ec1] = ec1 < E ? acc1[4 * i + j] + bias1 : -INFINITY;
            }
        }
    } else {
        for (int r = 0; r < kRouterTokens; r++) {
            logits[r][ebase + lane] = -INFINITY;
        }
    }
    __syncthreads();

    // ---- top-k per token: wave w ranks tokens 8w .. 8w+7 ----
    for (int r = wave * 8; r < wave * 8 + 8; r++) {
        const int t = t0 + r;
        if (t >= T) break;
        int ij;
        float wj;
        wave_topk([&](int e) { return logits[r][e]; }, E, top_k, lane, &ij, &wj);
        if (lane < top_k) {
            topk_idx[(size_t)t * top_k + lane] = ij;
            topk_w[(size_t)t * top_k + lane] = wj;
        }
    }

    if constexpr (kFused) {
        // float16 copy of x, 8-column blocks in dequantisation order
        const int nblk = H / 8;
        for (int i = threadIdx.x; i < kRouterTokens * nblk; i += blockDim.x) {
            const int r = i / nblk, blk = i % nblk;
            const int t = t0 + r;
            if (t >= T) break;
            uint4 raw = reinterpret_cast<const uint4*>(x + (size_t)t * H)[blk];
            const uint16_t* hb = reinterpret_cast<const uint16_t*>(&raw);
            half8_t o;
#pragma unroll
            for (int e = 0; e < 8; e++) o[e] = (_Float16)bf16_to_f32(hb[nibble_of(e)]);
            reinterpret_cast<half8_t*>(x16 + (size_t)t * H)[blk] = o;
        }
        const int n4 = H / 4;
        const float4 zero = {0.f, 0.f, 0.f, 0.f};
        for (int i = threadIdx.x; out_clear && i < kRouterTokens * n4; i += blockDim.x) {
            const int r = i / n4, c = i % n4;
            const int t = t0 + r;
            if (t >= T) break;
            reinterpret_cast<float4*>(out_clear + (size_t)t * H)[c] = zero;
        }
    }
}

}  // namespace

hipError_t launch_router(const uint16_t* x, const uint16_t* wr, const float* logit_bias, int T, int H,
                         int E, int top_k, int32_t* topk_idx, float* topk_w, _Float16* x16,
                         float* out_clear, hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    dim3 grid((T + kRouterTokens - 1) / kRouterTokens);
    if (x16) {
        hipLaunchKernelGGL(router_kernel<true>, grid, dim3(256), 0, stream, x, wr, logit_bias, T, H, E,
                           top_k, topk_idx, topk_w, x16, out_clear);
    } else {
        hipLaunchKernelGGL(router_kernel<false>, grid, dim3(256), 0, stream, x, wr, logit_bias, T, H, E,
                           top_k, topk_idx, topk_w, x16, out_clear);
    }
    return hipGetLastError();
}

}  // namespace bitmoe
