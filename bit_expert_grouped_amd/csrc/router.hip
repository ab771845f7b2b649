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
// That single kernel serves the step-by-step moe_route call.  The whole-layer
// call spreads the router over the chip instead (a workgroup reading the whole
// 1 MiB router on its own is bound by one compute unit's bandwidth):
//   - logits_kernel: one workgroup per (32 tokens, 32 experts); its four waves
//     split K and sum through LDS; logits go to the workspace;
//   - topk_kernel: one wave per token ranks its logits, writes the routing,
//     counts the expert histogram with atomics and writes the float16 copy of
//     the token's row (8-column blocks in dequantisation order) that the expert
//     products read.
#include "common.h"
#include "kernels.h"

namespace bitmoe {

namespace {

constexpr int kRouterTokens = 32;
constexpr int kWaves4 = 4;  // waves per workgroup of the spread router kernels

__global__ __launch_bounds__(256) void router_kernel(const uint16_t* __restrict__ x,
                                                     const uint16_t* __restrict__ wr,
                                                     const float* __restrict__ logit_bias, int T,
                                                     int H, int E, int top_k,
                                                     int32_t* __restrict__ topk_idx,
                                                     float* __restrict__ topk_w) {
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
}

constexpr int kLT = 32;  // tokens per logits workgroup
constexpr int kLE = 32;  // experts per logits workgroup
constexpr int kLSteps = 8;  // K steps (16 columns each) per load batch

__global__ __launch_bounds__(256) void logits_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                                                     const float* __restrict__ logit_bias, int T, int H, int E,
                                                     float* __restrict__ logits, int32_t* __restrict__ zero0,
                                                     int32_t* __restrict__ zero1) {
    __shared__ float part[kWaves4][kLT][kLE + 1];
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int row = lane % 32, half = lane / 32;
    const int t0 = blockIdx.x * kLT, e0 = blockIdx.y * kLE;
    if (blockIdx.x == 0 && blockIdx.y == 0) {
        for (int i = tid; i < E; i += blockDim.x) {
            if (zero0) __hip_atomic_store(zero0 + i * kCounterStride, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (zero1) __hip_atomic_store(zero1 + i * kCounterStride, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // wave w takes K columns [w H/4, (w+1) H/4): 16-byte chunk 2 kk + half of its range
    const int kq = H / 4;
    const int nk = kq / 16;
    const uint4* arow = reinterpret_cast<const uint4*>(x + (size_t)min(t0 + row, T - 1) * H + wave * kq);
    const uint4* brow = reinterpret_cast<const uint4*>(wr + (size_t)min(e0 + row, E - 1) * H + wave * kq);
    floatx16 acc = {0};
    uint4 a[kLSteps], b[kLSteps], an[kLSteps], bn[kLSteps];
#pragma unroll
    for (int j = 0; j < kLSteps; j++) {
        const int c = 2 * min(j, nk - 1) + half;
        a[j] = arow[c];
        b[j] = brow[c];
    }
    for (int kb = 0; kb < nk; kb += kLSteps) {
        const bool more = kb + kLSteps < nk;
        if (more) {
#pragma unroll
            for (int j = 0; j < kLSteps; j++) {
                const int c = 2 * min(kb + kLSteps + j, nk - 1) + half;
                an[j] = arow[c];
                bn[j] = brow[c];
            }
        }
#pragma unroll
        for (int j = 0; j < kLSteps; j++)
            if (kb + j < nk)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[j]),
                                                              __builtin_bit_cast(bf16x8_t, b[j]), acc, 0, 0, 0);
        if (more) {
#pragma unroll
            for (int j = 0; j < kLSteps; j++) {
                a[j] = an[j];
                b[j] = bn[j];
            }
        }
    }
    // C layout of 32x32 MFMA: lane holds column (lane%32) = expert, rows 8i + 4*(lane/32) + j = tokens
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) part[wave][8 * i + 4 * half + j][row] = acc[4 * i + j];
    __syncthreads();
    for (int i = tid; i < kLT * kLE; i += blockDim.x) {
        const int r = i / kLE, c = i % kLE;
        const int t = t0 + r, e = e0 + c;
        if (t < T && e < E) {
            float v = part[0][r][c] + part[1][r][c] + part[2][r][c] + part[3][r][c];
            if (logit_bias) v += logit_bias[e];
            logits[(size_t)t * E + e] = v;
        }
    }
}

__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, const uint16_t* __restrict__ x,
                                                   int T, int H, int E, int top_k, int32_t* __restrict__ topk_idx,
                                                   float* __restrict__ topk_w, int32_t* __restrict__ hist,
                                                   _Float16* __restrict__ x16) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int t = blockIdx.x * kWaves4 + wave;
    if (t >= T) return;  // no workgroup barrier below
    const float* lt = logits + (size_t)t * E;
    int ij;
    float wj;
    wave_topk([&](int e) { return lt[e]; }, E, top_k, lane, &ij, &wj);
    if (lane < top_k) {
        topk_idx[(size_t)t * top_k + lane] = ij;
        topk_w[(size_t)t * top_k + lane] = wj;
        if (hist && ij >= 0 && ij < E) atomicAdd(hist + ij * kCounterStride, 1);
    }
    if (x16) {
        const int nblk = H / 8;
        for (int blk = lane; blk < nblk; blk += kWave) {
            const uint4 raw = reinterpret_cast<const uint4*>(x + (size_t)t * H)[blk];
            const uint16_t* hb = reinterpret_cast<const uint16_t*>(&raw);
            half8_t o;
#pragma unroll
            for (int e = 0; e < 8; e++) o[e] = (_Float16)bf16_to_f32(hb[nibble_of(e)]);
            reinterpret_cast<half8_t*>(x16 + (size_t)t * H)[blk] = o;
        }
    }
}

}  // namespace

hipError_t launch_router(const uint16_t* x, const uint16_t* wr, const float* logit_bias, int T, int H,
                         int E, int top_k, int32_t* topk_idx, float* topk_w, hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    dim3 grid((T + kRouterTokens - 1) / kRouterTokens);
    hipLaunchKernelGGL(router_kernel, grid, dim3(256), 0, stream, x, wr, logit_bias, T, H, E, top_k, topk_idx,
                       topk_w);
    return hipGetLastError();
}

hipError_t launch_logits(const uint16_t* x, const uint16_t* wr, const float* logit_bias, int T, int H, int E,
                         float* logits, int32_t* zero0, int32_t* zero1, hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    const dim3 grid((T + kLT - 1) / kLT, (E + kLE - 1) / kLE);
    hipLaunchKernelGGL(logits_kernel, grid, dim3(256), 0, stream, x, wr, logit_bias, T, H, E, logits, zero0, zero1);
    return hipGetLastError();
}

hipError_t launch_topk(const float* logits, const uint16_t* x, int T, int H, int E, int top_k, int32_t* topk_idx,
                       float* topk_w, int32_t* hist, _Float16* x16, hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(topk_kernel, dim3((T + kWaves4 - 1) / kWaves4), dim3(256), 0, stream, logits, x, T, H, E,
                       top_k, topk_idx, topk_w, hist, x16);
    return hipGetLastError();
}

}  // namespace bitmoe
