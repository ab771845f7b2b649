// Small elementwise kernels for gfx950: the float16 activation copy used by the
// expert products of the step-by-step API, the stand-alone weighted combine,
// and the layer's combine over float16 expert rows.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace bitmoe {

namespace {

// x [T][H] bf16 -> x16 [T][H] float16 with 8-column blocks in dequantisation order.
__global__ __launch_bounds__(256) void convert_x_kernel(const uint16_t* __restrict__ x, int64_t nblk,
                                                        _Float16* __restrict__ x16) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nblk; i += (int64_t)gridDim.x * blockDim.x) {
        const uint4 raw = reinterpret_cast<const uint4*>(x)[i];
        const uint16_t* hb = reinterpret_cast<const uint16_t*>(&raw);
        half8_t o;
#pragma unroll
        for (int e = 0; e < 8; e++) o[e] = (_Float16)bf16_to_f32(hb[nibble_of(e)]);
        reinterpret_cast<half8_t*>(x16)[i] = o;
    }
}

// Pages: one shared expert is added to the routed experts' output (aimanavo.com
// page, section "Qwen3.6's 256 experts and two layer types make the MLX-Lily gap").
// out[t][h] = sum_j w[t][j] * y_slot[t*k+j][h] + s[t] * y_shared[t][h]; s[t] =
// shared_w[t] (an optional shared-expert gate, a checkpoint detail), else 1;
// 4 columns per thread.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_slot,
                                                      const float* __restrict__ topk_w,
                                                      const float* __restrict__ y_shared,
                                                      const float* __restrict__ shared_w, int T, int H, int k,
                                                      float* __restrict__ out) {
    const int h4 = H / 4;
    const int64_t n = (int64_t)T * h4;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int t = (int)(i / h4), c = (int)(i % h4);
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        if (y_shared) {
            const float s = shared_w ? shared_w[t] : 1.0f;
            const float4 y = reinterpret_cast<const float4*>(y_shared + (size_t)t * H)[c];
            acc = make_float4(s * y.x, s * y.y, s * y.z, s * y.w);
        }
        for (int j = 0; j < k; j++) {
            const float w = topk_w[(size_t)t * k + j];
            const float4 y = reinterpret_cast<const float4*>(y_slot + ((size_t)t * k + j) * H)[c];
            acc.x += w * y.x;
            acc.y += w * y.y;
            acc.z += w * y.z;
            acc.w += w * y.w;
        }
        reinterpret_cast<float4*>(out + (size_t)t * H)[c] = acc;
    }
}

// n 16-byte units from p on set to zero (a kernel rather than a memset, so that
// a captured graph replays it exactly)
__global__ __launch_bounds__(256) void zero_kernel(uint4* __restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// float32 -> bfloat16, round to nearest even (finite values)
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// 8 float32 values plus 8 bf16 residuals (nullable) -> 8 bf16, one rounding each
__device__ __forceinline__ uint4 residual_bf16x8(const float (&v)[8], const uint16_t* res) {
    float r[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (res) {
        const uint4 rr = *reinterpret_cast<const uint4*>(res);
        const uint16_t* rb = reinterpret_cast<const uint16_t*>(&rr);
#pragma unroll
        for (int e = 0; e < 8; e++) r[e] = bf16_to_f32(rb[e]);
    }
    uint32_t b[8];
#pragma unroll
    for (int e = 0; e < 8; e++) b[e] = bf16_bits_rne(v[e] + r[e]);
    return make_uint4(b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16), b[6] | (b[7] << 16));
}

// The layer's combine over float16 expert rows: 8 columns per thread, float32
// accumulation in slot order, then the shared expert's row (times shared_w[t]
// when the shared expert is gated).  out16 != nullptr: the result goes to the
// bf16 residual stream instead, out16 = bf16(residual + sum) (residual
// nullable, and it may be the same buffer as out16: each thread reads its 8
// residuals before it writes them).
template <int K, bool kShared>
__global__ __launch_bounds__(256) void combine16_kernel(const _Float16* __restrict__ y16,
                                                        const float* __restrict__ topk_w,
                                                        const float* __restrict__ shared_w, int T, int H,
                                                        float* __restrict__ out, const uint16_t* residual,
                                                        uint16_t* out16) {
    const int h8 = H / 8;
    const int64_t n = (int64_t)T * h8;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int t = (int)(i / h8), c = (int)(i % h8);
        // all K routed rows (and the shared row) go out before the first add,
        // so their latencies overlap; each row is read exactly once, so the
        // loads and stores are nontemporal and do not displace other data
        half8_t y[K + 1];
        float w[K];
        const float s = !kShared ? 0.0f : shared_w ? shared_w[t] : 1.0f;
#pragma unroll
        for (int j = 0; j < K; j++) {
            w[j] = topk_w[(size_t)t * K + j];
            y[j] = __builtin_nontemporal_load(reinterpret_cast<const half8_t*>(y16 + ((size_t)t * K + j) * H) + c);
        }
        if (kShared)
            y[K] = __builtin_nontemporal_load(reinterpret_cast<const half8_t*>(y16 + ((size_t)T * K + t) * H) + c);
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < K; j++)
#pragma unroll
            for (int e = 0; e < 8; e++) acc[e] += w[j] * (float)y[j][e];
        if (kShared) {
#pragma unroll
            for (int e = 0; e < 8; e++) acc[e] += s * (float)y[K][e];
        }
        if (out16) {
            const size_t at = (size_t)t * H + 8 * (size_t)c;
            *reinterpret_cast<uint4*>(out16 + at) = residual_bf16x8(acc, residual ? residual + at : nullptr);
            continue;
        }
        typedef float fx4 __attribute__((ext_vector_type(4)));
        fx4* o = reinterpret_cast<fx4*>(out + (size_t)t * H) + 2 * c;
        __builtin_nontemporal_store(fx4{acc[0], acc[1], acc[2], acc[3]}, o);
        __builtin_nontemporal_store(fx4{acc[4], acc[5], acc[6], acc[7]}, o + 1);
    }
}

// Weight of the shared expert per token under an optional shared-expert gate g
// (a checkpoint detail): shared_w[t] = sigmoid(sum_h x[t][h] * g[h]), float32 sum
// of exact bf16 products; one wave per token.
__global__ __launch_bounds__(256) void shared_gate_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ g, int T, int H,
                                                          float* __restrict__ shared_w) {
    const int t = blockIdx.x * (256 / kWave) + threadIdx.x / kWave, lane = threadIdx.x % kWave;
    if (t >= T) return;
    float z = 0.0f;
    for (int blk = lane; blk < H / 8; blk += kWave) {
        const uint4 xr = reinterpret_cast<const uint4*>(x + (size_t)t * H)[blk];
        const uint4 gr = reinterpret_cast<const uint4*>(g)[blk];
        const uint16_t* xb = reinterpret_cast<const uint16_t*>(&xr);
        const uint16_t* gb = reinterpret_cast<const uint16_t*>(&gr);
#pragma unroll
        for (int e = 0; e < 8; e++) z += bf16_to_f32(xb[e]) * bf16_to_f32(gb[e]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off);
    if (lane == 0) shared_w[t] = 1.0f / (1.0f + expf(-z));
}

// out16 = bf16(residual + y) for n8 blocks of 8 elements (the decode path's
// float32 layer output into the bf16 residual stream; residual nullable, may
// alias out16)
__global__ __launch_bounds__(256) void residual_bf16_kernel(const float* __restrict__ y, const uint16_t* residual,
                                                            int64_t n8, uint16_t* out16) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
        float v[8];
        const float4 a = reinterpret_cast<const float4*>(y)[2 * i], b = reinterpret_cast<const float4*>(y)[2 * i + 1];
        v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
        *reinterpret_cast<uint4*>(out16 + 8 * i) = residual_bf16x8(v, residual ? residual + 8 * i : nullptr);
    }
}

int grid_for(int64_t n) {
    int64_t g = (n + 255) / 256;
    return (int)(g < 1 ? 1 : (g > 8192 ? 8192 : g));
}

}  // namespace

hipError_t launch_combine16(const _Float16* y16, const float* topk_w, bool shared, const float* shared_w, int T,
                            int H, int k, float* out, const uint16_t* residual, uint16_t* out16, hipStream_t stream) {
    const int64_t n = (int64_t)T * (H / 8);
    if (n <= 0) return hipSuccess;
#define BITMOE_COMBINE16(K)                                                                                  \
    case K:                                                                                                  \
        if (shared)                                                                                          \
            hipLaunchKernelGGL((combine16_kernel<K, true>), dim3(grid_for(n)), dim3(256), 0, stream, y16,     \
                               topk_w, shared_w, T, H, out, residual, out16);                                \
        else                                                                                                 \
            hipLaunchKernelGGL((combine16_kernel<K, false>), dim3(grid_for(n)), dim3(256), 0, stream, y16,    \
                               topk_w, shared_w, T, H, out, residual, out16);                                \
        break;
    switch (k) {
        BITMOE_COMBINE16(1) BITMOE_COMBINE16(2) BITMOE_COMBINE16(3) BITMOE_COMBINE16(4)
        BITMOE_COMBINE16(5) BITMOE_COMBINE16(6) BITMOE_COMBINE16(7) BITMOE_COMBINE16(8)
        default: return hipErrorInvalidValue;
    }
#undef BITMOE_COMBINE16
    return hipGetLastError();
}

hipError_t launch_residual_bf16(const float* y, const uint16_t* residual, int T, int H, uint16_t* out16,
                                hipStream_t stream) {
    const int64_t n8 = (int64_t)T * H / 8;
    if (n8 <= 0) return hipSuccess;
    hipLaunchKernelGGL(residual_bf16_kernel, dim3(grid_for(n8)), dim3(256), 0, stream, y, residual, n8, out16);
    return hipGetLastError();
}

hipError_t launch_shared_gate(const uint16_t* x, const uint16_t* g, int T, int H, float* shared_w,
                              hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(shared_gate_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, x, g, T, H, shared_w);
    return hipGetLastError();
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream) {
    const int64_t n = (int64_t)(bytes / 16);
    if (n == 0) return hipSuccess;
    const int blocks = (int)std::min<int64_t>((n + 255) / 256, 1024);
    hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<uint4*>(p), n);
    return hipGetLastError();
}

hipError_t launch_convert_x(const uint16_t* x, int T, int H, _Float16* x16, hipStream_t stream) {
    const int64_t nblk = (int64_t)T * H / 8;
    if (nblk <= 0) return hipSuccess;
    hipLaunchKernelGGL(convert_x_kernel, dim3(grid_for(nblk)), dim3(256), 0, stream, x, nblk, x16);
    return hipGetLastError();
}

hipError_t launch_combine(const float* y_slot, const float* topk_w, const float* y_shared, const float* shared_w,
                          int T, int H, int k, float* out, hipStream_t stream) {
    const int64_t n = (int64_t)T * (H / 4);
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(combine_kernel, dim3(grid_for(n)), dim3(256), 0, stream, y_slot, topk_w, y_shared, shared_w, T,
                       H, k, out);
    return hipGetLastError();
}

}  // namespace bitmoe
