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
//   - logits_kernel (small batches): one workgroup per (32 tokens, 32 experts,
//     1/S of K); its four waves split K and sum through LDS; logits_staged_kernel
//     (T >= 2048): one workgroup per (64 tokens, 64 experts), operands staged
//     through LDS; partial logits go to the workspace;
//   - topk_kernel: one wave per token sums and ranks its logits, writes the routing,
//     counts the expert histogram (in LDS per 4 or 16 tokens, then one atomic
//     per expert) and writes the float16 copy of the token's row (8-column blocks in dequantisation order) that the expert
//     products read.
#include <algorithm>

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

// The 8-bit router restored to bf16 (a checkpoint detail, not on the pages):
// one thread per 8 columns (two code words), fused multiply-add in float32,
// then round to nearest even.  The result is the matrix every router kernel
// here scores with.
template <typename SB>
__global__ __launch_bounds__(256) void router_dequant_kernel(const uint32_t* __restrict__ q,
                                                             const SB* __restrict__ s, const SB* __restrict__ b,
                                                             int E, int H, uint16_t* __restrict__ out) {
    const int64_t n = (int64_t)E * (H / 8);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int e = (int)(i / (H / 8)), c8 = (int)(i % (H / 8));  // columns 8 c8 .. 8 c8 + 7
        const uint2 w = reinterpret_cast<const uint2*>(q + (size_t)e * (H / 4))[c8];
        const size_t g = (size_t)e * (H / 64) + c8 / 8;
        reinterpret_cast<uint4*>(out + (size_t)e * H)[c8] = restore_q8x8(w, sb_to_f32<SB>(s[g]), sb_to_f32<SB>(b[g]));
    }
}

// logits_kernel: one workgroup per (TM tokens, TM experts, 1/S of K).  Its four
// waves split the workgroup's K range and sum through LDS; split z writes its
// partial logits to partial[z][T][E] (split 0 adds the bias) and topk_kernel
// sums the S splits in order.  It runs with TM = 32 for batches below 2048
// tokens, with K split S ways so that the router's 1 MiB is spread over a few
// hundred workgroups (larger batches use logits_staged_kernel below).
// kQ8: the router is 8-bit (codes wq, scales wsc and biases wbi per 64
// columns) and each lane restores its 8-column chunks to bf16 in registers.
template <int TM, typename SB, bool kQ8>
__global__ __launch_bounds__(256) void logits_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                                                     const uint32_t* __restrict__ wq, const SB* __restrict__ wsc,
                                                     const SB* __restrict__ wbi,
                                                     const float* __restrict__ logit_bias, int T, int H, int E, int S,
                                                     float* __restrict__ partial, int32_t* __restrict__ zero0,
                                                     int32_t* __restrict__ zero1) {
    constexpr int MB = TM / 32;               // 32-row MFMA blocks per side
    constexpr int kSteps = TM == 32 ? 8 : 4;  // K steps (16 columns each) per load batch
    __shared__ float part[kWaves4][TM][TM + 1];
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int row = lane % 32, half = lane / 32;
    const int t0 = blockIdx.x * TM, e0 = blockIdx.y * TM, z = blockIdx.z;
    if (blockIdx.x == 0 && blockIdx.y == 0 && z == 0) {
        for (int i = tid; i < E; i += blockDim.x) {
            if (zero0) __hip_atomic_store(zero0 + i * kCounterStride, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (zero1) __hip_atomic_store(zero1 + i * kCounterStride, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // wave w takes K columns [kb, kb + kq) of this split: 16-byte chunk 2 kk + half of its range
    const int kq = H / (kWaves4 * S);
    const int nk = kq / 16;
    const int kb = z * (H / S) + wave * kq;
    const uint4* arow[MB];
    const uint4* brow[MB];
    const uint2* qrow[MB];
    const SB* srow[MB];
    const SB* bsrow[MB];
#pragma unroll
    for (int m = 0; m < MB; m++) {
        const size_t er = (size_t)min(e0 + 32 * m + row, E - 1);
        arow[m] = reinterpret_cast<const uint4*>(x + (size_t)min(t0 + 32 * m + row, T - 1) * H + kb);
        if (kQ8) {
            qrow[m] = reinterpret_cast<const uint2*>(wq + er * (H / 4)) + kb / 8;
            srow[m] = wsc + er * (H / 64);
            bsrow[m] = wbi + er * (H / 64);
        } else {
            brow[m] = reinterpret_cast<const uint4*>(wr + er * H + kb);
        }
    }
    // router chunk c (8 columns from kb + 8 c): bf16 directly, or codes, scale
    // and bias to restore once they have landed
    struct RawB {
        uint2 q;
        SB s, b;
    };
    auto fetch_b = [&](int m, int c, uint4& bf, RawB& raw) {
        if (kQ8) {
            const int g = (kb / 8 + c) / 8;
            raw.q = qrow[m][c];
            raw.s = srow[m][g];
            raw.b = bsrow[m][g];
        } else {
            bf = brow[m][c];
        }
    };
    auto restore = [](const RawB& raw) { return restore_q8x8(raw.q, sb_to_f32<SB>(raw.s), sb_to_f32<SB>(raw.b)); };
    floatx16 acc[MB][MB];
#pragma unroll
    for (int m = 0; m < MB; m++)
#pragma unroll
        for (int n = 0; n < MB; n++) acc[m][n] = floatx16{0};
    uint4 a[kSteps][MB], b[kSteps][MB], an[kSteps][MB], bn[kSteps][MB];
    RawB rb[kSteps][MB], rbn[kSteps][MB];
#pragma unroll
    for (int j = 0; j < kSteps; j++) {
        const int c = 2 * min(j, nk - 1) + half;
#pragma unroll
        for (int m = 0; m < MB; m++) {
            a[j][m] = arow[m][c];
            fetch_b(m, c, b[j][m], rb[j][m]);
        }
    }
    if (kQ8) {
#pragma unroll
        for (int j = 0; j < kSteps; j++)
#pragma unroll
            for (int m = 0; m < MB; m++) b[j][m] = restore(rb[j][m]);
    }
    for (int kk = 0; kk < nk; kk += kSteps) {
        const bool more = kk + kSteps < nk;
        if (more) {
#pragma unroll
            for (int j = 0; j < kSteps; j++) {
                const int c = 2 * min(kk + kSteps + j, nk - 1) + half;
#pragma unroll
                for (int m = 0; m < MB; m++) {
                    an[j][m] = arow[m][c];
                    fetch_b(m, c, bn[j][m], rbn[j][m]);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kSteps; j++)
            if (kk + j < nk) {
#pragma unroll
                for (int m = 0; m < MB; m++)
#pragma unroll
                    for (int n = 0; n < MB; n++)
                        acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[j][m]),
                                                                            __builtin_bit_cast(bf16x8_t, b[j][n]),
                                                                            acc[m][n], 0, 0, 0);
            }
        if (more) {
#pragma unroll
            for (int j = 0; j < kSteps; j++)
#pragma unroll
                for (int m = 0; m < MB; m++) {
                    a[j][m] = an[j][m];
                    b[j][m] = kQ8 ? restore(rbn[j][m]) : bn[j][m];
                }
        }
    }
    // C layout of 32x32 MFMA: lane holds column (lane%32) = expert, rows 8i + 4*(lane/32) + j = tokens
#pragma unroll
    for (int m = 0; m < MB; m++)
#pragma unroll
        for (int n = 0; n < MB; n++)
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 4; j++) part[wave][32 * m + 8 * i + 4 * half + j][32 * n + row] = acc[m][n][4 * i + j];
    __syncthreads();
    for (int i = tid; i < TM * TM; i += blockDim.x) {
        const int r = i / TM, c = i % TM;
        const int t = t0 + r, e = e0 + c;
        if (t < T && e < E) {
            float v = part[0][r][c] + part[1][r][c] + part[2][r][c] + part[3][r][c];
            if (z == 0 && logit_bias) v += logit_bias[e];
            partial[((size_t)z * T + t) * E + e] = v;
        }
    }
}

// logits_staged_kernel: one workgroup per (64 tokens, 64 experts, 1/S of K),
// for large batches.  Its eight waves load 64-column chunks of the 64 x rows
// and the 64 router rows into LDS with direct loads (global_load_lds_dwordx4,
// whole 128-byte row segments per 8 lanes), several chunks in flight.  Wave w
// computes the 32 x 32 block (tokens 32 ((w / 2) % 2), experts 32 (w % 2)) on
// K steps 2 (w / 4) and 2 (w / 4) + 1 of every chunk; the two waves of a block
// add their sums through LDS at the end.  Two waves per SIMD let one wave's
// LDS reads overlap the other's matrix products.  A row's 16-byte chunk c sits
// at LDS position c ^ ((row / 2) % 8): the 16 rows that one LDS read cycle
// serves fall on distinct banks.  The loads are waited for by count (the
// compiler does not see the LDS reads, which are inline asm) and the stages
// are handed over with bare barriers, so no wait for the loads still in
// flight is inserted.
constexpr int kStagedTile = 64;     // tokens and experts per workgroup
constexpr int kStagedChunk = 64;    // K columns per stage
constexpr int kStagedStages = 4;    // 64 KiB of LDS: three chunks in flight
constexpr int kStagedThreads = 512;
constexpr int kStagedRowBytes = kStagedChunk * 2;
constexpr int kStagedOperandBytes = kStagedTile * kStagedRowBytes;  // 8 KiB

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 lds_read16(unsigned addr) {
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
    return v;
}
template <typename V>
__device__ __forceinline__ void after_wait(V& v) {
    asm volatile("" : "+v"(v));
}
__device__ __forceinline__ int staged_pos(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

__global__ __launch_bounds__(kStagedThreads) void logits_staged_kernel(const uint16_t* __restrict__ x,
                                                                       const uint16_t* __restrict__ wr,
                                                                       const float* __restrict__ logit_bias,
                                                                       int T, int H, int E, int S,
                                                                       float* __restrict__ partial,
                                                                       int32_t* __restrict__ zero0,
                                                                       int32_t* __restrict__ zero1) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[kStagedStages][2][kStagedOperandBytes];
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int t0 = blockIdx.x * kStagedTile, e0 = blockIdx.y * kStagedTile, z = blockIdx.z;
    if (blockIdx.x == 0 && blockIdx.y == 0 && z == 0) {
        for (int i = tid; i < E; i += blockDim.x) {
            if (zero0) __hip_atomic_store(zero0 + i * kCounterStride, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (zero1) __hip_atomic_store(zero1 + i * kCounterStride, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    const int kb = z * (H / S);
    const int nc = H / (S * kStagedChunk);

    // wave w fills rows 8 w .. 8 w + 7 of both operands: lane i -> row
    // 8 w + i / 8, LDS position i % 8, which holds the row's chunk
    // staged_pos(row, i % 8)
    const int lr = 8 * wave + lane / 8;
    const int lc = staged_pos(lr, lane % 8);
    const uint16_t* a_src = x + (size_t)min(t0 + lr, T - 1) * H + kb + lc * 8;
    const uint16_t* b_src = wr + (size_t)min(e0 + lr, E - 1) * H + kb + lc * 8;
    auto issue = [&](int chunk, int stage) {
        __builtin_amdgcn_global_load_lds(a_src + chunk * kStagedChunk, &smem[stage][0][wave * kWave * 16], 16, 0, 0);
        __builtin_amdgcn_global_load_lds(b_src + chunk * kStagedChunk, &smem[stage][1][wave * kWave * 16], 16, 0, 0);
    };

    // MFMA operands: lane -> row lane % 32 of the wave's block, 16-byte chunk
    // 2 s + lane / 32 of the stage for K step s of the wave's two
    const int row = lane % 32, half = lane / 32;
    const int mb = (wave / 2) % 2, nb = wave % 2, kh = wave / 4;
    unsigned a_off[2], b_off[2];
#pragma unroll
    for (int s = 0; s < 2; s++) {
        const int c = 2 * (2 * kh + s) + half;
        const int ar = mb * 32 + row, br = nb * 32 + row;
        a_off[s] = (unsigned)(ar * kStagedRowBytes + staged_pos(ar, c) * 16);
        b_off[s] = (unsigned)(kStagedOperandBytes + br * kStagedRowBytes + staged_pos(br, c) * 16);
    }
    const unsigned lds0 = (unsigned)reinterpret_cast<uintptr_t>(&smem[0][0][0]);
    constexpr unsigned kStageBytes = 2 * kStagedOperandBytes;

    // chunks i + 1 .. i + kAhead - 1 stay in flight while chunk i is used
    constexpr int kAhead = kStagedStages - 1;
    floatx16 acc = floatx16{0};
#pragma unroll
    for (int c = 0; c < kAhead; c++) issue(min(c, nc - 1), c);
    for (int i = 0; i < nc; i++) {
        // this wave's loads of chunk i have landed (the two of each later
        // chunk may be in flight); after the barrier every wave's have, and
        // every wave is done reading chunk i - 1, whose stage the loads of
        // chunk i + kAhead reuse (past the last chunk they reload it into a
        // stage that is no longer read)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * (kAhead - 1)) : "memory");
        asm volatile("s_barrier" ::: "memory");
        issue(min(i + kAhead, nc - 1), (i + kAhead) % kStagedStages);
        const unsigned base = lds0 + (unsigned)(i % kStagedStages) * kStageBytes;
        u32x4 a[2], b[2];
#pragma unroll
        for (int s = 0; s < 2; s++) {
            a[s] = lds_read16(base + a_off[s]);
            b[s] = lds_read16(base + b_off[s]);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int s = 0; s < 2; s++) {
            after_wait(a[s]);
            after_wait(b[s]);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[s]),
                                                          __builtin_bit_cast(bf16x8_t, b[s]), acc, 0, 0, 0);
        }
    }
    // no load may still write LDS: the stages are reused for the sums below
    // and must be quiet before the workgroup ends
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    float* red = reinterpret_cast<float*>(&smem[0][0][0]);  // [4 blocks][16][64 lanes]
    const int blk = wave % 4;
    if (kh == 1) {
#pragma unroll
        for (int q = 0; q < 16; q++) red[(blk * 16 + q) * kWave + lane] = acc[q];
    }
    __syncthreads();
    if (kh == 1) return;

    // C layout of 32x32 MFMA: lane holds column (lane % 32) = expert, rows
    // 8 i + 4 (lane / 32) + j = tokens
    const int e = e0 + nb * 32 + row;
    if (e < E) {
        const float bias = (z == 0 && logit_bias) ? logit_bias[e] : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int q = 4 * i + j;
                const int t = t0 + mb * 32 + 8 * i + 4 * half + j;
                if (t < T) partial[((size_t)z * T + t) * E + e] = (acc[q] + red[(blk * 16 + q) * kWave + lane]) + bias;
            }
    }
}

// kTW tokens per top-k workgroup: 16 for large batches (fewer atomics on hot
// experts' counters), 4 for small ones (more workgroups in flight)
template <int kTW, bool kGate>
__global__ __launch_bounds__(kTW * kWave) void topk_kernel(const float* __restrict__ logits, int S,
                                                   const uint16_t* __restrict__ x, int T, int H, int E, int top_k,
                                                   int32_t* __restrict__ topk_idx,
                                                   float* __restrict__ topk_w, int32_t* __restrict__ hist,
                                                   _Float16* __restrict__ x16, const uint16_t* __restrict__ sgate,
                                                   float* __restrict__ shared_w) {
    // the workgroup's expert counts gather in LDS first: one global atomic per
    // (workgroup, expert), so a hot expert's counter sees at most T / kTW adds
    __shared__ int lh[kMaxE];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int t = blockIdx.x * kTW + wave;
    if (threadIdx.x < kMaxE) lh[threadIdx.x] = 0;
    __syncthreads();
    // the first kXPre 16-byte blocks of each lane's part of the token's x row
    // (all of it for H <= 2048) go out before the logits, so their latency
    // overlaps the loads and the selection below
    constexpr int kXPre = 4;
    const int nblk = H / 8;
    uint4 xr[kXPre], gr[kXPre];
    {
        const uint4* xrow = reinterpret_cast<const uint4*>(x + (size_t)min(t, T - 1) * H);
#pragma unroll
        for (int i = 0; i < kXPre; i++) {
            xr[i] = xrow[min(lane + kWave * i, nblk - 1)];
            if (kGate) gr[i] = reinterpret_cast<const uint4*>(sgate)[min(lane + kWave * i, nblk - 1)];
        }
    }
    if (t < T) {
        const float* lt = logits + (size_t)t * E;
        const size_t split = (size_t)T * E;
        // this lane's experts lane + 64 i: sum of the S partial logits, in split
        // order; the loads of 8 splits go out before their adds
        constexpr int kPer = kMaxE / kWave;
        float v[kPer];
#pragma unroll
        for (int i = 0; i < kPer; i++) v[i] = lane + kWave * i < E ? lt[lane + kWave * i] : 0.0f;
        for (int z0 = 1; z0 < S; z0 += 8) {
            float p[8][kPer];
#pragma unroll
            for (int dz = 0; dz < 8; dz++)
#pragma unroll
                for (int i = 0; i < kPer; i++) {
                    const int e = lane + kWave * i;
                    p[dz][i] = (z0 + dz < S && e < E) ? lt[(size_t)(z0 + dz) * split + e] : 0.0f;
                }
#pragma unroll
            for (int dz = 0; dz < 8; dz++)
#pragma unroll
                for (int i = 0; i < kPer; i++) v[i] += p[dz][i];
        }
        int ij;
        float wj;
        wave_topk_held(v, E, top_k, lane, &ij, &wj);
        if (lane < top_k) {
            topk_idx[(size_t)t * top_k + lane] = ij;
            topk_w[(size_t)t * top_k + lane] = wj;
            if (ij >= 0 && ij < E) atomicAdd(&lh[ij], 1);
        }
        if (x16) {
            // the float16 copy of the row; with a shared-expert gate g, also the
            // shared expert's weight sigmoid(x . g) (float32 sum of exact bf16
            // products, reduced over the wave)
            float z = 0.0f;
            auto convert = [&](int blk, const uint4& raw, const uint4& graw) {
                const uint16_t* hb = reinterpret_cast<const uint16_t*>(&raw);
                half8_t o;
#pragma unroll
                for (int e = 0; e < 8; e++) o[e] = (_Float16)bf16_to_f32(hb[nibble_of(e)]);
                reinterpret_cast<half8_t*>(x16 + (size_t)t * H)[blk] = o;
                if (kGate) {
                    const uint16_t* gb = reinterpret_cast<const uint16_t*>(&graw);
#pragma unroll
                    for (int e = 0; e < 8; e++) z += bf16_to_f32(hb[e]) * bf16_to_f32(gb[e]);
                }
            };
#pragma unroll
            for (int i = 0; i < kXPre; i++)
                if (lane + kWave * i < nblk) convert(lane + kWave * i, xr[i], kGate ? gr[i] : xr[i]);
            for (int blk = lane + kWave * kXPre; blk < nblk; blk += kWave) {
                const uint4 raw = reinterpret_cast<const uint4*>(x + (size_t)t * H)[blk];
                convert(blk, raw, kGate ? reinterpret_cast<const uint4*>(sgate)[blk] : raw);
            }
            if (kGate) {
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off);
                if (lane == 0) shared_w[t] = 1.0f / (1.0f + expf(-z));
            }
        }
    }
    __syncthreads();
    if (hist && threadIdx.x < E && lh[threadIdx.x] > 0)
        atomicAdd(hist + threadIdx.x * kCounterStride, lh[threadIdx.x]);
}

}  // namespace

hipError_t launch_router_dequant(const uint32_t* q, const void* s, const void* b, bool sb_bf16, int E, int H,
                                 uint16_t* out, hipStream_t stream) {
    const int64_t n = (int64_t)E * (H / 8);
    if (n <= 0) return hipSuccess;
    const int grid = (int)std::min<int64_t>((n + 255) / 256, 4096);
    if (sb_bf16)
        hipLaunchKernelGGL(router_dequant_kernel<uint16_t>, dim3(grid), dim3(256), 0, stream, q,
                           static_cast<const uint16_t*>(s), static_cast<const uint16_t*>(b), E, H, out);
    else
        hipLaunchKernelGGL(router_dequant_kernel<float>, dim3(grid), dim3(256), 0, stream, q,
                           static_cast<const float*>(s), static_cast<const float*>(b), E, H, out);
    return hipGetLastError();
}

hipError_t launch_router(const uint16_t* x, const uint16_t* wr, const float* logit_bias, int T, int H,
                         int E, int top_k, int32_t* topk_idx, float* topk_w, hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    dim3 grid((T + kRouterTokens - 1) / kRouterTokens);
    hipLaunchKernelGGL(router_kernel, grid, dim3(256), 0, stream, x, wr, logit_bias, T, H, E, top_k, topk_idx,
                       topk_w);
    return hipGetLastError();
}

hipError_t launch_logits(const uint16_t* x, const uint16_t* wr, const uint32_t* wq, const void* wsc, const void* wbi,
                         bool sb_bf16, const float* logit_bias, int T, int H, int E, float* logits, int32_t* zero0,
                         int32_t* zero1, hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    const int tm = logits_tile(T);
    const int S = logits_splits(T, H, E);
    const dim3 grid((T + tm - 1) / tm, (E + tm - 1) / tm, S);
    if (tm == 64) {
        if (!wr) return hipErrorInvalidValue;  // the staged kernel reads a bf16 router
        hipLaunchKernelGGL(logits_staged_kernel, grid, dim3(kStagedThreads), 0, stream, x, wr, logit_bias, T, H, E, S,
                           logits, zero0, zero1);
    } else if (!wq) {
        hipLaunchKernelGGL((logits_kernel<32, uint16_t, false>), grid, dim3(256), 0, stream, x, wr, nullptr,
                           nullptr, nullptr, logit_bias, T, H, E, S, logits, zero0, zero1);
    } else if (sb_bf16) {
        hipLaunchKernelGGL((logits_kernel<32, uint16_t, true>), grid, dim3(256), 0, stream, x, nullptr, wq,
                           static_cast<const uint16_t*>(wsc), static_cast<const uint16_t*>(wbi), logit_bias, T, H, E,
                           S, logits, zero0, zero1);
    } else {
        hipLaunchKernelGGL((logits_kernel<32, float, true>), grid, dim3(256), 0, stream, x, nullptr, wq,
                           static_cast<const float*>(wsc), static_cast<const float*>(wbi), logit_bias, T, H, E, S,
                           logits, zero0, zero1);
    }
    return hipGetLastError();
}

hipError_t launch_topk(const float* logits, const uint16_t* x, int T, int H, int E, int top_k, int32_t* topk_idx,
                       float* topk_w, int32_t* hist, _Float16* x16, const uint16_t* sgate, float* shared_w,
                       hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    const int S = logits_splits(T, H, E);
    // the gate's dot product needs the f16 copy's pass over x
    if (sgate && !x16) return hipErrorInvalidValue;
#define BITMOE_TOPK(TW, GATE)                                                                              \
    hipLaunchKernelGGL((topk_kernel<TW, GATE>), dim3((T + TW - 1) / TW), dim3(TW * kWave), 0, stream, logits, S, x, \
                       T, H, E, top_k, topk_idx, topk_w, hist, x16, sgate, shared_w)
    if (T >= 1024) {
        if (sgate) BITMOE_TOPK(16, true); else BITMOE_TOPK(16, false);
    } else {
        if (sgate) BITMOE_TOPK(4, true); else BITMOE_TOPK(4, false);
    }
#undef BITMOE_TOPK
    return hipGetLastError();
}

}  // namespace bitmoe
