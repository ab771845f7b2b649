// Decode attention with grouped-query KV sharing for gfx950: one query token
// per sequence, Hq query heads over Hkv KV heads, every K and V row read from
// HBM once for all Hq / Hkv query heads that share it.
//
// Pages: the model's full-attention layers have 16 query heads over 2 KV
// heads (aimanavo.com page, section "Qwen3.6's 256 experts and two layer types
// make the MLX-Lily gap"); packing the query heads of a KV head so that each
// KV row is read once is the decode-side gain the pages quote at 32K context
// (aimanavo.com page, section "Lily does not treat prefill and decode as the
// same job"; dzen.guru page, section "Where does the speed-up come from?").
//
// For sequence b with n cached rows, query head h and KV head g = h / G
// (G = Hq / Hkv):  s_j = scale * q_h . k_j,  out_h = sum_j softmax(s)_j v_j.
//
// At decode the work is a stream of the cache (HBM-bound: 16 FLOP per byte of
// K at G = 8), so the design is about keeping every compute unit's loads in
// flight and touching each byte once:
//
//   - pass 1 (gqa_partial_kernel): one workgroup of 4 waves per (sequence, KV
//     head, run of 4 * RW rows); each wave issues all loads of its RW rows of K
//     and V at once.  Scores: v_mfma_f32_16x16x32_bf16 with the K rows as the A
//     operand straight from HBM (16 rows x 32 columns per step) and the group's
//     query heads as B (heads padded to 16), so lane (i, r) = (lane % 16,
//     lane / 16) holds the scores of head i at rows 4 r .. 4 r + 3 of each
//     16-row block.  That is exactly the A operand of v_mfma_f32_16x16x16_bf16
//     for P V, so the probabilities go from the score accumulators to the
//     second product without leaving the lane (rounded to bf16).  V is the B
//     operand, which needs 4 consecutive rows of one column per lane: each wave
//     writes its V rows transposed into LDS (rows padded against bank
//     conflicts) and reads 8-byte runs back.  The 4 waves' (max, sum, output)
//     are merged in LDS and the workgroup stores one partial: the running max
//     m (log2 units), the sum l of the rounded probabilities and the
//     unnormalised output o.
//   - merge: one wave per (sequence, query head, 8 output columns) combines
//     the partials of all runs, o_total = sum_s 2^(m_s - M) o_s over l_total
//     likewise, spread over ~B * Hq * D / 8 waves so that the merge is not bound
//     by one compute unit's bandwidth.  When the whole grid fits on the device
//     at once, the merge runs in the same launch: each workgroup counts itself
//     in on its (sequence, KV head)'s arrival counter after storing its
//     partial; the last to arrive resets the counter and raises the call's
//     epoch in 16 copies of a flag (so that no cache line has more than ~8
//     readers); the others wait (bounded) for their copy, and every workgroup
//     then merges its share of the head's outputs.  Otherwise a second kernel
//     (gqa_merge_kernel) merges.
//
// Rows past a sequence's length are never read: their loads are clamped to the
// last valid row (whose values are finite) and their scores set to -inf.
//
#include "common.h"
#include "kernels.h"

namespace bitmoe {

namespace {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr long kSpinLimit = 1l << 20;  // bound of the fused merge's wait (s_sleep rounds)
constexpr int kFlagCopies = 16;         // copies of the merge's completion flag
constexpr int kCtlWords = 64 + 32 * kFlagCopies;  // control words per (sequence, KV head)
static_assert(kCtlWords * 4 <= 4096, "control block of a (sequence, KV head)");

// rows per wave: D <= 128 keeps 64 rows (16 KB of K and 16 KB of V per wave in
// flight); D = 256 keeps 32
template <int D>
constexpr int rows_per_wave() { return D <= 128 ? 64 : 32; }

__device__ __forceinline__ uint16_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float bf16_value(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m); }

// Partials that another workgroup of the same launch merges go through
// agent-scope stores and loads, which pass the per-XCD L2 (written through on
// store, missed on load), so no L2 write-back or invalidation is needed; with
// the merge in a second kernel, plain accesses do.
template <bool kCoherent>
__device__ __forceinline__ void put_f(float* p, float v) {
    if (kCoherent)
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        *p = v;
}

template <bool kCoherent>
__device__ __forceinline__ float get_f(const float* p) {
    if (kCoherent) return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return *p;
}

// two consecutive floats (8-byte aligned)
template <bool kCoherent>
__device__ __forceinline__ void put_f2(float* p, float x, float y) {
    const unsigned long long w = ((unsigned long long)__float_as_uint(y) << 32) | __float_as_uint(x);
    if (kCoherent)
        __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        *reinterpret_cast<unsigned long long*>(p) = w;
}

template <bool kCoherent>
__device__ __forceinline__ float2 get_f2(const float* p) {
    unsigned long long w;
    if (kCoherent)
        w = __hip_atomic_load(reinterpret_cast<unsigned long long*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
    else
        w = *reinterpret_cast<const unsigned long long*>(p);
    return make_float2(__uint_as_float((uint32_t)w), __uint_as_float((uint32_t)(w >> 32)));
}

// One wave merges output columns [8 chunk, 8 chunk + 8) of query head h of
// sequence b over its ns partials.  Each lane takes two runs per round and
// issues both runs' loads before any arithmetic (clamped indices, unused runs
// weighted 0), keeping a running (max, sum, output) rescaled as it goes; the
// lanes are combined at the end.
template <int D, bool kCoherent>
__device__ void merge_item(const GqaArgs& a, int b, int h, int chunk, int ns, int lane) {
    const int G = a.G, g = h / G, hh = h % G;
    const size_t stride = (size_t)(G * D + 32);
    const float* base = a.part + ((size_t)b * a.Hkv + g) * a.n_split * stride;
    float M = -INFINITY, L = 0.0f;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int s0 = 0; s0 < ns; s0 += 2 * kWave) {
        float mr[2], lr[2], ov[2][8];
#pragma unroll
        for (int r = 0; r < 2; r++) {
            const float* p = base + (size_t)min(s0 + r * kWave + lane, ns - 1) * stride;
            mr[r] = get_f<kCoherent>(p + G * D + hh);
            lr[r] = get_f<kCoherent>(p + G * D + 16 + hh);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float2 v = get_f2<kCoherent>(p + hh * D + 8 * chunk + 2 * i);
                ov[r][2 * i] = v.x;
                ov[r][2 * i + 1] = v.y;
            }
        }
#pragma unroll
        for (int r = 0; r < 2; r++) {
            if (s0 + r * kWave + lane >= ns) continue;
            const float Mn = fmaxf(M, mr[r]);
            const float keep = M == -INFINITY ? 0.0f : exp2f(M - Mn);
            const float w = exp2f(mr[r] - Mn);
            M = Mn;
            L = L * keep + w * lr[r];
#pragma unroll
            for (int i = 0; i < 8; i++) acc[i] = acc[i] * keep + w * ov[r][i];
        }
    }
    float Mw = M;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) Mw = fmaxf(Mw, __shfl_xor(Mw, o));
    const float sc = M == -INFINITY ? 0.0f : exp2f(M - Mw);
    L *= sc;
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] *= sc;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        L += __shfl_xor(L, o);
#pragma unroll
        for (int i = 0; i < 8; i++) acc[i] += __shfl_xor(acc[i], o);
    }
    if (lane == 0) {
        float* out = a.out + ((size_t)b * a.Hq + h) * D + 8 * chunk;
        const float inv = ns > 0 ? 1.0f / L : 0.0f;
        *reinterpret_cast<float4*>(out) = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
        *reinterpret_cast<float4*>(out + 4) = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
    }
}

template <int D, bool kFused>
__global__ __launch_bounds__(kThreads) void gqa_partial_kernel(GqaArgs a) {
    constexpr int RW = rows_per_wave<D>();
    constexpr int KK = D / 32;           // score steps per 16-row block
    constexpr int NB = RW / 16;          // 16-row blocks per wave
    constexpr int ND = D / 16;           // output column blocks
    constexpr int VTS = RW + 4;          // bf16 per transposed-V row (8 bytes of padding)
    constexpr int NQ = RW / 4;           // row quads per wave
    constexpr int NI = NQ * (D / 8) / kWave;  // (row quad, 8-column chunk) items per lane
    static_assert(NI * kWave == NQ * (D / 8), "V items must fill the wave");
    // transposed V per wave; after the products the same bytes hold each
    // wave's unnormalised outputs for the workgroup merge
    constexpr int kVtElems = kWaves * D * VTS;
    static_assert(kVtElems * 2 >= kWaves * 16 * D * 4, "the merge buffer must fit in the V region");
    __shared__ __align__(16) uint16_t vt[kVtElems];
    __shared__ float red_m[kWaves][16], red_l[kWaves][16];

    const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int li = lane % 16, lg = lane / 16;
    const int n = min(max(a.seq_len[b], 0), a.S_max);
    const int row0 = split * kWaves * RW;
    const int G = a.G;
    if (row0 >= n) {
        // no rows of this sequence here; with the merge in this launch, the
        // first run of an empty sequence writes its zeros
        if (kFused && n == 0 && split == 0)
            for (int e = threadIdx.x; e < G * D; e += kThreads) a.out[((size_t)b * a.Hq + g * G) * D + e] = 0.0f;
        return;
    }
    const int wrow0 = row0 + wave * RW;
    // the merge's control words: arrival counter, epoch, 16 flag copies, one line each
    unsigned* ctl = a.cnt + ((size_t)b * a.Hkv + g) * kCtlWords;
    unsigned epoch = 0;
    if (kFused && threadIdx.x == 0) epoch = __hip_atomic_load(ctl + 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const size_t head_base = ((size_t)b * a.Hkv + g) * (size_t)a.S_max * D;
    const uint16_t* kb = a.k + head_base;
    const uint16_t* vb = a.v + head_base;

    // ---- loads: the group's queries, then K, then V (all in flight at once)
    uint4 qop[KK];
    {
        const int h = g * G + li;
        const uint16_t* qh = a.q + ((size_t)b * a.Hq + min(h, a.Hq - 1)) * D + 8 * lg;
#pragma unroll
        for (int kk = 0; kk < KK; kk++) qop[kk] = *reinterpret_cast<const uint4*>(qh + 32 * kk);
        if (li >= G)
#pragma unroll
            for (int kk = 0; kk < KK; kk++) qop[kk] = make_uint4(0, 0, 0, 0);
    }
    uint4 kop[NB][KK];
#pragma unroll
    for (int rb = 0; rb < NB; rb++) {
        const int row = min(wrow0 + 16 * rb + li, n - 1);
        const uint16_t* kr = kb + (size_t)row * D + 8 * lg;
#pragma unroll
        for (int kk = 0; kk < KK; kk++) kop[rb][kk] = *reinterpret_cast<const uint4*>(kr + 32 * kk);
    }
    uint4 vop[NI][4];
#pragma unroll
    for (int t = 0; t < NI; t++) {
        const int it = lane + kWave * t, rq = it % NQ, c = it / NQ;
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int row = min(wrow0 + 4 * rq + r, n - 1);
            vop[t][r] = *reinterpret_cast<const uint4*>(vb + (size_t)row * D + 8 * c);
        }
    }

    // ---- scores: S^T = K Q^T, 16 rows x 16 heads per block
    floatx4 sacc[NB];
#pragma unroll
    for (int rb = 0; rb < NB; rb++) {
        sacc[rb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < KK; kk++)
            sacc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kop[rb][kk]),
                                                               __builtin_bit_cast(bf16x8_t, qop[kk]), sacc[rb],
                                                               0, 0, 0);
    }
    // lane (li, lg) holds head li at rows wrow0 + 16 rb + 4 lg + i
    float m = -INFINITY;
#pragma unroll
    for (int rb = 0; rb < NB; rb++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const bool valid = wrow0 + 16 * rb + 4 * lg + i < n;
            const float sv = valid ? sacc[rb][i] * a.c : -INFINITY;
            sacc[rb][i] = sv;
            m = fmaxf(m, sv);
        }
    m = fmaxf(m, shfl_xor_f(m, 16));
    m = fmaxf(m, shfl_xor_f(m, 32));
    const float mu = m == -INFINITY ? 0.0f : m;  // a wave past the sequence: every p is 0
    short4_t pop[NB];
    float l = 0.0f;
#pragma unroll
    for (int rb = 0; rb < NB; rb++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint16_t pb = bf16_rne(exp2f(sacc[rb][i] - mu));
            pop[rb][i] = (short)pb;
            l += bf16_value(pb);
        }
    l += shfl_xor_f(l, 16);
    l += shfl_xor_f(l, 32);

    // ---- V transposed into this wave's LDS region: vt[d][j], 4 rows per 8 bytes
    uint16_t* myvt = vt + (size_t)wave * D * VTS;
#pragma unroll
    for (int t = 0; t < NI; t++) {
        const int it = lane + kWave * t, rq = it % NQ, c = it / NQ;
        const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&vop[t][0]);
        const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&vop[t][1]);
        const uint32_t* r2 = reinterpret_cast<const uint32_t*>(&vop[t][2]);
        const uint32_t* r3 = reinterpret_cast<const uint32_t*>(&vop[t][3]);
#pragma unroll
        for (int w = 0; w < 4; w++) {
            const uint2 lo = make_uint2((r0[w] & 0xFFFFu) | (r1[w] << 16), (r2[w] & 0xFFFFu) | (r3[w] << 16));
            const uint2 hi = make_uint2((r0[w] >> 16) | (r1[w] & 0xFFFF0000u), (r2[w] >> 16) | (r3[w] & 0xFFFF0000u));
            *reinterpret_cast<uint2*>(myvt + (8 * c + 2 * w) * VTS + 4 * rq) = lo;
            *reinterpret_cast<uint2*>(myvt + (8 * c + 2 * w + 1) * VTS + 4 * rq) = hi;
        }
    }
    __syncthreads();

    // ---- O = P V: 16 heads x 16 columns per block, 16 rows per step
    floatx4 oacc[ND];
#pragma unroll
    for (int db = 0; db < ND; db++) oacc[db] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int rb = 0; rb < NB; rb++)
#pragma unroll
        for (int db = 0; db < ND; db++) {
            const uint2 v4 = *reinterpret_cast<const uint2*>(myvt + (16 * db + li) * VTS + 16 * rb + 4 * lg);
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pop[rb], __builtin_bit_cast(short4_t, v4),
                                                                 oacc[db], 0, 0, 0);
        }
    // lane (li, lg) holds heads 4 lg + i at column 16 db + li

    // ---- merge the 4 waves in LDS and store the workgroup's partial
    if (lg == 0) {
        red_m[wave][li] = m;
        red_l[wave][li] = l;
    }
    __syncthreads();  // every wave is done reading vt
    float* ob = reinterpret_cast<float*>(vt);  // [wave][16][D]
#pragma unroll
    for (int db = 0; db < ND; db++)
#pragma unroll
        for (int i = 0; i < 4; i++) ob[((size_t)wave * 16 + 4 * lg + i) * D + 16 * db + li] = oacc[db][i];
    __syncthreads();
    float* part = a.part + (((size_t)b * a.Hkv + g) * a.n_split + split) * (size_t)(G * D + 32);
    for (int e = 2 * threadIdx.x; e < G * D; e += 2 * kThreads) {
        const int hh = e / D, d = e % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; w++) M = fmaxf(M, red_m[w][hh]);
        float o0 = 0.0f, o1 = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; w++) {
            const float sc = red_m[w][hh] == -INFINITY ? 0.0f : exp2f(red_m[w][hh] - M);
            o0 += sc * ob[((size_t)w * 16 + hh) * D + d];
            o1 += sc * ob[((size_t)w * 16 + hh) * D + d + 1];
        }
        put_f2<kFused>(part + e, o0, o1);
    }
    if (threadIdx.x < G) {
        const int hh = threadIdx.x;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; w++) M = fmaxf(M, red_m[w][hh]);
        float L = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; w++)
            L += (red_m[w][hh] == -INFINITY ? 0.0f : exp2f(red_m[w][hh] - M)) * red_l[w][hh];
        put_f<kFused>(part + G * D + hh, M);
        put_f<kFused>(part + G * D + 16 + hh, L);
    }
    if (!kFused) return;

    // ---- the merge in this launch: wait for every run of this (sequence, KV head)
    const int ns = (n + kWaves * RW - 1) / (kWaves * RW);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores acknowledged (written through)
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned next = epoch + 1u;
        if (atomicAdd(ctl, 1u) == (unsigned)ns - 1) {
            // the last run of this head: reset the counter, raise the epoch
            __hip_atomic_store(ctl, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(ctl + 32, next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int c = 0; c < kFlagCopies; c++)
                __hip_atomic_store(ctl + 64 + 32 * c, next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            unsigned* flag = ctl + 64 + 32 * (split % kFlagCopies);
            for (long spins = 0; __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != next;
                 spins++) {
                if (spins > kSpinLimit) {
                    __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
    }
    __syncthreads();
    const int items = G * (D / 8);
    for (int it = split + ns * wave; it < items; it += ns * kWaves)
        merge_item<D, true>(a, b, g * G + it / (D / 8), it % (D / 8), ns, lane);
}

// One wave per (sequence, query head, 8 output columns): merge the partials of
// every run of rows of that sequence.
template <int D>
__global__ __launch_bounds__(kThreads) void gqa_merge_kernel(GqaArgs a) {
    constexpr int RWG = kWaves * rows_per_wave<D>();  // rows per partial
    const int lane = threadIdx.x % kWave;
    const long item = (long)blockIdx.x * kWaves + threadIdx.x / kWave;
    const long n_items = (long)a.B * a.Hq * (D / 8);
    if (item >= n_items) return;
    const int chunk = (int)(item % (D / 8));
    const int h = (int)((item / (D / 8)) % a.Hq);
    const int b = (int)(item / ((long)(D / 8) * a.Hq));
    const int n = min(max(a.seq_len[b], 0), a.S_max);
    merge_item<D, false>(a, b, h, chunk, (n + RWG - 1) / RWG, lane);
}

template <int D>
hipError_t launch_gqa_d(const GqaArgs& a, hipStream_t stream, hipEvent_t* events) {
    hipError_t e;
    if (events && (e = hipEventRecord(events[0], stream)) != hipSuccess) return e;
    const dim3 grid1((unsigned)a.n_split, (unsigned)a.Hkv, (unsigned)a.B);
    if (a.fused) {
        hipLaunchKernelGGL((gqa_partial_kernel<D, true>), grid1, dim3(kThreads), 0, stream, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        for (int i = 1; i < 3 && events; i++)
            if ((e = hipEventRecord(events[i], stream)) != hipSuccess) return e;
        return hipSuccess;
    }
    hipLaunchKernelGGL((gqa_partial_kernel<D, false>), grid1, dim3(kThreads), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (events && (e = hipEventRecord(events[1], stream)) != hipSuccess) return e;
    const long items = (long)a.B * a.Hq * (D / 8);
    hipLaunchKernelGGL(gqa_merge_kernel<D>, dim3((unsigned)((items + kWaves - 1) / kWaves)), dim3(kThreads), 0,
                       stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (events && (e = hipEventRecord(events[2], stream)) != hipSuccess) return e;
    return hipSuccess;
}

}  // namespace

int gqa_rows_per_split(int D) { return kWaves * (D <= 128 ? 64 : 32); }

namespace {

template <int D>
int fused_capacity() {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(&gqa_partial_kernel<D, true>), kThreads, 0) != hipSuccess)
        return 0;
    return cus * per_cu;
}

}  // namespace

int gqa_fused_capacity(int D) {
    switch (D) {
        case 64: return fused_capacity<64>();
        case 128: return fused_capacity<128>();
        case 256: return fused_capacity<256>();
        default: return 0;
    }
}

hipError_t launch_gqa_decode(const GqaArgs& a, hipStream_t stream, hipEvent_t* events) {
    switch (a.D) {
        case 64: return launch_gqa_d<64>(a, stream, events);
        case 128: return launch_gqa_d<128>(a, stream, events);
        case 256: return launch_gqa_d<256>(a, stream, events);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace bitmoe
