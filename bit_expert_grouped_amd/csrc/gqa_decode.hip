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
//     at once, the merge runs in the same launch.  Each workgroup stores its
//     partial with agent-scope stores, which write through the per-XCD L2, in
//     the order the merge reads it (per output item: 8 values, then the head's
//     m and l, 48 bytes), waits for the stores to be acknowledged and raises
//     the run's ready flag (its own cache line) to this call's epoch.  It then
//     merges its share of the head's outputs: it polls (bounded) only the
//     flags of every run, then reads each run's 48 bytes with three plain
//     16-byte loads.  No cache holds a line of a partial before its flag is up
//     (the kernel boundary drops what the previous call left), so plain loads
//     after the flag see the data.  Polling one word per run instead of every
//     value cut the merge from ~4 us to ~1 us.  The epoch is one more than a
//     per-(sequence, KV head) word that every workgroup reads when it starts;
//     the first run's workgroup raises it after its merge, when every run's
//     flag (so every workgroup's read of it) is in.  Otherwise a second kernel
//     (gqa_merge_kernel) merges plain partials.
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
constexpr long kSpinLimit = 1l << 20;  // bound of the fused merge's polls (s_sleep rounds)
constexpr int kCtlWords = 64;           // control words per (sequence, KV head): the epoch, its own line

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

template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_f(float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); }
// the wave's largest value / total, wave-uniform: DPP within each row of 16
// lanes (quad_perm 1,0,3,2; quad_perm 2,3,0,1; row_half_mirror; row_mirror),
// then the four row results through readlane
__device__ __forceinline__ float wave_max_f(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x141>(v));
    v = fmaxf(v, dpp_f<0x140>(v));
    return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ float wave_sum_f(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);
    v += dpp_f<0x140>(v);
    return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

__device__ __forceinline__ unsigned long long peek(const unsigned long long* p) {
    return __hip_atomic_load(const_cast<unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Bytes of one run's partial in the fused layout: a 128-byte line for the
// ready flag, then per output item (query head hh, 8 columns) 8 values, m and
// l of head hh and 2 words of padding (48 bytes).
__host__ __device__ constexpr size_t fused_part_bytes(int G, int D) { return 128 + (size_t)G * (D / 8) * 48; }

// two float32 values with one agent-scope (L2 write-through) store
__device__ __forceinline__ void put2_wt(char* p, float x, float y) {
    __hip_atomic_store(reinterpret_cast<unsigned long long*>(p),
                       ((unsigned long long)__float_as_uint(y) << 32) | __float_as_uint(x), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// One wave merges output columns [8 chunk, 8 chunk + 8) of query head h of
// sequence b over its ns partials.  Each lane takes two runs per round and
// issues both runs' loads before any arithmetic (clamped indices, unused runs
// weighted 0), keeping a running (max, sum, output) rescaled as it goes; the
// lanes are combined at the end.  Tagged partials are polled until every word
// the wave needs carries `tag` (bounded: on timeout the error word is set).
template <int D, bool kTagged>
__device__ void merge_item(const GqaArgs& a, int b, int h, int chunk, int ns, int lane, unsigned tag) {
    const int G = a.G, g = h / G, hh = h % G;
    const size_t stride = (size_t)(G * D + 32);  // values per partial
    const size_t base_i = ((size_t)b * a.Hkv + g) * a.n_split * stride;
    float M = -INFINITY, L = 0.0f;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int s0 = 0; s0 < ns; s0 += 2 * kWave) {
        float mr[2], lr[2], ov[2][8];
        if (kTagged) {
            // the flags of this round's runs, then their items' 48 bytes
            const char* blk0 = reinterpret_cast<const char*>(a.part) +
                               ((size_t)b * a.Hkv + g) * a.n_split * fused_part_bytes(G, D);
            for (long spins = 0;; spins++) {
                bool have = true;
#pragma unroll
                for (int r = 0; r < 2; r++) {
                    const unsigned* f = reinterpret_cast<const unsigned*>(
                        blk0 + (size_t)min(s0 + r * kWave + lane, ns - 1) * fused_part_bytes(G, D));
                    have = have && __hip_atomic_load(const_cast<unsigned*>(f), __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT) == tag;
                }
                if (__ballot(!have) == 0) break;
                if (spins > kSpinLimit) {
                    if (lane == 0) __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            const int item = hh * (D / 8) + chunk;
#pragma unroll
            for (int r = 0; r < 2; r++) {
                const float4* q = reinterpret_cast<const float4*>(
                    blk0 + (size_t)min(s0 + r * kWave + lane, ns - 1) * fused_part_bytes(G, D) + 128 + item * 48);
                const float4 o0 = q[0], o1 = q[1], ml = q[2];
                ov[r][0] = o0.x, ov[r][1] = o0.y, ov[r][2] = o0.z, ov[r][3] = o0.w;
                ov[r][4] = o1.x, ov[r][5] = o1.y, ov[r][6] = o1.z, ov[r][7] = o1.w;
                mr[r] = ml.x;
                lr[r] = ml.y;
            }
        } else {
#pragma unroll
            for (int r = 0; r < 2; r++) {
                const float* p = a.part + base_i + (size_t)min(s0 + r * kWave + lane, ns - 1) * stride;
                mr[r] = p[G * D + hh];
                lr[r] = p[G * D + 16 + hh];
                const float4 o0 = *reinterpret_cast<const float4*>(p + hh * D + 8 * chunk);
                const float4 o1 = *reinterpret_cast<const float4*>(p + hh * D + 8 * chunk + 4);
                ov[r][0] = o0.x, ov[r][1] = o0.y, ov[r][2] = o0.z, ov[r][3] = o0.w;
                ov[r][4] = o1.x, ov[r][5] = o1.y, ov[r][6] = o1.z, ov[r][7] = o1.w;
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
    const float Mw = wave_max_f(M);
    const float sc = M == -INFINITY ? 0.0f : exp2f(M - Mw);
    L = wave_sum_f(L * sc);
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] = wave_sum_f(acc[i] * sc);
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
    __shared__ unsigned epoch_sh;

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
    // the merge's epoch word of this (sequence, KV head)
    unsigned* ctl = a.cnt + ((size_t)b * a.Hkv + g) * kCtlWords;
    if (kFused && threadIdx.x == 0) epoch_sh = __hip_atomic_load(ctl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

    // ---- V transposed into this wave's LDS region (vt[d][j], 4 rows per 8
    // bytes) and O = P V (16 heads x 16 columns per block, 16 rows per step),
    // a group of columns at a time: item t covers columns [32 t, 32 t + 32) of
    // every row, so the products of those columns run as soon as it is written
    // and V's later loads land meanwhile.  The region is this wave's alone and
    // a wave's LDS accesses complete in order, so no barrier is needed.
    static_assert((8 * kWave / NQ) % 16 == 0 && NI * (8 * kWave / NQ) == D, "items cover whole column blocks");
    uint16_t* myvt = vt + (size_t)wave * D * VTS;
    floatx4 oacc[ND];
#pragma unroll
    for (int db = 0; db < ND; db++) oacc[db] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
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
        asm volatile("" ::: "memory");  // the reads below after this wave's writes
        // item t wrote columns [8 (kWave t / NQ), 8 (kWave (t + 1) / NQ))
        constexpr int kColsPerItem = 8 * kWave / NQ;
#pragma unroll
        for (int db = t * kColsPerItem / 16; db < (t + 1) * kColsPerItem / 16; db++)
#pragma unroll
            for (int rb = 0; rb < NB; rb++) {
                const uint2 v4 = *reinterpret_cast<const uint2*>(myvt + (16 * db + li) * VTS + 16 * rb + 4 * lg);
                oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pop[rb], __builtin_bit_cast(short4_t, v4),
                                                                     oacc[db], 0, 0, 0);
            }
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
    const size_t part_i = (((size_t)b * a.Hkv + g) * a.n_split + split) * (size_t)(G * D + 32);
    char* fblk = reinterpret_cast<char*>(a.part) + (((size_t)b * a.Hkv + g) * a.n_split + split) * fused_part_bytes(G, D);
    const unsigned tag = kFused ? epoch_sh + 1u : 0u;  // read after the barriers above
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
        if (kFused) {
            char* it = fblk + 128 + (size_t)(hh * (D / 8) + d / 8) * 48;
            put2_wt(it + (d % 8) * 4, o0, o1);
            if (d % 8 == 0) {  // the head's m and l beside each of its items
                float L = 0.0f;
#pragma unroll
                for (int w = 0; w < kWaves; w++)
                    L += (red_m[w][hh] == -INFINITY ? 0.0f : exp2f(red_m[w][hh] - M)) * red_l[w][hh];
                put2_wt(it + 32, M, L);
            }
        } else {
            a.part[part_i + e] = o0;
            a.part[part_i + e + 1] = o1;
        }
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
        if (!kFused) {
            a.part[part_i + G * D + hh] = M;
            a.part[part_i + G * D + 16 + hh] = L;
        }
    }
    if (!kFused) return;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores acknowledged (written through)
    __syncthreads();
    if (threadIdx.x == 0)
        __hip_atomic_store(reinterpret_cast<unsigned*>(fblk), tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // ---- the merge in this launch: poll the flags of every run of this
    // (sequence, KV head), read their items; the first run's workgroup then
    // raises the epoch
    const int ns = (n + kWaves * RW - 1) / (kWaves * RW);
    const int items = G * (D / 8);
    for (int it = split + ns * wave; it < items; it += ns * kWaves)
        merge_item<D, true>(a, b, g * G + it / (D / 8), it % (D / 8), ns, lane, tag);
    if (split == 0) {
        __syncthreads();  // every item of this workgroup merged: every run's partial was in
        if (threadIdx.x == 0) __hip_atomic_store(ctl, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
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
    merge_item<D, false>(a, b, h, chunk, (n + RWG - 1) / RWG, lane, 0u);
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
