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

// Sum over the wave, as a wave-uniform value: DPP butterflies inside each row of
// 16 lanes, then the four row totals through readlane (no LDS round trip, as
// the last two steps of group_sum take).
__device__ __forceinline__ float wave_total(float v) {
    v += dpp<0xB1>(v);   // quad_perm 1,0,3,2
    v += dpp<0x4E>(v);   // quad_perm 2,3,0,1
    v += dpp<0x141>(v);  // row_half_mirror
    v += dpp<0x140>(v);  // row_mirror
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

// ---- top k of a token's E <= 256 logits, selected by one workgroup whose
// threads 0..255 (4 waves) hold one order key each (thread t: expert t; key 0
// for t >= E).  Rank order: larger logit first, equal logits by lower expert
// index.  Three steps with a workgroup barrier between them:
//   topk_keys        every thread 0..255: its key into LDS, each wave's two
//                    largest keys;
//   topk_candidates  keys at or above the least of the four waves' second
//                    largest: at least two keys of every wave reach it, so the
//                    k <= 8 largest are among them and no key below it ranks in
//                    the top k (fewer than 194 experts can leave a wave with
//                    under two keys: then every expert is a candidate).  Each
//                    wave lists its own candidates;
//   topk_rank        up to kRankCands candidates are ranked in parallel, 8
//                    threads each (the candidates above one, and the equal ones
//                    of lower index); more take a radix search for the k-th
//                    key in one wave.  Writes sel_e / sel_key for ranks < k.
constexpr int kRankCands = 32;

struct TopkShared {
    uint32_t keys[kMaxE];
    uint32_t m2[4];
    uint32_t ckey[4][kWave];
    int cidx[4][kWave];
    int ccnt[4];
    uint32_t tkey[kMaxTopK];
    int tidx[kMaxTopK];
    int sel_e[kMaxTopK];
    uint32_t sel_key[kMaxTopK];
};

__device__ __forceinline__ void topk_keys(TopkShared& s, uint32_t mykey, int tid, int lane, int wave) {
    s.keys[tid] = mykey;
    const uint32_t m1 = wave_max_u32(mykey);
    const int first = (int)__builtin_ctzll(__ballot(mykey == m1));
    const uint32_t m2 = wave_max_u32(lane == first ? 0u : mykey);
    if (lane == 0) s.m2[wave] = m2;
}

__device__ __forceinline__ void topk_candidates(TopkShared& s, uint32_t mykey, int E, int tid, int lane, int wave) {
    const uint32_t lim = E >= 194 ? min(min(s.m2[0], s.m2[1]), min(s.m2[2], s.m2[3])) : 1u;
    const bool c = mykey != 0u && mykey >= lim;
    const uint64_t bal = __ballot(c);
    if (c) {
        const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
        s.ckey[wave][pos] = mykey;
        s.cidx[wave][pos] = tid;
    }
    if (lane == 0) s.ccnt[wave] = __popcll(bal);
}

// Top k of the E <= 256 order keys one wave holds (key[i] of lane l: expert
// l + 64 i, 0 for a missing expert) by a radix search for the k-th largest
// key: the keys above it, then the equal ones of lowest index, ranked among
// themselves.  Wave-local (uses tkey / tidx); writes sel_e / sel_key.
__device__ __forceinline__ void topk_radix_wave(TopkShared& s, const uint32_t (&key)[kMaxE / kWave], int k, int lane) {
    uint32_t theta = 0;
    for (int b = 31; b >= 0; b--) {
        const uint32_t cand = theta | (1u << b);
        int c = 0;
#pragma unroll
        for (int i = 0; i < kMaxE / kWave; i++) c += __popcll(__ballot(key[i] >= cand));
        if (c >= k) theta = cand;
    }
    uint64_t sel[kMaxE / kWave];
    int need = k;
#pragma unroll
    for (int i = 0; i < kMaxE / kWave; i++) {
        sel[i] = __ballot(key[i] > theta);
        need -= __popcll(sel[i]);
    }
#pragma unroll
    for (int i = 0; i < kMaxE / kWave; i++) {
        uint64_t eq = __ballot(key[i] == theta);
        while (need > 0 && eq) {
            const uint64_t bit = eq & (~eq + 1);
            sel[i] |= bit;
            eq ^= bit;
            need--;
        }
    }
    int base = 0;
#pragma unroll
    for (int i = 0; i < kMaxE / kWave; i++) {
        if ((sel[i] >> lane) & 1ull) {
            const int pos = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(sel[i] >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)sel[i], 0));
            s.tkey[pos] = key[i];
            s.tidx[pos] = lane + kWave * i;
        }
        base += __popcll(sel[i]);
    }
    if (lane < k) {
        const uint32_t mk = s.tkey[lane];
        const int me = s.tidx[lane];
        int rank = 0;
        for (int m = 0; m < k; m++) {
            const uint32_t om = s.tkey[m];
            rank += (om > mk || (om == mk && s.tidx[m] < me)) ? 1 : 0;
        }
        s.sel_e[rank] = me;
        s.sel_key[rank] = mk;
    }
}

// Top k (k <= 8) of the E <= 256 order keys one wave holds (as above), with no
// workgroup barrier.  The keys of each of the 8 groups of 32 (slot i, lanes
// 0..31 or 32..63) have a maximum; every key at or above the least of those 8
// maxima is a candidate.  Each group holds one, so at least 8 >= k keys are
// candidates and no key below the bound ranks in the top k.  The candidates
// (~21 of 256 typically) move to lanes 0..n-1 through LDS, and lane c counts
// the candidates that rank above its own (larger key, or equal key and lower
// expert index).  More than 64 candidates (many equal logits, or E small enough
// that a group is empty) take the radix search.  Writes sel_e / sel_key for
// ranks < k and returns, in lane j < k, the key of rank j (0 in other lanes).
__device__ __forceinline__ uint32_t topk_wave_select(TopkShared& s, const uint32_t (&key)[kMaxE / kWave], int k, int lane) {
    uint32_t lim = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < kMaxE / kWave; i++) {
        uint32_t m = key[i];
        m = max_dpp<0xB1>(m);   // quad_perm 1,0,3,2
        m = max_dpp<0x4E>(m);   // quad_perm 2,3,0,1
        m = max_dpp<0x141>(m);  // row_half_mirror
        m = max_dpp<0x140>(m);  // row_mirror
        const uint32_t a = __builtin_amdgcn_readlane(m, 0), b = __builtin_amdgcn_readlane(m, 16);
        const uint32_t c = __builtin_amdgcn_readlane(m, 32), d = __builtin_amdgcn_readlane(m, 48);
        lim = min(lim, min(max(a, b), max(c, d)));  // unsigned compares
    }
    uint64_t bal[kMaxE / kWave];
    int n = 0;
#pragma unroll
    for (int i = 0; i < kMaxE / kWave; i++) {
        bal[i] = __ballot(key[i] != 0u && key[i] >= lim);
        n += __popcll(bal[i]);
    }
    if (n > kWave) {
        topk_radix_wave(s, key, k, lane);
    } else {
        int base = 0;
#pragma unroll
        for (int i = 0; i < kMaxE / kWave; i++) {
            if ((bal[i] >> lane) & 1ull) {
                const int pos = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal[i] >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)bal[i], 0));
                s.ckey[0][pos] = key[i];
                s.cidx[0][pos] = lane + kWave * i;
            }
            base += __popcll(bal[i]);
        }
        // candidate c (lane c < n) as one 64-bit value that orders as the rank
        // order: the key above 255 - expert index.  Lanes past n hold 0, below
        // every candidate.  The broadcasts take constant lane indices.
        const uint32_t ck = lane < n ? s.ckey[0][lane] : 0u;
        const int ce = lane < n ? s.cidx[0][lane] : 0;
        const uint64_t mine = lane < n ? ((uint64_t)ck << 8) | (uint32_t)(255 - ce) : 0ull;
        const uint32_t mlo = (uint32_t)mine, mhi = (uint32_t)(mine >> 32);
        int rank = 0;
#pragma unroll
        for (int c0 = 0; c0 < kWave; c0 += 8) {
            if (c0 >= n) break;
#pragma unroll
            for (int m = 0; m < 8; m++) {
                const uint64_t km = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(mhi, c0 + m) << 32) |
                                    (uint32_t)__builtin_amdgcn_readlane(mlo, c0 + m);
                rank += km > mine ? 1 : 0;
            }
        }
        if (lane < n && rank < k) {
            s.sel_e[rank] = ce;
            s.sel_key[rank] = ck;
        }
    }
    return lane < k ? s.sel_key[lane] : 0u;
}

__device__ __forceinline__ void topk_rank(TopkShared& s, int k, int tid, int lane, int wave) {
    const int n0 = s.ccnt[0], n1 = s.ccnt[1], n2 = s.ccnt[2], n3 = s.ccnt[3];
    const int n = n0 + n1 + n2 + n3;
    if (n <= kRankCands) {
        if (tid < 8 * kRankCands) {
            auto cand = [&](int q, uint32_t& key, int& e) {
                const int w = q < n0 ? 0 : q < n0 + n1 ? 1 : q < n0 + n1 + n2 ? 2 : 3;
                const int r = q - (w > 0 ? n0 : 0) - (w > 1 ? n1 : 0) - (w > 2 ? n2 : 0);
                key = s.ckey[w][r];
                e = s.cidx[w][r];
            };
            const int i = tid / 8;
            uint32_t ck = 0;
            int ce = 0;
            if (i < n) cand(i, ck, ce);
            int rank = 0;
#pragma unroll
            for (int m = 0; m < kRankCands / 8; m++) {
                const int jj = tid % 8 + 8 * m;
                if (jj < n) {
                    uint32_t kj;
                    int ej;
                    cand(jj, kj, ej);
                    rank += (kj > ck || (kj == ck && ej < ce)) ? 1 : 0;
                }
            }
            rank = (int)group_sum((float)rank, 8);
            if (tid % 8 == 0 && i < n && rank < k) {
                s.sel_e[rank] = ce;
                s.sel_key[rank] = ck;
            }
        }
    } else if (wave == 0) {
        uint32_t key[kMaxE / kWave];
#pragma unroll
        for (int i = 0; i < kMaxE / kWave; i++) key[i] = s.keys[lane + kWave * i];
        topk_radix_wave(s, key, k, lane);
    }
}

// Routing weight of every rank (lane j < k: rank j), softmax of the kept
// logits summed in rank order, from the ranks' keys (rk of lane j < k: rank j's
// key); one wave.
__device__ __forceinline__ float topk_weight_of_keys(uint32_t rk, int k) {
    const float top = key_float(__builtin_amdgcn_readlane(rk, 0));
    const float pr = expf(key_float(rk) - top);
    float z = 0.0f;
    for (int m = 0; m < k; m++) z += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pr), m));
    return pr / z;
}
// the same from sel_key, after topk_rank and a barrier
__device__ __forceinline__ float topk_weight_of_lane(const TopkShared& s, int k, int lane) {
    return topk_weight_of_keys(lane < k ? s.sel_key[lane] : 0u, k);
}

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
