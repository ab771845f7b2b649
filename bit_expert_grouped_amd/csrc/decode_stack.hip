// Persistent multi-layer decode for gfx950: ONE kernel launch carries a decode
// step (one token) through L stacked MoE layers of a pre-norm decoder,
//     x(l+1) = bf16(x(l) + layer_l(n(l))),  n(l) = bf16(x(l) / rms(x(l)) * gamma_l),
// rms(x) = sqrt(mean(x^2) + 1e-6): each layer reads the root-mean-square
// normalisation of the bf16 residual stream and adds its output to it.
//
// Pages: decode reads the weights every step and is bound by memory bandwidth;
// the engine overlaps the dependent stages of a decode step (hundreds of
// kernels in fewer sequential stages) instead of running them one after the
// other (aimanavo.com page, section "Lily does not treat prefill and decode as
// the same job"); routing stays on the GPU (same section; dzen.guru page,
// section "Where does the speed-up come from?").
//
// What one layer needs at T = 1 is a chain: x -> its normalisation -> router logits -> top-k ->
// the k experts' gate/up -> their down -> x of the next layer.  Only the k
// routed experts' weights (14 MB at the Qwen shapes) depend on the data; the
// router (1 MiB) and the shared expert (1.8 MB) do not, so they are read ahead
// of the layer that uses them.  The kernel keeps every hand-over inside one
// launch and takes as few of them as the chain allows:
//
//   - the grid is kStackGrid workgroups of 8 waves, one per compute unit, all
//     resident at once (the host checks the device can hold them), and every
//     wait is bounded;
//   - router: workgroup w scores expert w and publishes its logit ({epoch,
//     logit} words, kStackLogitCopies copies); every workgroup then reads all
//     E logits and selects the top k itself, so the routing costs one
//     hand-over, not two.  Each of four waves holds 64 order keys; their two
//     largest give at least 8 keys at or above the smallest of the four
//     second-largest, so the top k (k <= 8) are among the keys at or above it.
//     Those few candidates are ranked by counting (ties to the lower expert
//     index); a radix search over all keys serves the rare case of more than
//     64 candidates or of under two experts per wave;
//   - gate/up: workgroup w takes 16 rows of the intermediate dim of one routed
//     slot (2 rows per wave, gate and up) and publishes h as float16 pairs; the
//     shared expert's gate/up (2 rows per workgroup) runs on weights read ahead;
//   - down and output: workgroup w owns output columns [8 w, 8 w + 8) and
//     computes them for every slot: wave j the 8 rows of routed slot j (one
//     64-column group per lane), waves 4-7 the 8 rows of the shared expert.
//     Every workgroup therefore reads every slot's h (each gate/up unit
//     publishes its h in kStackRoutedHCopies copies).  The k + 1
//     contributions of a column are summed in LDS in slot order (so the output
//     is the same bit for bit on every call) and the workgroup forms the next
//     layer's stream x(l+1) = bf16(x(l) + sum) for its columns and publishes
//     it packed ({16-bit tag, 3 bf16} words) in kStackXCopies copies; every
//     workgroup then reads the whole stream from its copy.  Broadcasting a few
//     KB to 256 workgroups costs what its most-read cache line costs, so every
//     value all workgroups read is replicated until each copy has ~8 readers.
//   - every exchange region is kept twice, by the parity of the layer's epoch:
//     a workgroup can run at most one layer ahead of the slowest (each layer's
//     logits come from all of them), so a word is never rewritten while a
//     reader may still wait for its previous value.
//
// Loads of one wave complete in order (the vmcnt counter), so a poll waits
// behind every load its wave issued before.  Each wave therefore issues the
// next layer's read-ahead (router row, shared expert slices, logit bias, into
// registers) only after the last poll of the layer, and polls follow the loads
// whose data they must wait for anyway.
//
#include "common.h"
#include "decode_common.h"
#include "kernels.h"

namespace bitmoe {

namespace {

using namespace dec;

constexpr int kWorkers = 8;
constexpr int kThreads = kWorkers * kWave;
constexpr int kGURows = 16;  // intermediate rows of a routed gate/up unit: 2 per wave
constexpr long kSpinLimit = 1l << 20;
constexpr int kHWords = kStackMaxI / 2;  // h words per slot (float16 pairs)
constexpr int kPollThreads = kStackMaxH / 8;  // threads that poll the output, one 8-column block each

// control words (uint32 indices) of the stack kernel inside the decode control block
constexpr int kCtlStEpoch = 2048;         // epoch of the last layer of the last call
constexpr int kCtlStDone = 2048 + 64;     // groups of workgroups finished in this call
constexpr int kCtlStGroupDone = 2048 + 128;  // + 32 g: workgroups of group g finished
constexpr int kDoneGroups = 8;

constexpr float kNormEps = 1e-6f;  // epsilon of the stream's normalisation

struct StackShared {
    uint4 xp[kStackMaxH / 8];    // the layer's input as float16 pairs in nibble order, per 8 columns
    float2 xs[kStackMaxH / 8];   // low/high nibble sums of each 8 columns
    uint16_t xb[kStackMaxH];     // the residual stream entering the layer, bf16
    uint16_t xn[kStackMaxH];     // its normalisation, the layer's input, bf16
    float ssq[4];                // sums of squares of the stream, one per polling wave
    uint4 hsp[kStackMaxI / 8];   // shared expert's h, pairs per 8 columns
    float2 hss[kStackMaxI / 8];
    uint4 hrp[8][kStackMaxI / 8];  // routed h of every slot, pairs per 8 columns
    float2 hrs[8][kStackMaxI / 8];
    float ycon[8 + 1][8];        // contributions to the owned columns: routed slots, then the shared expert
    uint32_t keys[kMaxE];        // order keys of the logits
    uint32_t tkey[kMaxTopK];     // the selected keys, in expert order
    int tidx[kMaxTopK];
    float red[kWorkers];         // router partial sums, one per wave
    float sred[kWorkers];        // shared gate/up partial sums, two waves per row
    int sel_e[kMaxTopK];         // the top k in rank order
    uint32_t sel_key[kMaxTopK];
    float sel_w[kMaxTopK];
    uint32_t m2[4];              // second largest key of each wave's 64
    int ncand;                   // candidates of the top k (keys >= min of m2)
    uint32_t ckey[kWave];
    int cidx[kWave];
    int last;
};

template <typename T>
__device__ __forceinline__ const T* layer_ptr(const T* p, int64_t stride, int l) {
    return reinterpret_cast<const T*>(reinterpret_cast<const char*>(p) + stride * (int64_t)l);
}

template <typename SB>
__device__ __forceinline__ const SB* sb_ptr(const void* p, int64_t stride, int l) {
    return reinterpret_cast<const SB*>(reinterpret_cast<const char*>(p) + stride * (int64_t)l);
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// tag of the stream words of epoch ep: 16 bits, never 0 (a zero-filled workspace's)
__device__ __forceinline__ unsigned xtag(unsigned ep) { return ep % 65535u + 1u; }

// 8 values of one 8-column block -> float16 pairs in nibble order and their
// low/high nibble sums (taken over the float16 values the products use)
__device__ __forceinline__ void block_pairs(const float (&v)[8], uint4& pairs, float2& sums) {
    _Float16 h[8];
#pragma unroll
    for (int i = 0; i < 8; i++) h[i] = (_Float16)v[i];
    pairs.x = as_u32(half2_t{h[0], h[4]});
    pairs.y = as_u32(half2_t{h[1], h[5]});
    pairs.z = as_u32(half2_t{h[2], h[6]});
    pairs.w = as_u32(half2_t{h[3], h[7]});
    sums = make_float2(((float)h[0] + (float)h[4]) + ((float)h[2] + (float)h[6]),
                       ((float)h[1] + (float)h[5]) + ((float)h[3] + (float)h[7]));
}

// Poll the {epoch, float16 pair} words [n v, n v + n) of an h vector of
// n_words words (lanes 0..n-1 of wave v, one word each; n = kPer <= 64) and
// place the values in LDS as pairs in nibble order; then lanes 0..n/4-1 form
// the low/high sums of the wave's blocks.  Returns false on timeout (then sets
// the error word).
template <int kPer>
__device__ bool poll_h(const unsigned long long* src, int n_words, unsigned epoch, uint4* pairs, float2* sums,
                       int v, int lane, bool failed, unsigned* ctl) {
    const int wd = kPer * v + lane;
    const bool mine = lane < kPer && wd < n_words;
    bool ok = true;
    unsigned long long val = 0;
    if (!failed) {
        for (long spins = 0;; spins++) {
            bool have = true;
            if (mine) {
                val = peek(src + wd);
                have = (unsigned)(val >> 32) == epoch;
            }
            if (__ballot(!have) == 0) break;
            if (spins > kSpinLimit) {
                if (lane == 0) flag_error(ctl);
                ok = false;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    _Float16* hh = reinterpret_cast<_Float16*>(pairs);
    if (mine) {
        const half2_t pr = as_half2((uint32_t)val);
        const int c0 = 2 * wd, c1 = 2 * wd + 1;
        hh[(c0 >> 3) * 8 + slot_of_column(c0 & 7)] = pr.x;
        hh[(c1 >> 3) * 8 + slot_of_column(c1 & 7)] = pr.y;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's values are in LDS
    const int blk = (kPer / 4) * v + lane;
    if (lane < kPer / 4 && blk * 4 < n_words) {
        const uint4 p = pairs[blk];
        const half2_t a = as_half2(p.x), b = as_half2(p.y), c = as_half2(p.z), d = as_half2(p.w);
        sums[blk] = make_float2(((float)a.x + (float)a.y) + ((float)c.x + (float)c.y),
                                ((float)b.x + (float)b.y) + ((float)d.x + (float)d.y));
    }
    return ok;
}

// s * (sum of code * a over a word or words) + b * (sum of a), from the
// exponent-trick partial sums of dot_word
__device__ __forceinline__ float affine(float s, float b, float alo, float ahi, float lo, float hi) {
    return s * ((alo - 1024.0f * lo) + (ahi - 64.0f * hi)) + b * (lo + hi);
}

// Addressing.  Every load, poll and atomic of the loop takes a base address
// that is uniform over the wave (kernel arguments, the layer, the expert: kept
// in scalar registers) plus a per-lane byte offset computed once before the
// loop.  The loop then writes no vector register that a memory operation in
// flight still reads as its address, which would make the compiler wait for
// that operation to complete.  Every load is issued whatever the shape
// (indices clamped into the tensors), so that each wave's count of loads in
// flight is the same on every path and the compiler's waits stay exact.
__device__ __forceinline__ const char* lay(const void* p, int64_t stride, int l) {
    return reinterpret_cast<const char*>(p) + stride * (int64_t)l;
}
template <typename T>
__device__ __forceinline__ T ld(const char* base, uint32_t off) {
    return *reinterpret_cast<const T*>(base + off);
}
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Read-ahead of one layer's data-independent weights, held in the registers of
// waves 4-7 until the layer runs.  Thread u = tid - 256 of those waves holds:
//   router  columns [8 u, 8 u + 8) of expert w's router row, and its logit bias;
//   sgu     columns [32 lane, 32 lane + 32) of shared gate row 2w (wave 4), 2w+1
//           (wave 5), shared up row 2w (wave 6), 2w+1 (wave 7), with the
//           group's scale and bias;
//   sdn     words 2 (lane % 32), +1 of shared down row 8w + 2 (wave - 4) + lane / 32.
template <typename SB>
struct Ahead {
    uint4 router;
    float bias;
    uint4 sgu;
    SB sgu_s, sgu_b;
    uint2 sdn;
    SB sdn_s, sdn_b;
};

struct AheadOffsets {
    uint32_t router, bias, sgu_q, sgu_sb, sdn_q, sdn_sb;
};

template <typename SB>
__device__ __forceinline__ void read_ahead(const StackArgs& a, int l, int hw, const AheadOffsets& o, Ahead<SB>& r) {
    r.router = ld<uint4>(lay(a.router, a.router_stride, l), o.router);
    if (a.logit_bias) r.bias = ld<float>(lay(a.logit_bias, a.bias_stride, l), o.bias);
    if (a.I_shared > 0) {
        const QMatPtr& m = hw < 2 ? a.shared.gate : a.shared.up;
        const QMatStride& st = hw < 2 ? a.shared_stride.gate : a.shared_stride.up;
        r.sgu = ld<uint4>(lay(m.q, st.q, l), o.sgu_q);
        r.sgu_s = ld<SB>(lay(m.s, st.s, l), o.sgu_sb);
        r.sgu_b = ld<SB>(lay(m.b, st.b, l), o.sgu_sb);
        const QMatStride& sd = a.shared_stride.down;
        r.sdn = ld<uint2>(lay(a.shared.down.q, sd.q, l), o.sdn_q);
        r.sdn_s = ld<SB>(lay(a.shared.down.s, sd.s, l), o.sdn_sb);
        r.sdn_b = ld<SB>(lay(a.shared.down.b, sd.b, l), o.sdn_sb);
    }
}

// Publish the owned block of the stream of epoch ep_next (wave 0; lane c < 8
// holds column 8 w + c in xn): the block's 8 values in every lane, packed 3 to
// a word under the tag, in every copy.
__device__ void publish_x(const StackArgs& a, int w, int lane, unsigned ep_next, uint16_t xn) {
    uint32_t b[8];
#pragma unroll
    for (int c = 0; c < 8; c++) b[c] = (uint32_t)__shfl((int)xn, c);
    const unsigned long long tag = (unsigned long long)xtag(ep_next) << 48;
    const unsigned long long words[3] = {
        tag | ((unsigned long long)b[2] << 32) | ((unsigned long long)b[1] << 16) | b[0],
        tag | ((unsigned long long)b[5] << 32) | ((unsigned long long)b[4] << 16) | b[3],
        tag | ((unsigned long long)b[7] << 16) | b[6]};
    unsigned long long* dst = a.xpub + (size_t)(ep_next & 1) * kStackXCopies * kStackXWords + 3 * w;
    for (int i = lane; i < 3 * kStackXCopies; i += kWave) {
        const int q = i % 3, copy = i / 3;
        const unsigned long long word = q == 0 ? words[0] : q == 1 ? words[1] : words[2];
        if (8 * w < a.H)
            __hip_atomic_store(dst + (size_t)copy * kStackXWords + q, word, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Poll the n_words {epoch, float16 pair} words of one slot's h (the whole wave:
// 4 words per lane, all in flight at once) into LDS as pairs in nibble order,
// then form the low/high sums of every block (lane b: block b).  Returns false
// on timeout (then sets the error word).
__device__ bool poll_slot_h(const unsigned long long* src, int n_words, unsigned epoch, uint4* pairs, float2* sums,
                            int lane, bool failed, unsigned* ctl) {
    constexpr int kPer = kHWords / kWave;  // words per lane
    bool ok = true;
    unsigned long long val[kPer] = {};
    if (!failed) {
        for (long spins = 0;; spins++) {
            bool have = true;
#pragma unroll
            for (int t = 0; t < kPer; t++) val[t] = peek(src + min(kWave * t + lane, n_words - 1));
#pragma unroll
            for (int t = 0; t < kPer; t++) have = have && (unsigned)(val[t] >> 32) == epoch;
            if (__ballot(!have) == 0) break;
            if (spins > kSpinLimit) {
                if (lane == 0) flag_error(ctl);
                ok = false;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    _Float16* hh = reinterpret_cast<_Float16*>(pairs);
#pragma unroll
    for (int t = 0; t < kPer; t++) {
        const int wd = kWave * t + lane;
        if (wd < n_words) {
            const half2_t pr = as_half2((uint32_t)val[t]);
            const int c0 = 2 * wd, c1 = 2 * wd + 1;
            hh[(c0 >> 3) * 8 + slot_of_column(c0 & 7)] = pr.x;
            hh[(c1 >> 3) * 8 + slot_of_column(c1 & 7)] = pr.y;
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's values are in LDS
    if (lane * 4 < n_words) {
        const uint4 p = pairs[lane];
        const half2_t a = as_half2(p.x), b = as_half2(p.y), c = as_half2(p.z), d = as_half2(p.w);
        sums[lane] = make_float2(((float)a.x + (float)a.y) + ((float)c.x + (float)c.y),
                                 ((float)b.x + (float)b.y) + ((float)d.x + (float)d.y));
    }
    return ok;
}

template <typename SB>
__global__ __launch_bounds__(kThreads) void decode_stack_kernel(StackArgs a) {
    __shared__ StackShared sh;
    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = uniform(tid / kWave);
    const int w = blockIdx.x;
    const int H = a.H, I = a.I, E = a.E, k = a.top_k, L = a.L;
    const bool shared = a.I_shared > 0;
    const int n_slots = k + (shared ? 1 : 0);  // contributions per output column
    constexpr uint32_t kSB = sizeof(SB);
    // a plain load: stored by the previous call, which has ended
    const unsigned e0 = a.ctl[kCtlStEpoch];
    const bool holder = wave >= 4;  // waves 4-7 hold the read-ahead
    const int hw = wave - 4;        // their index 0..3
    const int u = tid - 4 * kWave;  // their thread index 0..255

    // this workgroup's units
    const int gu_per_slot = I / kGURows;
    const bool has_gu = w < k * gu_per_slot;
    const int gu_slot = min(w / gu_per_slot, k - 1), gu_i0 = (w % gu_per_slot) * kGURows;
    const bool owns = 8 * w < H;  // output columns [8 w, 8 w + 8)
    const int own0 = min(8 * w, H - 8);
    const bool has_sgu = shared && w < a.I_shared / 2;
    const int nblk = H / 8;
    const int chunks = H / 32;
    bool failed = false;

    // per-lane byte offsets, fixed for the whole call
    AheadOffsets ao{};
    {
        const int e = min(w, E - 1), c = min(u, nblk - 1);
        ao.router = (uint32_t)((e * H + 8 * c) * 2);
        ao.bias = (uint32_t)(e * 4);
        if (shared) {
            const int Is = a.I_shared;
            const int row = min(2 * w + (hw & 1), Is - 1), cc = min(lane, chunks - 1);
            ao.sgu_q = (uint32_t)(row * (H / 2) + cc * 16);
            ao.sgu_sb = (uint32_t)((row * (H / kGroup) + cc / 2) * kSB);
            const int drow = min(kWorkers * w + 2 * hw + lane / 32, H - 1), wd = min(2 * (lane % 32), I / 8 - 2);
            ao.sdn_q = (uint32_t)(drow * (I / 2) + wd * 4);
            ao.sdn_sb = (uint32_t)((drow * (I / kGroup) + wd / 8) * kSB);
        }
    }
    const int gchunk = min(lane, chunks - 1);
    const uint32_t off_gq = (uint32_t)(gchunk * 16), off_gsb = (uint32_t)((gchunk / 2) * kSB);
    const int ia = min(gu_i0 + 2 * wave, I - 2);  // this wave's two intermediate rows
    const int dgrp = lane % 8, dgrp_c = min(dgrp, I / kGroup - 1);
    const uint32_t off_dq = (uint32_t)((lane / 8) * (I / 2) + dgrp_c * 32);
    const uint32_t off_dsb = (uint32_t)(((lane / 8) * (I / kGroup) + dgrp_c) * kSB);
    const bool dmine = owns && wave < k && dgrp < I / kGroup;  // routed slot `wave`, row own0 + lane / 8

    Ahead<SB> ah{};
    if (holder) read_ahead<SB>(a, 0, hw, ao, ah);
    uint32_t mykey = 0;  // waves 0-3: the order key of expert tid's logit
    if (tid == 0) sh.ncand = 0;

    // the normalisation weight of each block of 8 columns, read ahead a layer
    // at a time by waves 0-3 (thread t: block t)
    const uint32_t off_norm = (uint32_t)(min(tid, nblk - 1) * 16);
    uint4 gam = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);  // bf16 ones
    if (tid < kPollThreads && a.norm_w) gam = ld<uint4>(lay(a.norm_w, a.norm_stride, 0), off_norm);
    // this thread's block of the stream entering the layer (waves 0-3)
    float xv[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};

    // the first layer's input
    if (tid < nblk) {
        const uint4 raw = reinterpret_cast<const uint4*>(a.x_in)[tid];
        const uint16_t* b = reinterpret_cast<const uint16_t*>(&raw);
#pragma unroll
        for (int i = 0; i < 8; i++) xv[i] = bf16_to_f32(b[i]);
        reinterpret_cast<uint4*>(sh.xb)[tid] = raw;
        if (a.layer_x && tid == w) reinterpret_cast<uint4*>(a.layer_x)[tid] = raw;
    }

    for (int l = 0; l < L; l++) {
        const unsigned ep = e0 + 1 + (unsigned)l;
        // this layer's halves of the exchange regions
        const size_t par = ep & 1;
        unsigned long long* logits_p = a.logits + par * (kStackLogitCopies * kMaxE);
        unsigned long long* sh_h_p = a.sh_h + par * (kStackSharedHCopies * kHWords);
        unsigned long long* rt_h_p = a.rt_h + par * (8 * kStackRoutedHCopies * kHWords);

        // ---- x of this layer: every block of the stream from this workgroup's
        // copy (waves 0-3, thread t: block t)
        if (l > 0) {
            if (tid < kPollThreads) {
                const unsigned long long* src =
                    a.xpub + (par * kStackXCopies + (size_t)(w % kStackXCopies)) * kStackXWords + 3 * tid;
                const unsigned tag = xtag(ep);
                const bool mine = tid < nblk;
                unsigned long long q0 = 0, q1 = 0, q2 = 0;
                for (long spins = 0;; spins++) {
                    bool have = true;
                    if (mine && !failed) {
                        q0 = peek(src);
                        q1 = peek(src + 1);
                        q2 = peek(src + 2);
                        have = (unsigned)(q0 >> 48) == tag && (unsigned)(q1 >> 48) == tag &&
                               (unsigned)(q2 >> 48) == tag;
                    }
                    if (__ballot(!have) == 0) break;
                    if (spins > kSpinLimit) {
                        if (lane == 0) flag_error(a.ctl);
                        failed = true;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                if (mine) {
                    const uint32_t nb[8] = {(uint32_t)(q0 & 0xFFFF), (uint32_t)((q0 >> 16) & 0xFFFF),
                                            (uint32_t)((q0 >> 32) & 0xFFFF), (uint32_t)(q1 & 0xFFFF),
                                            (uint32_t)((q1 >> 16) & 0xFFFF), (uint32_t)((q1 >> 32) & 0xFFFF),
                                            (uint32_t)(q2 & 0xFFFF), (uint32_t)((q2 >> 16) & 0xFFFF)};
#pragma unroll
                    for (int i = 0; i < 8; i++) xv[i] = __uint_as_float(nb[i] << 16);
                    reinterpret_cast<uint4*>(sh.xb)[tid] =
                        make_uint4(nb[0] | (nb[1] << 16), nb[2] | (nb[3] << 16), nb[4] | (nb[5] << 16),
                                   nb[6] | (nb[7] << 16));
                }
            }
        }
        // ---- the layer's input: the stream's RMS normalisation (waves 0-3)
        if (tid < kPollThreads) {
            float ss = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; i++) ss += xv[i] * xv[i];
            ss = group_sum(ss, kWave);
            if (lane == 0) sh.ssq[wave] = ss;
        }
        __syncthreads();  // B1: the stream and its sums of squares in LDS
        if (tid < nblk) {
            const float r = 1.0f / sqrtf(((sh.ssq[0] + sh.ssq[1]) + (sh.ssq[2] + sh.ssq[3])) / (float)H + kNormEps);
            const uint32_t gw[4] = {gam.x, gam.y, gam.z, gam.w};
            float v[8];
            uint16_t nb[8];
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const float g = __uint_as_float(i & 1 ? gw[i / 2] & 0xFFFF0000u : gw[i / 2] << 16);
                nb[i] = bf16_rne(xv[i] * r * g);
                v[i] = bf16_to_f32(nb[i]);
            }
            const uint4 raw = make_uint4(nb[0] | ((uint32_t)nb[1] << 16), nb[2] | ((uint32_t)nb[3] << 16),
                                         nb[4] | ((uint32_t)nb[5] << 16), nb[6] | ((uint32_t)nb[7] << 16));
            reinterpret_cast<uint4*>(sh.xn)[tid] = raw;
            block_pairs(v, sh.xp[tid], sh.xs[tid]);
            if (a.layer_in && tid == w) reinterpret_cast<uint4*>(a.layer_in + (size_t)l * H)[tid] = raw;
        }
        __syncthreads();  // the layer's input in LDS

        // ---- router logit of expert w and the shared expert's gate/up (waves 4-7)
        if (holder) {
            float p = 0.0f;
            if (w < E && u < nblk) {
                // bf16 pairs as words: the low half widens by a shift, the high
                // half by masking (exact, as bf16 -> float32 is)
                const uint4 xr = reinterpret_cast<const uint4*>(sh.xn)[u];
                const uint4 rr = ah.router;
                const uint32_t xw[4] = {xr.x, xr.y, xr.z, xr.w}, rw[4] = {rr.x, rr.y, rr.z, rr.w};
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    p += __uint_as_float(xw[i] << 16) * __uint_as_float(rw[i] << 16);
                    p += __uint_as_float(xw[i] & 0xFFFF0000u) * __uint_as_float(rw[i] & 0xFFFF0000u);
                }
            }
            p = group_sum(p, kWave);
            float q = 0.0f;
            if (has_sgu && lane < chunks) {
                float alo = 0.0f, ahi = 0.0f, lo = 0.0f, hi = 0.0f;
                const uint32_t qw[4] = {ah.sgu.x, ah.sgu.y, ah.sgu.z, ah.sgu.w};
#pragma unroll
                for (int m = 0; m < 4; m++) {
                    dot_word(qw[m], pairs_of(sh.xp[4 * lane + m]), alo, ahi);
                    const float2 sm = sh.xs[4 * lane + m];
                    lo += sm.x;
                    hi += sm.y;
                }
                q = affine(sb_to_f32<SB>(ah.sgu_s), sb_to_f32<SB>(ah.sgu_b), alo, ahi, lo, hi);
            }
            q = group_sum(q, kWave);
            if (lane == 0) {
                sh.red[hw] = p;
                sh.sred[hw] = q;
            }
        }
        __syncthreads();  // B2: partial sums in LDS
        if (wave == 4 && w < E) {  // lanes 0..7 publish one copy each of the logit
            const float lg = ((sh.red[0] + sh.red[1]) + (sh.red[2] + sh.red[3])) + (a.logit_bias ? ah.bias : 0.0f);
            if (lane < kStackLogitCopies) publish(logits_p + (size_t)lane * kMaxE + w, ep, __float_as_uint(lg));
        } else if (wave == 5 && has_sgu) {  // rows 2w, 2w+1 of the shared expert's h
            const half2_t hp = {(_Float16)(silu(sh.sred[0]) * sh.sred[2]), (_Float16)(silu(sh.sred[1]) * sh.sred[3])};
            if (lane < kStackSharedHCopies) publish(sh_h_p + (size_t)lane * kHWords + w, ep, as_u32(hp));
        }

        // ---- every logit of the layer (waves 0-3 poll one word each)
        if (tid < kMaxE) {
            const unsigned long long* src = logits_p + (size_t)(w % kStackLogitCopies) * kMaxE;
            const bool mine = tid < E;
            unsigned long long v = 0;
            for (long spins = 0;; spins++) {
                bool have = true;
                if (mine && !failed) {
                    v = peek(src + tid);
                    have = (unsigned)(v >> 32) == ep;
                }
                if (__ballot(!have) == 0) break;
                if (spins > kSpinLimit) {
                    if (lane == 0) flag_error(a.ctl);
                    failed = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            mykey = mine ? order_key(__uint_as_float((uint32_t)v)) : 0u;
            sh.keys[tid] = mykey;
            // the two largest keys of this wave's 64 (equal keys count apart)
            const uint32_t m1 = wave_max_u32(mykey);
            const int first = (int)__builtin_ctzll(__ballot(mykey == m1));
            const uint32_t m2 = wave_max_u32(lane == first ? 0u : mykey);
            if (lane == 0) sh.m2[wave] = m2;
        }
        __syncthreads();  // B3: keys in LDS
        // candidates of the top k: keys >= the least of the four waves' second
        // largest keys.  At least two keys of every wave reach it, so the k <= 8
        // largest are among the candidates, and no key below it ranks in the
        // top k.  (Fewer than 194 experts leave a wave with under two keys: then
        // every expert is a candidate.)
        if (tid < kMaxE) {
            const uint32_t lim = E >= 194 ? min(min(sh.m2[0], sh.m2[1]), min(sh.m2[2], sh.m2[3])) : 1u;
            if (mykey != 0u && mykey >= lim) {
                const int pos = atomicAdd(&sh.ncand, 1);
                if (pos < kWave) {
                    sh.ckey[pos] = mykey;
                    sh.cidx[pos] = tid;
                }
            }
        }
        __syncthreads();  // candidates in LDS

        // ---- top k: every workgroup selects for itself, from the same words
        if (wave == 0) {
            const int n = sh.ncand;
            if (n <= kWave) {
                // rank of each candidate: the candidates above it, and the equal
                // ones of lower expert index; every other key is below them all
                const uint32_t ck = lane < n ? sh.ckey[lane] : 0u;
                const int ce = lane < n ? sh.cidx[lane] : 0;
                int rank = 0;
                for (int j = 0; j < n; j++) {
                    const uint32_t kj = __builtin_amdgcn_readlane(ck, j);
                    const int ej = __builtin_amdgcn_readlane(ce, j);
                    rank += (kj > ck || (kj == ck && ej < ce)) ? 1 : 0;
                }
                if (lane < n && rank < k) {
                    sh.sel_e[rank] = ce;
                    sh.sel_key[rank] = ck;
                }
            } else {
                // many equal keys: the k-th largest key by a radix search, then
                // every key above it and the equal ones by ascending index
                uint32_t key[kMaxE / kWave];
#pragma unroll
                for (int i = 0; i < kMaxE / kWave; i++) key[i] = sh.keys[lane + kWave * i];
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
                        sh.tkey[pos] = key[i];
                        sh.tidx[pos] = lane + kWave * i;
                    }
                    base += __popcll(sel[i]);
                }
                if (lane < k) {
                    const uint32_t mk = sh.tkey[lane];
                    const int me = sh.tidx[lane];
                    int rank = 0;
                    for (int m = 0; m < k; m++) {
                        const uint32_t om = sh.tkey[m];
                        rank += (om > mk || (om == mk && sh.tidx[m] < me)) ? 1 : 0;
                    }
                    sh.sel_e[rank] = me;
                    sh.sel_key[rank] = mk;
                }
            }
            // weights: softmax of the kept logits, summed in rank order
            const uint32_t rk = lane < k ? sh.sel_key[lane] : 0u;
            const float top = key_float(__builtin_amdgcn_readlane(rk, 0));
            const float pr = expf(key_float(rk) - top);
            float z = 0.0f;
            for (int m = 0; m < k; m++) z += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pr), m));
            if (lane < k) sh.sel_w[lane] = pr / z;
            if (lane == 0) sh.ncand = 0;  // for the next layer (past several barriers)
        }
        __syncthreads();  // B4: the routing in LDS

        // ---- routed loads, gate/up rows first, then down rows
        const int ex_gu = uniform(sh.sel_e[gu_slot]), ex_dn = uniform(sh.sel_e[min(wave, k - 1)]);
        uint4 gq[4];
        SB gs[4], gb[4];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const QMatPtr& m = r < 2 ? a.experts.gate : a.experts.up;
            const QMatStride& st = r < 2 ? a.experts_stride.gate : a.experts_stride.up;
            const size_t row = (size_t)ex_gu * I + ia + (r & 1);
            gs[r] = ld<SB>(lay(m.s, st.s, l) + row * (H / kGroup) * kSB, off_gsb);
            gb[r] = ld<SB>(lay(m.b, st.b, l) + row * (H / kGroup) * kSB, off_gsb);
            gq[r] = ld<uint4>(lay(m.q, st.q, l) + row * (H / 2), off_gq);
        }
        __builtin_amdgcn_sched_barrier(0);  // the gate/up products wait for their loads only
        uint4 dq0, dq1;
        SB ds, db;
        {
            const size_t row0 = (size_t)ex_dn * H + own0;  // this wave's slot, the owned rows
            const QMatStride& st = a.experts_stride.down;
            ds = ld<SB>(lay(a.experts.down.s, st.s, l) + row0 * (I / kGroup) * kSB, off_dsb);
            db = ld<SB>(lay(a.experts.down.b, st.b, l) + row0 * (I / kGroup) * kSB, off_dsb);
            const char* qb = lay(a.experts.down.q, st.q, l) + row0 * (I / 2);
            dq0 = ld<uint4>(qb, off_dq);
            dq1 = ld<uint4>(qb, off_dq + 16);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (w == 0 && tid < k) {
            if (a.idx_out) a.idx_out[(size_t)l * k + tid] = sh.sel_e[tid];
            if (a.w_out) a.w_out[(size_t)l * k + tid] = sh.sel_w[tid];
        }

        // ---- routed gate/up: rows ia, ia + 1 of h per wave
        if (has_gu) {
            float acc4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (lane < chunks) {
                float lo = 0.0f, hi = 0.0f;
                Pairs8 px[4];
#pragma unroll
                for (int m = 0; m < 4; m++) {
                    px[m] = pairs_of(sh.xp[4 * lane + m]);
                    const float2 sm = sh.xs[4 * lane + m];
                    lo += sm.x;
                    hi += sm.y;
                }
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    float alo = 0.0f, ahi = 0.0f;
                    dot_word(gq[r].x, px[0], alo, ahi);
                    dot_word(gq[r].y, px[1], alo, ahi);
                    dot_word(gq[r].z, px[2], alo, ahi);
                    dot_word(gq[r].w, px[3], alo, ahi);
                    acc4[r] = affine(sb_to_f32<SB>(gs[r]), sb_to_f32<SB>(gb[r]), alo, ahi, lo, hi);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; r++) acc4[r] = group_sum(acc4[r], kWave);
            if (lane < kStackRoutedHCopies) {  // one copy per lane
                const half2_t hp = {(_Float16)(silu(acc4[0]) * acc4[2]), (_Float16)(silu(acc4[1]) * acc4[3])};
                publish(rt_h_p + ((size_t)gu_slot * kStackRoutedHCopies + lane) * kHWords + gu_i0 / 2 + wave, ep,
                        as_u32(hp));
            }
        }

        // ---- shared expert's down (waves 4-7: 2 rows each, 2 words per lane)
        if (shared && holder) {
            const bool ok = poll_h<2 * 32>(sh_h_p + (size_t)(w % kStackSharedHCopies) * kHWords, a.I_shared / 2, ep,
                                           sh.hsp, sh.hss, hw, lane, failed, a.ctl);
            failed = failed || !ok;
        }
        __syncthreads();  // shared h in LDS
        if (shared && holder) {
            const int row = kWorkers * w + 2 * hw + lane / 32, wd = 2 * (lane % 32);
            float y = 0.0f;
            if (row < H && wd < I / 8) {
                float alo = 0.0f, ahi = 0.0f;
                dot_word(ah.sdn.x, pairs_of(sh.hsp[wd]), alo, ahi);
                dot_word(ah.sdn.y, pairs_of(sh.hsp[wd + 1]), alo, ahi);
                const float2 s0 = sh.hss[wd], s1 = sh.hss[wd + 1];
                y = affine(sb_to_f32<SB>(ah.sdn_s), sb_to_f32<SB>(ah.sdn_b), alo, ahi, s0.x + s1.x, s0.y + s1.y);
            }
            y = group_sum(y, 32);
            if (lane % 32 == 0) sh.ycon[k][2 * hw + lane / 32] = y;
        }

        // ---- routed down: wave j polls slot j's h, then 8 rows x one group per lane
        if (owns && wave < k) {
            const bool ok = poll_slot_h(rt_h_p + ((size_t)wave * kStackRoutedHCopies + w % kStackRoutedHCopies) *
                                                     kHWords,
                                        I / 2, ep, sh.hrp[wave], sh.hrs[wave], lane, failed, a.ctl);
            failed = failed || !ok;
        }
        float y = 0.0f;
        if (dmine) {
            const uint32_t wv[8] = {dq0.x, dq0.y, dq0.z, dq0.w, dq1.x, dq1.y, dq1.z, dq1.w};
            float alo = 0.0f, ahi = 0.0f, lo = 0.0f, hi = 0.0f;
#pragma unroll
            for (int m = 0; m < 8; m++) {
                dot_word(wv[m], pairs_of(sh.hrp[wave][8 * dgrp + m]), alo, ahi);
                const float2 sm = sh.hrs[wave][8 * dgrp + m];
                lo += sm.x;
                hi += sm.y;
            }
            y = affine(sb_to_f32<SB>(ds), sb_to_f32<SB>(db), alo, ahi, lo, hi);
        }
        y = group_sum(y, 8);  // the row's groups: 8 lanes
        if (dgrp == 0 && wave < k) sh.ycon[wave][lane / 8] = sh.sel_w[wave] * y;
        // every poll and product of this layer is done: waves 4-7 read the next
        // layer's data-independent weights ahead; they land while this layer's
        // output completes
        __builtin_amdgcn_sched_barrier(0);
        if (holder) read_ahead<SB>(a, min(l + 1, L - 1), hw, ao, ah);
        if (tid < kPollThreads && a.norm_w) gam = ld<uint4>(lay(a.norm_w, a.norm_stride, min(l + 1, L - 1)), off_norm);
        __syncthreads();  // every contribution to the owned columns in LDS

        // ---- the owned columns of the layer's output and of the next stream
        // (wave 0, lane c < 8: column 8 w + c), summed in slot order
        if (wave == 0) {
            float o = 0.0f;
            uint16_t xn = 0;
            if (lane < 8 && owns) {
                for (int j = 0; j < n_slots; j++) o += sh.ycon[j][lane];
                xn = bf16_rne(bf16_to_f32(sh.xb[8 * w + lane]) + o);
                if (a.layer_out) a.layer_out[(size_t)l * H + 8 * w + lane] = o;
                if (l + 1 < L) {
                    if (a.layer_x) a.layer_x[(size_t)(l + 1) * H + 8 * w + lane] = xn;
                } else {
                    a.x_out[8 * w + lane] = xn;
                }
            }
            if (l + 1 < L) publish_x(a, w, lane, ep + 1, xn);
        }
    }

    // the last workgroup to finish resets the counters and records the epoch
    // of the last layer for the next call (two-level count, as in the
    // one-layer decode kernel)
    __syncthreads();
    if (tid == 0) {
        const unsigned g = blockIdx.x % kDoneGroups;
        const unsigned members = (gridDim.x - g + kDoneGroups - 1) / kDoneGroups;
        const unsigned groups = min(gridDim.x, (unsigned)kDoneGroups);
        bool last = false;
        const unsigned old = __hip_atomic_fetch_add(a.ctl + kCtlStGroupDone + 32 * g, 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        if (old == members - 1)
            last = __hip_atomic_fetch_add(a.ctl + kCtlStDone, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   groups - 1;
        if (last) {
            for (int gg = 0; gg < kDoneGroups; gg++)
                __hip_atomic_store(a.ctl + kCtlStGroupDone + 32 * gg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.ctl + kCtlStDone, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.ctl + kCtlStEpoch, e0 + (unsigned)L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

}  // namespace

int stack_resident_capacity() {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(
                                                                  &decode_stack_kernel<uint16_t>),
                                                     kThreads, 0) != hipSuccess)
        return 0;
    int per_cu_f = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_f, reinterpret_cast<const void*>(&decode_stack_kernel<float>),
                                                     kThreads, 0) != hipSuccess)
        return 0;
    return cus * min(per_cu, per_cu_f);
}

hipError_t launch_decode_stack(const StackArgs& a, bool sb_bf16, hipStream_t stream) {
    if (sb_bf16)
        hipLaunchKernelGGL(decode_stack_kernel<uint16_t>, dim3(kStackGrid), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(decode_stack_kernel<float>, dim3(kStackGrid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace bitmoe
