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
// What one layer needs at T = 1 is a chain: x -> its normalisation -> router
// logits -> top-k -> the k experts' gate/up -> their down -> x of the next
// layer.  Only the k routed experts' weights (14 MB at the Qwen shapes) depend
// on the data; the router (1 MiB) and the shared expert (1.8 MB) do not, so
// they are read ahead of the layer that uses them.  Each link of the chain is a
// hand-over between workgroups, and its cost is a round trip to wherever the
// two workgroups share memory: the L2 of their XCD (~0.4 us for an all-gather
// among an XCD's 32 workgroups), or, across XCDs, the memory side of the
// fabric (~1-2 us).  So the layer is laid out along the device's XCDs:
//
//   - the grid is kStackGrid workgroups of 8 waves, one per compute unit, all
//     resident at once (the host checks the device can hold them), and every
//     wait is bounded.  Each workgroup reads the id of the XCD it runs on from
//     the hardware and takes an index j among that XCD's 32 workgroups;
//   - every XCD carries the layer up to the routed experts on its own: its 32
//     workgroups score all E experts (workgroup j experts 8 j .. 8 j + 7, from
//     router rows read ahead), read all E logits from their XCD's L2, and each
//     selects the top k itself.  The XCDs compute the same logits with the same
//     arithmetic, so they select the same experts;
//   - XCD x computes routed slot x (k <= 8 slots for 8 XCDs): workgroup j the
//     16 intermediate rows [16 j, 16 j + 16) of the slot's gate/up, published
//     in the XCD's L2; then every workgroup reads the slot's whole h and
//     computes its 64 owned output columns [64 j, 64 j + 64) of the slot's
//     down.  The shared expert is cut along its intermediate dimension: XCD x
//     takes rows [x I_s / 8, (x + 1) I_s / 8), gate/up and the matching slice of
//     down, so every XCD adds one eighth of it;
//   - the one hand-over across XCDs: workgroup j of XCD x publishes its partial
//     sum p_x = w_x y_x + y_shared,x for its 64 columns, and reads the 8 XCDs'
//     partials of the same columns.  Every XCD adds them in XCD order, so the
//     next stream x(l+1) = bf16(x(l) + sum_x p_x) is the same bits in every XCD,
//     and each XCD gathers it from its own L2;
//   - values handed within an XCD are stored with workgroup-scope stores, which
//     pass through the compute unit's write-through L1 into the XCD's L2, and
//     read with agent-scope loads, which miss the L1 and are served by the L2
//     line the store wrote (lines no other XCD touches).  Values crossing XCDs
//     are stored and read with agent-scope accesses, which write through to and
//     read from the memory side.  Each value carries its epoch, so a reader
//     waits for the value itself, with no flags or counters;
//   - every exchange region is kept twice, by the parity of the layer's epoch:
//     a workgroup can run at most one layer ahead of any other (each layer's
//     logits come from all 32 workgroups of its XCD, and its output from the
//     same workgroup index in all 8 XCDs), so a word is never rewritten while a
//     reader may still wait for its previous value.
//
// Loads of one wave complete in order (the vmcnt counter), so a poll waits
// behind every load its wave issued before.  Waves 0-3 do every poll but one
// (the shared expert's h, polled by wave 6 long after its read-ahead landed);
// waves 4-7 hold the read-ahead (router rows, the shared expert's slices, the
// logit bias and the normalisation weight, in registers) and issue the next
// layer's as soon as their gate/up products are done.
#include "common.h"
#include "decode_common.h"
#include "kernels.h"

namespace bitmoe {

namespace {

using namespace dec;

constexpr int kWorkers = 8;
constexpr int kThreads = kWorkers * kWave;
constexpr int kXcds = kStackXcds;
constexpr int kPerXcd = kStackGrid / kStackXcds;  // workgroups per XCD
constexpr int kGURows = 16;                       // routed gate/up rows of a workgroup: 2 per wave
constexpr int kOwn = 64;                          // output columns a workgroup owns: 8 per wave
constexpr int kLogitsPerWg = 8;                   // experts a workgroup scores: 2 per holding wave
constexpr long kSpinLimit = 1l << 20;
constexpr int kPollThreads = kStackMaxH / 8;  // threads that poll the stream, one 8-column block each
constexpr int kCopies = kStackLocalCopies;

// control words (uint32 indices) of the stack kernel inside the decode control block
constexpr int kCtlStEpoch = 2048;            // epoch of the last layer of the last call
constexpr int kCtlStDone = 2048 + 64;        // groups of workgroups finished in this call
constexpr int kCtlStGroupDone = 2048 + 128;  // + 32 g: workgroups of group g finished
constexpr int kCtlStClaim = 2048 + 512;      // + 32 x: workgroups that ever started on XCD x
constexpr int kDoneGroups = 8;

constexpr float kNormEps = 1e-6f;  // epsilon of the stream's normalisation

struct StackShared {
    uint4 xp[kStackMaxH / 8];    // the layer's input as float16 pairs in nibble order, per 8 columns
    float2 xs[kStackMaxH / 8];   // low/high nibble sums of each 8 columns
    uint16_t xb[kStackMaxH];     // the residual stream entering the layer, bf16
    uint16_t xn[kStackMaxH];     // its normalisation, the layer's input, bf16
    float ssq[4];                // sums of squares of the stream, one per polling wave
    uint4 hsp[kStackMaxI / 64];  // the XCD's share of the shared expert's h, pairs per 8 values
    float2 hss[kStackMaxI / 64];
    uint4 hrp[kStackMaxI / 8];   // the XCD's routed slot's h, pairs per 8 values
    float2 hrs[kStackMaxI / 64];  // its even- and odd-column sums per 64-column group
    float yr[kOwn];              // the routed slot's rows of the owned columns
    float ysh[kOwn];             // the shared expert's share of the same rows
    float pp[kXcds][kOwn];       // every XCD's partial sums of the owned columns
    TopkShared tk;               // the top-k selection
    float sred[4];               // shared gate/up rows of this workgroup (gate 2j, 2j+1, up 2j, 2j+1)
    float sel_w[kMaxTopK];       // routing weights in rank order
    uint4 gam[kStackMaxH / 8];   // the layer's normalisation weight, per 8 columns
    unsigned xcd, idx;           // this workgroup's XCD and its index there
};

__device__ __forceinline__ uint16_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// LDS positions of 16-byte blocks, transposed so that the lanes of one read
// instruction touch consecutive blocks (no bank conflicts): the layer's input
// (block 4 l + i, read by lane l as its i-th block, at i * 64 + l) and the
// routed h (block 8 g + m, read by the lanes of group g as their m-th block,
// at m * 8 + g)
__device__ __forceinline__ int xpos(int b) { return (b & 3) * (kStackMaxH / 32) + (b >> 2); }
__device__ __forceinline__ int hpos(int b) { return (b & 7) * (kStackMaxI / 64) + (b >> 3); }

// tag of the stream words of epoch ep: 16 bits, never 0 (a zero-filled workspace's)
__device__ __forceinline__ unsigned xtag(unsigned ep) { return ep % 65535u + 1u; }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// c + a.lo b.lo + a.hi b.hi over bf16 pairs (v_dot2_f32_bf16)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// the XCD this wave runs on (hardware register)
__device__ __forceinline__ unsigned xcc_id() {
    unsigned v;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
    return v & 0xFu;
}

// an {epoch, value} word (or a tagged stream word) for the workgroups of this
// XCD: a workgroup-scope store, through the write-through L1 into the XCD's L2
__device__ __forceinline__ void put_local(unsigned long long* p, unsigned long long v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

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
// place the values in LDS as pairs in nibble order.  Then the low/high sums
// that dot_word's exponent-trick codes need: the sums of the even and of the
// odd columns (the two values of a word).  With kT (the routed h, n = 64) they
// are formed per 64-column group by DPP sums over the words the wave holds
// (group 2v in lanes 0..31, group 2v + 1 in lanes 32..63) and sums[g] is group
// g's; otherwise lanes 0..n/4-1 form them per block of 8 columns.  Returns false
// on timeout (then sets the error word).
template <int kPer, bool kT>
__device__ bool poll_h(const unsigned long long* src, int n_words, unsigned epoch, uint4* pairs, float2* sums,
                       int v, int lane, bool failed, unsigned* ctl) {
    auto pos = [](int b) { return kT ? hpos(b) : b; };
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
    float ev = 0.0f, od = 0.0f;
    if (mine) {
        const half2_t pr = as_half2((uint32_t)val);
        const int c0 = 2 * wd, c1 = 2 * wd + 1;
        hh[pos(c0 >> 3) * 8 + slot_of_column(c0 & 7)] = pr.x;
        hh[pos(c1 >> 3) * 8 + slot_of_column(c1 & 7)] = pr.y;
        ev = (float)pr.x;
        od = (float)pr.y;
    }
    if constexpr (kT) {
        static_assert(kPer == kWave, "one word per lane of the whole wave");
        ev += dpp<0xB1>(ev);  // quad_perm 1,0,3,2
        od += dpp<0xB1>(od);
        ev += dpp<0x4E>(ev);  // quad_perm 2,3,0,1
        od += dpp<0x4E>(od);
        ev += dpp<0x141>(ev);  // row_half_mirror
        od += dpp<0x141>(od);
        ev += dpp<0x140>(ev);  // row_mirror
        od += dpp<0x140>(od);
        // the row totals are read by the whole wave: under a one-lane branch the
        // compiler may finish the sums in that lane only
        auto at = [](float f, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), l)); };
        const float2 g0 = make_float2(at(ev, 0) + at(ev, 16), at(od, 0) + at(od, 16));
        const float2 g1 = make_float2(at(ev, 32) + at(ev, 48), at(od, 32) + at(od, 48));
        if (lane == 0) {
            sums[2 * v] = g0;
            sums[2 * v + 1] = g1;
        }
        return ok;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's values are in LDS
    const int blk = (kPer / 4) * v + lane;
    if (lane < kPer / 4 && blk * 4 < n_words) {
        const uint4 p = pairs[pos(blk)];
        const half2_t a = as_half2(p.x), b = as_half2(p.y), c = as_half2(p.z), d = as_half2(p.w);
        sums[pos(blk)] = make_float2(((float)a.x + (float)a.y) + ((float)c.x + (float)c.y),
                                ((float)b.x + (float)b.y) + ((float)d.x + (float)d.y));
    }
    return ok;
}

// s * (sum of code * a over a word or words) + b * (sum of a), from the
// exponent-trick partial sums of dot_word
__device__ __forceinline__ float affine(float s, float b, float alo, float ahi, float lo, float hi) {
    return s * ((alo - 1024.0f * lo) + (ahi - 64.0f * hi)) + b * (lo + hi);
}

// Addressing.  Every load of the loop takes a base address that is uniform over
// the wave (kernel arguments, the layer, the expert: kept in scalar registers)
// plus a per-lane byte offset computed once before the loop.  The loop then
// writes no vector register that a memory operation in flight still reads as
// its address, which would make the compiler wait for that operation to
// complete.  Every load is issued whatever the shape (indices clamped into the
// tensors), so that each wave's count of loads in flight is the same on every
// path and the compiler's waits stay exact.
__device__ __forceinline__ const char* lay(const void* p, int64_t stride, int l) {
    return reinterpret_cast<const char*>(p) + stride * (int64_t)l;
}
template <typename T>
__device__ __forceinline__ T ld(const char* base, uint32_t off) {
    return *reinterpret_cast<const T*>(base + off);
}
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Read-ahead of one layer's data-independent weights, held in the registers of
// waves 4-7 until the layer runs.  Thread u = tid - 256 of those waves (lane,
// hw = wave - 4) holds:
//   rt      8-column blocks [4 lane, 4 lane + 4) of the router rows of experts
//           8 j + 2 hw and 8 j + 2 hw + 1;
//   bias    the logit bias of expert 8 j + 2 hw + lane % 2;
//   sgu     columns [32 lane, 32 lane + 32) of the XCD's shared gate row 2 j
//           (hw 0), 2 j + 1 (hw 1), shared up row 2 j (hw 2), 2 j + 1 (hw 3),
//           with the group's scale and bias;
//   sdn     words 2 (u % 4), +1 of owned column 64 j + u / 4 of the shared down
//           rows over the XCD's intermediate slice, with its scale and bias;
//   gam     the normalisation weight of 8-column block u.
template <typename SB>
struct Ahead {
    uint4 rt[2][4];
    float bias;
    uint4 sgu;
    SB sgu_s, sgu_b;
    uint32_t sdn0, sdn1;
    SB sdn_s, sdn_b;
    uint4 gam;
};

struct AheadOffsets {
    uint32_t rt0, rt1, bias, sgu_q, sgu_sb, sdn_q0, sdn_q1, sdn_sb, gam;
};

template <typename SB>
__device__ __forceinline__ void read_ahead(const StackArgs& a, int l, int hw, const AheadOffsets& o, Ahead<SB>& r) {
    // every load is issued on every path (an absent tensor is replaced by one
    // that exists, its value unused), so that the waves' counts of loads in
    // flight, and the compiler's waits on them, do not depend on the shape
    const bool shared = a.I_shared > 0;
    const char* rb = lay(a.router, a.router_stride, l);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        r.rt[0][i] = ld<uint4>(rb, o.rt0 + 16 * i);
        r.rt[1][i] = ld<uint4>(rb, o.rt1 + 16 * i);
    }
    r.bias = a.logit_bias ? ld<float>(lay(a.logit_bias, a.bias_stride, l), o.bias) : ld<float>(rb, o.bias);
    r.gam = a.norm_w ? ld<uint4>(lay(a.norm_w, a.norm_stride, l), o.gam) : ld<uint4>(rb, o.gam);
    const QMatPtr& m = shared ? (hw < 2 ? a.shared.gate : a.shared.up) : a.experts.gate;
    const QMatStride& st = shared ? (hw < 2 ? a.shared_stride.gate : a.shared_stride.up) : a.experts_stride.gate;
    r.sgu = ld<uint4>(lay(m.q, st.q, l), o.sgu_q);
    r.sgu_s = ld<SB>(lay(m.s, st.s, l), o.sgu_sb);
    r.sgu_b = ld<SB>(lay(m.b, st.b, l), o.sgu_sb);
    const QMatPtr& d = shared ? a.shared.down : a.experts.down;
    const QMatStride& sd = shared ? a.shared_stride.down : a.experts_stride.down;
    const char* dq = lay(d.q, sd.q, l);
    r.sdn0 = ld<uint32_t>(dq, o.sdn_q0);
    r.sdn1 = ld<uint32_t>(dq, o.sdn_q1);
    r.sdn_s = ld<SB>(lay(d.s, sd.s, l), o.sdn_sb);
    r.sdn_b = ld<SB>(lay(d.b, sd.b, l), o.sdn_sb);
}

template <typename SB>
__global__ __launch_bounds__(kThreads) void decode_stack_kernel(StackArgs a) {
    __shared__ StackShared sh;
    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = uniform(tid / kWave);
    const int H = a.H, I = a.I, E = a.E, k = a.top_k, L = a.L;
    const bool shared = a.I_shared > 0;
    constexpr uint32_t kSB = sizeof(SB);
    // a plain load: stored by the previous call, which has ended
    const unsigned e0 = a.ctl[kCtlStEpoch];
    const bool holder = wave >= 4;  // waves 4-7 hold the read-ahead
    const int hw = wave - 4;        // their index 0..3
    const int u = tid - 4 * kWave;  // their thread index 0..255

    // this workgroup's XCD x and its index j among the XCD's workgroups (each
    // call starts kPerXcd workgroups on every XCD, which count themselves)
    if (tid == 0) {
        const unsigned xc = xcc_id();
        unsigned idx = 0;
        if (xc < (unsigned)kXcds)
            idx = __hip_atomic_fetch_add(a.ctl + kCtlStClaim + 32 * xc, 1u, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT) % (unsigned)kPerXcd;
        else
            flag_error(a.ctl);
        sh.xcd = xc;
        sh.idx = idx;
    }
    __syncthreads();
    bool failed = sh.xcd >= (unsigned)kXcds;
    const int x = uniform((int)min(sh.xcd, (unsigned)kXcds - 1)), j = uniform((int)sh.idx);

    // this workgroup's units
    const int nblk = H / 8, chunks = H / 32;
    const int Ix = a.I_shared / kXcds;          // the XCD's share of the shared expert's rows
    const bool has_slot = x < k;                // XCD x computes routed slot x
    const bool has_gu = has_slot && kGURows * j < I;
    const int ia = min(kGURows * j + 2 * wave, I - 2);  // this wave's two intermediate rows
    const bool owns = kOwn * j < H;             // output columns [64 j, 64 j + 64)
    const int own0 = min(kOwn * j, H - kOwn);
    const bool has_sgu = shared && 2 * j < Ix;  // shared rows x Ix + 2 j, + 1
    const int sgrow = x * Ix + min(2 * j, max(Ix - 2, 0));
    const bool zero_rank = x == 0 && j == 0;    // writes the routing outputs
    const bool recorder = x == 0;               // XCD 0 writes the per-layer outputs

    // per-lane byte offsets, fixed for the whole call
    AheadOffsets ao{};
    {
        const int e0r = min(kLogitsPerWg * j + 2 * hw, E - 1), e1r = min(kLogitsPerWg * j + 2 * hw + 1, E - 1);
        const int rb = min(4 * lane, nblk - 4);
        ao.rt0 = (uint32_t)((e0r * H + 8 * rb) * 2);
        ao.rt1 = (uint32_t)((e1r * H + 8 * rb) * 2);
        ao.bias = (uint32_t)(min(kLogitsPerWg * j + 2 * hw + (lane & 1), E - 1) * 4);
        ao.gam = (uint32_t)(min(u, nblk - 1) * 16);
        if (shared) {
            const int Is = a.I_shared;
            const int row = min(sgrow + (hw & 1), Is - 1), cc = min(lane, chunks - 1);
            ao.sgu_q = (uint32_t)(row * (H / 2) + cc * 16);
            ao.sgu_sb = (uint32_t)((row * (H / kGroup) + cc / 2) * kSB);
            // shared down: row (output column) own0 + u / 4, words 2 (u % 4), +1
            // of the slice [x Ix, x Ix + Ix) of its Is values (Ix / 8 words)
            const int drow = own0 + u / 4, wpr = Ix / 8;
            const int w0 = min(2 * (u % 4), wpr - 1), w1 = min(2 * (u % 4) + 1, wpr - 1);
            ao.sdn_q0 = (uint32_t)(drow * (Is / 2) + (x * Ix) / 2 + 4 * w0);
            ao.sdn_q1 = (uint32_t)(drow * (Is / 2) + (x * Ix) / 2 + 4 * w1);
            ao.sdn_sb = (uint32_t)((drow * (Is / kGroup) + (x * Ix) / kGroup) * kSB);
        }
    }
    const bool rt_mine = 4 * lane < nblk;  // the router blocks this lane holds are real
    const int gchunk = min(lane, chunks - 1);
    const uint32_t off_gq = (uint32_t)(gchunk * 16), off_gsb = (uint32_t)((gchunk / 2) * kSB);
    const int dgrp = lane % 8, dgrp_c = min(dgrp, I / kGroup - 1);
    const uint32_t off_dq = (uint32_t)((lane / 8) * (I / 2) + dgrp_c * 32);
    const uint32_t off_dsb = (uint32_t)(((lane / 8) * (I / kGroup) + dgrp_c) * kSB);
    const bool dmine = owns && has_slot && dgrp < I / kGroup;  // row own0 + 8 wave + lane / 8, group dgrp
    const bool sdmine = shared && owns && 2 * (u % 4) < Ix / 8;  // (waves 4-7) the first of the two words
    const bool sdmine1 = shared && owns && 2 * (u % 4) + 1 < Ix / 8;

    Ahead<SB> ah{};
    if (holder) read_ahead<SB>(a, 0, hw, ao, ah);

    // this thread's block of the stream entering the layer (waves 0-3)
    float xv[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    if (tid < nblk) {
        const uint4 raw = reinterpret_cast<const uint4*>(a.x_in)[tid];
        const uint16_t* b = reinterpret_cast<const uint16_t*>(&raw);
#pragma unroll
        for (int i = 0; i < 8; i++) xv[i] = bf16_to_f32(b[i]);
        reinterpret_cast<uint4*>(sh.xb)[tid] = raw;
        if (a.layer_x && recorder && tid / 8 == j) reinterpret_cast<uint4*>(a.layer_x)[tid] = raw;
    }
    uint32_t mykey = 0;  // waves 0-3: the order key of expert tid's logit

    for (int l = 0; l < L; l++) {
        const unsigned ep = e0 + 1 + (unsigned)l;
        const size_t par = ep & 1;
        // this layer's halves of the exchange regions
        unsigned long long* loc_x = a.local + ((size_t)x * 2 + par) * kStackLocWords;
        unsigned long long* loc_logits = loc_x + (size_t)kCopies * kStackXWords;
        unsigned long long* loc_h = loc_logits + (size_t)kCopies * kMaxE;
        unsigned long long* loc_sh = loc_h + (size_t)kCopies * (kStackMaxI / 2);
        unsigned long long* part = a.part + par * ((size_t)kStackGrid * kOwn);

        // ---- x of this layer: every block of the stream from this XCD's copy
        // (waves 0-3, thread t: block t)
        if (l > 0 && tid < kPollThreads) {
            const unsigned long long* src = loc_x + (size_t)(j % kCopies) * kStackXWords + 3 * tid;
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
                reinterpret_cast<uint4*>(sh.xb)[tid] = make_uint4(nb[0] | (nb[1] << 16), nb[2] | (nb[3] << 16),
                                                                  nb[4] | (nb[5] << 16), nb[6] | (nb[7] << 16));
            }
        }
        // ---- the layer's normalisation weight, read ahead (waves 4-7)
        if (holder && u < nblk) sh.gam[u] = a.norm_w ? ah.gam : make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
        // ---- the stream's sum of squares (waves 0-3)
        if (tid < kPollThreads) {
            float ss = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; i++) ss += xv[i] * xv[i];
            ss = wave_total(ss);
            if (lane == 0) sh.ssq[wave] = ss;
        }
        __syncthreads();  // B1: the stream and its sums of squares in LDS

        // ---- the layer's input: the stream's RMS normalisation (waves 0-3, thread t: block t)
        if (tid < nblk) {
            const float r = 1.0f / sqrtf(((sh.ssq[0] + sh.ssq[1]) + (sh.ssq[2] + sh.ssq[3])) / (float)H + kNormEps);
            const uint4 gm = sh.gam[tid];
            const uint32_t gw[4] = {gm.x, gm.y, gm.z, gm.w};
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
            reinterpret_cast<uint4*>(sh.xn)[xpos(tid)] = raw;
            block_pairs(v, sh.xp[xpos(tid)], sh.xs[xpos(tid)]);
            if (a.layer_in && recorder && tid / 8 == j) reinterpret_cast<uint4*>(a.layer_in + (size_t)l * H)[tid] = raw;
        }
        __syncthreads();  // the layer's input in LDS

        // ---- router logits of experts 8 j + 2 hw, + 1 and the shared gate/up (waves 4-7)
        if (holder) {
            // two partial sums per row (blocks 4 lane, +2 and 4 lane + 1, +3), bf16
            // pairs against bf16 pairs
            float p0a = 0.0f, p0b = 0.0f, p1a = 0.0f, p1b = 0.0f;
            if (rt_mine) {
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const uint4 xr = reinterpret_cast<const uint4*>(sh.xn)[xpos(4 * lane + i)];
                    const uint32_t xw[4] = {xr.x, xr.y, xr.z, xr.w};
                    const uint32_t r0[4] = {ah.rt[0][i].x, ah.rt[0][i].y, ah.rt[0][i].z, ah.rt[0][i].w};
                    const uint32_t r1[4] = {ah.rt[1][i].x, ah.rt[1][i].y, ah.rt[1][i].z, ah.rt[1][i].w};
#pragma unroll
                    for (int m = 0; m < 4; m++) {
                        if (i & 1) {
                            p0b = dot2_bf16(xw[m], r0[m], p0b);
                            p1b = dot2_bf16(xw[m], r1[m], p1b);
                        } else {
                            p0a = dot2_bf16(xw[m], r0[m], p0a);
                            p1a = dot2_bf16(xw[m], r1[m], p1a);
                        }
                    }
                }
            }
            const float p0 = wave_total(p0a + p0b), p1 = wave_total(p1a + p1b);
            // lane: expert 8 j + 2 hw + lane % 2, copy lane / 2
            {
                const int e = kLogitsPerWg * j + 2 * hw + (lane & 1);
                if (lane < 2 * kCopies && e < E) {
                    const float lg = ((lane & 1) ? p1 : p0) + (a.logit_bias ? ah.bias : 0.0f);
                    put_local(loc_logits + (size_t)(lane / 2) * kMaxE + e,
                              ((unsigned long long)ep << 32) | __float_as_uint(lg));
                }
            }
            float q = 0.0f;
            if (has_sgu && lane < chunks) {
                float alo = 0.0f, ahi = 0.0f, lo = 0.0f, hi = 0.0f;
                const uint32_t qw[4] = {ah.sgu.x, ah.sgu.y, ah.sgu.z, ah.sgu.w};
#pragma unroll
                for (int m = 0; m < 4; m++) {
                    dot_word(qw[m], pairs_of(sh.xp[xpos(4 * lane + m)]), alo, ahi);
                    const float2 sm = sh.xs[xpos(4 * lane + m)];
                    lo += sm.x;
                    hi += sm.y;
                }
                q = affine(sb_to_f32<SB>(ah.sgu_s), sb_to_f32<SB>(ah.sgu_b), alo, ahi, lo, hi);
            }
            q = wave_total(q);
            if (lane == 0) sh.sred[hw] = q;
        }
        __syncthreads();  // B2: this workgroup's shared gate/up rows in LDS
        if (wave == 5 && has_sgu) {  // shared rows x Ix + 2 j, + 1 of h
            const half2_t hp = {(_Float16)(silu(sh.sred[0]) * sh.sred[2]), (_Float16)(silu(sh.sred[1]) * sh.sred[3])};
            if (lane < kCopies)
                put_local(loc_sh + (size_t)lane * kStackShWords + j, ((unsigned long long)ep << 32) | as_u32(hp));
        }

        // ---- every logit of the layer (waves 0-3 poll one word each) and the
        // XCD's share of the shared expert's h (wave 6)
        if (tid < kMaxE) {
            const unsigned long long* src = loc_logits + (size_t)(j % kCopies) * kMaxE;
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
            topk_keys(sh.tk, mykey, tid, lane, wave);
        } else if (wave == 6 && shared) {
            const bool ok = poll_h<kStackShWords, false>(loc_sh + (size_t)(j % kCopies) * kStackShWords, Ix / 2, ep, sh.hsp,
                                                  sh.hss, 0, lane, failed, a.ctl);
            failed = failed || !ok;
        }
        __syncthreads();  // B3: keys and the shared share's h in LDS
        // ---- top k: every workgroup selects for itself, from the same words
        if (tid < kMaxE) topk_candidates(sh.tk, mykey, E, tid, lane, wave);
        __syncthreads();  // candidates in LDS
        topk_rank(sh.tk, k, tid, lane, wave);
        __syncthreads();  // B4: the routing in LDS

        // ---- routed loads of the XCD's slot: gate/up rows first, then down rows
        const int ex = uniform(sh.tk.sel_e[min(x, k - 1)]);
        uint4 gq[4];
        SB gs[4], gb[4];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const QMatPtr& m = r < 2 ? a.experts.gate : a.experts.up;
            const QMatStride& st = r < 2 ? a.experts_stride.gate : a.experts_stride.up;
            const size_t row = (size_t)ex * I + ia + (r & 1);
            gs[r] = ld<SB>(lay(m.s, st.s, l) + row * (H / kGroup) * kSB, off_gsb);
            gb[r] = ld<SB>(lay(m.b, st.b, l) + row * (H / kGroup) * kSB, off_gsb);
            gq[r] = ld<uint4>(lay(m.q, st.q, l) + row * (H / 2), off_gq);
        }
        __builtin_amdgcn_sched_barrier(0);  // the gate/up products wait for their loads only
        // every wave's gate/up loads go out before any down load: the older
        // waves 0-3 would otherwise issue their down rows ahead of the gate/up
        // rows of waves 4-7, whose h then comes last (10.48 against 10.64 us)
        __syncthreads();
        uint4 dq0, dq1;
        SB ds, db;
        {
            const size_t row0 = (size_t)ex * H + own0 + 8 * wave;  // this wave's 8 owned rows
            const QMatStride& st = a.experts_stride.down;
            ds = ld<SB>(lay(a.experts.down.s, st.s, l) + row0 * (I / kGroup) * kSB, off_dsb);
            db = ld<SB>(lay(a.experts.down.b, st.b, l) + row0 * (I / kGroup) * kSB, off_dsb);
            const char* qb = lay(a.experts.down.q, st.q, l) + row0 * (I / 2);
            dq0 = ld<uint4>(qb, off_dq);
            dq1 = ld<uint4>(qb, off_dq + 16);
        }
        __builtin_amdgcn_sched_barrier(0);
        // ---- the shared expert's share of the owned columns (waves 4-7, while
        // their routed loads are in flight; its weights were read ahead during
        // the previous layer and are replaced by the next layer's after the gate/up)
        if (holder && shared && owns) {
            float alo = 0.0f, ahi = 0.0f, lo = 0.0f, hi = 0.0f;
            const int w0 = 2 * (u % 4);
            if (sdmine) {
                dot_word(ah.sdn0, pairs_of(sh.hsp[w0]), alo, ahi);
                const float2 s0 = sh.hss[w0];
                lo += s0.x;
                hi += s0.y;
            }
            if (sdmine1) {
                dot_word(ah.sdn1, pairs_of(sh.hsp[w0 + 1]), alo, ahi);
                const float2 s1 = sh.hss[w0 + 1];
                lo += s1.x;
                hi += s1.y;
            }
            float y = sdmine ? affine(sb_to_f32<SB>(ah.sdn_s), sb_to_f32<SB>(ah.sdn_b), alo, ahi, lo, hi) : 0.0f;
            y = group_sum(y, 4);  // the row's 4 threads
            if (u % 4 == 0) sh.ysh[u / 4] = y;
        }

        // ---- routed gate/up: rows ia, ia + 1 of the slot's h per wave
        if (has_gu) {
            float acc4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (lane < chunks) {
                float lo = 0.0f, hi = 0.0f;
                Pairs8 px[4];
#pragma unroll
                for (int m = 0; m < 4; m++) {
                    px[m] = pairs_of(sh.xp[xpos(4 * lane + m)]);
                    const float2 sm = sh.xs[xpos(4 * lane + m)];
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
            for (int r = 0; r < 4; r++) acc4[r] = wave_total(acc4[r]);
            if (lane < kCopies) {  // one copy per lane
                const half2_t hp = {(_Float16)(silu(acc4[0]) * acc4[2]), (_Float16)(silu(acc4[1]) * acc4[3])};
                put_local(loc_h + (size_t)lane * (kStackMaxI / 2) + ia / 2, ((unsigned long long)ep << 32) | as_u32(hp));
            }
        }
        // ---- the routing weights: softmax of the kept logits, summed in rank
        // order (wave 0; used from the down on)
        if (wave == 0) {
            const float wr = topk_weight_of_lane(sh.tk, k, lane);
            if (lane < k) sh.sel_w[lane] = wr;
            if (zero_rank && lane < k) {
                if (a.idx_out) a.idx_out[(size_t)l * k + lane] = sh.tk.sel_e[lane];
                if (a.w_out) a.w_out[(size_t)l * k + lane] = wr;
            }
        }
        // every poll of this layer by waves 4-7 is done: they read the next
        // layer's data-independent weights ahead; the loads land while this
        // layer's down and output hand-over complete
        __builtin_amdgcn_sched_barrier(0);
        if (holder) read_ahead<SB>(a, min(l + 1, L - 1), hw, ao, ah);
        __builtin_amdgcn_sched_barrier(0);

        // ---- the slot's whole h (waves 0-3: 64 words each)
        if (has_slot && owns && wave < 4) {
            const bool ok = poll_h<kWave, true>(loc_h + (size_t)(j % kCopies) * (kStackMaxI / 2), I / 2, ep, sh.hrp, sh.hrs,
                                          wave, lane, failed, a.ctl);
            failed = failed || !ok;
        }
        __syncthreads();  // the slot's h in LDS

        // ---- the routed slot's down for the owned columns: 8 rows per wave, one
        // 64-value group per lane
        if (has_slot && owns) {
            float y = 0.0f;
            if (dmine) {
                const uint32_t wv[8] = {dq0.x, dq0.y, dq0.z, dq0.w, dq1.x, dq1.y, dq1.z, dq1.w};
                // the group's 8 blocks of h and its sums, read together
                uint4 hv[8];
#pragma unroll
                for (int m = 0; m < 8; m++) hv[m] = sh.hrp[hpos(8 * dgrp + m)];
                const float2 gs = sh.hrs[dgrp];
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                float alo0 = 0.0f, ahi0 = 0.0f, alo1 = 0.0f, ahi1 = 0.0f;
#pragma unroll
                for (int m = 0; m < 8; m += 2) {
                    dot_word(wv[m], pairs_of(hv[m]), alo0, ahi0);
                    dot_word(wv[m + 1], pairs_of(hv[m + 1]), alo1, ahi1);
                }
                y = affine(sb_to_f32<SB>(ds), sb_to_f32<SB>(db), alo0 + alo1, ahi0 + ahi1, gs.x, gs.y);
            }
            y = group_sum(y, 8);  // the row's groups: 8 lanes
            if (dgrp == 0) sh.yr[8 * wave + lane / 8] = y;
        }
        __syncthreads();  // the owned rows of both products in LDS

        // ---- this XCD's partial sums of the owned columns, to the 8 workgroups
        // that own them (wave 0, lane c: column own0 + c)
        if (wave == 0 && owns) {
            const float pr = (has_slot ? sh.sel_w[x] * sh.yr[lane] : 0.0f) + (shared ? sh.ysh[lane] : 0.0f);
            publish(part + ((size_t)x * kPerXcd + j) * kOwn + lane, ep, __float_as_uint(pr));
        }
        // every XCD's partials of the owned columns (waves 0-3: XCDs 2 wave, + 1)
        if (owns && wave < 4) {
            const unsigned long long* s0 = part + ((size_t)(2 * wave) * kPerXcd + j) * kOwn + lane;
            const unsigned long long* s1 = s0 + (size_t)kPerXcd * kOwn;
            unsigned long long v0 = 0, v1 = 0;
            if (!failed) {
                for (long spins = 0;; spins++) {
                    v0 = peek(s0);
                    v1 = peek(s1);
                    const bool have = (unsigned)(v0 >> 32) == ep && (unsigned)(v1 >> 32) == ep;
                    if (__ballot(!have) == 0) break;
                    if (spins > kSpinLimit) {
                        if (lane == 0) flag_error(a.ctl);
                        failed = true;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
            }
            sh.pp[2 * wave][lane] = __uint_as_float((uint32_t)v0);
            sh.pp[2 * wave + 1][lane] = __uint_as_float((uint32_t)v1);
        }
        __syncthreads();  // every partial of the owned columns in LDS

        // ---- the owned columns of the layer's output and of the next stream
        // (wave 0, lane c: column own0 + c), summed in XCD order
        if (wave == 0 && owns) {
            float o = 0.0f;
#pragma unroll
            for (int xx = 0; xx < kXcds; xx++) o += sh.pp[xx][lane];
            const int col = own0 + lane;
            const uint16_t xn = bf16_rne(bf16_to_f32(sh.xb[col]) + o);
            if (recorder) {
                if (a.layer_out) a.layer_out[(size_t)l * H + col] = o;
                if (l + 1 < L) {
                    if (a.layer_x) a.layer_x[(size_t)(l + 1) * H + col] = xn;
                } else {
                    a.x_out[col] = xn;
                }
            }
            if (l + 1 < L) {
                // block lane / 8 of the owned columns: 3 tagged words, written by
                // lanes 8 b .. 8 b + 2 into every copy of the next layer's stream
                const int b = lane / 8, q = lane % 8;
                uint32_t v[8];
#pragma unroll
                for (int c = 0; c < 8; c++) v[c] = (uint32_t)__shfl((int)xn, 8 * b + c);
                const unsigned long long tag = (unsigned long long)xtag(ep + 1) << 48;
                const unsigned long long w0 =
                    tag | ((unsigned long long)v[2] << 32) | ((unsigned long long)v[1] << 16) | v[0];
                const unsigned long long w1 =
                    tag | ((unsigned long long)v[5] << 32) | ((unsigned long long)v[4] << 16) | v[3];
                const unsigned long long w2 = tag | ((unsigned long long)v[7] << 16) | v[6];
                const unsigned long long word = q == 0 ? w0 : q == 1 ? w1 : w2;
                if (q < 3) {
                    unsigned long long* nx = a.local + ((size_t)x * 2 + ((ep + 1) & 1)) * kStackLocWords;
                    const size_t wd = (size_t)3 * (own0 / 8 + b) + q;
#pragma unroll
                    for (int c = 0; c < kCopies; c++) put_local(nx + (size_t)c * kStackXWords + wd, word);
                }
            }
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
