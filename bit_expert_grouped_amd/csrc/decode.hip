// Decode path (a handful of tokens) for gfx950: ONE kernel per layer call, no
// host sync.
//
// Pages: decode reads the weights every step, so it is bound by memory
// bandwidth, not arithmetic; the engine treats it as a different workload from
// prefill and overlaps the dependent stages of a decode step (aimanavo.com page,
// section "Lily does not treat prefill and decode as the same job"); routing
// stays on the GPU (same section; dzen.guru page, section "Where does the
// speed-up come from?").
//
// At T <= kDecodeMaxT only ~9 of 257 experts are touched and every product is a
// matrix-vector product, so there is no MFMA here.  Two facts of the hardware
// shape the kernel: a compute unit sustains only a few tens of GB/s on its own
// (its outstanding misses times the ~1-2 us memory latency), so the ~17 MB of a
// step must be spread over every compute unit; and every hop between
// workgroups costs a memory round trip, so the chain router -> gate/up -> down
// has as few hops as possible and no arrival counters on it.
//
// Workgroup roles, in grid order (the grid is dispatched in order and every
// role waits only on roles before it, so waits always terminate):
//   router  [0, R)     R = E: one expert per workgroup (its 256 threads split
//                      the row), its logit for every token; also clears the
//                      output rows, then publishes the logits.
//   gate/up [R, R+G)   one per (slot, 16-row block of the intermediate dim);
//                      the shared expert is one more slot per token.  Reads
//                      all E logits of its token and selects the top k itself
//                      (so routing is one hand-over), then computes 16 values
//                      of h = silu(gate x) * (up x).
//   down    [R+G, ...) one per (slot, 64 output rows).  Selects like gate/up,
//                      has its 16 KB of whole down rows land in LDS
//                      (direct loads), turns its rows' codes into float16
//                      values in registers and forms the routing weight while
//                      it waits for the slot's h, then adds w * (W_down h) for
//                      its rows to the float32 output with atomics (the fused
//                      combine: k+1 adds per output element).
// Hand-over between workgroups.  Polling is what costs here: a poll waits
// behind every load its compute unit has in flight, and hundreds of
// workgroups polling many words flood the memory system that the weights are
// streaming through.  So every poll is a few lanes on a few words:
//   - values go out as 64-bit words {epoch, value} written with L2-bypassing
//     (agent-scope) stores; a reader waits for the words themselves.  The
//     epoch comes from control words every workgroup counts itself in on when
//     it starts (count_in / counted_in), so nothing is left to do when the
//     work is done.
//   - the expert workgroups read one of kXchReplicas copies of the logits
//     (wave 0 polls them all, four experts per lane).
//   - h goes out as float16 pairs, one pair per {epoch, pair} word; a gate/up
//     workgroup's 16 values are 8 words stored by 8 lanes of one wave.  Each
//     wave of a down workgroup polls the words of its own 64-column groups of
//     the slot's h (the poll is the read), sleeping between rounds; once all
//     are in, the products need only broadcast reads of h.
// Waits are bounded: after kSpinLimit polls a workgroup sets the error control
// word and carries on (that call's output is then invalid).
//
// Dot products run v_dot2_f32_f16 directly on exponent-trick codes: a word's low
// nibbles become 1024+q and its high nibbles 64+q as float16, so
//   sum_k q_k a_k = (sum over low of (1024+q) a) - 1024 * (sum over low of a)
//                 + (sum over high of (64+q) a) -   64 * (sum over high of a)
// and a group contributes scale * sum q a + bias * sum a: 9 VALU ops per word
// (the router and gate/up products).  The down products take codes turned into
// exact float16 q before h arrives (one packed subtract of 1024 or 64 per pair).
#include "common.h"
#include "decode_common.h"
#include "kernels.h"

namespace bitmoe {

namespace {

using namespace dec;

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kXchReplicas = kDecodeXchReplicas;
constexpr size_t kXchWords = (size_t)kDecodeMaxT * kMaxE;     // one copy of the logits: [T][E]
constexpr int kGURows = 16;  // gate and up rows per gate/up workgroup
constexpr int kDRows = 64;   // output rows per down workgroup
constexpr long kSpinLimit = 1l << 20;


// control words (uint32 indices into the workspace control block); words that
// many workgroups touch sit on lines of their own.  Workgroup b counts itself
// in on the 64-bit word of group b % kArriveGroups, at kCtlArrive + 32 g: the
// group's workgroups of the running call that have started (low half) and the
// calls started before it (high half, one copy per group).  One word for every
// workgroup would serialize hundreds of atomics at the start of each call: one
// word 19.5 us per call, 8 words 11.6, 16 words 11.1, 32 words 11.0.
constexpr int kCtlArrive = 512;
constexpr int kArriveGroups = 32;  // the grid has at least this many workgroups

// A call's epoch: the count of calls before it with the top bit set, so that
// it is never 0 (the epoch of the words of a zero-filled workspace) and two
// consecutive calls never share one, across the count's wrap too.
__device__ __forceinline__ unsigned epoch_of_calls(unsigned calls) { return calls | 0x80000000u; }

// Counting a workgroup in: count_in() adds it to its group's word and returns
// the word as it was; counted_in() then returns the call's epoch, and in the
// last workgroup of the group to start moves the word on to the next call
// (calls + 1, started 0) with an add whose result it does not wait for.  The
// next call's workgroups start only after this kernel has ended, and every
// call has workgroups in every group, so the groups' counts of calls stay
// equal and every workgroup of a call reads the same one, whatever the grid
// size of either call.  Two steps, so that a workgroup can put work between
// the atomic and the use of its result.
__device__ __forceinline__ unsigned long long* arrive_word(unsigned* ctl) {
    return reinterpret_cast<unsigned long long*>(ctl + kCtlArrive + 32 * (blockIdx.x % kArriveGroups));
}
__device__ __forceinline__ unsigned long long count_in(unsigned* ctl) {
    // an offset the compiler cannot prove uniform: it would otherwise merge the
    // lanes' atomics into one and read the result back at once
    unsigned zero = 0;
    asm volatile("" : "+v"(zero));
    return __hip_atomic_fetch_add(arrive_word(ctl) + zero, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned counted_in(unsigned* ctl, unsigned long long old) {
    const unsigned g = blockIdx.x % kArriveGroups;
    const unsigned members = (gridDim.x - g + kArriveGroups - 1) / kArriveGroups;
    if ((unsigned)old == members - 1)
        __hip_atomic_fetch_add(arrive_word(ctl), (1ull << 32) - members, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return epoch_of_calls((unsigned)(old >> 32));
}

// Sum each of 8 per-lane values over the 64 lanes of a wave through an LDS
// transpose (red: 64*9 floats of this wave).  Lane 8v receives the total of value v.
__device__ __forceinline__ float wave_sum8(const float (&v)[8], float* red, int lane) {
#pragma unroll
    for (int i = 0; i < 8; i++) red[lane * 9 + i] = v[i];
    const int which = lane / 8, part = lane % 8;
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; j++) s += red[(part * 8 + j) * 9 + which];
    return group_sum(s, 8);
}

struct RoleShared {
    union {
        float red[kWaves][kWave * 9];  // gate/up role: cross-lane sums
        struct {
            uint4 drows[kDRows * 16];  // 64 whole rows of up to 512 columns, landed by direct loads
            uint4 dsb[2][256];         // scale and bias of those rows (when they fit)
            _Float16 hh[kMaxDecodeI];  // the slot's h, 8-column blocks in nibble order, blocks rotated per group
            float2 hsum[kMaxDecodeI / 8];  // low/high sums of h per 8 columns
            float part[kWaves][kDRows];    // each wave's part of every row's dot product
            int wave_ok[kWaves];           // each wave saw its part of h in time
        } down;
        TopkShared tk;  // gate/up and down roles: the token's top k (before the roles' own LDS use)
    };
    float rsum[kDecodeMaxT][kWaves];  // router role: each wave's part of the logits
    float hrow[kGURows];  // gate/up role: this workgroup's h
    int ex;
    float gatew;  // down role of the shared expert: its weight under an optional gate
    int ok;       // routing read in time
    int wait_ok;  // result of the last wait on published values
    unsigned epoch;  // this call's epoch
};

// Poll n published words until every one carries `epoch`; each thread handles
// indices tid, tid + kThreads, ...; value i goes to keep(i, bits).  Returns
// false (and sets the error word) on timeout.
template <typename Keep>
__device__ bool await_published(const unsigned long long* src, int n, unsigned epoch, Keep keep, unsigned* ctl) {
    long spins = 0;
    for (;;) {
        int missing = 0;
        for (int i = threadIdx.x; i < n; i += kThreads) {
            const unsigned long long w = peek(src + i);
            if ((unsigned)(w >> 32) == epoch) {
                keep(i, (uint32_t)w);
            } else {
                missing = 1;
            }
        }
        if (__syncthreads_or(missing) == 0) return true;
        if (++spins > kSpinLimit) {
            if (threadIdx.x == 0) flag_error(ctl);
            return false;
        }
        __builtin_amdgcn_s_sleep(2);
    }
}

// The expert of `slot`: wave 0 of the workgroup polls its token's E logits
// (copy blockIdx % kXchReplicas; lane l: experts l, l + 64, l + 128, l + 192),
// selects the top k in registers and keeps rank slot % top_k; the other waves
// only meet it at the closing barrier.  Returns, in wave 0's lane j < top_k,
// the order key of rank j (the routing weight is formed from these later, off
// the path to the expert's loads).  The shared expert's slots wait for the
// logits too (so that its down workgroups never add into rows not yet cleared)
// and take expert 0 of the shared stack.
__device__ uint32_t route_slot(const DecodeArgs& p, int slot, int t, bool routed, unsigned epoch, RoleShared& sh) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    constexpr int kPer = kMaxE / kWave;
    uint32_t rk = 0;
    if (wave == 0) {
        const unsigned long long* src = p.xch64 + (blockIdx.x % kXchReplicas) * kXchWords + (size_t)t * p.E;
        // wait on one word first (the last expert's), so that hundreds of
        // workgroups do not poll every word while the router works: that traffic
        // slows the router's own loads (13.5 against 15.0 us per call)
        if (lane == 0) {
            for (long spins = 0; spins <= kSpinLimit; spins++) {
                if ((unsigned)(peek(src + p.E - 1) >> 32) == epoch) break;
                __builtin_amdgcn_s_sleep(2);
            }
        }
        // the four loads go out together (a lane past E reads expert E-1 again)
        unsigned long long v[kPer];
        bool ok = true;
        for (long spins = 0;; spins++) {
#pragma unroll
            for (int i = 0; i < kPer; i++) v[i] = peek(src + min(lane + kWave * i, p.E - 1));
            bool have = true;
#pragma unroll
            for (int i = 0; i < kPer; i++) have &= (unsigned)(v[i] >> 32) == epoch;
            if (__ballot(!have) == 0) break;
            if (spins > kSpinLimit) {
                if (lane == 0) flag_error(p.ctl);
                ok = false;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        int ex = 0;
        if (routed) {
            uint32_t key[kPer];
#pragma unroll
            for (int i = 0; i < kPer; i++)
                key[i] = lane + kWave * i < p.E ? order_key(__uint_as_float((uint32_t)v[i])) : 0u;
            rk = topk_wave_select(sh.tk, key, p.top_k, lane);
            ex = min(max(sh.tk.sel_e[slot % p.top_k], 0), p.E - 1);  // in range whatever was read
        }
        if (lane == 0) {
            sh.ex = ex;
            sh.ok = ok;
        }
    }
    __syncthreads();
    return rk;
}

// ------------------------------------------------------------------ router role

template <typename SB, bool kQ8>
__device__ void router_role(const DecodeArgs& p, int b, RoleShared& sh) {
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int H = p.H, T = p.T, E = p.E;
    const int e = b;  // one expert per workgroup
    const int nblk = H / 8;  // 16-byte chunks of a row
    // clear the output rows (write-through); they are complete before any logit
    // goes out, which every down workgroup reads before it adds into them
    for (int i = b * kThreads + tid; i < T * H; i += p.router_wgs * kThreads) put(p.out + i, 0.0f);

    float acc[kDecodeMaxT];
#pragma unroll
    for (int t = 0; t < kDecodeMaxT; t++) acc[t] = 0.0f;
    unsigned long long arrived = 0;
    const int er = min(e, E - 1);
    const uint4* wr = reinterpret_cast<const uint4*>(p.router + (size_t)er * H);
    // 8-bit router: the row's codes (8 per 8-byte pair of words) and the scale
    // and bias of each 64-column group
    const uint2* wq = reinterpret_cast<const uint2*>(p.router_q8 + (size_t)er * (H / 4));
    const SB* rs = static_cast<const SB*>(p.router_s) + (size_t)er * (H / 64);
    const SB* rb = static_cast<const SB*>(p.router_b) + (size_t)er * (H / 64);
    for (int c0 = 0; c0 < nblk; c0 += kThreads) {
        const int c = min(c0 + tid, nblk - 1);
        uint4 a, xv[kDecodeMaxT];
        uint2 aq;
        SB sq, bq;
        if (kQ8) {
            aq = wq[c];
            sq = rs[c / 8];
            bq = rb[c / 8];
        } else {
            a = wr[c];
        }
#pragma unroll
        for (int t = 0; t < kDecodeMaxT; t++) xv[t] = reinterpret_cast<const uint4*>(p.x + (size_t)min(t, T - 1) * H)[c];
        // count the workgroup in after this wave's loads, so that the atomic's
        // return (in order with them) does not delay the products
        if (c0 == 0 && tid == 0) arrived = count_in(p.ctl);
        __builtin_amdgcn_sched_barrier(0);
        if (kQ8) a = restore_q8x8(aq, sb_to_f32<SB>(sq), sb_to_f32<SB>(bq));
        if (c0 + tid < nblk) {
            const uint16_t* ab = reinterpret_cast<const uint16_t*>(&a);
#pragma unroll
            for (int t = 0; t < kDecodeMaxT; t++) {
                const uint16_t* xb = reinterpret_cast<const uint16_t*>(&xv[t]);
#pragma unroll
                for (int i = 0; i < 8; i++) acc[t] += bf16_to_f32(xb[i]) * bf16_to_f32(ab[i]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < kDecodeMaxT; t++) {
        const float w = wave_total(acc[t]);
        if (lane == 0) sh.rsum[t][wave] = w;
    }
    if (tid == 0) sh.epoch = counted_in(p.ctl, arrived);
    __builtin_amdgcn_s_waitcnt(0);  // the clearing stores are out
    __syncthreads();
    const unsigned epoch = sh.epoch;
    const float bias = (p.logit_bias && e < E) ? p.logit_bias[e] : 0.0f;
    if (tid < kXchReplicas && e < E) {  // thread r writes copy r
#pragma unroll
        for (int t = 0; t < kDecodeMaxT; t++) {
            if (t >= T) break;
            const float lg = ((sh.rsum[t][0] + sh.rsum[t][1]) + (sh.rsum[t][2] + sh.rsum[t][3])) + bias;
            publish(p.xch64 + tid * kXchWords + (size_t)t * E + e, epoch, __float_as_uint(lg));
        }
    }
}

// ------------------------------------------------------------------ gate/up role

// kRouted: the slot belongs to a routed expert (else to the shared expert); a
// template parameter so that each instantiation reads one weight set directly
template <typename SB, bool kRouted>
__device__ void gateup_role(const DecodeArgs& p, int slot, int blk, unsigned epoch, RoleShared& sh) {
    const int H = p.H, I = p.I;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int TK = p.T * p.top_k;
    constexpr bool routed = kRouted;
    const int t = routed ? slot / p.top_k : slot - TK;
    const int i0 = blk * kGURows;

    // the shared expert waits for the logits too, so that its loads do not
    // compete with the router's (13.38 against 13.46 us per call)
    route_slot(p, slot, t, routed, epoch, sh);
    const size_t ex = (size_t)sh.ex;

    const FfnPtr& f = kRouted ? p.experts : p.shared;
    const uint32_t* g_q = f.gate.q;
    const void* g_s = f.gate.s;
    const void* g_b = f.gate.b;
    const uint32_t* u_q = f.up.q;
    const void* u_s = f.up.s;
    const void* u_b = f.up.b;

    // wave w owns rows i0+4w .. i0+4w+3 of gate and of up; lane l covers the
    // input columns [32 l, 32 l + 32) (+2048 per further chunk pass)
    constexpr int kRowsPerWave = kGURows / kWaves;  // 4
    const int n_chunks = H / 32;
    const int ng = H / kGroup;
    const size_t row0 = ex * I + i0 + wave * kRowsPerWave;
    const uint32_t* gq = g_q + row0 * (size_t)(H / 8);
    const uint32_t* uq = u_q + row0 * (size_t)(H / 8);
    const SB* gs = reinterpret_cast<const SB*>(g_s) + row0 * ng;
    const SB* gb = reinterpret_cast<const SB*>(g_b) + row0 * ng;
    const SB* us = reinterpret_cast<const SB*>(u_s) + row0 * ng;
    const SB* ub = reinterpret_cast<const SB*>(u_b) + row0 * ng;
    const uint4* xrow = reinterpret_cast<const uint4*>(p.x + (size_t)t * H);

    float acc[8];  // gate rows 0..3, up rows 0..3
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] = 0.0f;
    for (int c0 = 0; c0 < n_chunks; c0 += kWave) {
        const bool valid = c0 + lane < n_chunks;
        const int c = min(c0 + lane, n_chunks - 1);
        uint4 gv[kRowsPerWave], uv[kRowsPerWave], xr[4];
        SB gsr[kRowsPerWave], gbr[kRowsPerWave], usr[kRowsPerWave], ubr[kRowsPerWave];
#pragma unroll
        for (int r = 0; r < kRowsPerWave; r++) {
            gsr[r] = gs[(size_t)r * ng + c / 2];
            gbr[r] = gb[(size_t)r * ng + c / 2];
            usr[r] = us[(size_t)r * ng + c / 2];
            ubr[r] = ub[(size_t)r * ng + c / 2];
        }
#pragma unroll
        for (int r = 0; r < kRowsPerWave; r++) {
            gv[r] = reinterpret_cast<const uint4*>(gq + (size_t)r * (H / 8))[c];
            uv[r] = reinterpret_cast<const uint4*>(uq + (size_t)r * (H / 8))[c];
        }
#pragma unroll
        for (int m = 0; m < 4; m++) xr[m] = xrow[c * 4 + m];
        __builtin_amdgcn_sched_barrier(0);  // every load above is issued before the math

        Pairs8 pr[4];
        float lo = 0.0f, hi = 0.0f;
#pragma unroll
        for (int m = 0; m < 4; m++) pr[m] = pairs_from_bf16(xr[m], lo, hi);
        const float vmask = valid ? 1.0f : 0.0f;
#pragma unroll
        for (int r = 0; r < kRowsPerWave; r++) {
            float glo = 0.0f, ghi = 0.0f, ulo = 0.0f, uhi = 0.0f;
            dot_word(gv[r].x, pr[0], glo, ghi);
            dot_word(gv[r].y, pr[1], glo, ghi);
            dot_word(gv[r].z, pr[2], glo, ghi);
            dot_word(gv[r].w, pr[3], glo, ghi);
            dot_word(uv[r].x, pr[0], ulo, uhi);
            dot_word(uv[r].y, pr[1], ulo, uhi);
            dot_word(uv[r].z, pr[2], ulo, uhi);
            dot_word(uv[r].w, pr[3], ulo, uhi);
            const float gqx = (glo - 1024.0f * lo) + (ghi - 64.0f * hi);
            const float uqx = (ulo - 1024.0f * lo) + (uhi - 64.0f * hi);
            acc[r] += vmask * (sb_to_f32<SB>(gsr[r]) * gqx + sb_to_f32<SB>(gbr[r]) * (lo + hi));
            acc[4 + r] += vmask * (sb_to_f32<SB>(usr[r]) * uqx + sb_to_f32<SB>(ubr[r]) * (lo + hi));
        }
    }
    const float total = wave_sum8(acc, sh.red[wave], lane);
    // lane 8v holds value v: v < 4 gate row v, v >= 4 up row v-4
    const float upv = __shfl(total, (lane + 32) & 63);
    if (lane < 32 && lane % 8 == 0) sh.hrow[wave * kRowsPerWave + lane / 8] = silu(total) * upv;
    __syncthreads();
    // the 16 values as 8 words {epoch, float16 pair}, one 64-byte store of one wave
    if (tid < kGURows / 2) {
        const half2_t pr = {(_Float16)sh.hrow[2 * tid], (_Float16)sh.hrow[2 * tid + 1]};
        publish(p.h64 + ((size_t)slot * I + i0) / 2 + tid, epoch, as_u32(pr));
    }
}

// ------------------------------------------------------------------ down role

template <typename SB, bool kRouted>
__device__ void down_role(const DecodeArgs& p, int slot, int blk, unsigned epoch, RoleShared& sh) {
    const int H = p.H, I = p.I;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int TK = p.T * p.top_k;
    constexpr bool routed = kRouted;
    const int t = routed ? slot / p.top_k : slot - TK;
    const int n0 = blk * kDRows;

    // the shared expert's weight under an optional gate g (a checkpoint detail):
    // sigmoid(x[t] . g), float32 sum of exact bf16 products, by wave 1 while
    // wave 0 waits for the routing (route_slot ends with a barrier)
    if (!kRouted && p.shared_gate && wave == 1) {
        const uint4* xr = reinterpret_cast<const uint4*>(p.x + (size_t)t * H);
        const uint4* gr = reinterpret_cast<const uint4*>(p.shared_gate);
        float z = 0.0f;
        for (int blk = lane; blk < H / 8; blk += kWave) {
            const uint4 a = xr[blk], g = gr[blk];
            const uint16_t* ab = reinterpret_cast<const uint16_t*>(&a);
            const uint16_t* gb = reinterpret_cast<const uint16_t*>(&g);
#pragma unroll
            for (int e = 0; e < 8; e++) z += bf16_to_f32(ab[e]) * bf16_to_f32(gb[e]);
        }
        z = group_sum(z, kWave);
        if (lane == 0) sh.gatew = 1.0f / (1.0f + expf(-z));
    }
    // every down workgroup waits for its token's logits, shared ones too: the
    // router clears the output rows before it publishes them
    const uint32_t rk = route_slot(p, slot, t, routed, epoch, sh);
    const size_t ex = (size_t)sh.ex;
    const FfnPtr& f = kRouted ? p.experts : p.shared;
    const uint32_t* d_q = f.down.q;
    const void* d_s = f.down.s;
    const void* d_b = f.down.b;

    // rows [n0, n0+128) land in LDS through direct loads: instruction j of wave w
    // fills 64 consecutive 16-byte units of the row-major [row][I/32] block
    const int gd = I / kGroup;
    const int u_per_row = I / 32;  // 16-byte units per row
    const int n_rows = min(kDRows, H - n0);
    const int n_units = n_rows * u_per_row;
    const uint4* dq = reinterpret_cast<const uint4*>(d_q + (ex * (size_t)H + n0) * (I / 8));
    const bool rows_in_lds = u_per_row <= 16;  // I <= 512
    // 16-unit rows are stored rotated (unit u of row r at u ^ (r % 16)) so that
    // the 8 rows a wave reads at once hit different LDS banks
    const int swz_mask = u_per_row == 16 ? 15 : 0;
    if (rows_in_lds) {
        for (int f0 = wave * kWave; f0 < n_units; f0 += kThreads) {
            const int f = min(f0 + lane, n_units - 1);
            const int r = f / u_per_row, u = f % u_per_row;
            __builtin_amdgcn_global_load_lds(dq + r * u_per_row + (u ^ (r & swz_mask)), &sh.down.drows[f0], 16, 0, 0);
        }
    }
    const SB* ds = reinterpret_cast<const SB*>(d_s) + (ex * (size_t)H + n0) * gd;
    const SB* db = reinterpret_cast<const SB*>(d_b) + (ex * (size_t)H + n0) * gd;
    // scale and bias of the rows are contiguous too: land them beside the rows
    const int sb_units = n_rows * gd * (int)sizeof(SB) / 16;
    const bool sb_in_lds = sb_units <= 256;
    if (sb_in_lds && wave < 2) {
        const uint4* src = reinterpret_cast<const uint4*>(wave == 0 ? ds : db);
        for (int f0 = 0; f0 < sb_units; f0 += kWave)
            __builtin_amdgcn_global_load_lds(src + min(f0 + lane, sb_units - 1), &sh.down.dsb[wave][f0], 16, 0, 0);
    }
    const SB* lds_s = reinterpret_cast<const SB*>(sh.down.dsb[0]);
    const SB* lds_b = reinterpret_cast<const SB*>(sh.down.dsb[1]);

    // the slot's routing weight, by wave 0 (which adds the rows at the end)
    // while the loads are in flight
    float wgt = 1.0f;
    if (kRouted && wave == 0) {
        const float w = topk_weight_of_keys(rk, p.top_k);
        wgt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), slot % p.top_k));
    }

    // every wave's direct loads of rows and scales have landed
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();


    // h of the slot, by 64-column groups: wave w takes groups w, w + 4, ...
    // (32 words {epoch, float16 pair} each), polls their words itself and, once
    // they all carry this call's epoch, moves on to the products.  Lane i of
    // the poll holds word i of the wave's words and returns the sum of its pair
    // (0 for a lane past the groups).  h is kept in LDS as float16 in nibble
    // order; 8-column block m of group g sits at block g * 8 + (m + g) % 8, so
    // the 8 groups the lanes read at once hit different banks.
    const unsigned long long* hsrc = p.h64 + (size_t)slot * I / 2;
    _Float16* hh = sh.down.hh;
    auto h_pos = [](int i) {
        const int b = i >> 3, g = b >> 3, m = b & 7;
        return ((g << 3) + ((m + g) & 7)) * 8 + slot_of_column(i & 7);
    };
    const int gpw = (gd + kWaves - 1) / kWaves;  // groups per wave
    const int nw = 32 * gpw;                      // words this wave polls
    auto poll_h = [&](float& pair_sum) -> int {
        for (long spins = 0;; spins++) {
            bool have = true;
            for (int idx = lane; idx < nw; idx += kWave) {
                const int g = wave + kWaves * (idx / 32);
                if (g >= gd) continue;
                const int wd = 32 * g + idx % 32;
                const unsigned long long v = peek(hsrc + wd);
                if ((unsigned)(v >> 32) == epoch) {
                    const half2_t pr = as_half2((uint32_t)v);
                    hh[h_pos(2 * wd)] = pr.x;
                    hh[h_pos(2 * wd + 1)] = pr.y;
                    pair_sum = (float)pr.x + (float)pr.y;
                } else {
                    have = false;
                }
            }
            if (__ballot(!have) == 0) return 1;
            if (spins > kSpinLimit) {
                if (lane == 0) flag_error(p.ctl);
                return 0;
            }
            __builtin_amdgcn_s_sleep(4);
        }
    };
    const int r = lane;  // lane r: this wave's groups of row r
    float y = 0.0f;
    int ok_h;
    if (rows_in_lds) {
        // I <= 512, so at most two groups per wave.  While h is on its way each
        // lane turns its row's codes of those groups into exact float16 values
        // (the exponent trick, then one packed subtract of 1024 or 64) and
        // takes their scales and biases, so that once h is in only the dot
        // products remain: y += s * sum(q * h) + b * sum(h) per group.
        half2_t qv[2][32];
        float sv[2] = {0.0f, 0.0f}, bv[2] = {0.0f, 0.0f};
        const half2_t k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
        const half2_t k64 = {(_Float16)64.0f, (_Float16)64.0f};
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int g = wave + kWaves * j;
            const int gc = min(g, gd - 1), rr = min(r, n_rows - 1);  // in bounds for every lane
            const uint4 v0 = sh.down.drows[rr * u_per_row + ((2 * gc) ^ (rr & swz_mask))];
            const uint4 v1 = sh.down.drows[rr * u_per_row + ((2 * gc + 1) ^ (rr & swz_mask))];
            const uint32_t wv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
            for (int m = 0; m < 8; m++) {
                const uint32_t w8 = wv[m] >> 8;
                qv[j][4 * m + 0] = as_half2(and_or(wv[m], 0x000F000Fu, 0x64006400u)) - k1024;
                qv[j][4 * m + 1] = as_half2(and_or(wv[m], 0x00F000F0u, 0x54005400u)) - k64;
                qv[j][4 * m + 2] = as_half2(and_or(w8, 0x000F000Fu, 0x64006400u)) - k1024;
                qv[j][4 * m + 3] = as_half2(and_or(w8, 0x00F000F0u, 0x54005400u)) - k64;
            }
            if (g < gd) {
                sv[j] = sb_to_f32<SB>(lds_s[rr * gd + g]);
                bv[j] = sb_to_f32<SB>(lds_b[rr * gd + g]);
            }
        }
        // keep the compiler from sinking this work past the wait for h
#pragma unroll
        for (int j = 0; j < 2; j++) {
#pragma unroll
            for (int i = 0; i < 32; i++) {
                uint32_t u = as_u32(qv[j][i]);
                asm volatile("" : "+v"(u));
                qv[j][i] = as_half2(u);
            }
            asm volatile("" : "+v"(sv[j]), "+v"(bv[j]));
        }
        float pair_sum = 0.0f;
        ok_h = poll_h(pair_sum);
        // sum of h over each of the wave's groups: lanes 0..31 polled group
        // wave, lanes 32..63 group wave + 4
        float t = pair_sum;
        t += dpp<0xB1>(t);   // quad_perm 1,0,3,2
        t += dpp<0x4E>(t);   // quad_perm 2,3,0,1
        t += dpp<0x141>(t);  // row_half_mirror
        t += dpp<0x140>(t);  // row_mirror
        const float hs[2] = {__int_as_float(__builtin_amdgcn_readlane(__float_as_int(t), 0)) +
                                 __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t), 16)),
                             __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t), 32)) +
                                 __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t), 48))};
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's h is in LDS
        // all 16 blocks of h the wave needs (broadcast reads), then one wait
        const uint4* hp4 = reinterpret_cast<const uint4*>(hh);
        uint4 hv[2][8];
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int g = min(wave + kWaves * j, gd - 1);
#pragma unroll
            for (int m = 0; m < 8; m++) hv[j][m] = hp4[g * 8 + ((m + g) & 7)];
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int j = 0; j < 2; j++) {
            if (wave + kWaves * j >= gd) break;
            float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
#pragma unroll
            for (int m = 0; m < 8; m++) {
                a0 = __builtin_amdgcn_fdot2(qv[j][4 * m + 0], as_half2(hv[j][m].x), a0, false);
                a1 = __builtin_amdgcn_fdot2(qv[j][4 * m + 1], as_half2(hv[j][m].y), a1, false);
                a2 = __builtin_amdgcn_fdot2(qv[j][4 * m + 2], as_half2(hv[j][m].z), a2, false);
                a3 = __builtin_amdgcn_fdot2(qv[j][4 * m + 3], as_half2(hv[j][m].w), a3, false);
            }
            y += sv[j] * ((a0 + a1) + (a2 + a3)) + bv[j] * hs[j];
        }
        if (r >= n_rows) y = 0.0f;
    } else {
        // rows of more than 512 columns stay in global memory
        float unused = 0.0f;
        ok_h = poll_h(unused);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's h is in LDS
        for (int idx = lane; idx < 8 * gpw; idx += kWave) {
            const int g = wave + kWaves * (idx / 8), m = idx % 8;
            if (g >= gd) continue;
            const _Float16* hv = hh + ((g << 3) + ((m + g) & 7)) * 8;  // 0,4,1,5,2,6,3,7
            sh.down.hsum[g * 8 + m] = make_float2((float)hv[0] + (float)hv[1] + (float)hv[4] + (float)hv[5],
                                                  (float)hv[2] + (float)hv[3] + (float)hv[6] + (float)hv[7]);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (r < n_rows) {
            for (int j = 0; j < gpw; j++) {
                const int g = wave + kWaves * j;
                if (g >= gd) break;
                const uint4 v0 = dq[(size_t)r * u_per_row + 2 * g];
                const uint4 v1 = dq[(size_t)r * u_per_row + 2 * g + 1];
                const uint4* hp4 = reinterpret_cast<const uint4*>(hh) + g * 8;  // blocks rotated by g
                float alo = 0.0f, ahi = 0.0f, lo = 0.0f, hi = 0.0f;
                const uint32_t wv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
                for (int m = 0; m < 8; m++) {
                    dot_word(wv[m], pairs_of(hp4[(m + g) & 7]), alo, ahi);
                    const float2 sm = sh.down.hsum[g * 8 + m];
                    lo += sm.x;
                    hi += sm.y;
                }
                const SB sv = sb_in_lds ? lds_s[r * gd + g] : ds[(size_t)r * gd + g];
                const SB bv = sb_in_lds ? lds_b[r * gd + g] : db[(size_t)r * gd + g];
                y += sb_to_f32<SB>(sv) * ((alo - 1024.0f * lo) + (ahi - 64.0f * hi)) + sb_to_f32<SB>(bv) * (lo + hi);
            }
        }
    }
    sh.down.part[wave][lane] = y;
    if (lane == 0) sh.down.wave_ok[wave] = ok_h;
    __syncthreads();
    if (wave == 0 && r < n_rows) {
        const bool ok = sh.ok && sh.down.wave_ok[0] && sh.down.wave_ok[1] && sh.down.wave_ok[2] && sh.down.wave_ok[3];
        const float yt = (sh.down.part[0][r] + sh.down.part[1][r]) + (sh.down.part[2][r] + sh.down.part[3][r]);
        const float wt = (!kRouted && p.shared_gate) ? sh.gatew : wgt;
        if (ok) atomicAdd(p.out + (size_t)t * H + n0 + r, wt * yt);
    }
}

template <typename SB, bool kQ8>
__global__ __launch_bounds__(kThreads) void decode_layer_kernel(DecodeArgs p) {
    __shared__ RoleShared sh;
    const int b = blockIdx.x;
    if (b < p.router_wgs) {
        router_role<SB, kQ8>(p, b, sh);
        return;
    }
    // the expert workgroups need the epoch first for the logits, which take
    // longer to come than the count
    if (threadIdx.x == 0) sh.epoch = counted_in(p.ctl, count_in(p.ctl));
    if (b >= p.router_wgs + p.gateup_wgs + p.down_wgs) return;  // padding up to kArriveGroups
    __syncthreads();
    const unsigned epoch = sh.epoch;
    if (b < p.router_wgs + p.gateup_wgs) {
        const int unit = b - p.router_wgs, nblk = p.I / kGURows;
        const int slot = unit / nblk, blk = unit % nblk;
        if (slot < p.T * p.top_k)
            gateup_role<SB, true>(p, slot, blk, epoch, sh);
        else
            gateup_role<SB, false>(p, slot, blk, epoch, sh);
    } else {
        const int unit = b - p.router_wgs - p.gateup_wgs, nblk = (p.H + kDRows - 1) / kDRows;
        const int slot = unit / nblk, blk = unit % nblk;
        if (slot < p.T * p.top_k)
            down_role<SB, true>(p, slot, blk, epoch, sh);
        else
            down_role<SB, false>(p, slot, blk, epoch, sh);
    }
}

// Routing outputs requested by the caller: the top k of the logits the layer
// kernel published (copy 0), selected by one wave with the same ranking and
// weight arithmetic as the expert workgroups (a tiny second kernel, only when
// asked).
__global__ __launch_bounds__(kWave) void decode_routing_out_kernel(DecodeArgs p) {
    __shared__ int counts[kMaxE];
    const int lane = threadIdx.x;
    // the layer kernel's epoch: it counted its call in when it started
    const unsigned calls = __hip_atomic_load(p.ctl + kCtlArrive + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // group 0's
    const unsigned epoch = epoch_of_calls(calls - 1u);
    const int k = p.top_k, E = p.E;
    for (int e = lane; e < kMaxE; e += kWave) counts[e] = 0;
    __syncthreads();
#pragma unroll
    for (int t = 0; t < kDecodeMaxT; t++) {
        if (t >= p.T) break;
        float held[kMaxE / kWave];
        bool ok = true;
#pragma unroll
        for (int i = 0; i < kMaxE / kWave; i++) {
            const int e = lane + kWave * i;
            const unsigned long long wd = e < E ? peek(p.xch64 + (size_t)t * E + e) : 0ull;
            ok = ok && (e >= E || (unsigned)(wd >> 32) == epoch);
            held[i] = e < E ? __uint_as_float((uint32_t)wd) : -INFINITY;
        }
        int ex;
        float w;
        wave_topk_held(held, E, k, lane, &ex, &w);
        if (__ballot(!ok) != 0) {
            if (lane == 0) flag_error(p.ctl);
        }
        if (lane < k) {
            if (p.idx_out) p.idx_out[t * k + lane] = ex;
            if (p.w_out) p.w_out[t * k + lane] = w;
            if (ex >= 0 && ex < E) atomicAdd(&counts[ex], 1);
        }
    }
    __syncthreads();
    if (p.counts_out)
        for (int e = lane; e < p.E; e += kWave) p.counts_out[e] = counts[e];
}

}  // namespace

int decode_router_wgs(int E) { return E; }
int decode_gateup_wgs(int T, int k, bool shared, int I) { return (T * k + (shared ? T : 0)) * (I / kGURows); }
int decode_down_wgs(int T, int k, bool shared, int H) {
    return (T * k + (shared ? T : 0)) * ((H + kDRows - 1) / kDRows);
}

hipError_t launch_decode(const DecodeArgs& a, bool sb_bf16, hipStream_t stream) {
    const dim3 grid(max(a.router_wgs + a.gateup_wgs + a.down_wgs, kArriveGroups));
    const bool q8 = a.router_q8 != nullptr;
    if (sb_bf16 && !q8)
        hipLaunchKernelGGL((decode_layer_kernel<uint16_t, false>), grid, dim3(kThreads), 0, stream, a);
    else if (sb_bf16)
        hipLaunchKernelGGL((decode_layer_kernel<uint16_t, true>), grid, dim3(kThreads), 0, stream, a);
    else if (!q8)
        hipLaunchKernelGGL((decode_layer_kernel<float, false>), grid, dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((decode_layer_kernel<float, true>), grid, dim3(kThreads), 0, stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (a.idx_out || a.w_out || a.counts_out) {
        hipLaunchKernelGGL(decode_routing_out_kernel, dim3(1), dim3(kWave), 0, stream, a);
        err = hipGetLastError();
    }
    return err;
}

}  // namespace bitmoe
