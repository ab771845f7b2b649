// Grouped expert products with affine 4-bit dequantisation inside the MFMA
// main loop (gfx950).
//
// Pages: the 4-bit weights are restored inside the grouped GEMM and the
// restored values stay in the compute unit's fast memory, never written out
// (aimanavo.com page, section "Lily does not treat prefill and decode as the
// same job"; dzen.guru page, section "Where does the speed-up come from?").
// Weight format: MLX affine 4-bit, group size 64 (aimanavo.com page, section on
// the single supported 4-bit checkpoint).
//
// Design (gfx950):
//   - A workgroup owns one row tile of one expert group (<= 128 rows, from
//     the device tile map) and one slab of output columns.  Three variants:
//     8 waves of 2 stripes on 128-row tiles (gate/up at large T: two waves
//     per SIMD cover each other's stalls); 4 waves of 2 stripes on tiles of
//     at most 64 rows with half the LDS (two workgroups per compute unit: both
//     products of small batches, and down at large T); 4 waves on 128-row
//     tiles (the float32 rows of the step-by-step down).  The grid is
//     sized from T alone; workgroups read the tile count written by the permute
//     kernel and leave when there is no work.  Workgroups are dispatched
//     round-robin over the 8 XCDs; tiles are dealt to XCDs the same way in map
//     order (the map lists long tiles first, so the grid ends on short work and
//     every XCD gets an equal share), and the slabs of a tile stay on one XCD,
//     so they share its activation rows in that XCD's L2.
//   - Operands stream through a ring of LDS stages, one 64-column group of K
//     per stage, filled by direct-to-LDS loads (global_load_lds_dwordx4): the
//     activation rows (float16, XOR-swizzled so the 32-row MFMA operand reads
//     are conflict free; gate/up gathers token rows through the slot
//     permutation, so the permuted matrix is never materialised) and, every
//     second stage, 64 bytes of each weight row (two groups; requests of 64
//     bytes stream ~1.4x faster than 32-byte row slices), also XOR-swizzled.
//     The loads of a later stage go out between the MFMAs of the current one.
//     The ring is deeper for shorter tiles (less arithmetic per stage), so HBM
//     stays busy at every batch size.  The waits are counted by hand
//     (s_waitcnt vmcnt(loads of the stages issued since)) and the ring reads
//     are inline-asm ds_reads, so the compiler's conservative waits for LDS
//     DMA never drain the ring.
//   - A lane's 8 consecutive K values of one output column are exactly one
//     packed word: it is dequantised in registers (dequant_word: 13 VALU ops
//     per 8 weights) straight into the B operand of v_mfma_f32_32x32x16_f16.
//   - gate/up: a wave computes a 32-column stripe of gate and the same stripe of
//     up, so SwiGLU is elementwise on the accumulators; h goes to global memory
//     as float16 through an LDS transpose (16-byte stores), 8-column blocks in
//     dequantisation order, which is the K order the down product reads.
//   - down: a wave computes four 32-column stripes (512 output columns per
//     workgroup, so the activations staged once feed four times the MFMAs of
//     one stripe pair); the epilogue stores each row to its slot's row
//     (un-permute on store): float16 rows for the layer's combine kernel, or
//     float32 rows for the step-by-step API.
#include "common.h"
#include "kernels.h"

namespace bitmoe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMT = kTileRows / 32;              // 32-row MFMA tiles per full row tile
constexpr int kStageRowBytes = kGroup * 2;       // one group of float16 per row

enum Mode { kGateUp = 0, kDownY16 = 1, kDownStore = 2 };

// Geometry of a mode: a wave owns NS stripes of 32 weight rows.  gate/up:
// stripes 0 .. NS/2-1 of gate and the same rows of up (SwiGLU pairs them), so
// a wave owns 32 NS/2 columns of h; down: NS consecutive stripes, 4 for the
// layer's float16 rows (the activations staged once feed 512 output columns),
// 2 for the float32 rows of the step-by-step call.
// Scales and biases of a wave's rows stay in LDS for a block of groups: per
// (stripe, array), 32 rows x kSBRowDwords dwords (a row's block plus one
// dword, so that a block starting at a 2-byte offset fits), loaded with dword
// direct loads.
// Variants: kBig (4 waves), kSmall (tiles of at most 64 rows: 2 stripes per
// wave and at most 80 KB of LDS, so that two workgroups share a compute unit
// and twice the loads are in flight per unit where the weights stream for few
// rows), kWide (8 waves of 2 stripes: the same tile and LDS as kBig with two
// waves per SIMD, so one wave's waits are covered by the other's MFMAs).
enum Variant { kBig = 0, kSmall = 1, kWide = 2 };
template <int kMode, int kV = kBig>
struct Geo {
    static constexpr int kWavesV = kV == kWide ? 8 : kWaves;
    static constexpr int kThreadsV = kWavesV * kWave;
    static constexpr int NS = kV != kBig || kMode == kDownStore ? 2 : 4;
    static constexpr int kWaveCols = kMode == kGateUp ? 32 * NS / 2 : 32 * NS;  // output columns per wave
    static constexpr int kSlabCols = kWavesV * kWaveCols;
    static constexpr int kBStageBytes = kWavesV * NS * kWave * 16;  // each lane's 16 bytes per stripe
    static constexpr int kSBRowDwords = 5;  // 8 bf16 (or 4 fp32) groups per block
    static constexpr int kSBArrayDwords = (32 * kSBRowDwords + kWave - 1) / kWave * kWave;
    static constexpr int kSBWaveBytes = NS * 2 * kSBArrayDwords * 4;
    static constexpr int kSBBytes = kWavesV * kSBWaveBytes;
    // the ring (and the epilogue tiles): what the 160 KB of LDS leaves beside
    // the scale block and the row tables, in whole KB
    static constexpr int kLdsBytes = kV == kSmall ? 80 * 1024 : 160 * 1024;
    static constexpr int kRingBytes = (kLdsBytes - kSBBytes - 2 * kTileRows * 4) / 1024 * 1024;
    static constexpr int kMaxMT = kV == kSmall ? 2 : kMT;  // tallest tile
};

// Ring of stages for a row tile of MT 32-row MFMA tiles, one 64-column group
// of K per stage.  Loads per wave, all direct-to-LDS: every stage brings MT
// activation chunks; every even stage also brings the weights of its group and
// the next one (64 bytes of each weight row in one request, 2 per stripe), so
// a pair of slots holds [A | B of two groups] [A].
template <int kMode, int MT, int kV = kBig>
struct Ring {
    using G = Geo<kMode, kV>;
    // the 4 MT 1-KB activation loads of a stage, dealt round-robin to the
    // waves: at most kALoadsMax per wave, at least kALoads (what the counted
    // waits assume, so a wave with one more only waits longer)
    static constexpr int kALoadsMax = (4 * MT + G::kWavesV - 1) / G::kWavesV;
    static constexpr int kALoads = 4 * MT / G::kWavesV;
    static constexpr int kABytes = MT * 32 * kStageRowBytes;
    static constexpr int kEven = kABytes + 2 * G::kBStageBytes;
    static constexpr int kPair = kEven + kABytes;
    static constexpr int DP = G::kRingBytes / kPair > 5 ? 5 : G::kRingBytes / kPair;
    static constexpr int D = 2 * DP;  // slots; stage j goes to slot j % D
    static constexpr int kLoadsEven = kALoads + 2 * G::NS;
    static constexpr int kLoadsOdd = kALoads;
    static_assert(DP >= 2, "ring too shallow");
    static_assert((D - 2) / 2 * kLoadsEven + (D - 2) / 2 * kLoadsOdd <= 48, "wait_vm covers 48 loads");
    static __device__ __forceinline__ int slot_offset(int slot) { return (slot >> 1) * kPair + (slot & 1) * kEven; }
    static __device__ __forceinline__ int loads(int j) { return (j & 1) ? kLoadsOdd : kLoadsEven; }
};

struct GemmArgs {
    const Tile* tiles;
    const int32_t* n_tiles;
    int slabs;
    const _Float16* a;  // x16 [T][H] (gate/up) or h [rows][I] (down)
    int lda;
    int K;              // contraction length
    int N;              // output columns of each group's matrices
    int k, TK, T, H;
    const int32_t* sorted_slot;
    QMatPtr m0, m1;     // routed stacks used by stripe 0 / stripe 1
    QMatPtr s0, s1;     // shared-expert matrices used by stripe 0 / stripe 1
    int E;
    _Float16* h;        // gate/up output [rows][N]
    _Float16* y16;      // down output [T*k + T][H] float16: slot rows, then shared rows
    float* y_slot;      // down output [T*k][H] float32 (step-by-step API)
    float* y_shared;    // [T][H] float32, nullable
};

template <typename SB>
struct Stripe {
    const uint4* q;  // row of packed words, 16-byte units
    const SB* s;
    const SB* b;
};

template <typename SB>
__device__ __forceinline__ Stripe<SB> stripe_of(const QMatPtr& routed, const QMatPtr& shared, int group,
                                                int E, int N, int K, int row) {
    const bool sh = group >= E;
    const QMatPtr& m = sh ? shared : routed;
    const size_t r = (size_t)(sh ? 0 : group) * N + row;
    Stripe<SB> st;
    st.q = reinterpret_cast<const uint4*>(m.q + r * (K / 8));
    st.s = reinterpret_cast<const SB*>(m.s) + r * (K / kGroup);
    st.b = reinterpret_cast<const SB*>(m.b) + r * (K / kGroup);
    return st;
}

__device__ __forceinline__ uint32_t word_of(const uint32_t __attribute__((ext_vector_type(4))) & v, int s) {
    return v[s];
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

__device__ __forceinline__ unsigned lds_addr(const void* p) {
    return (unsigned)reinterpret_cast<uintptr_t>(p);
}

// all but this wave's n newest loads have landed (a smaller n is always safe)
#define GEMM_VM_CASE(N) \
    case N: asm volatile("s_waitcnt vmcnt(" #N ")" ::: "memory"); break;
__device__ __forceinline__ void wait_vm(int n) {
    switch (n) {
        GEMM_VM_CASE(1) GEMM_VM_CASE(2) GEMM_VM_CASE(3) GEMM_VM_CASE(4) GEMM_VM_CASE(5) GEMM_VM_CASE(6)
        GEMM_VM_CASE(7) GEMM_VM_CASE(8) GEMM_VM_CASE(9) GEMM_VM_CASE(10) GEMM_VM_CASE(11) GEMM_VM_CASE(12)
        GEMM_VM_CASE(13) GEMM_VM_CASE(14) GEMM_VM_CASE(15) GEMM_VM_CASE(16) GEMM_VM_CASE(17) GEMM_VM_CASE(18)
        GEMM_VM_CASE(19) GEMM_VM_CASE(20) GEMM_VM_CASE(21) GEMM_VM_CASE(22) GEMM_VM_CASE(23) GEMM_VM_CASE(24)
        GEMM_VM_CASE(25) GEMM_VM_CASE(26) GEMM_VM_CASE(27) GEMM_VM_CASE(28) GEMM_VM_CASE(29) GEMM_VM_CASE(30)
        GEMM_VM_CASE(31) GEMM_VM_CASE(32) GEMM_VM_CASE(33) GEMM_VM_CASE(34) GEMM_VM_CASE(35) GEMM_VM_CASE(36)
        GEMM_VM_CASE(37) GEMM_VM_CASE(38) GEMM_VM_CASE(39) GEMM_VM_CASE(40) GEMM_VM_CASE(41) GEMM_VM_CASE(42)
        GEMM_VM_CASE(43) GEMM_VM_CASE(44) GEMM_VM_CASE(45) GEMM_VM_CASE(46) GEMM_VM_CASE(47) GEMM_VM_CASE(48)
        default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
}
#undef GEMM_VM_CASE

__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ half8_t ds_read16(unsigned addr) {
    half8_t v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
    return v;
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 ds_read16u(unsigned addr) {
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
    return v;
}
template <int N>
__device__ __forceinline__ void wait_lds() {
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N > 15 ? 15 : N) : "memory");
}
// the same for a count known after unrolling
__device__ __forceinline__ void wait_lds_n(int n) {
    switch (n) {
        case 0: wait_lds<0>(); break;
        case 1: wait_lds<1>(); break;
        case 2: wait_lds<2>(); break;
        case 3: wait_lds<3>(); break;
        case 4: wait_lds<4>(); break;
        case 5: wait_lds<5>(); break;
        case 6: wait_lds<6>(); break;
        case 7: wait_lds<7>(); break;
        default: wait_lds<8>(); break;
    }
}
// make a value produced by an inline-asm LDS read depend on the wait above
template <typename V>
__device__ __forceinline__ void landed(V& v) {
    asm volatile("" : "+v"(v));
}

__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t mask, uint32_t magic) {
    // (w & mask) | magic in one VALU op; one scalar operand is allowed, so the
    // magic constant sits in a VGPR
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(mask), "v"(magic));
    return r;
}

// dequant_word (common.h) with the code extraction in v_and_or_b32: 13 VALU ops
__device__ __forceinline__ half8_t dequant_fast(uint32_t w, half2_t s, half2_t b, uint32_t m1024, uint32_t m64) {
    const half2_t k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
    const half2_t k64 = {(_Float16)64.0f, (_Float16)64.0f};
    const uint32_t w8 = w >> 8;
    const half2_t q04 = as_half2(and_or(w, 0x000F000Fu, m1024)) - k1024;
    const half2_t q15 = as_half2(and_or(w, 0x00F000F0u, m64)) - k64;
    const half2_t q26 = as_half2(and_or(w8, 0x000F000Fu, m1024)) - k1024;
    const half2_t q37 = as_half2(and_or(w8, 0x00F000F0u, m64)) - k64;
    const half2_t r0 = __builtin_elementwise_fma(q04, s, b);
    const half2_t r1 = __builtin_elementwise_fma(q15, s, b);
    const half2_t r2 = __builtin_elementwise_fma(q26, s, b);
    const half2_t r3 = __builtin_elementwise_fma(q37, s, b);
    return half8_t{r0.x, r0.y, r1.x, r1.y, r2.x, r2.y, r3.x, r3.y};
}

template <typename SB>
__device__ __forceinline__ float sb_bits_to_f32(uint32_t v);
template <>
__device__ __forceinline__ float sb_bits_to_f32<uint16_t>(uint32_t v) {
    return __uint_as_float(v << 16);
}
template <>
__device__ __forceinline__ float sb_bits_to_f32<float>(uint32_t v) {
    return __uint_as_float(v);
}
template <typename SB>
__device__ __forceinline__ uint32_t ds_read_sb(unsigned addr) {
    uint32_t v;
    if constexpr (sizeof(SB) == 2)
        asm volatile("ds_read_u16 %0, %1" : "=v"(v) : "v"(addr));
    else
        asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(addr));
    return v;
}

// One row tile x column slab, MT 32-row MFMA tiles.
template <typename SB, int kMode, int MT, int kV>
__device__ void gemm_tile(const GemmArgs& p, const Tile& tl, int slab, unsigned char* smem, const int* row_src,
                          const int* row_dst) {
    using G = Geo<kMode, kV>;
    using R = Ring<kMode, MT, kV>;
    constexpr int kW = G::kWavesV;
    constexpr int kNT = G::kThreadsV;
    constexpr int NS = G::NS;
    constexpr int D = R::D;
    constexpr int kWaveCols = G::kWaveCols;
    constexpr int kSlabCols = G::kSlabCols;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
    const int col = lane % 32, half = lane / 32;
    const int n_groups = p.K / kGroup;
    const bool sh = tl.group >= p.E;

    // ---- weight rows of this wave's stripes; a stripe past N reads a valid row and drops it ----
    // gate/up: stripe i < NS/2 = gate rows [c0 + 32 i, c0 + 32 i + 32), stripe
    // NS/2 + i = the same rows of up; down: stripe i = rows [c0 + 32 i, c0 + 32 i + 32)
    const int c0 = slab * kSlabCols + wave * kWaveCols;
    bool s_active[NS];
    int row0[NS];                 // first weight row of each stripe (0 for a dropped stripe)
    const char* q_row[NS];        // first packed row of each stripe
    const SB* arr_start[2 * NS];  // the group's rows of each scale/bias array (loads are clamped to them)
    const size_t grp = (size_t)(sh ? 0 : tl.group) * p.N;
#pragma unroll
    for (int i = 0; i < NS; i++) {
        const bool up = kMode == kGateUp && i >= NS / 2;
        const int r0 = c0 + 32 * (up ? i - NS / 2 : i);
        s_active[i] = r0 < p.N;
        row0[i] = s_active[i] ? r0 : 0;
        const QMatPtr& m = sh ? (up ? p.s1 : p.s0) : (up ? p.m1 : p.m0);
        q_row[i] = reinterpret_cast<const char*>(m.q + (grp + row0[i]) * (p.K / 8));
        arr_start[2 * i] = reinterpret_cast<const SB*>(m.s) + grp * n_groups;
        arr_start[2 * i + 1] = reinterpret_cast<const SB*>(m.b) + grp * n_groups;
    }

    // ---- activation chunk of each of this lane's direct loads per stage ----
    // load i of wave w is the stage's load j = i kW + w (if j < 4 MT); it fills
    // LDS chunks u = j * 64 + lane: row u / 8, stored position u % 8, which
    // holds the row's chunk (u % 8) ^ ((row / 2) % 8).  A row is 128 bytes (32
    // banks), so rows two apart start on the same bank; the XOR by row / 2
    // puts the 16 rows of one LDS read cycle on 16 distinct 16-byte bank groups
    constexpr int kAL = R::kALoadsMax;
    const char* a_src[kAL];
#pragma unroll
    for (int i = 0; i < kAL; i++) {
        const int j = min(i * kW + wave, 4 * MT - 1);
        const int u = j * kWave + lane;
        const int r = u >> 3, c = (u & 7) ^ ((r >> 1) & 7);
        const int src = row_src[r] >= 0 ? row_src[r] : row_src[0];
        a_src[i] = reinterpret_cast<const char*>(p.a + (size_t)src * p.lda) + c * 16;
    }

    // weights: load h of stripe i, lane L -> row 16 h + L / 4 of the stripe,
    // LDS position L % 4 of that row's 64 bytes, which holds the row's 16-byte
    // chunk c = (L % 4) ^ ((L / 16) % 4) (group kg + c / 2, half c % 2): the
    // XOR keeps the 16 rows that one LDS read cycle serves on distinct banks
    const int row_bytes = p.K / 2;
    const int b_chunk = (lane & 3) ^ ((lane >> 4) & 3);
    const int b_lane = (lane >> 2) * row_bytes + (b_chunk & 1) * 16;
    const int b_grp = b_chunk >> 1;

    // load q of stage kg (q < kAL: activations; then 2 per stripe on even stages)
    auto issue_one = [&](int kg, int slot, int q) {
        unsigned char* base = smem + R::slot_offset(slot);
        if (q < kAL) {
            const int j = q * kW + wave;
            if (j < 4 * MT)
                __builtin_amdgcn_global_load_lds(a_src[q] + kg * kStageRowBytes, base + j * kWave * 16, 16, 0, 0);
        } else if (q < kAL + 2 * NS && (kg & 1) == 0) {
            const int i = (q - kAL) >> 1, h = (q - kAL) & 1;
            const int g = min(kg + b_grp, n_groups - 1);
            __builtin_amdgcn_global_load_lds(q_row[i] + 16 * h * row_bytes + b_lane + g * 32,
                                             base + R::kABytes + ((wave * NS + i) * 2 + h) * kWave * 16, 16, 0, 0);
        }
    };
    auto issue = [&](int kg, int slot) {
#pragma unroll
        for (int q = 0; q < kAL + 2 * NS; q++) issue_one(kg, slot, q);
    };

    // ---- scales and biases of this wave's rows, one block of groups at a time ----
    // array i: (stripe i / 2, scale or bias); rows of a stripe are consecutive,
    // so array i of group block g0 is read dword by dword from where each of
    // the 32 rows' blocks starts
    constexpr int kBlk = (G::kSBRowDwords - 1) * 4 / (int)sizeof(SB);  // groups per block
    const int ng = n_groups;
    const size_t group_elems = (size_t)p.N * ng;
    unsigned char* sb_lds = smem + G::kRingBytes + wave * G::kSBWaveBytes;
    auto arr_row = [&](int i, int r) {  // first element of row r of the stripe, array i
        return arr_start[i] + (size_t)(row0[i / 2] + r) * ng;
    };
    auto load_scales = [&](int g0) {
#pragma unroll
        for (int i = 0; i < 2 * NS; i++) {
            const uintptr_t lo = reinterpret_cast<uintptr_t>(arr_start[i]) & ~uintptr_t(3);
            const uintptr_t hi = (reinterpret_cast<uintptr_t>(arr_start[i] + group_elems) - 4) & ~uintptr_t(3);
#pragma unroll
            for (int j = 0; j < G::kSBArrayDwords / kWave; j++) {
                const int u = j * kWave + lane;
                const int r = min(u / G::kSBRowDwords, 31), dw = u - r * G::kSBRowDwords;
                const uintptr_t row_blk = reinterpret_cast<uintptr_t>(arr_row(i, r) + g0) & ~uintptr_t(3);
                uintptr_t a = row_blk + (uintptr_t)dw * 4;
                a = a < lo ? lo : (a > hi ? hi : a);
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(a),
                                                 sb_lds + i * G::kSBArrayDwords * 4 + j * kWave * 4, 4, 0, 0);
            }
        }
    };
    // LDS byte offset of this lane's element g of block g0, array i
    auto sb_off = [&](int i, int g0, int g) -> unsigned {
        const uintptr_t e = reinterpret_cast<uintptr_t>(arr_row(i, col) + g0);
        return lds_addr(sb_lds) + i * G::kSBArrayDwords * 4 + col * G::kSBRowDwords * 4 + (unsigned)(e & 3) +
               (unsigned)(g - g0) * (unsigned)sizeof(SB);
    };

    floatx16 acc[NS][MT];
#pragma unroll
    for (int i = 0; i < NS; i++)
#pragma unroll
        for (int m = 0; m < MT; m++) acc[i][m] = floatx16{0};

    // LDS offsets of this lane's operand reads: weights of row `col`, chunk
    // 2 (kg % 2) + half, in the even slot of the pair
    const int b_row = R::kABytes + wave * NS * 2 * kWave * 16 + (col >> 4) * kWave * 16 + (col & 15) * 64;
    const unsigned b_off[2] = {(unsigned)(b_row + ((half ^ ((col >> 2) & 3)) * 16)),
                               (unsigned)(b_row + (((2 + half) ^ ((col >> 2) & 3)) * 16))};
    unsigned a_off[4];
#pragma unroll
    for (int s = 0; s < 4; s++) a_off[s] = col * kStageRowBytes + (((4 * half + s) ^ ((col >> 1) & 7)) * 16);

    // exponent-trick constants held in VGPRs (v_and_or_b32 takes one scalar)
    uint32_t m1024 = 0x64006400u, m64 = 0x54005400u;
    asm volatile("" : "+v"(m1024), "+v"(m64));

    // compute stage kg; the loads of stage nk (< 0: none) into slot nslot go
    // out one after each MFMA, so their issue hides under the matrix cores.
    // g_next >= 0: once this stage's scales are read, this wave's scale block
    // is refilled with the block starting at group g_next (each wave owns its
    // block, so no barrier is needed).
    auto compute = [&](int slot, int kg, int g0, int nk, int nslot, int g_next) {
        int q = 0;
        auto mfma_then_load = [&](const half8_t& a, const half8_t& w, floatx16& c) {
            c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, w, c, 0, 0, 0);
            if (q < kAL + 2 * NS && nk >= 0) issue_one(nk, nslot, q);
            q++;
        };
        const unsigned base = lds_addr(smem) + R::slot_offset(slot);
        const unsigned b_base = lds_addr(smem) + R::slot_offset(slot & ~1) + b_off[kg & 1];
        u32x4 bq[NS];
        uint32_t sv[NS], bv[NS];
#pragma unroll
        for (int i = 0; i < NS; i++) bq[i] = ds_read16u(b_base + i * 2 * kWave * 16);
#pragma unroll
        for (int i = 0; i < NS; i++) {
            sv[i] = ds_read_sb<SB>(sb_off(2 * i, g0, kg));
            bv[i] = ds_read_sb<SB>(sb_off(2 * i + 1, g0, kg));
        }
        half2_t sc[NS], bi[NS];
        auto scales_landed = [&]() {
#pragma unroll
            for (int i = 0; i < NS; i++) {
                landed(bq[i]);
                landed(sv[i]);
                landed(bv[i]);
                sc[i] = splat_half2(sb_bits_to_f32<SB>(sv[i]));
                bi[i] = splat_half2(sb_bits_to_f32<SB>(bv[i]));
            }
        };
        if constexpr (MT <= 2) {
            // short tiles: every LDS read of the stage goes out at once; the
            // weights are dequantised while the activation reads land
            half8_t a[4][MT];
#pragma unroll
            for (int s = 0; s < 4; s++)
#pragma unroll
                for (int m = 0; m < MT; m++) a[s][m] = ds_read16(base + a_off[s] + m * 32 * kStageRowBytes);
            wait_lds<4 * MT>();  // the weights and scales (the 3 NS oldest reads)
            scales_landed();
            if (g_next >= 0) load_scales(g_next);
            half8_t w[NS][4];
#pragma unroll
            for (int s = 0; s < 4; s++)
#pragma unroll
                for (int i = 0; i < NS; i++) w[i][s] = dequant_fast(word_of(bq[i], s), sc[i], bi[i], m1024, m64);
#pragma unroll
            for (int s = 0; s < 4; s++) {
                wait_lds_n((3 - s) * MT);
#pragma unroll
                for (int m = 0; m < MT; m++) {
                    landed(a[s][m]);
#pragma unroll
                    for (int i = 0; i < NS; i++) mfma_then_load(a[s][m], w[i][s], acc[i][m]);
                }
            }
        } else {
            // tall tiles: activation reads one K step ahead of the MFMAs, and
            // the next K step's weights dequantised between this step's MFMAs
            half8_t a_cur[MT], a_nxt[MT];
            half8_t w_cur[NS], w_nxt[NS];
#pragma unroll
            for (int m = 0; m < MT; m++) a_cur[m] = ds_read16(base + a_off[0] + m * 32 * kStageRowBytes);
#pragma unroll
            for (int s = 0; s < 4; s++) {
                if (s < 3) {
#pragma unroll
                    for (int m = 0; m < MT; m++) a_nxt[m] = ds_read16(base + a_off[s + 1] + m * 32 * kStageRowBytes);
                    wait_lds<MT>();
                } else {
                    wait_lds<0>();
                }
                if (s == 0) {
                    scales_landed();
                    if (g_next >= 0) load_scales(g_next);
#pragma unroll
                    for (int i = 0; i < NS; i++) w_cur[i] = dequant_fast(word_of(bq[i], 0), sc[i], bi[i], m1024, m64);
                }
#pragma unroll
                for (int m = 0; m < MT; m++) landed(a_cur[m]);
#pragma unroll
                for (int m = 0; m < MT; m++)
#pragma unroll
                    for (int i = 0; i < NS; i++) {
                        mfma_then_load(a_cur[m], w_cur[i], acc[i][m]);
                        if (m == 0 && s < 3)
                            w_nxt[i] = dequant_fast(word_of(bq[i], s + 1), sc[i], bi[i], m1024, m64);
                    }
                if (s < 3) {
#pragma unroll
                    for (int m = 0; m < MT; m++) a_cur[m] = a_nxt[m];
#pragma unroll
                    for (int i = 0; i < NS; i++) w_cur[i] = w_nxt[i];
                }
            }
        }
    };

    // ---- main loop: stage kg in slot kg % D; D - 2 stages in flight ----
    // A slot is refilled two iterations after its stage was computed, so the
    // weights of an even stage stay for the odd stage after it.  The first
    // scale block goes out before the ring, so waiting for stage 0 also waits
    // for it (loads of a wave complete in order); later blocks go out during
    // the last stage of the block before, so the ring never drains.
    // gate/up synchronises the workgroup once per pair of stages (an even
    // stage and the odd one after it): compute(kg) refills the slot of stage
    // kg - 2, which belongs to the pair before, so one barrier per pair covers
    // every refill, and the wave that finishes a stage first goes on to the
    // next instead of waiting at a barrier for its SIMD's other wave.  down,
    // with 8 stages per item at I = 512, waits per stage: waiting for a whole
    // pair at its start costs it more than the barriers saved.
    constexpr bool kPairs = kMode == kGateUp;
    static_assert(!kPairs || kBlk % 2 == 0, "a scale block starts on the first stage of a pair");
    load_scales(0);
#pragma unroll
    for (int j = 0; j < D - 2; j++)
        if (j < n_groups) issue(j, j);
    int g0 = 0;
    int slot = 0, fill = D - 2;  // slot of stage kg; slot that stage kg + D - 2 goes to
#pragma unroll 1
    for (int kg = 0; kg < n_groups; kg++) {
        if (!kPairs || (kg & 1) == 0) {
            // this wait covers stages kg .. last: the loads of the stages
            // issued after `last` (up to kg + D - 3, those that exist) may be
            // outstanding
            const int last = kPairs ? kg + 1 : kg;
            int younger = 0;
            if (kg == g0 + kBlk) {
                // first stage of the next scale block: the block went out in
                // the previous iteration, after the loads of stages up to
                // kg + D - 4 and before those of stage kg + D - 3, so all but
                // stage kg + D - 3's loads must have landed (and all of them
                // when that stage is one the wait covers)
                g0 = kg;
                if (kg + D - 3 > last && kg + D - 3 < n_groups) younger = R::loads(kg + D - 3);
            } else {
#pragma unroll
                for (int j = 1; j <= D - 3; j++)
                    if (kg + j > last && kg + j < n_groups) younger += R::loads(kg + j);
            }
            wait_vm(younger);
            barrier();  // every wave's stages kg .. last have landed; every wave is done with the stages before kg
        }
        const int g_next = kg + 1 == g0 + kBlk && kg + 1 < n_groups ? kg + 1 : -1;
        compute(slot, kg, g0, kg + D - 2 < n_groups ? kg + D - 2 : -1, fill, g_next);
        slot = slot == D - 1 ? 0 : slot + 1;
        fill = fill == D - 1 ? 0 : fill + 1;
    }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    barrier();  // the ring is free for the epilogue

    // ---- epilogues.  Accumulator element 4i+j of a lane: row 8i + 4*half + j, column `col` ----
    if constexpr (kMode == kGateUp) {
        // LDS tile [128 rows][kSlabCols columns] float16 (64 KB), columns in dequantisation order
        _Float16* ht = reinterpret_cast<_Float16*>(smem);
#pragma unroll
        for (int si = 0; si < NS / 2; si++) {
            if (!s_active[si]) continue;
            const int cl = wave * kWaveCols + 32 * si + col;  // column within the slab
            const int pos = (cl & ~7) + slot_of_column(cl & 7);
#pragma unroll
            for (int m = 0; m < MT; m++) {
#pragma unroll
                for (int i = 0; i < 4; i++) {
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        const int r = m * 32 + 8 * i + 4 * half + j;
                        ht[r * kSlabCols + pos] =
                            (_Float16)(silu(acc[si][m][4 * i + j]) * acc[si + NS / 2][m][4 * i + j]);
                    }
                }
            }
        }
        __syncthreads();
        constexpr int kChunks = kSlabCols / 8;  // 16-byte chunks per row
        const int col_chunks = min(kChunks, (p.N - slab * kSlabCols) / 8);
        for (int idx = tid; idx < tl.rows * kChunks; idx += kNT) {
            const int r = idx / kChunks, c = idx % kChunks;
            if (c < col_chunks) {
                const uint4 v = *reinterpret_cast<const uint4*>(ht + r * kSlabCols + c * 8);
                *reinterpret_cast<uint4*>(p.h + (size_t)(tl.row0 + r) * p.N + slab * kSlabCols + c * 8) = v;
            }
        }
    } else if constexpr (kMode == kDownY16) {
        // LDS tile [64 rows][kSlabCols columns] float16 in natural column order,
        // one half of the row tile at a time
        _Float16* yt = reinterpret_cast<_Float16*>(smem);
        constexpr int kChunks = kSlabCols / 8;
        const int col_chunks = min(kChunks, (p.N - slab * kSlabCols) / 8);
#pragma unroll
        for (int hh = 0; hh < (MT + 1) / 2; hh++) {
            if (hh > 0) __syncthreads();  // the previous half is stored
#pragma unroll
            for (int m = 2 * hh; m < 2 * hh + 2 && m < MT; m++) {
#pragma unroll
                for (int si = 0; si < NS; si++) {
                    if (!s_active[si]) continue;
                    const int cl = wave * kWaveCols + 32 * si + col;
#pragma unroll
                    for (int i = 0; i < 4; i++) {
#pragma unroll
                        for (int j = 0; j < 4; j++) {
                            const int r = (m - 2 * hh) * 32 + 8 * i + 4 * half + j;
                            yt[r * kSlabCols + cl] = (_Float16)acc[si][m][4 * i + j];
                        }
                    }
                }
            }
            __syncthreads();
            const int r_lo = 64 * hh, r_hi = min(tl.rows, 64 * hh + 64);
            for (int idx = tid; idx < (r_hi - r_lo) * kChunks; idx += kNT) {
                const int r = idx / kChunks, c = idx % kChunks;
                if (c < col_chunks) {
                    const uint4 v = *reinterpret_cast<const uint4*>(yt + r * kSlabCols + c * 8);
                    *reinterpret_cast<uint4*>(p.y16 + (size_t)row_dst[r_lo + r] * p.H + slab * kSlabCols + c * 8) = v;
                }
            }
        }
    } else {
#pragma unroll
        for (int m = 0; m < MT; m++) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const int r = m * 32 + 8 * i + 4 * half + j;
                    if (r < tl.rows) {
                        const int d = row_dst[r];
                        float* o = d < p.TK ? p.y_slot + (size_t)d * p.H
                                            : (p.y_shared ? p.y_shared + (size_t)(d - p.TK) * p.H : nullptr);
                        if (o) {
#pragma unroll
                            for (int si = 0; si < NS; si++)
                                if (s_active[si]) o[c0 + 32 * si + col] = acc[si][m][4 * i + j];
                        }
                    }
                }
            }
        }
    }
}

template <typename SB, int kMode, int kV>
__global__ __launch_bounds__((Geo<kMode, kV>::kThreadsV), (kV == kSmall ? 2 : 1)) void expert_gemm_kernel(GemmArgs p) {
    using G = Geo<kMode, kV>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[G::kRingBytes + G::kSBBytes];
    __shared__ int row_src[kTileRows];
    __shared__ int row_dst[kTileRows];

    // ---- workgroup -> (tile, slab): tiles dealt round-robin to the 8 XCDs in
    // map order (longest first), the slabs of a tile on one XCD ----
    const int xcd = blockIdx.x % 8, local = blockIdx.x / 8;
    const int tile = (local / p.slabs) * 8 + xcd;
    const int slab = local % p.slabs;
    if (tile >= *p.n_tiles) return;
    const Tile tl = p.tiles[tile];
    const int mt_count = min((tl.rows + 31) / 32, G::kMaxMT);

    // row r of the tile: where its activations come from and where its output goes
    // (-1: padding).  Grouped row gp < T*k is slot sorted_slot[gp] of token slot / k;
    // rows from T*k on are the shared expert's tokens.
    const int tid = threadIdx.x;
    if (kMode != kGateUp) {
        // down reads grouped row gp itself; only its epilogue needs the slot,
        // which lands by a direct load that the main loop's final wait covers
        if (tid < kTileRows) {
            const int r = tid, gp = tl.row0 + r;
            row_src[r] = r < tl.rows ? gp : -1;
            if (r < tl.rows && gp < p.TK)
                __builtin_amdgcn_global_load_lds(p.sorted_slot + gp, &row_dst[tid / kWave * kWave], 4, 0, 0);
            else
                row_dst[r] = r < tl.rows ? gp : -1;  // shared rows: slot T*k + t = gp
        }
    } else if (tid < kTileRows) {
        const int r = tid;
        int src = -1, dst = -1;
        if (r < tl.rows) {
            const int gp = tl.row0 + r;
            int slot, t;
            if (gp < p.TK) {
                slot = p.sorted_slot[gp];
                t = slot / p.k;
            } else {
                t = gp - p.TK;
                slot = p.TK + t;
            }
            src = kMode == kGateUp ? t : gp;
            dst = slot;
        }
        row_src[r] = src;
        row_dst[r] = dst;
    }
    __syncthreads();

    if constexpr (kV == kSmall) {
        if (mt_count == 1)
            gemm_tile<SB, kMode, 1, kV>(p, tl, slab, smem, row_src, row_dst);
        else
            gemm_tile<SB, kMode, 2, kV>(p, tl, slab, smem, row_src, row_dst);
    } else {
        switch (mt_count) {
            case 1: gemm_tile<SB, kMode, 1, kV>(p, tl, slab, smem, row_src, row_dst); break;
            case 2: gemm_tile<SB, kMode, 2, kV>(p, tl, slab, smem, row_src, row_dst); break;
            case 3: gemm_tile<SB, kMode, 3, kV>(p, tl, slab, smem, row_src, row_dst); break;
            default: gemm_tile<SB, kMode, kMT, kV>(p, tl, slab, smem, row_src, row_dst); break;
        }
    }
}

template <int kMode, int kV>
hipError_t launch_mode(GemmArgs a, int64_t max_tiles, int cols, bool sb_bf16, hipStream_t stream) {
    using G = Geo<kMode, kV>;
    a.slabs = (a.N + G::kSlabCols - 1) / G::kSlabCols;
    const int64_t grid = (max_tiles + 7) / 8 * 8 * a.slabs;
    (void)cols;
    if (sb_bf16)
        hipLaunchKernelGGL((expert_gemm_kernel<uint16_t, kMode, kV>), dim3((unsigned)grid), dim3(G::kThreadsV), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((expert_gemm_kernel<float, kMode, kV>), dim3((unsigned)grid), dim3(G::kThreadsV), 0,
                           stream, a);
    return hipGetLastError();
}

GemmArgs common_args(const GemmProblem& pr) {
    GemmArgs a = {};
    a.tiles = pr.tiles;
    a.n_tiles = pr.n_tiles;
    a.k = pr.k;
    a.TK = pr.T * pr.k;
    a.T = pr.T;
    a.H = pr.H;
    a.E = pr.E;
    a.sorted_slot = pr.sorted_slot;
    return a;
}

}  // namespace

hipError_t launch_gateup(const GemmProblem& pr, const _Float16* x16, _Float16* h, hipStream_t stream) {
    GemmArgs a = common_args(pr);
    a.a = x16;
    a.lda = pr.H;
    a.K = pr.H;
    a.N = pr.I;
    a.m0 = pr.experts.gate;
    a.m1 = pr.experts.up;
    a.s0 = pr.shared_w.gate;
    a.s1 = pr.shared_w.up;
    a.h = h;
    return pr.small_tiles ? launch_mode<kGateUp, kSmall>(a, pr.max_tiles, 0, pr.sb_bf16, stream)
                          : launch_mode<kGateUp, kWide>(a, pr.max_tiles, 0, pr.sb_bf16, stream);
}

hipError_t launch_down(const GemmProblem& pr, const _Float16* h, _Float16* y16, float* y_slot, float* y_shared,
                       hipStream_t stream) {
    GemmArgs a = common_args(pr);
    a.a = h;
    a.lda = pr.I;
    a.K = pr.I;
    a.N = pr.H;
    a.m0 = pr.experts.down;
    a.m1 = pr.experts.down;
    a.s0 = pr.shared_w.down;
    a.s1 = pr.shared_w.down;
    a.y16 = y16;
    a.y_slot = y_slot;
    a.y_shared = y_shared;
    if (!y16) return launch_mode<kDownStore, kBig>(a, pr.max_tiles, 0, pr.sb_bf16, stream);
    return pr.small_tiles ? launch_mode<kDownY16, kSmall>(a, pr.max_tiles, 0, pr.sb_bf16, stream)
                          : launch_mode<kDownY16, kWide>(a, pr.max_tiles, 0, pr.sb_bf16, stream);
}

}  // namespace bitmoe
