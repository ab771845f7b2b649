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
//   - A workgroup (4 waves) owns one row tile of one expert group (<= 128 rows,
//     from the device tile map) and one slab of output columns.  The grid is
//     sized from T alone; workgroups read the tile count written by the permute
//     kernel and leave when there is no work.  Work ids are handed out in
//     contiguous ranges per XCD (workgroups are dispatched round-robin over the
//     8 XCDs), so the slabs of one tile and the tiles of one expert share an L2.
//   - Activations (float16) are staged through LDS, one 64-column group per
//     stage, double-buffered, rows XOR-swizzled so the 32-row MFMA operand reads
//     are bank-conflict free.  Gate/up gathers token rows through the slot
//     permutation (the permuted activation matrix is never materialised).
//   - Weights never touch LDS: every lane of the 32x32x16 MFMA B operand needs 8
//     consecutive K values of one output row, which is exactly one packed word.
//     A lane loads 4 words (16 bytes) per group, dequantises them in registers
//     (dequant_word: 13 VALU ops per 8 weights) and feeds four MFMAs.  Weight
//     loads run two groups ahead of the math.
//   - gate/up: a wave computes a 32-column stripe of gate and the same stripe of
//     up, so SwiGLU is elementwise on the accumulators; h goes to global memory
//     as float16 through an LDS transpose (16-byte stores).
//   - down: a wave computes two 32-column stripes; the epilogue either scales by
//     the routing weight and adds into the float32 output with atomics (the
//     fused combine) or stores the slot rows.
#include "common.h"
#include "kernels.h"

namespace bitmoe {

namespace {

constexpr int kThreads = 256;
constexpr int kMT = kTileRows / 32;          // 32-row MFMA tiles per row tile
constexpr int kStageRowBytes = kGroup * 2;   // one group of float16 per row
constexpr int kStageBytes = kTileRows * kStageRowBytes;

enum Mode { kGateUp = 0, kDownCombine = 1, kDownStore = 2 };

struct GemmArgs {
    const Tile* tiles;
    const int32_t* n_tiles;
    int slabs;
    const _Float16* a;  // x16 [T][H] (gate/up) or h [rows][I] (down)
    int lda;
    int K;              // contraction length
    int N;              // output columns of each group's matrices
    int k, TK, H;
    const int32_t* sorted_slot;
    QMatPtr m0, m1;     // routed stacks used by stripe 0 / stripe 1
    QMatPtr s0, s1;     // shared-expert matrices used by stripe 0 / stripe 1
    int E;
    _Float16* h;        // gate/up output [rows][N]
    const float* topk_w;
    float* out;
    float* y_slot;
    float* y_shared;
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

template <typename SB>
struct BRegs {
    uint4 q0, q1;
    SB s0, b0, s1, b1;
};

template <typename SB>
__device__ __forceinline__ void load_b(BRegs<SB>& r, const Stripe<SB>& st0, const Stripe<SB>& st1, int kg,
                                       int half) {
    r.q0 = st0.q[kg * 2 + half];
    r.q1 = st1.q[kg * 2 + half];
    r.s0 = st0.s[kg];
    r.b0 = st0.b[kg];
    r.s1 = st1.s[kg];
    r.b1 = st1.b[kg];
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int s) {
    return s == 0 ? v.x : (s == 1 ? v.y : (s == 2 ? v.z : v.w));
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

template <typename SB, int kMode>
__global__ __launch_bounds__(kThreads) void expert_gemm_kernel(GemmArgs p) {
    constexpr int kWaveCols = kMode == kGateUp ? 32 : 64;  // output columns per wave
    constexpr int kStripeStep = kMode == kGateUp ? 0 : 32;  // row offset of stripe 1
    constexpr int kSlabCols = 4 * kWaveCols;

    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kStageBytes];
    __shared__ int row_src[kTileRows];
    __shared__ int row_t[kTileRows];
    __shared__ int row_slot[kTileRows];
    __shared__ float row_w[kTileRows];

    // ---- work id -> (tile, slab), contiguous ranges per XCD ----
    const int n_work = *p.n_tiles * p.slabs;
    const int xcd = blockIdx.x % 8, local = blockIdx.x / 8;
    const int per = (n_work + 7) / 8;
    const int work = xcd * per + local;
    if (local >= per || work >= n_work) return;
    const int slab = work % p.slabs;
    const Tile tl = p.tiles[work / p.slabs];
    const int mt_count = (tl.rows + 31) / 32;
    const int rows_pad = mt_count * 32;

    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const int col = lane % 32, half = lane / 32;

    if (tid < kTileRows) {
        const int r = tid;
        int src = -1, t = 0, slot = -1;
        float w = 1.0f;
        if (r < tl.rows) {
            const int gp = tl.row0 + r;
            if (gp < p.TK) {
                slot = p.sorted_slot[gp];
                t = slot / p.k;
                if (kMode == kDownCombine) w = p.topk_w[slot];
            } else {
                t = gp - p.TK;
            }
            src = kMode == kGateUp ? t : gp;
        }
        row_src[r] = src;
        row_t[r] = t;
        row_slot[r] = slot;
        row_w[r] = w;
    }
    __syncthreads();

    // ---- operands of this wave ----
    const int c0 = slab * kSlabCols + wave * kWaveCols;
    const bool active = c0 < p.N;
    const int brow = active ? c0 + col : 0;
    const Stripe<SB> st0 = stripe_of<SB>(p.m0, p.s0, tl.group, p.E, p.N, p.K, brow);
    const Stripe<SB> st1 = stripe_of<SB>(p.m1, p.s1, tl.group, p.E, p.N, p.K, brow + (active ? kStripeStep : 0));
    const int n_groups = p.K / kGroup;

    // A staging: thread -> 16-byte chunk (tid % 8) of rows tid/8 + 32j
    const int a_chunk = tid % 8;
    const int a_row0 = tid / 8;
    const _Float16* a_ptr[kMT];
#pragma unroll
    for (int j = 0; j < kMT; j++) {
        const int r = a_row0 + 32 * j;
        const int src = row_src[r];
        a_ptr[j] = src >= 0 ? p.a + (size_t)src * p.lda + a_chunk * 8 : nullptr;
    }
    uint4 a_regs[kMT];
    auto load_a = [&](int kg) {
#pragma unroll
        for (int j = 0; j < kMT; j++) {
            const int r = a_row0 + 32 * j;
            if (r < rows_pad && a_ptr[j]) {
                a_regs[j] = *reinterpret_cast<const uint4*>(a_ptr[j] + kg * kGroup);
            } else {
                a_regs[j] = make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int j = 0; j < kMT; j++) {
            const int r = a_row0 + 32 * j;
            if (r < rows_pad) {
                unsigned char* dst = smem + buf * kStageBytes + r * kStageRowBytes + ((a_chunk ^ (r & 7)) * 16);
                *reinterpret_cast<uint4*>(dst) = a_regs[j];
            }
        }
    };

    floatx16 acc0[kMT], acc1[kMT];
#pragma unroll
    for (int m = 0; m < kMT; m++) {
        acc0[m] = floatx16{0};
        acc1[m] = floatx16{0};
    }

    BRegs<SB> bc = {}, bn = {}, bnn = {};
    if (active) {
        load_b(bc, st0, st1, 0, half);
        if (n_groups > 1) load_b(bn, st0, st1, 1, half);
    }
    load_a(0);
    store_a(0);
    if (n_groups > 1) load_a(1);

    for (int kg = 0; kg < n_groups; kg++) {
        __syncthreads();
        const int buf = kg & 1;
        if (kg + 1 < n_groups) store_a(buf ^ 1);
        if (kg + 2 < n_groups) {
            load_a(kg + 2);
            if (active) load_b(bnn, st0, st1, kg + 2, half);
        }
        if (active) {
            const half2_t sc0 = splat_half2(sb_to_f32<SB>(bc.s0));
            const half2_t bi0 = splat_half2(sb_to_f32<SB>(bc.b0));
            const half2_t sc1 = splat_half2(sb_to_f32<SB>(bc.s1));
            const half2_t bi1 = splat_half2(sb_to_f32<SB>(bc.b1));
            const unsigned char* abase = smem + buf * kStageBytes;
#pragma unroll
            for (int s = 0; s < 4; s++) {
                const half8_t w0 = dequant_word(word_of(bc.q0, s), sc0, bi0);
                const half8_t w1 = dequant_word(word_of(bc.q1, s), sc1, bi1);
                const int chunk = 4 * half + s;
#pragma unroll
                for (int m = 0; m < kMT; m++) {
                    if (m < mt_count) {
                        const int r = m * 32 + col;
                        const half8_t av = *reinterpret_cast<const half8_t*>(
                            abase + r * kStageRowBytes + ((chunk ^ (r & 7)) * 16));
                        acc0[m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, w0, acc0[m], 0, 0, 0);
                        acc1[m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, w1, acc1[m], 0, 0, 0);
                    }
                }
            }
        }
        bc = bn;
        bn = bnn;
    }

    // ---- epilogues.  Accumulator element 4i+j of a lane: row 8i + 4*half + j, column `col` ----
    if constexpr (kMode == kGateUp) {
        __syncthreads();  // every wave is done reading the activation stages
        // LDS tile [128 rows][kSlabCols columns] float16, columns in dequantisation order
        _Float16* ht = reinterpret_cast<_Float16*>(smem);
        if (active) {
            const int cl = wave * kWaveCols + col;  // column within the slab
            const int pos = (cl & ~7) + slot_of_column(cl & 7);
#pragma unroll
            for (int m = 0; m < kMT; m++) {
                if (m < mt_count) {
#pragma unroll
                    for (int i = 0; i < 4; i++) {
#pragma unroll
                        for (int j = 0; j < 4; j++) {
                            const int r = m * 32 + 8 * i + 4 * half + j;
                            const float g = acc0[m][4 * i + j];
                            const float u = acc1[m][4 * i + j];
                            ht[r * kSlabCols + pos] = (_Float16)(silu(g) * u);
                        }
                    }
                }
            }
        }
        __syncthreads();
        constexpr int kChunks = kSlabCols / 8;  // 16-byte chunks per row
        const int col_chunks = min(kChunks, (p.N - slab * kSlabCols) / 8);
        for (int idx = tid; idx < tl.rows * kChunks; idx += kThreads) {
            const int r = idx / kChunks, c = idx % kChunks;
            if (c < col_chunks) {
                const uint4 v = *reinterpret_cast<const uint4*>(ht + r * kSlabCols + c * 8);
                *reinterpret_cast<uint4*>(p.h + (size_t)(tl.row0 + r) * p.N + slab * kSlabCols + c * 8) = v;
            }
        }
    } else {
        if (active) {
#pragma unroll
            for (int m = 0; m < kMT; m++) {
                if (m < mt_count) {
#pragma unroll
                    for (int i = 0; i < 4; i++) {
#pragma unroll
                        for (int j = 0; j < 4; j++) {
                            const int r = m * 32 + 8 * i + 4 * half + j;
                            if (r < tl.rows) {
                                const int n0 = c0 + col;
                                const int n1 = c0 + kStripeStep + col;
                                if constexpr (kMode == kDownCombine) {
                                    float* o = p.out + (size_t)row_t[r] * p.H;
                                    const float w = row_w[r];
                                    atomicAdd(o + n0, w * acc0[m][4 * i + j]);
                                    atomicAdd(o + n1, w * acc1[m][4 * i + j]);
                                } else {
                                    const int slot = row_slot[r];
                                    float* o = slot >= 0 ? p.y_slot + (size_t)slot * p.H
                                                         : p.y_shared + (size_t)row_t[r] * p.H;
                                    if (slot >= 0 || p.y_shared) {
                                        o[n0] = acc0[m][4 * i + j];
                                        o[n1] = acc1[m][4 * i + j];
                                    }
                                }
                            }
                        }
                    }
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_gateup(const GemmProblem& pr, const _Float16* x16, _Float16* h, hipStream_t stream) {
    GemmArgs a = {};
    a.a = x16;
    a.lda = pr.H;
    a.K = pr.H;
    a.N = pr.I;
    a.m0 = pr.experts.gate;
    a.m1 = pr.experts.up;
    a.s0 = pr.shared_w.gate;
    a.s1 = pr.shared_w.up;
    a.h = h;
    a.tiles = pr.tiles;
    a.n_tiles = pr.n_tiles;
    a.slabs = (pr.I + 127) / 128;
    a.k = pr.k;
    a.TK = pr.T * pr.k;
    a.H = pr.H;
    a.E = pr.E;
    a.sorted_slot = pr.sorted_slot;
    const int64_t grid = (pr.max_tiles * a.slabs + 7) / 8 * 8;
    if (pr.sb_bf16) {
        hipLaunchKernelGGL((expert_gemm_kernel<uint16_t, kGateUp>), dim3((unsigned)grid), dim3(kThreads), 0,
                           stream, a);
    } else {
        hipLaunchKernelGGL((expert_gemm_kernel<float, kGateUp>), dim3((unsigned)grid), dim3(kThreads), 0,
                           stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_down(const GemmProblem& pr, const _Float16* h, const float* topk_w, bool combine, float* out,
                       float* y_slot, float* y_shared, hipStream_t stream) {
    GemmArgs a = {};
    a.a = h;
    a.lda = pr.I;
    a.K = pr.I;
    a.N = pr.H;
    a.m0 = pr.experts.down;
    a.m1 = pr.experts.down;
    a.s0 = pr.shared_w.down;
    a.s1 = pr.shared_w.down;
    a.topk_w = topk_w;
    a.out = out;
    a.y_slot = y_slot;
    a.y_shared = y_shared;
    a.tiles = pr.tiles;
    a.n_tiles = pr.n_tiles;
    a.slabs = (pr.H + 255) / 256;
    a.k = pr.k;
    a.TK = pr.T * pr.k;
    a.H = pr.H;
    a.E = pr.E;
    a.sorted_slot = pr.sorted_slot;
    const int64_t grid = (pr.max_tiles * a.slabs + 7) / 8 * 8;
    if (combine) {
        if (pr.sb_bf16)
            hipLaunchKernelGGL((expert_gemm_kernel<uint16_t, kDownCombine>), dim3((unsigned)grid), dim3(kThreads),
                               0, stream, a);
        else
            hipLaunchKernelGGL((expert_gemm_kernel<float, kDownCombine>), dim3((unsigned)grid), dim3(kThreads), 0,
                               stream, a);
    } else {
        if (pr.sb_bf16)
            hipLaunchKernelGGL((expert_gemm_kernel<uint16_t, kDownStore>), dim3((unsigned)grid), dim3(kThreads), 0,
                               stream, a);
        else
            hipLaunchKernelGGL((expert_gemm_kernel<float, kDownStore>), dim3((unsigned)grid), dim3(kThreads), 0,
                               stream, a);
    }
    return hipGetLastError();
}

}  // namespace bitmoe
