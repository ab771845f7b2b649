// Launchers of the gfx950 MoE kernels (internal to libbitmoe; the public ABI is
// include/moe.h).  Every launcher only enqueues on `stream` and returns the
// launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bitmoe {

// One stack of affine 4-bit matrices [n][N][K]: q [n][N][K/8] words,
// scale/bias [n][N][K/64].
struct QMatPtr {
    const uint32_t* q;
    const void* s;
    const void* b;
};

struct FfnPtr {
    QMatPtr gate, up, down;
};

// A row tile of one expert group: group g (0..E-1 routed, E shared), the first
// row in the grouped row space, the number of rows (1..kTileRows).
// Grouped row space: rows [0, T*k) are the routed slots in expert order
// (row p holds slot sorted_slot[p]); rows [T*k, T*k+T) are the shared expert's
// tokens in order.
struct Tile {
    int32_t group, row0, rows, pad;
};

constexpr int kTileRows = 128;  // rows of the grouped products handled by one workgroup

// Upper bound of the number of tiles for T tokens (host side).
// Tiles of the grouped rows at most: one partial tile per group plus full
// tiles of tile_rows rows.
inline int64_t max_tiles(int64_t T, int64_t k, int64_t E, bool shared, int tile_rows) {
    return (T * k + (shared ? T : 0)) / tile_rows + E + (shared ? 1 : 0) + 1;
}
// The layer's tile height: 64 rows when groups average at most 32 rows (small
// batches; the grouped products then run two workgroups per compute unit),
// else kTileRows.
inline bool layer_small_tiles(int64_t T, int64_t k, int64_t E) { return T * k <= 32 * E; }
inline int64_t max_tiles(int64_t T, int64_t k, int64_t E, bool shared) {
    return max_tiles(T, k, E, shared, kTileRows);
}

// Tokens (and experts) per workgroup of the layer's logits kernel (64: the
// LDS-staged kernel for large batches; 32: the register-fed one), and the
// number of K slices it splits the router product into (a power of two with
// H / (64 S) whole; more slices for small batches, so that a few hundred
// workgroups share the router's rows).  The logits workspace holds S x T x E
// floats.
inline int logits_tile(int64_t T) { return T >= 2048 ? 64 : 32; }
inline int logits_splits(int64_t T, int64_t H, int64_t E) {
    const int64_t tm = logits_tile(T);
    const int64_t blocks = ((T + tm - 1) / tm) * ((E + tm - 1) / tm);
    int S = 1;
    while (blocks * S < 256 && H % (64 * 2 * S) == 0) S *= 2;
    return S;
}

// An 8-bit router (four codes per word, low byte first; a scale and a bias per
// 64 columns) restored to bf16: out = bf16_nearest_even(fmaf(s, code, b)).
hipError_t launch_router_dequant(const uint32_t* q, const void* s, const void* b, bool sb_bf16, int E, int H,
                                 uint16_t* out, hipStream_t stream);

// Router + top-k in one kernel (32 tokens x all experts per workgroup).
hipError_t launch_router(const uint16_t* x, const uint16_t* wr, const float* logit_bias, int T, int H,
                         int E, int top_k, int32_t* topk_idx, float* topk_w, hipStream_t stream);

// The layer's spread router: logits [T][E] float32 (workspace), then one wave
// per token for the top-k, the expert histogram and the float16 copy of x.
// Counters that thousands of atomics hit are padded to one per 128-byte line
// (kCounterStride ints apart); launch_logits zeroes zero0[e * kCounterStride]
// and zero1[e * kCounterStride].
constexpr int kCounterStride = 32;
// The router is the bf16 matrix wr, or (wq non-null, batches below 2048 tokens)
// an 8-bit one that the logits kernel restores in registers; the staged kernel
// of larger batches needs wr.
hipError_t launch_logits(const uint16_t* x, const uint16_t* wr, const uint32_t* wq, const void* wsc, const void* wbi,
                         bool sb_bf16, const float* logit_bias, int T, int H, int E, float* logits, int32_t* zero0,
                         int32_t* zero1, hipStream_t stream);
// sgate (nullable, needs x16): the shared expert's gate vector [H] bf16; then
// shared_w [T] receives sigmoid(x[t] . sgate)
hipError_t launch_topk(const float* logits, const uint16_t* x, int T, int H, int E, int top_k, int32_t* topk_idx,
                       float* topk_w, int32_t* hist, _Float16* x16, const uint16_t* sgate, float* shared_w,
                       hipStream_t stream);

hipError_t launch_convert_x(const uint16_t* x, int T, int H, _Float16* x16, hipStream_t stream);

// Histogram, exclusive scan, scatter and tile map (one workgroup).
hipError_t launch_permute(const int32_t* topk_idx, int T, int k, int E, bool shared, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_slot, Tile* tiles, int32_t* n_tiles,
                          hipStream_t stream);

// Scan, tile map and scatter from the padded histogram of launch_topk; also
// writes counts [E] (nullable).  cursor: padded like the histogram, zeroed
// beforehand (launch_logits' zero1).  tiles64 (nullable): a second tile map of
// 64-row tiles over the same groups.
hipError_t launch_scatter(const int32_t* topk_idx, const int32_t* hist, int T, int k, int E, bool shared,
                          int32_t* counts, int32_t* offsets, int32_t* cursor, int32_t* sorted_slot, Tile* tiles,
                          int32_t* n_tiles, int tile_rows, Tile* tiles64, int32_t* n_tiles64,
                          hipStream_t stream);

// Tile map only, from caller-provided offsets [E+1].
hipError_t launch_tiles(const int32_t* offsets, int T, int k, int E, bool shared, Tile* tiles,
                        int32_t* n_tiles, hipStream_t stream);

struct GemmProblem {
    int T, H, E, k, I;
    bool shared;
    bool sb_bf16;
    const Tile* tiles;
    const int32_t* n_tiles;
    int64_t max_tiles;
    const int32_t* sorted_slot;  // [T*k]
    FfnPtr experts, shared_w;
    bool small_tiles;  // every tile has at most 64 rows: two workgroups per compute unit
};

// gate/up products with SwiGLU: h [T*k + T][I] float16 in grouped row order,
// 8-column blocks in dequantisation order.
hipError_t launch_gateup(const GemmProblem& p, const _Float16* x16, _Float16* h, hipStream_t stream);

// down products; each row goes to its slot's row (un-permute on store).
// y16 != nullptr: y16 [T*k + T][H] float16, routed slots then the shared
// expert's tokens (the layer path; launch_combine16 finishes it).  Else
// y_slot [T*k][H] float32 and, when not null, y_shared [T][H] float32.
hipError_t launch_down(const GemmProblem& p, const _Float16* h, _Float16* y16, float* y_slot, float* y_shared,
                       hipStream_t stream);

// Decode path (T <= kDecodeMaxT, I <= kMaxDecodeI): one kernel per call whose
// router workgroups publish the logits (each expert workgroup selects its
// token's top k from them), whose gate/up workgroups
// publish h, and whose down workgroups combine into `out` with float32
// atomics.  It uses the decode region at the start of the workspace
// (kDecodeRegionBytes, the same offsets for every dims, zero before the first
// call): control words, then the values handed between workgroups.
constexpr int kDecodeMaxT = 4;
constexpr int kMaxDecodeI = 4096;
constexpr int kDecodeXchReplicas = 32;  // copies of the logits, each read by a share of the expert workgroups
constexpr int kDecodeControlBytes = 16384;
constexpr size_t kDecodeXchBytes = (size_t)kDecodeXchReplicas * kDecodeMaxT * 256 * 8;
constexpr size_t kDecodeHBytes = (size_t)kDecodeMaxT * (8 + 1) * kMaxDecodeI * 8;
constexpr size_t kDecodeRegionBytes = kDecodeControlBytes + kDecodeXchBytes + kDecodeHBytes;

struct DecodeArgs {
    int T, H, E, top_k, I;
    int router_wgs, gateup_wgs, down_wgs;  // workgroups per role (decode_*_wgs)
    const uint16_t* x;
    const uint16_t* router;
    const uint32_t* router_q8;   // or an 8-bit router, restored in the router workgroups
    const void* router_s;        // its scales and biases [E][H/64] (the experts' dtype)
    const void* router_b;
    const float* logit_bias;
    unsigned* ctl;               // control words and counters
    unsigned long long* xch64;   // kDecodeXchReplicas copies of [kDecodeMaxT][256] {epoch, logit}
    unsigned long long* h64;     // [slots][I] {epoch, h}; slots = T*k routed, then T shared
    int32_t* idx_out;            // optional copies of the routing
    float* w_out;
    int32_t* counts_out;
    float* out;                  // [T][H]
    FfnPtr experts, shared;      // shared.gate.q == nullptr: no shared expert
    const uint16_t* shared_gate; // [H] bf16 gate vector of the shared expert, or nullptr (weight 1)
};

// Persistent multi-layer decode (one token through L stacked layers in one
// launch, each layer reading the RMS-normalised residual stream): a grid of
// kStackGrid workgroups, all resident at once, spread by the hardware over the
// device's kStackXcds XCDs (kStackGrid / kStackXcds on each).  Each XCD carries
// one routed slot of the layer; its workgroups hand values to each other
// through words in that XCD's L2 (the local region below), and the XCDs meet
// once per layer, in the cross region.  Both regions sit at fixed offsets after
// the one-layer decode region and are zero before the first call.  Limits:
// T = 1, H <= kStackMaxH, I a power of two in [64, kStackMaxI], top_k <= 8.
constexpr int kStackGrid = 256;
constexpr int kStackXcds = 8;
constexpr int kStackMaxH = 2048;
constexpr int kStackMaxI = 512;
// Copies of each XCD-local vector, so that each copy has 8 of the XCD's 32
// workgroups polling it.
constexpr int kStackLocalCopies = 4;
constexpr int kStackXWords = kStackMaxH / 8 * 3;   // the stream: 3 words {16-bit tag, 3 bf16} per 8 columns
constexpr int kStackShWords = kStackMaxI / 16;     // an XCD's share of the shared expert's h, float16 pairs
// one XCD's local words of one parity: [copies][stream] [copies][logits]
// [copies][routed h] [copies][shared h share], each vector a whole number of
// 128-byte lines
constexpr size_t kStackLocWords =
    (size_t)kStackLocalCopies * (kStackXWords + 256 + kStackMaxI / 2 + kStackShWords);
constexpr size_t kStackLocalWords = (size_t)kStackXcds * 2 * kStackLocWords;
// cross region: [2 parities][XCD][workgroup of the XCD][64 owned columns] {epoch, float32}
constexpr size_t kStackPartWords = (size_t)2 * kStackGrid * 64;
constexpr size_t kStackRegionBytes = 8 * (kStackLocalWords + kStackPartWords);
// every region at fixed offsets at the start of the workspace
constexpr size_t kFixedRegionBytes = kDecodeRegionBytes + kStackRegionBytes;

struct QMatStride {
    int64_t q, s, b;  // bytes from one layer's tensor to the next layer's
};
struct FfnStride {
    QMatStride gate, up, down;
};

struct StackArgs {
    int H, E, top_k, I, I_shared, L;
    const uint16_t* x_in;   // [H] bf16, the first layer's input
    uint16_t* x_out;        // [H] bf16, x after the last layer (may alias x_in)
    float* layer_out;       // [L][H] float32 layer outputs, or nullptr
    uint16_t* layer_x;      // [L][H] bf16 residual stream entering every layer, or nullptr
    uint16_t* layer_in;     // [L][H] bf16 normalised input of every layer, or nullptr
    const uint16_t* norm_w;  // [H] bf16 normalisation weight of layer 0 (layer l at + l * norm_stride), or nullptr
    int64_t norm_stride;
    int32_t* idx_out;       // [L][top_k] routing per layer, or nullptr
    float* w_out;           // [L][top_k], or nullptr
    const uint16_t* router;  // layer 0; layer l at + l * router_stride bytes
    int64_t router_stride;
    const float* logit_bias;  // or nullptr
    int64_t bias_stride;
    FfnPtr experts, shared;   // shared.gate.q == nullptr: no shared expert
    FfnStride experts_stride, shared_stride;
    unsigned* ctl;               // the workspace's control words
    unsigned long long* local;   // [kStackXcds][2 parities][kStackLocWords] XCD-local words
    unsigned long long* part;    // [2 parities][kStackXcds][kStackGrid / kStackXcds][64] partial sums
};

// Workgroups the stack kernel can keep resident on the current device (0 on error).
int stack_resident_capacity();
hipError_t launch_decode_stack(const StackArgs& a, bool sb_bf16, hipStream_t stream);

int decode_router_wgs(int E);
int decode_gateup_wgs(int T, int k, bool shared, int I);
int decode_down_wgs(int T, int k, bool shared, int H);
hipError_t launch_decode(const DecodeArgs& a, bool sb_bf16, hipStream_t stream);

// out[t] = sum_j topk_w[t][j] * y_slot[t*k+j] + s[t] * y_shared[t] (y_shared
// nullable); s = shared_w (nullable: 1)
hipError_t launch_combine(const float* y_slot, const float* topk_w, const float* y_shared, const float* shared_w,
                          int T, int H, int k, float* out, hipStream_t stream);

// out[t] = sum_j topk_w[t][j] * y16[t*k+j] (+ s[t] * y16[T*k+t] when shared; s =
// shared_w, nullable: 1), float32.  out16 != nullptr: out16 = bf16(residual +
// that sum) instead (residual nullable, may alias out16).
hipError_t launch_combine16(const _Float16* y16, const float* topk_w, bool shared, const float* shared_w, int T,
                            int H, int k, float* out, const uint16_t* residual, uint16_t* out16, hipStream_t stream);

// out16 [T][H] = bf16(residual + y) (residual nullable, may alias out16)
hipError_t launch_residual_bf16(const float* y, const uint16_t* residual, int T, int H, uint16_t* out16,
                                hipStream_t stream);

// bytes (a multiple of 16) from p on set to zero, by a kernel
hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream);

// Decode attention with grouped-query KV sharing (two passes: per-run
// partials, then their merge).  q [B][Hq][D], k/v [B][Hkv][S_max][D] bf16,
// seq_len [B]; part: B * Hkv * n_split partials of G * D + 32 floats (o [G][D],
// then m and l, 16 slots each); out [B][Hq][D] float32.  c = scale * log2(e).
// With fused set (every workgroup of the grid resident at once), one kernel
// also merges: part then holds {epoch, float32} words, cnt 64 control words
// per (sequence, KV head) (word 0: the epoch; zero before the first call);
// err is set if a poll timed out.
struct GqaArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* seq_len;
    float* part;
    float* out;
    unsigned* cnt;
    unsigned* err;
    int B, Hq, Hkv, G, D, S_max, n_split;
    int fused;
    float c;
};

// rows of the cache one pass-1 workgroup covers (the run length of a partial)
int gqa_rows_per_split(int D);
// workgroups of the fused kernel the current device holds at once (0 on error)
int gqa_fused_capacity(int D);
// events (nullable): 3 events recorded before pass 1, between the passes and after pass 2
hipError_t launch_gqa_decode(const GqaArgs& a, hipStream_t stream, hipEvent_t* events);

// shared_w[t] = sigmoid(x[t] . g), x [T][H] and g [H] bf16
hipError_t launch_shared_gate(const uint16_t* x, const uint16_t* g, int T, int H, float* shared_w,
                              hipStream_t stream);

}  // namespace bitmoe
