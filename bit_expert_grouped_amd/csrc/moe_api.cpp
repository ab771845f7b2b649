// C ABI of the gfx950 MoE layer (include/moe.h): host-side validation,
// workspace layout and kernel dispatch on the caller's stream.  Nothing here
// allocates, frees or synchronises; every check runs before the first launch.
#include "../../include/moe.h"

#include <stdint.h>

#include <mutex>

#include "common.h"
#include "kernels.h"

using namespace bitmoe;

namespace {

constexpr int kMaxH = 16384;
constexpr int kMaxI = 4096;
constexpr int64_t kMaxT = int64_t(1) << 22;
constexpr int64_t kMaxPermuteSlots = int64_t(1) << 22;  // T * top_k of one moe_permute call

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

moe_status check_dims(const moe_dims* d) {
    if (!d) return MOE_ERR_NULL;
    if (d->T < 0 || d->H <= 0 || d->E <= 0 || d->top_k <= 0 || d->I <= 0 || d->I_shared < 0 || d->group <= 0)
        return MOE_ERR_SHAPE;
    if (d->top_k > d->E) return MOE_ERR_SHAPE;
    if (d->H % d->group != 0 || d->I % d->group != 0 || d->I_shared % d->group != 0) return MOE_ERR_SHAPE;
    if (d->sb_dtype != MOE_BF16 && d->sb_dtype != MOE_F32) return MOE_ERR_SHAPE;
    if (d->out_dtype != MOE_BF16 && d->out_dtype != MOE_F32) return MOE_ERR_SHAPE;
    if (d->group != kGroup) return MOE_ERR_UNSUPPORTED;
    if (d->E > kMaxE || d->top_k > kMaxTopK) return MOE_ERR_UNSUPPORTED;
    if (d->H > kMaxH || d->I > kMaxI) return MOE_ERR_UNSUPPORTED;
    if (d->I_shared != 0 && d->I_shared != d->I) return MOE_ERR_UNSUPPORTED;
    if ((int64_t)d->T > kMaxT) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

// Workspace layout; every region starts on a 256-byte boundary.
struct Layout {
    size_t ctl, xch, hbuf, stack;                        // decode regions (fixed offsets)
    size_t x16, h, y16, logits, hist, cursor;            // prefill buffers
    size_t idx, w, counts, offsets, sorted, tiles, n_tiles, tiles64, n_tiles64, shared_w, yacc, router16, total;
};

size_t up256(size_t v) { return (v + 255) & ~size_t(255); }

Layout layout_of(const moe_dims* d) {
    const size_t T = (size_t)d->T, H = (size_t)d->H, k = (size_t)d->top_k, E = (size_t)d->E, I = (size_t)d->I;
    const bool shared = d->I_shared > 0;
    Layout L;
    size_t o = 0;
    // decode region: the same offsets for every dims, so that what one call
    // leaves there is what the next call expects, whatever the dims of either
    L.ctl = o;
    o += kDecodeControlBytes;
    L.xch = o;
    o += kDecodeXchBytes;
    L.hbuf = o;
    o = up256(o + kDecodeHBytes);
    L.stack = o;  // exchange words of the persistent multi-layer decode kernel
    o = up256(o + kStackRegionBytes);
    L.x16 = o;
    o = up256(o + T * H * 2);
    L.h = o;
    o = up256(o + (T * k + (shared ? T : 0)) * I * 2);
    L.y16 = o;
    o = up256(o + (T * k + (shared ? T : 0)) * H * 2);
    L.logits = o;
    o = up256(o + (size_t)logits_splits(d->T, d->H, d->E) * T * E * 4);
    L.hist = o;
    o = up256(o + E * kCounterStride * 4);
    L.cursor = o;
    o = up256(o + E * kCounterStride * 4);
    L.idx = o;
    o = up256(o + T * k * 4);
    L.w = o;
    o = up256(o + T * k * 4);
    L.counts = o;
    o = up256(o + E * 4);
    L.offsets = o;
    o = up256(o + (E + 1) * 4);
    L.sorted = o;
    o = up256(o + T * k * 4);
    L.tiles = o;
    o = up256(o + (size_t)max_tiles(d->T, d->top_k, d->E, shared, 64) * sizeof(Tile));  // room for either height
    L.n_tiles = o;
    o = up256(o + 4);
    L.tiles64 = o;
    o = up256(o + (size_t)max_tiles(d->T, d->top_k, d->E, shared, 64) * sizeof(Tile));
    L.n_tiles64 = o;
    o = up256(o + 4);
    L.shared_w = o;  // the shared expert's weight per token under its optional gate
    o = up256(o + T * 4);
    L.yacc = o;  // decode with a bf16 output: the float32 layer output before the residual add
    o = up256(o + (T <= (size_t)kDecodeMaxT ? T * H * 4 : 0));
    L.router16 = o;  // an 8-bit router restored to bf16 [E][H]
    o = up256(o + E * H * 2);
    L.total = o;
    return L;
}

template <typename T>
T* at(void* ws, size_t off) {
    return reinterpret_cast<T*>(static_cast<unsigned char*>(ws) + off);
}

moe_status check_ws(const moe_dims* d, const void* ws, size_t ws_bytes) {
    if (!ws) return MOE_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return MOE_ERR_ALIGN;
    if (ws_bytes < layout_of(d).total) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

moe_status check_qmat(const moe_qmat& m) {
    if (!m.q || !m.scale || !m.bias) return MOE_ERR_NULL;
    if (!aligned16(m.q) || !aligned16(m.scale) || !aligned16(m.bias)) return MOE_ERR_ALIGN;
    return MOE_OK;
}

moe_status check_ffn(const moe_ffn* f) {
    if (!f) return MOE_ERR_NULL;
    moe_status s;
    if ((s = check_qmat(f->gate)) != MOE_OK) return s;
    if ((s = check_qmat(f->up)) != MOE_OK) return s;
    return check_qmat(f->down);
}

moe_status check_ptrs(std::initializer_list<const void*> ptrs) {
    for (const void* p : ptrs)
        if (!p) return MOE_ERR_NULL;
    for (const void* p : ptrs)
        if (!aligned16(p)) return MOE_ERR_ALIGN;
    return MOE_OK;
}

moe_status check_opt(std::initializer_list<const void*> ptrs) {
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MOE_ERR_ALIGN;
    return MOE_OK;
}

QMatPtr to_ptr(const moe_qmat& m) { return QMatPtr{m.q, m.scale, m.bias}; }

FfnPtr to_ptr(const moe_ffn* f) {
    if (!f) return FfnPtr{};
    return FfnPtr{to_ptr(f->gate), to_ptr(f->up), to_ptr(f->down)};
}

#define MOE_TRY(expr)                          \
    do {                                       \
        moe_status _s = (expr);                \
        if (_s != MOE_OK) return _s;           \
    } while (0)

#define HIP_TRY(expr)                          \
    do {                                       \
        if ((expr) != hipSuccess) return MOE_ERR_HIP; \
    } while (0)

}  // namespace

extern "C" {

size_t moe_workspace_size(const moe_dims* dims) {
    if (check_dims(dims) != MOE_OK) return 0;
    return layout_of(dims).total;
}

const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULL: return "a required pointer is NULL";
        case MOE_ERR_SHAPE: return "inconsistent or non-positive sizes";
        case MOE_ERR_UNSUPPORTED: return "sizes outside the supported limits";
        case MOE_ERR_ALIGN: return "a pointer is not 16-byte aligned (workspace: 256-byte)";
        case MOE_ERR_WORKSPACE: return "workspace smaller than moe_workspace_size()";
        case MOE_ERR_HIP: return "a kernel launch failed";
    }
    return "unknown status";
}

moe_status moe_route(const moe_dims* d, const uint16_t* x, const uint16_t* router, const float* logit_bias,
                     int32_t* topk_idx, float* topk_w, hipStream_t stream) {
    MOE_TRY(check_dims(d));
    if (d->T == 0) return MOE_OK;
    MOE_TRY(check_ptrs({x, router, topk_idx, topk_w}));
    MOE_TRY(check_opt({logit_bias}));
    HIP_TRY(launch_router(x, router, logit_bias, d->T, d->H, d->E, d->top_k, topk_idx, topk_w, stream));
    return MOE_OK;
}

moe_status moe_permute(const moe_dims* d, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                       int32_t* sorted_slot, void* ws, size_t ws_bytes, hipStream_t stream) {
    MOE_TRY(check_dims(d));
    if (d->T == 0) return MOE_OK;
    // one workgroup sorts every slot of this call, so its run time grows with
    // T * top_k; the header bounds that product
    if ((int64_t)d->T * d->top_k > kMaxPermuteSlots) return MOE_ERR_UNSUPPORTED;
    MOE_TRY(check_ptrs({topk_idx, counts, offsets, sorted_slot}));
    MOE_TRY(check_ws(d, ws, ws_bytes));
    const Layout L = layout_of(d);
    HIP_TRY(launch_permute(topk_idx, d->T, d->top_k, d->E, d->I_shared > 0, counts, offsets, sorted_slot,
                           at<Tile>(ws, L.tiles), at<int32_t>(ws, L.n_tiles), stream));
    return MOE_OK;
}

moe_status moe_expert_ffn(const moe_dims* d, const uint16_t* x, const int32_t* offsets, const int32_t* sorted_slot,
                          const moe_ffn* experts, const moe_ffn* shared, float* y_slot, float* y_shared, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
    MOE_TRY(check_dims(d));
    if (d->T == 0) return MOE_OK;
    MOE_TRY(check_ptrs({x, offsets, sorted_slot, y_slot}));
    MOE_TRY(check_ffn(experts));
    const bool use_shared = shared != nullptr && y_shared != nullptr;
    if (use_shared) {
        if (d->I_shared == 0) return MOE_ERR_SHAPE;
        MOE_TRY(check_ffn(shared));
        MOE_TRY(check_ptrs({y_shared}));
    }
    MOE_TRY(check_ws(d, ws, ws_bytes));
    const Layout L = layout_of(d);
    GemmProblem p;
    p.T = d->T;
    p.H = d->H;
    p.E = d->E;
    p.k = d->top_k;
    p.I = d->I;
    p.shared = use_shared;
    p.sb_bf16 = d->sb_dtype == MOE_BF16;
    p.tiles = at<Tile>(ws, L.tiles);
    p.n_tiles = at<int32_t>(ws, L.n_tiles);
    p.max_tiles = max_tiles(d->T, d->top_k, d->E, use_shared);
    p.sorted_slot = sorted_slot;
    p.small_tiles = false;  // caller-provided offsets: no bound on rows per expert
    p.experts = to_ptr(experts);
    p.shared_w = use_shared ? to_ptr(shared) : FfnPtr{};
    _Float16* x16 = at<_Float16>(ws, L.x16);
    _Float16* h = at<_Float16>(ws, L.h);
    HIP_TRY(launch_tiles(offsets, d->T, d->top_k, d->E, use_shared, at<Tile>(ws, L.tiles),
                         at<int32_t>(ws, L.n_tiles), stream));
    HIP_TRY(launch_convert_x(x, d->T, d->H, x16, stream));
    HIP_TRY(launch_gateup(p, x16, h, stream));
    HIP_TRY(launch_down(p, h, nullptr, y_slot, use_shared ? y_shared : nullptr, stream));
    return MOE_OK;
}

moe_status moe_combine(const moe_dims* d, const float* y_slot, const float* topk_w, const float* y_shared, void* out,
                       hipStream_t stream) {
    MOE_TRY(check_dims(d));
    if (d->T == 0) return MOE_OK;
    MOE_TRY(check_ptrs({y_slot, topk_w, out}));
    MOE_TRY(check_opt({y_shared}));
    HIP_TRY(launch_combine(y_slot, topk_w, y_shared, nullptr, d->T, d->H, d->top_k, static_cast<float*>(out),
                           stream));
    return MOE_OK;
}

moe_status moe_combine_gated(const moe_dims* d, const float* y_slot, const float* topk_w, const float* y_shared,
                             const float* shared_w, void* out, hipStream_t stream) {
    MOE_TRY(check_dims(d));
    if (d->T == 0) return MOE_OK;
    MOE_TRY(check_ptrs({y_slot, topk_w, out}));
    MOE_TRY(check_opt({y_shared, shared_w}));
    HIP_TRY(launch_combine(y_slot, topk_w, y_shared, shared_w, d->T, d->H, d->top_k, static_cast<float*>(out),
                           stream));
    return MOE_OK;
}

moe_status moe_shared_gate(const moe_dims* d, const uint16_t* x, const uint16_t* gate, float* shared_w,
                           hipStream_t stream) {
    MOE_TRY(check_dims(d));
    if (d->T == 0) return MOE_OK;
    MOE_TRY(check_ptrs({x, gate, shared_w}));
    HIP_TRY(launch_shared_gate(x, gate, d->T, d->H, shared_w, stream));
    return MOE_OK;
}

moe_status moe_router_dequant(const moe_dims* d, const uint32_t* router_q8, const void* scale, const void* bias,
                              uint16_t* router_out, hipStream_t stream) {
    MOE_TRY(check_dims(d));
    MOE_TRY(check_ptrs({router_q8, scale, bias, router_out}));
    HIP_TRY(launch_router_dequant(router_q8, scale, bias, d->sb_dtype == MOE_BF16, d->E, d->H, router_out, stream));
    return MOE_OK;
}

namespace {

const char* const kPrefillStages[] = {"router", "topk", "permute", "gate_up", "down", "combine"};
constexpr int kPrefillStageCount = 6;
const char* const kDecodeStages[] = {"decode_layer"};
constexpr int kDecodeStageCount = 1;

bool use_decode_path(const moe_dims* d) { return d->T <= kDecodeMaxT && d->I <= kMaxDecodeI; }

int stage_count(const moe_dims* d) { return use_decode_path(d) ? kDecodeStageCount : kPrefillStageCount; }

// out16 != nullptr: the bf16 residual-stream output (out unused), out16 =
// bf16(residual + layer); else the float32 output `out`
moe_status layer_impl(const moe_dims* d, const moe_weights* wts, const uint16_t* x, void* out,
                      int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out, void* ws, size_t ws_bytes,
                      hipStream_t stream, hipEvent_t* events, int32_t n_events, const uint16_t* residual = nullptr,
                      uint16_t* out16 = nullptr, bool validate_only = false) {
    MOE_TRY(check_dims(d));
    if (d->out_dtype != (out16 ? MOE_BF16 : MOE_F32)) return MOE_ERR_UNSUPPORTED;
    if (d->T == 0) return MOE_OK;
    if (!wts) return MOE_ERR_NULL;
    // exactly one router: the bf16 matrix, or the 8-bit one restored per call
    if (wts->router && wts->router_q8) return MOE_ERR_SHAPE;
    MOE_TRY(check_ptrs({x, out16 ? static_cast<const void*>(out16) : out,
                        wts->router_q8 ? static_cast<const void*>(wts->router_q8) : wts->router}));
    if (wts->router_q8) MOE_TRY(check_ptrs({wts->router_scale, wts->router_bias}));
    MOE_TRY(check_opt({residual}));
    MOE_TRY(check_opt({wts->logit_bias, topk_idx_out, topk_w_out, counts_out}));
    MOE_TRY(check_ffn(&wts->experts));
    const bool shared = d->I_shared > 0;
    if (shared) {
        MOE_TRY(check_ffn(&wts->shared));
    } else if (wts->shared.gate.q || wts->shared_expert_gate) {
        return MOE_ERR_SHAPE;
    }
    MOE_TRY(check_opt({wts->shared_expert_gate}));
    MOE_TRY(check_ws(d, ws, ws_bytes));
    const int n_stages = stage_count(d);
    if (events) {
        if (n_events < n_stages + 1) return MOE_ERR_SHAPE;
        for (int i = 0; i <= n_stages; i++)
            if (!events[i]) return MOE_ERR_NULL;
    }
    if (validate_only) return MOE_OK;
    const Layout L = layout_of(d);
    auto mark = [&](int i) -> bool { return !events || hipEventRecord(events[i], stream) == hipSuccess; };
    // the router the kernels score with; an 8-bit one is restored first, inside
    // the first stage
    const uint16_t* router = wts->router_q8 ? at<uint16_t>(ws, L.router16) : wts->router;
    auto restore_router = [&]() -> hipError_t {
        if (!wts->router_q8) return hipSuccess;
        return launch_router_dequant(wts->router_q8, wts->router_scale, wts->router_bias, d->sb_dtype == MOE_BF16,
                                     d->E, d->H, at<uint16_t>(ws, L.router16), stream);
    };

    if (use_decode_path(d)) {
        DecodeArgs a;
        a.T = d->T;
        a.H = d->H;
        a.E = d->E;
        a.top_k = d->top_k;
        a.I = d->I;
        a.router_wgs = decode_router_wgs(d->E);
        a.gateup_wgs = decode_gateup_wgs(d->T, d->top_k, shared, d->I);
        a.down_wgs = decode_down_wgs(d->T, d->top_k, shared, d->H);
        a.x = x;
        // the router workgroups restore an 8-bit router themselves
        a.router = wts->router;
        a.router_q8 = wts->router_q8;
        a.router_s = wts->router_scale;
        a.router_b = wts->router_bias;
        a.logit_bias = wts->logit_bias;
        a.ctl = at<unsigned>(ws, L.ctl);
        a.xch64 = at<unsigned long long>(ws, L.xch);
        a.h64 = at<unsigned long long>(ws, L.hbuf);
        a.idx_out = topk_idx_out;
        a.w_out = topk_w_out;
        a.counts_out = counts_out;
        a.out = out16 ? at<float>(ws, L.yacc) : static_cast<float*>(out);
        a.experts = to_ptr(&wts->experts);
        a.shared = shared ? to_ptr(&wts->shared) : FfnPtr{};
        a.shared_gate = wts->shared_expert_gate;
        if (!mark(0)) return MOE_ERR_HIP;
        HIP_TRY(launch_decode(a, d->sb_dtype == MOE_BF16, stream));
        if (out16) HIP_TRY(launch_residual_bf16(a.out, residual, d->T, d->H, out16, stream));
        if (!mark(1)) return MOE_ERR_HIP;
        return MOE_OK;
    }

    int32_t* idx = topk_idx_out ? topk_idx_out : at<int32_t>(ws, L.idx);
    float* w = topk_w_out ? topk_w_out : at<float>(ws, L.w);
    int32_t* counts = counts_out ? counts_out : at<int32_t>(ws, L.counts);
    int32_t* offsets = at<int32_t>(ws, L.offsets);
    int32_t* sorted = at<int32_t>(ws, L.sorted);
    _Float16* x16 = at<_Float16>(ws, L.x16);
    _Float16* h = at<_Float16>(ws, L.h);
    _Float16* y16 = at<_Float16>(ws, L.y16);
    float* o = static_cast<float*>(out);

    GemmProblem p;
    p.T = d->T;
    p.H = d->H;
    p.E = d->E;
    p.k = d->top_k;
    p.I = d->I;
    p.shared = shared;
    p.sb_bf16 = d->sb_dtype == MOE_BF16;
    p.tiles = at<Tile>(ws, L.tiles);
    p.n_tiles = at<int32_t>(ws, L.n_tiles);
    // small batches: 64-row tiles, two workgroups per compute unit
    const bool small = layer_small_tiles(d->T, d->top_k, d->E);
    const int tile_rows = small ? 64 : kTileRows;
    p.max_tiles = max_tiles(d->T, d->top_k, d->E, shared, tile_rows);
    p.sorted_slot = sorted;
    p.small_tiles = small;
    p.experts = to_ptr(&wts->experts);
    p.shared_w = shared ? to_ptr(&wts->shared) : FfnPtr{};

    if (!mark(0)) return MOE_ERR_HIP;
    int32_t* hist = at<int32_t>(ws, L.hist);
    int32_t* cursor = at<int32_t>(ws, L.cursor);
    // an 8-bit router: the register-fed logits kernel restores it in place;
    // the staged one (large batches) reads the copy restored into the workspace
    const bool restore_in_logits = wts->router_q8 && logits_tile(d->T) != 64;
    if (!restore_in_logits) HIP_TRY(restore_router());
    HIP_TRY(launch_logits(x, restore_in_logits ? nullptr : router, restore_in_logits ? wts->router_q8 : nullptr,
                          wts->router_scale, wts->router_bias, d->sb_dtype == MOE_BF16, wts->logit_bias, d->T, d->H,
                          d->E, at<float>(ws, L.logits), hist, cursor, stream));
    if (!mark(1)) return MOE_ERR_HIP;
    float* shared_w = wts->shared_expert_gate ? at<float>(ws, L.shared_w) : nullptr;
    HIP_TRY(launch_topk(at<float>(ws, L.logits), x, d->T, d->H, d->E, d->top_k, idx, w, hist, x16,
                        wts->shared_expert_gate, shared_w, stream));
    if (!mark(2)) return MOE_ERR_HIP;
    // large batches: down (short K, so per-tile overheads weigh more) runs on
    // a second map of 64-row tiles with two workgroups per compute unit
    HIP_TRY(launch_scatter(idx, hist, d->T, d->top_k, d->E, shared, counts, offsets, cursor, sorted,
                           at<Tile>(ws, L.tiles), at<int32_t>(ws, L.n_tiles), tile_rows,
                           small ? nullptr : at<Tile>(ws, L.tiles64), small ? nullptr : at<int32_t>(ws, L.n_tiles64),
                           stream));
    if (!mark(3)) return MOE_ERR_HIP;
    HIP_TRY(launch_gateup(p, x16, h, stream));
    if (!mark(4)) return MOE_ERR_HIP;
    GemmProblem pd = p;
    if (!small) {
        pd.tiles = at<Tile>(ws, L.tiles64);
        pd.n_tiles = at<int32_t>(ws, L.n_tiles64);
        pd.max_tiles = max_tiles(d->T, d->top_k, d->E, shared, 64);
        pd.small_tiles = true;
    }
    HIP_TRY(launch_down(pd, h, y16, nullptr, nullptr, stream));
    if (!mark(5)) return MOE_ERR_HIP;
    HIP_TRY(launch_combine16(y16, w, shared, shared_w, d->T, d->H, d->top_k, o, residual, out16, stream));
    if (!mark(6)) return MOE_ERR_HIP;
    return MOE_OK;
}

}  // namespace

moe_status moe_layer(const moe_dims* d, const moe_weights* wts, const uint16_t* x, void* out, int32_t* topk_idx_out,
                     float* topk_w_out, int32_t* counts_out, void* ws, size_t ws_bytes, hipStream_t stream) {
    return layer_impl(d, wts, x, out, topk_idx_out, topk_w_out, counts_out, ws, ws_bytes, stream, nullptr, 0);
}

moe_status moe_layer_residual(const moe_dims* d, const moe_weights* wts, const uint16_t* x, const uint16_t* residual,
                              uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream) {
    MOE_TRY(check_dims(d));
    if (d->out_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (d->T == 0) return MOE_OK;
    if (!out) return MOE_ERR_NULL;
    return layer_impl(d, wts, x, nullptr, nullptr, nullptr, nullptr, ws, ws_bytes, stream, nullptr, 0, residual, out);
}

moe_status moe_layer_events(const moe_dims* d, const moe_weights* wts, const uint16_t* x, void* out,
                            int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out, void* ws, size_t ws_bytes,
                            hipStream_t stream, hipEvent_t* events, int32_t n_events) {
    if (!events) return MOE_ERR_NULL;
    return layer_impl(d, wts, x, out, topk_idx_out, topk_w_out, counts_out, ws, ws_bytes, stream, events,
                      n_events);
}

}  // extern "C"

namespace {

// ------------------------------------------------------- moe_decode_stack

bool stride16(int64_t v) { return v % 16 == 0; }

moe_status check_stride(const moe_qmat_stride& s) {
    return stride16(s.q) && stride16(s.scale) && stride16(s.bias) ? MOE_OK : MOE_ERR_ALIGN;
}

QMatStride to_stride(const moe_qmat_stride& s) { return QMatStride{s.q, s.scale, s.bias}; }

FfnStride to_stride(const moe_ffn_stride& s) { return FfnStride{to_stride(s.gate), to_stride(s.up), to_stride(s.down)}; }

// strides of tensors stacked contiguously over layers: one layer's size
moe_layer_strides contiguous_strides(const moe_dims* d) {
    const int64_t H = d->H, I = d->I, E = d->E, Is = d->I_shared, sb = d->sb_dtype == MOE_BF16 ? 2 : 4;
    auto mat = [&](int64_t n, int64_t N, int64_t K) {
        return moe_qmat_stride{n * N * K / 2, n * N * (K / kGroup) * sb, n * N * (K / kGroup) * sb};
    };
    moe_layer_strides s;
    s.router = E * H * 2;
    s.logit_bias = E * 4;
    s.norm_weight = H * 2;
    s.experts = moe_ffn_stride{mat(E, I, H), mat(E, I, H), mat(E, H, I)};
    s.shared = moe_ffn_stride{mat(1, Is, H), mat(1, Is, H), mat(1, H, Is)};
    return s;
}

// workgroups of the stack kernel the current device holds at once (looked up
// once per device; a property of the device and the kernel)
std::mutex g_capacity_mu;
int g_capacity[64];

int resident_capacity() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lock(g_capacity_mu);
    if (g_capacity[dev] == 0) g_capacity[dev] = stack_resident_capacity();
    return g_capacity[dev];
}

}  // namespace

extern "C" {

moe_status moe_decode_stack(const moe_dims* d, const moe_weights* wts, const uint16_t* norm_weight,
                            const moe_layer_strides* strides, int32_t n_layers, const uint16_t* x_in,
                            uint16_t* x_out, uint16_t* layer_x, uint16_t* layer_in, float* layer_out,
                            int32_t* topk_idx_out, float* topk_w_out, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
    MOE_TRY(check_dims(d));
    if (d->T == 0) return MOE_OK;
    if (n_layers < 1) return MOE_ERR_SHAPE;
    if (d->T != 1 || d->out_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    // one routed slot per XCD; the intermediate dim a power of two, so that an
    // XCD's eighth of the shared expert sits inside one scale group
    if (d->H > kStackMaxH || d->I > kStackMaxI || d->top_k > kStackXcds) return MOE_ERR_UNSUPPORTED;
    if (d->I < kGroup || (d->I & (d->I - 1)) != 0) return MOE_ERR_UNSUPPORTED;
    if (!wts) return MOE_ERR_NULL;
    if (wts->router_q8 || wts->shared_expert_gate) return MOE_ERR_UNSUPPORTED;
    MOE_TRY(check_ptrs({x_in, x_out, wts->router}));
    MOE_TRY(check_opt({wts->logit_bias, norm_weight, layer_out, layer_x, layer_in, topk_idx_out, topk_w_out}));
    MOE_TRY(check_ffn(&wts->experts));
    const bool shared = d->I_shared > 0;
    if (shared) {
        MOE_TRY(check_ffn(&wts->shared));
    } else if (wts->shared.gate.q) {
        return MOE_ERR_SHAPE;
    }
    const moe_layer_strides st = strides ? *strides : contiguous_strides(d);
    if (!stride16(st.router) || !stride16(st.norm_weight) || st.logit_bias % 4 != 0) return MOE_ERR_ALIGN;
    MOE_TRY(check_stride(st.experts.gate));
    MOE_TRY(check_stride(st.experts.up));
    MOE_TRY(check_stride(st.experts.down));
    MOE_TRY(check_stride(st.shared.gate));
    MOE_TRY(check_stride(st.shared.up));
    MOE_TRY(check_stride(st.shared.down));
    MOE_TRY(check_ws(d, ws, ws_bytes));
    if (resident_capacity() < kStackGrid) return MOE_ERR_UNSUPPORTED;
    const Layout L = layout_of(d);
    StackArgs a;
    a.H = d->H;
    a.E = d->E;
    a.top_k = d->top_k;
    a.I = d->I;
    a.I_shared = d->I_shared;
    a.L = n_layers;
    a.x_in = x_in;
    a.x_out = x_out;
    a.layer_out = layer_out;
    a.layer_x = layer_x;
    a.layer_in = layer_in;
    a.norm_w = norm_weight;
    a.norm_stride = st.norm_weight;
    a.idx_out = topk_idx_out;
    a.w_out = topk_w_out;
    a.router = wts->router;
    a.router_stride = st.router;
    a.logit_bias = wts->logit_bias;
    a.bias_stride = st.logit_bias;
    a.experts = to_ptr(&wts->experts);
    a.shared = shared ? to_ptr(&wts->shared) : FfnPtr{};
    a.experts_stride = to_stride(st.experts);
    a.shared_stride = to_stride(st.shared);
    a.ctl = at<unsigned>(ws, L.ctl);
    unsigned long long* sw = at<unsigned long long>(ws, L.stack);
    a.local = sw;
    a.part = sw + kStackLocalWords;
    HIP_TRY(launch_decode_stack(a, d->sb_dtype == MOE_BF16, stream));
    return MOE_OK;
}

}  // extern "C"

namespace {

// ------------------------------------------------------- moe_layer_no_alloc
// The workspace of moe_layer_no_alloc: a file-scope device array, one copy per
// device, held until the process ends.  Host code never passes `scratch`
// itself to a kernel (in host code the name only stands for the device
// variable); it looks up each device's address once with hipGetSymbolAddress
// and uses that.
constexpr size_t kNoAllocBytes = MOE_NO_ALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device, once looked up
bool g_scratch_ready[kMaxDevices];  // its decode region was cleared by a call outside graph capture

// The current device's scratch address (looked up on the device's first call).
moe_status scratch_address(int* dev_out, void** ptr_out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *dev_out = dev;
    *ptr_out = g_scratch_ptr[dev];
    return MOE_OK;
}

// The layer's workspace contract needs zero decode regions before the first
// call (the rest of the workspace is written before it is read in every call).
// Until a call outside graph capture has cleared it, every call clears it
// first with a kernel on its stream; a captured clearing kernel then runs on
// every replay, which leaves the region as consistent as a first call does.
moe_status scratch_prepare(int dev, void* ptr, hipStream_t stream) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ready[dev]) return MOE_OK;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return MOE_ERR_HIP;
    if (launch_zero(ptr, kFixedRegionBytes, stream) != hipSuccess) return MOE_ERR_HIP;
    if (cs == hipStreamCaptureStatusNone) g_scratch_ready[dev] = true;
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_layer_no_alloc(const moe_dims* d, const moe_weights* wts, const uint16_t* x, void* out,
                              int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out, hipStream_t stream) {
    MOE_TRY(check_dims(d));
    if (d->out_dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
    if (d->T == 0) return MOE_OK;
    if (layout_of(d).total > kNoAllocBytes) return MOE_ERR_WORKSPACE;
    int dev = 0;
    void* ws = nullptr;
    MOE_TRY(scratch_address(&dev, &ws));
    // every argument is checked before anything is enqueued
    MOE_TRY(layer_impl(d, wts, x, out, topk_idx_out, topk_w_out, counts_out, ws, kNoAllocBytes, stream, nullptr, 0,
                       nullptr, nullptr, true));
    MOE_TRY(scratch_prepare(dev, ws, stream));
    return layer_impl(d, wts, x, out, topk_idx_out, topk_w_out, counts_out, ws, kNoAllocBytes, stream, nullptr, 0);
}

int32_t moe_layer_stage_count(const moe_dims* d) {
    if (check_dims(d) != MOE_OK || d->T == 0) return 0;
    return stage_count(d);
}

const char* moe_layer_stage_name(const moe_dims* d, int32_t i) {
    const int32_t n = moe_layer_stage_count(d);
    if (i < 0 || i >= n) return nullptr;
    return use_decode_path(d) ? kDecodeStages[i] : kPrefillStages[i];
}

// ---------------------------------------------------------------- decode attention

}  // extern "C"

namespace {

constexpr int64_t kMaxGqaSeq = int64_t(1) << 24;

moe_status check_gqa_dims(const moe_gqa_dims* d) {
    if (!d) return MOE_ERR_NULL;
    if (d->B < 0 || d->n_q_heads <= 0 || d->n_kv_heads <= 0 || d->head_dim <= 0 || d->max_seq <= 0)
        return MOE_ERR_SHAPE;
    if (d->n_q_heads % d->n_kv_heads != 0) return MOE_ERR_SHAPE;
    if (d->n_q_heads / d->n_kv_heads > 16) return MOE_ERR_UNSUPPORTED;
    if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256) return MOE_ERR_UNSUPPORTED;
    if (d->B > 65535 || d->n_kv_heads > 65535 || (int64_t)d->max_seq > kMaxGqaSeq) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

int gqa_splits(const moe_gqa_dims* d) {
    const int r = gqa_rows_per_split(d->head_dim);
    return (d->max_seq + r - 1) / r;
}

// workspace: the partials (the fused merge's layout, 128 + 6 G D bytes per
// run: a flag line, then 48 bytes per 8-column item; the second kernel's plain
// float32 layout, 4 G D + 128 bytes per run, fits in it), then 256 bytes of
// control words per (sequence, KV head) (the fused merge's epoch), then the
// timeout word
size_t gqa_part_bytes(const moe_gqa_dims* d) {
    const size_t G = (size_t)(d->n_q_heads / d->n_kv_heads);
    const size_t bytes = (size_t)d->B * d->n_kv_heads * (size_t)gqa_splits(d) * (128 + 6 * G * d->head_dim);
    return (bytes + 255) & ~(size_t)255;
}

size_t gqa_ws_bytes(const moe_gqa_dims* d) {
    return gqa_part_bytes(d) + (size_t)d->B * d->n_kv_heads * 256 + 256;
}

// workgroups of the fused attention kernel the current device holds at once
int gqa_capacity(int D) {
    static std::mutex mu;
    static int cap[64][3];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    const int i = D == 64 ? 0 : D == 128 ? 1 : 2;
    std::lock_guard<std::mutex> lock(mu);
    if (cap[dev][i] == 0) cap[dev][i] = gqa_fused_capacity(D);
    return cap[dev][i];
}

}  // namespace

extern "C" {

size_t moe_gqa_workspace_size(const moe_gqa_dims* dims) {
    if (check_gqa_dims(dims) != MOE_OK) return 0;
    return gqa_ws_bytes(dims);
}

}  // extern "C"

namespace {

moe_status gqa_impl(const moe_gqa_dims* d, const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                    const int32_t* seq_len, float scale, float* out, void* ws, size_t ws_bytes, hipStream_t stream,
                    hipEvent_t* events) {
    MOE_TRY(check_gqa_dims(d));
    const float c = scale * 1.4426950408889634f;  // scores in log2 units
    if (!(c == c) || c - c != 0.0f) return MOE_ERR_SHAPE;  // NaN or infinite
    if (d->B == 0) return MOE_OK;
    MOE_TRY(check_ptrs({q, k_cache, v_cache, out}));
    if (!seq_len) return MOE_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(seq_len) & 3u) != 0) return MOE_ERR_ALIGN;
    if (!ws) return MOE_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return MOE_ERR_ALIGN;
    if (ws_bytes < gqa_ws_bytes(d)) return MOE_ERR_WORKSPACE;
    GqaArgs a;
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.seq_len = seq_len;
    a.part = static_cast<float*>(ws);
    a.cnt = reinterpret_cast<unsigned*>(static_cast<char*>(ws) + gqa_part_bytes(d));
    a.err = reinterpret_cast<unsigned*>(static_cast<char*>(ws) + gqa_part_bytes(d) + (size_t)d->B * d->n_kv_heads * 256);
    a.out = out;
    a.B = d->B;
    a.Hq = d->n_q_heads;
    a.Hkv = d->n_kv_heads;
    a.G = d->n_q_heads / d->n_kv_heads;
    a.D = d->head_dim;
    a.S_max = d->max_seq;
    a.n_split = gqa_splits(d);
    a.fused = moe_gqa_decode_kernels(d) == 1 ? 1 : 0;
    a.c = c;
    HIP_TRY(launch_gqa_decode(a, stream, events));
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_gqa_decode(const moe_gqa_dims* d, const uint16_t* q, const uint16_t* k_cache,
                          const uint16_t* v_cache, const int32_t* seq_len, float scale, float* out, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
    return gqa_impl(d, q, k_cache, v_cache, seq_len, scale, out, ws, ws_bytes, stream, nullptr);
}

int32_t moe_gqa_decode_kernels(const moe_gqa_dims* d) {
    if (check_gqa_dims(d) != MOE_OK || d->B == 0) return 0;
    return (int64_t)gqa_splits(d) * d->n_kv_heads * d->B <= (int64_t)gqa_capacity(d->head_dim) ? 1 : 2;
}

moe_status moe_gqa_decode_events(const moe_gqa_dims* d, const uint16_t* q, const uint16_t* k_cache,
                                 const uint16_t* v_cache, const int32_t* seq_len, float scale, float* out, void* ws,
                                 size_t ws_bytes, hipStream_t stream, hipEvent_t* events, int32_t n_events) {
    if (!events) return MOE_ERR_NULL;
    if (n_events < 3) return MOE_ERR_SHAPE;
    return gqa_impl(d, q, k_cache, v_cache, seq_len, scale, out, ws, ws_bytes, stream, events);
}

}  // extern "C"
