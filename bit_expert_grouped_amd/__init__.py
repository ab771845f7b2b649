"""Python binding of libbitmoe (include/moe.h): the gfx950 4-bit grouped-expert MoE layer.

Argument marshalling only: torch tensors in device memory are turned into
pointers and the current torch stream into a ``hipStream_t``; every step of
the layer runs in the HIP kernels of ``libbitmoe.so``.  There is no fallback:
if the library is missing or a call fails, an exception is raised.

Names follow the C ABI: ``moe_workspace_size``, ``moe_route``,
``moe_permute``, ``moe_expert_ffn``, ``moe_combine``, ``moe_layer``,
``moe_status_string``.
"""
from __future__ import annotations

import ctypes as C
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbitmoe.so")

MOE_BF16, MOE_F32 = 0, 1
STATUS = {0: "MOE_OK", -1: "MOE_ERR_NULL", -2: "MOE_ERR_SHAPE", -3: "MOE_ERR_UNSUPPORTED",
          -4: "MOE_ERR_ALIGN", -5: "MOE_ERR_WORKSPACE", -6: "MOE_ERR_HIP"}
EXPORTS = ("moe_workspace_size", "moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_shared_gate",
           "moe_combine_gated", "moe_router_dequant", "moe_layer", "moe_layer_residual", "moe_layer_events", "moe_layer_stage_count", "moe_layer_stage_name",
           "moe_layer_no_alloc", "moe_decode_stack", "moe_gqa_workspace_size", "moe_gqa_decode", "moe_gqa_decode_events",
           "moe_gqa_decode_kernels",
           "moe_status_string")


class MoeError(RuntimeError):
    def __init__(self, status: int, call: str):
        super().__init__("%s failed: %s (%s)" % (call, STATUS.get(status, status), status_string(status)))
        self.status = status


class Dims(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("T", "H", "E", "top_k", "I", "I_shared", "group", "sb_dtype",
                                          "out_dtype")]


class GqaDims(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("B", "n_q_heads", "n_kv_heads", "head_dim", "max_seq")]


class QMat(C.Structure):
    _fields_ = [("q", C.c_void_p), ("scale", C.c_void_p), ("bias", C.c_void_p)]


class Ffn(C.Structure):
    _fields_ = [("gate", QMat), ("up", QMat), ("down", QMat)]


class QMatStride(C.Structure):
    _fields_ = [("q", C.c_int64), ("scale", C.c_int64), ("bias", C.c_int64)]


class FfnStride(C.Structure):
    _fields_ = [("gate", QMatStride), ("up", QMatStride), ("down", QMatStride)]


class LayerStrides(C.Structure):
    _fields_ = [("router", C.c_int64), ("logit_bias", C.c_int64), ("norm_weight", C.c_int64), ("experts", FfnStride),
                ("shared", FfnStride)]


class Weights(C.Structure):
    _fields_ = [("router", C.c_void_p), ("logit_bias", C.c_void_p), ("experts", Ffn), ("shared", Ffn),
                ("shared_expert_gate", C.c_void_p), ("router_q8", C.c_void_p), ("router_scale", C.c_void_p),
                ("router_bias", C.c_void_p)]


_lib = None


def lib():
    """Load libbitmoe.so (built in-tree by ``python -m bit_expert_grouped_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libbitmoe.so is not built; run `python -m bit_expert_grouped_amd.build`")
        # torch ships its own HIP runtime under the same soname as the system's
        # (libamdhip64.so.7), and the first one loaded serves the whole process;
        # load torch's first so that the library and torch's streams share it
        import torch  # noqa: F401

        L = C.CDLL(LIB_PATH)
        P, D = C.c_void_p, C.POINTER(Dims)
        L.moe_workspace_size.argtypes = [D]
        L.moe_workspace_size.restype = C.c_size_t
        L.moe_status_string.argtypes = [C.c_int]
        L.moe_status_string.restype = C.c_char_p
        L.moe_route.argtypes = [D, P, P, P, P, P, P]
        L.moe_permute.argtypes = [D, P, P, P, P, P, C.c_size_t, P]
        L.moe_expert_ffn.argtypes = [D, P, P, P, C.POINTER(Ffn), C.POINTER(Ffn), P, P, P, C.c_size_t, P]
        L.moe_combine.argtypes = [D, P, P, P, P, P]
        L.moe_combine_gated.argtypes = [D, P, P, P, P, P, P]
        L.moe_shared_gate.argtypes = [D, P, P, P, P]
        L.moe_router_dequant.argtypes = [D, P, P, P, P, P]
        L.moe_layer.argtypes = [D, C.POINTER(Weights), P, P, P, P, P, P, C.c_size_t, P]
        L.moe_layer_residual.argtypes = [D, C.POINTER(Weights), P, P, P, P, C.c_size_t, P]
        L.moe_layer_events.argtypes = [D, C.POINTER(Weights), P, P, P, P, P, P, C.c_size_t, P, P, C.c_int32]
        L.moe_layer_no_alloc.argtypes = [D, C.POINTER(Weights), P, P, P, P, P, P]
        L.moe_decode_stack.argtypes = [D, C.POINTER(Weights), P, C.POINTER(LayerStrides), C.c_int32, P, P, P, P, P,
                                       P, P, P, C.c_size_t, P]
        L.moe_gqa_workspace_size.argtypes = [C.POINTER(GqaDims)]
        L.moe_gqa_workspace_size.restype = C.c_size_t
        L.moe_gqa_decode.argtypes = [C.POINTER(GqaDims), P, P, P, P, C.c_float, P, P, C.c_size_t, P]
        L.moe_gqa_decode_kernels.argtypes = [C.POINTER(GqaDims)]
        L.moe_gqa_decode_kernels.restype = C.c_int32
        L.moe_gqa_decode_events.argtypes = [C.POINTER(GqaDims), P, P, P, P, C.c_float, P, P, C.c_size_t, P, P,
                                            C.c_int32]
        L.moe_layer_stage_count.argtypes = [D]
        L.moe_layer_stage_count.restype = C.c_int32
        L.moe_layer_stage_name.argtypes = [D, C.c_int32]
        L.moe_layer_stage_name.restype = C.c_char_p
        for name in ("moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_combine_gated",
                     "moe_shared_gate", "moe_layer", "moe_layer_residual", "moe_layer_events", "moe_layer_no_alloc",
                     "moe_decode_stack", "moe_gqa_decode", "moe_gqa_decode_events"):
            getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


moe_status_string = status_string


def _check(status: int, call: str):
    if status != 0:
        raise MoeError(status, call)


def _p(t):
    return None if t is None else t.data_ptr()


def _stream():
    import torch

    return torch.cuda.current_stream().cuda_stream


def dims(T, H, E, top_k, I, I_shared, sb_bf16=True, group=64, out_dtype=MOE_F32) -> Dims:
    return Dims(T, H, E, top_k, I, I_shared, group, MOE_BF16 if sb_bf16 else MOE_F32, out_dtype)


def moe_workspace_size(d: Dims) -> int:
    return lib().moe_workspace_size(C.byref(d))


def workspace(d: Dims, device="cuda"):
    """A zeroed workspace tensor of moe_workspace_size(d) bytes (torch allocations are 256-byte aligned)."""
    import torch

    n = moe_workspace_size(d)
    if n == 0:
        raise MoeError(-2, "moe_workspace_size")
    # the library requires a zero-filled workspace before its first use
    return torch.zeros(n, dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- weights


class LayerWeights:
    """Device tensors of one layer (router, stacked experts, shared expert) plus the C structs."""

    def __init__(self, tensors: dict):
        self.t = tensors
        self.sb_bf16 = tensors["gate_s"].element_size() == 2
        self.E, self.I, hw = tensors["gate_q"].shape
        self.H = hw * 8
        self.I_shared = tensors["shared_gate_q"].shape[1] if tensors.get("shared_gate_q") is not None else 0

        def qm(prefix, name):
            return QMat(_p(tensors[prefix + name + "_q"]), _p(tensors[prefix + name + "_s"]),
                        _p(tensors[prefix + name + "_b"]))

        self.experts = Ffn(qm("", "gate"), qm("", "up"), qm("", "down"))
        self.shared = (Ffn(qm("shared_", "gate"), qm("shared_", "up"), qm("shared_", "down"))
                       if self.I_shared else Ffn())
        self.struct = Weights(_p(tensors.get("router")), _p(tensors.get("logit_bias")), self.experts, self.shared,
                              _p(tensors.get("shared_expert_gate")), _p(tensors.get("router_q8")),
                              _p(tensors.get("router_scale")), _p(tensors.get("router_bias")))

    def dims(self, T, top_k) -> Dims:
        return dims(T, self.H, self.E, top_k, self.I, self.I_shared, self.sb_bf16)


def upload_weights(w: dict, device="cuda") -> LayerWeights:
    """numpy weights (moe_synth layout: uint32 codes, bf16 bits as uint16 or float32) -> device tensors."""
    import numpy as np
    import torch

    t = {}
    for k, v in w.items():
        if v is None:
            t[k] = None
            continue
        a = np.ascontiguousarray(v)
        if a.dtype == np.uint32:
            t[k] = torch.from_numpy(a.view(np.int32)).to(device)
        elif a.dtype == np.uint16:
            t[k] = torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
        else:
            t[k] = torch.from_numpy(a).to(device)
    return LayerWeights(t)


def bf16_tensor(x_bits, device="cuda"):
    """bf16 bit patterns (numpy uint16) -> torch.bfloat16 tensor on device."""
    import numpy as np
    import torch

    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to(device).view(torch.bfloat16)


# ---------------------------------------------------------------- calls


def moe_route(x, router, top_k, logit_bias=None, topk_idx=None, topk_w=None):
    import torch

    T, H = x.shape
    E = router.shape[0]
    d = dims(T, H, E, top_k, 64, 0)
    if topk_idx is None:
        topk_idx = torch.empty(T, top_k, dtype=torch.int32, device=x.device)
    if topk_w is None:
        topk_w = torch.empty(T, top_k, dtype=torch.float32, device=x.device)
    _check(lib().moe_route(C.byref(d), _p(x), _p(router), _p(logit_bias), _p(topk_idx), _p(topk_w), _stream()),
           "moe_route")
    return topk_idx, topk_w


def moe_permute(topk_idx, E, ws=None, d=None):
    import torch

    T, k = topk_idx.shape
    if d is None:
        d = dims(T, 64, E, k, 64, 0)
    if ws is None:
        ws = workspace(d, topk_idx.device)
    counts = torch.empty(E, dtype=torch.int32, device=topk_idx.device)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=topk_idx.device)
    sorted_slot = torch.empty(max(T * k, 1), dtype=torch.int32, device=topk_idx.device)
    _check(lib().moe_permute(C.byref(d), _p(topk_idx), _p(counts), _p(offsets), _p(sorted_slot), _p(ws),
                             ws.numel(), _stream()), "moe_permute")
    return counts, offsets, sorted_slot


def moe_expert_ffn(x, offsets, sorted_slot, weights: LayerWeights, top_k, with_shared=True, ws=None):
    import torch

    T, H = x.shape
    d = weights.dims(T, top_k)
    if ws is None:
        ws = workspace(d, x.device)
    y_slot = torch.empty(max(T * top_k, 1), H, dtype=torch.float32, device=x.device)
    y_shared = torch.empty(T, H, dtype=torch.float32, device=x.device) if (with_shared and weights.I_shared) else None
    shared = C.byref(weights.shared) if y_shared is not None else None
    _check(lib().moe_expert_ffn(C.byref(d), _p(x), _p(offsets), _p(sorted_slot), C.byref(weights.experts), shared,
                                _p(y_slot), _p(y_shared), _p(ws), ws.numel(), _stream()), "moe_expert_ffn")
    return y_slot, y_shared


def moe_combine(y_slot, topk_w, y_shared=None, out=None, shared_w=None):
    """shared_w [T] float32 (optional): the shared expert's weight per token (moe_combine_gated)."""
    import torch

    T, k = topk_w.shape
    H = y_slot.shape[1]
    d = dims(T, H, max(k, 1), k, 64, 0)
    if out is None:
        out = torch.empty(T, H, dtype=torch.float32, device=y_slot.device)
    if shared_w is None:
        _check(lib().moe_combine(C.byref(d), _p(y_slot), _p(topk_w), _p(y_shared), _p(out), _stream()),
               "moe_combine")
    else:
        _check(lib().moe_combine_gated(C.byref(d), _p(y_slot), _p(topk_w), _p(y_shared), _p(shared_w), _p(out),
                                       _stream()), "moe_combine_gated")
    return out


def moe_shared_gate(x, gate, shared_w=None):
    """shared_w [T] float32 = sigmoid(x[t] . gate): the shared expert's weight under its optional gate."""
    import torch

    T, H = x.shape
    d = dims(T, H, 1, 1, 64, 0)
    if shared_w is None:
        shared_w = torch.empty(T, dtype=torch.float32, device=x.device)
    _check(lib().moe_shared_gate(C.byref(d), _p(x), _p(gate), _p(shared_w), _stream()), "moe_shared_gate")
    return shared_w


def moe_router_dequant(router_q8, scale, bias, out=None):
    """The 8-bit router (codes [E][H/4] int32, scale/bias [E][H/64]) restored to bf16 [E][H]."""
    import torch

    E, H = router_q8.shape[0], router_q8.shape[1] * 4
    d = dims(1, H, E, 1, 64, 0, scale.element_size() == 2)
    if out is None:
        out = torch.empty(E, H, dtype=torch.bfloat16, device=router_q8.device)
    _check(lib().moe_router_dequant(C.byref(d), _p(router_q8), _p(scale), _p(bias), _p(out), _stream()),
           "moe_router_dequant")
    return out


def moe_layer_residual(x, weights: "LayerWeights", top_k, residual=None, out=None, ws=None):
    """out [T][H] bf16 = bf16(residual + layer(x)); residual (bf16, optional) may be ``out`` itself."""
    import torch

    T, H = x.shape
    d = weights.dims(T, top_k)
    d.out_dtype = MOE_BF16
    if ws is None:
        ws = workspace(d, x.device)
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=x.device)
    _check(lib().moe_layer_residual(C.byref(d), C.byref(weights.struct), _p(x), _p(residual), _p(out), _p(ws),
                                    ws.numel(), _stream()), "moe_layer_residual")
    return out


class StackWeights:
    """Device tensors of n_layers stacked layers (every tensor with a leading
    layer dimension, as moe_synth.device_stack draws them) plus the C structs
    of moe_decode_stack: layer 0's pointers and each tensor's layer stride."""

    def __init__(self, tensors: dict):
        self.t = tensors
        self.n_layers = tensors["gate_q"].shape[0]
        self.layer0 = LayerWeights({k: (None if v is None else v[0]) for k, v in tensors.items()
                                    if k != "norm_weight"})
        self.E, self.I, self.H, self.I_shared = self.layer0.E, self.layer0.I, self.layer0.H, self.layer0.I_shared
        self.sb_bf16 = self.layer0.sb_bf16

        def st(name):
            v = tensors.get(name)
            return 0 if v is None else v.stride(0) * v.element_size()

        def qs(prefix, name):
            return QMatStride(st(prefix + name + "_q"), st(prefix + name + "_s"), st(prefix + name + "_b"))

        self.norm_weight = tensors.get("norm_weight")
        self.strides = LayerStrides(st("router"), st("logit_bias"), st("norm_weight"),
                                    FfnStride(qs("", "gate"), qs("", "up"), qs("", "down")),
                                    FfnStride(qs("shared_", "gate"), qs("shared_", "up"), qs("shared_", "down"))
                                    if self.I_shared else FfnStride())

    def dims(self, top_k) -> Dims:
        return dims(1, self.H, self.E, top_k, self.I, self.I_shared, self.sb_bf16, out_dtype=MOE_BF16)


def moe_decode_stack(x, stack: StackWeights, top_k, x_out=None, ws=None, record=False):
    """One token x [1][H] bf16 through every layer of ``stack`` in one kernel:
    x(l+1) = bf16(x(l) + layer_l(rmsnorm(x(l)))).  Returns x_out, or with
    record=True (x_out, layer_x [L][H] bf16, layer_in [L][H] bf16, layer_out
    [L][H] float32, topk_idx [L][k], topk_w [L][k])."""
    import torch

    d = stack.dims(top_k)
    H, L = stack.H, stack.n_layers
    if ws is None:
        ws = workspace(d, x.device)
    if x_out is None:
        x_out = torch.empty(1, H, dtype=torch.bfloat16, device=x.device)
    rec = [None] * 5
    if record:
        rec = [torch.empty(L, H, dtype=torch.bfloat16, device=x.device),
               torch.empty(L, H, dtype=torch.bfloat16, device=x.device),
               torch.empty(L, H, dtype=torch.float32, device=x.device),
               torch.empty(L, top_k, dtype=torch.int32, device=x.device),
               torch.empty(L, top_k, dtype=torch.float32, device=x.device)]
    nw = stack.norm_weight
    _check(lib().moe_decode_stack(C.byref(d), C.byref(stack.layer0.struct), _p(nw[0]) if nw is not None else None,
                                  C.byref(stack.strides), L, _p(x), _p(x_out), *[_p(r) for r in rec], _p(ws),
                                  ws.numel(), _stream()), "moe_decode_stack")
    if record:
        return tuple([x_out] + rec)
    return x_out


NO_ALLOC_SCRATCH_BYTES = 32 << 20  # MOE_NO_ALLOC_SCRATCH_BYTES


def moe_layer_no_alloc(x, weights: "LayerWeights", top_k, out=None, want_routing=False):
    """moe_layer on the library's static per-device scratch (no workspace argument)."""
    import torch

    T, H = x.shape
    d = weights.dims(T, top_k)
    if out is None:
        out = torch.empty(T, H, dtype=torch.float32, device=x.device)
    idx = w = counts = None
    if want_routing:
        idx = torch.empty(T, top_k, dtype=torch.int32, device=x.device)
        w = torch.empty(T, top_k, dtype=torch.float32, device=x.device)
        counts = torch.empty(weights.E, dtype=torch.int32, device=x.device)
    _check(lib().moe_layer_no_alloc(C.byref(d), C.byref(weights.struct), _p(x), _p(out), _p(idx), _p(w),
                                    _p(counts), _stream()), "moe_layer_no_alloc")
    if want_routing:
        return out, idx, w, counts
    return out


def moe_layer_stages(d: Dims):
    """Names of the kernels moe_layer launches for these dims."""
    n = lib().moe_layer_stage_count(C.byref(d))
    return [lib().moe_layer_stage_name(C.byref(d), i).decode() for i in range(n)]


def moe_layer(x, weights: LayerWeights, top_k, out=None, ws=None, want_routing=False, events=None,
              topk_idx_out=None, topk_w_out=None, counts_out=None):
    """out [T][H] float32 = the whole MoE layer on bf16 activations x [T][H].

    want_routing: also return (topk_idx, topk_w, counts), allocated here unless
    given.  events: optional list of torch.cuda.Event (enable_timing=True), one
    more than the number of stages; recorded around each kernel by
    moe_layer_events."""
    import torch

    T, H = x.shape
    d = weights.dims(T, top_k)
    if ws is None:
        ws = workspace(d, x.device)
    if out is None:
        out = torch.empty(T, H, dtype=torch.float32, device=x.device)
    idx, w, counts = topk_idx_out, topk_w_out, counts_out
    if want_routing:
        if idx is None:
            idx = torch.empty(T, top_k, dtype=torch.int32, device=x.device)
        if w is None:
            w = torch.empty(T, top_k, dtype=torch.float32, device=x.device)
        if counts is None:
            counts = torch.empty(weights.E, dtype=torch.int32, device=x.device)
    if events is None:
        _check(lib().moe_layer(C.byref(d), C.byref(weights.struct), _p(x), _p(out), _p(idx), _p(w), _p(counts),
                               _p(ws), ws.numel(), _stream()), "moe_layer")
    else:
        for e in events:
            if not e.cuda_event:  # torch creates the HIP event lazily, on first record
                e.record()
        arr = (C.c_void_p * len(events))(*[e.cuda_event for e in events])
        _check(lib().moe_layer_events(C.byref(d), C.byref(weights.struct), _p(x), _p(out), _p(idx), _p(w),
                                      _p(counts), _p(ws), ws.numel(), _stream(), C.cast(arr, C.c_void_p),
                                      len(events)), "moe_layer_events")
    if want_routing:
        return out, idx, w, counts
    return out


# ---------------------------------------------------------------- decode attention


def gqa_dims(B, n_q_heads, n_kv_heads, head_dim, max_seq) -> GqaDims:
    return GqaDims(B, n_q_heads, n_kv_heads, head_dim, max_seq)


def gqa_workspace(d: GqaDims, device="cuda"):
    """A zeroed workspace tensor of moe_gqa_workspace_size(d) bytes."""
    import torch

    n = lib().moe_gqa_workspace_size(C.byref(d))
    if n == 0:
        raise MoeError(-2, "moe_gqa_workspace_size")
    # the library requires a zero-filled workspace before its first use
    return torch.zeros(n, dtype=torch.uint8, device=device)


def gqa_decode_kernels(d: GqaDims) -> int:
    """Kernels a moe_gqa_decode call with dims d launches on the current device (1: merge fused)."""
    return lib().moe_gqa_decode_kernels(C.byref(d))


def gqa_timed_out(ws, d: GqaDims) -> bool:
    """The workspace's sticky timeout word, the first of its last 256 bytes (a
    device-side wait of a call gave up; that call's output is invalid)."""
    import torch

    n = lib().moe_gqa_workspace_size(C.byref(d))
    return bool(int(ws[n - 256:n - 252].view(torch.int32).item()))


def gqa_decode(q, k_cache, v_cache, seq_len, scale=None, out=None, ws=None, events=None):
    """out [B][Hq][D] float32 = decode attention of q [B][Hq][D] over k_cache,
    v_cache [B][Hkv][S_max][D] (bf16 tensors) with seq_len [B] int32 rows each;
    scale defaults to 1/sqrt(D).  events: optional 3 torch.cuda.Event (timing
    enabled) recorded around the two kernels (moe_gqa_decode_events)."""
    import torch

    B, Hq, D = q.shape
    _, Hkv, S_max, _ = k_cache.shape
    d = gqa_dims(B, Hq, Hkv, D, S_max)
    if out is None:
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=q.device)
    if ws is None:
        ws = gqa_workspace(d, q.device)
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if events is None:
        _check(lib().moe_gqa_decode(C.byref(d), _p(q), _p(k_cache), _p(v_cache), _p(seq_len), sc, _p(out), _p(ws),
                                    ws.numel(), _stream()), "moe_gqa_decode")
    else:
        for e in events:
            if not e.cuda_event:  # torch creates the HIP event lazily, on first record
                e.record()
        ev = (C.c_void_p * len(events))(*[e.cuda_event for e in events])
        _check(lib().moe_gqa_decode_events(C.byref(d), _p(q), _p(k_cache), _p(v_cache), _p(seq_len), sc, _p(out),
                                           _p(ws), ws.numel(), _stream(), C.cast(ev, C.c_void_p), len(events)),
               "moe_gqa_decode_events")
    return out
