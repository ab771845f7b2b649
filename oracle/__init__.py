"""CPU oracle for the 4-bit grouped-expert MoE layer (Qwen3.6-35B-A3B shapes).

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the CPU-baseline
leg of the benchmark call this package; the HIP product path never does.  It
shares no code with ``bit_expert_grouped_amd``.

The arithmetic lives in ``moe_oracle.c`` (plain C, double precision, compiled
with gcc into ``liboracle.so``); this module only marshals numpy arrays.  The
readings R1-R7 listed at the top of ``moe_oracle.c`` say what is computed and
which page passage each step follows.  ``oracle.brute`` is a second, dense,
numpy-only evaluation used to check this one on tiny shapes.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile moe_oracle.c with gcc into liboracle.so (no GPU code involved)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class QMat(C.Structure):
    _fields_ = [("q", C.c_void_p), ("s", C.c_void_p), ("b", C.c_void_p), ("sb_bf16", C.c_int32),
                ("N", C.c_int32), ("K", C.c_int32), ("group", C.c_int32)]


class Layer(C.Structure):
    _fields_ = ([(n, C.c_int32) for n in ("T", "H", "E", "top_k", "I", "I_shared", "group", "sb_bf16")]
                + [(n, C.c_void_p) for n in (
                    "x", "router", "logit_bias",
                    "gate_q", "up_q", "down_q", "gate_s", "gate_b", "up_s", "up_b", "down_s", "down_b",
                    "sh_gate_q", "sh_up_q", "sh_down_q", "sh_gate_s", "sh_gate_b", "sh_up_s", "sh_up_b",
                    "sh_down_s", "sh_down_b", "sh_expert_gate")])


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = C.CDLL(_LIB_PATH)
        P = C.c_void_p
        i32 = C.c_int32
        L.oracle_code.argtypes = [C.POINTER(QMat), i32, i32]
        L.oracle_code.restype = i32
        L.oracle_dequant.argtypes = [C.POINTER(QMat), P]
        L.oracle_dequant.restype = None
        L.oracle_router_dequant_q8.argtypes = [i32, i32, P, P, P, i32, P]
        L.oracle_router_dequant_q8.restype = None
        L.oracle_router_logits.argtypes = [i32, i32, i32, P, P, P, P]
        L.oracle_router_logits.restype = None
        L.oracle_select.argtypes = [i32, i32, i32, P, P, P]
        L.oracle_select.restype = None
        L.oracle_permute.argtypes = [i32, i32, i32, P, P, P, P]
        L.oracle_permute.restype = None
        L.oracle_expert_ffn.argtypes = [C.POINTER(QMat)] * 3 + [i32, P, P, P, P]
        L.oracle_expert_ffn.restype = None
        L.oracle_combine.argtypes = [i32, i32, i32, P, P, P, P, P]
        L.oracle_shared_gate.argtypes = [i32, i32, P, P, P]
        L.oracle_shared_gate.restype = None
        L.oracle_combine.restype = None
        L.oracle_rmsnorm.argtypes = [i32, P, P, C.c_double, P]
        L.oracle_rmsnorm.restype = None
        L.oracle_moe_layer.argtypes = [C.POINTER(Layer), i32, P, P, P, P, P, P, P, P]
        L.oracle_moe_layer.restype = C.c_int
        L.oracle_gqa_decode.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, C.c_double, P]
        L.oracle_gqa_decode.restype = C.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _sb(a):
    """Scales/biases: uint16 arrays are bfloat16 bits, float32 arrays are values."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return a, 1
    return np.ascontiguousarray(a, dtype=np.float32), 0


def qmat(q, s, b, group=64):
    """Wrap one [N][K/8] matrix; returns (struct, keep-alive list)."""
    q = _c(q, np.uint32)
    s, bf = _sb(s)
    b, bf2 = _sb(b)
    assert bf == bf2 and q.ndim == 2
    N, K = q.shape[0], q.shape[1] * 8
    assert s.shape == (N, K // group) and b.shape == s.shape
    return QMat(q.ctypes.data, s.ctypes.data, b.ctypes.data, bf, N, K, group), [q, s, b]


def code(q, s, b, n, k, group=64):
    m, keep = qmat(q, s, b, group)
    return lib().oracle_code(C.byref(m), n, k)


def dequant(q, s, b, group=64):
    m, keep = qmat(q, s, b, group)
    W = np.empty((m.N, m.K), dtype=np.float64)
    lib().oracle_dequant(C.byref(m), W.ctypes.data)
    return W


def router_dequant_q8(codes, scale, bias):
    """8-bit router (R16): codes [E][H/4] uint32, scale/bias [E][H/64] (bf16 bits
    as uint16, or float32) -> the bfloat16 router [E][H] as uint16 bits."""
    codes = _c(codes, np.uint32)
    sb_bf16 = np.asarray(scale).dtype == np.uint16
    dt = np.uint16 if sb_bf16 else np.float32
    scale, bias = _c(scale, dt), _c(bias, dt)
    E, H = codes.shape[0], codes.shape[1] * 4
    out = np.empty((E, H), dtype=np.uint16)
    lib().oracle_router_dequant_q8(E, H, codes.ctypes.data, scale.ctypes.data, bias.ctypes.data, int(sb_bf16),
                                   out.ctypes.data)
    return out


def layer_router(weights):
    """The layer's bfloat16 router: the dense one, or the 8-bit one restored (R16)."""
    if weights.get("router_q8") is not None:
        return router_dequant_q8(weights["router_q8"], weights["router_scale"], weights["router_bias"])
    return weights["router"]


def router_logits(x, router, logit_bias=None):
    x = _c(x, np.uint16)
    router = _c(router, np.uint16)
    lb = _c(logit_bias, np.float32)
    T, H = x.shape
    E = router.shape[0]
    out = np.empty((T, E), dtype=np.float64)
    lib().oracle_router_logits(T, H, E, x.ctypes.data, router.ctypes.data, _ptr(lb), out.ctypes.data)
    return out


def select(logits, k):
    logits = _c(logits, np.float64)
    T, E = logits.shape
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    lib().oracle_select(T, E, k, logits.ctypes.data, idx.ctypes.data, w.ctypes.data)
    return idx, w


def permute(idx, E):
    idx = _c(idx, np.int32)
    T, k = idx.shape
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    ss = np.empty(T * k, dtype=np.int32)
    lib().oracle_permute(T, k, E, idx.ctypes.data, counts.ctypes.data, offsets.ctypes.data, ss.ctypes.data)
    return counts, offsets, ss


def expert_ffn(gate, up, down, x_rows, group=64, want_gu=False):
    """gate/up/down: (q, s, b) tuples of one expert; x_rows [n][H] bf16 bits."""
    mg, k1 = qmat(*gate, group=group)
    mu, k2 = qmat(*up, group=group)
    md, k3 = qmat(*down, group=group)
    x_rows = _c(x_rows, np.uint16)
    n, H = x_rows.shape
    I = mg.N
    ptrs = (C.c_void_p * max(n, 1))(*[x_rows.ctypes.data + r * H * 2 for r in range(n)])
    y = np.empty((n, H), dtype=np.float64)
    g = np.empty((n, I), dtype=np.float64) if want_gu else None
    u = np.empty((n, I), dtype=np.float64) if want_gu else None
    lib().oracle_expert_ffn(C.byref(mg), C.byref(mu), C.byref(md), n, C.cast(ptrs, C.c_void_p),
                            _ptr(g), _ptr(u), y.ctypes.data)
    return (y, g, u) if want_gu else y


def combine(y_slot, w, y_shared=None, shared_w=None):
    """y_slot [n][k][H], w [n][k], y_shared [n][H] or None, shared_w [n] or None (weight 1)."""
    y_slot = _c(y_slot, np.float64)
    w = _c(w, np.float64)
    ys = _c(y_shared, np.float64)
    sw = _c(shared_w, np.float64)
    n, k, H = y_slot.shape
    out = np.empty((n, H), dtype=np.float64)
    lib().oracle_combine(n, k, H, y_slot.ctypes.data, w.ctypes.data, _ptr(ys), _ptr(sw), out.ctypes.data)
    return out


def shared_gate(x, gate):
    """Weight of the shared expert per token: sigmoid(x[t] . gate), x [T][H] and gate [H] bf16 bits."""
    x = _c(x, np.uint16)
    g = _c(gate, np.uint16)
    out = np.empty(x.shape[0], dtype=np.float64)
    lib().oracle_shared_gate(x.shape[0], x.shape[1], x.ctypes.data, g.ctypes.data, out.ctypes.data)
    return out


RMSNORM_EPS = 1e-6  # the epsilon of the decode stack's normalisation (R17)


def rmsnorm(x, gamma=None, eps=RMSNORM_EPS):
    """R17: bf16(x / sqrt(mean(x^2) + eps) * gamma) of each row of x [n][H] (bf16
    bits); gamma [H] bf16 bits or None (1).  Returns bf16 bits [n][H]."""
    x = _c(np.atleast_2d(x), np.uint16)
    g = _c(gamma, np.uint16)
    out = np.empty_like(x)
    for r in range(x.shape[0]):
        lib().oracle_rmsnorm(x.shape[1], x[r].ctypes.data, _ptr(g), float(eps), out[r].ctypes.data)
    return out


def gqa_decode(q, k, v, seq_len, scale=None):
    """R19: decode attention with grouped-query KV sharing.  q [B][Hq][D], k and v
    [B][Hkv][S_max][D] (bf16 bits), seq_len [B]; scale defaults to 1/sqrt(D).
    Returns out [B][Hq][D] float64."""
    q = _c(q, np.uint16)
    k = _c(k, np.uint16)
    v = _c(v, np.uint16)
    B, Hq, D = q.shape
    _, Hkv, S_max, _ = k.shape
    if k.shape != (B, Hkv, S_max, D) or v.shape != k.shape or Hq % Hkv:
        raise ValueError("gqa_decode: inconsistent shapes")
    n = _c(seq_len, np.int32)
    out = np.empty((B, Hq, D), dtype=np.float64)
    sc = 1.0 / np.sqrt(D) if scale is None else float(scale)
    if lib().oracle_gqa_decode(B, Hq, Hkv, D, S_max, q.ctypes.data, k.ctypes.data, v.ctypes.data, n.ctypes.data,
                               sc, out.ctypes.data) != 0:
        raise MemoryError("oracle_gqa_decode could not allocate its working buffer")
    return out


def moe_layer(weights: dict, x, top_k: int, group: int = 64, tokens=None, want_logits=False):
    """Whole layer on ``x`` [T][H] (bf16 bits) with the weights dict of ``moe_synth.layer_weights``.

    ``tokens``: indices whose outputs are computed (all when None); routing,
    counts and offsets always cover every token.  Returns a dict with ``out``
    [n][H] float64, ``idx`` [T][k], ``w`` [T][k], ``counts`` [E], ``offsets``
    [E+1], ``sorted_slot`` [T*k] and optionally ``logits`` [T][E].
    """
    x = _c(x, np.uint16)
    T, H = x.shape
    router = _c(layer_router(weights), np.uint16)
    E = router.shape[0]
    gq = _c(weights["gate_q"], np.uint32)
    I = gq.shape[1]
    keep = [x, router, gq]

    def arr(name, dtype=None):
        a = weights.get(name)
        if a is None:
            return None
        a = np.ascontiguousarray(a) if dtype is None else np.ascontiguousarray(a, dtype=dtype)
        keep.append(a)
        return a

    sb_bf16 = 1 if np.asarray(weights["gate_s"]).dtype == np.uint16 else 0
    sbd = np.uint16 if sb_bf16 else np.float32
    L = Layer()
    L.T, L.H, L.E, L.top_k, L.I, L.group, L.sb_bf16 = T, H, E, top_k, I, group, sb_bf16
    L.x, L.router = x.ctypes.data, router.ctypes.data
    lb = arr("logit_bias", np.float32)
    L.logit_bias = _ptr(lb)
    L.gate_q = gq.ctypes.data
    for name in ("up_q", "down_q"):
        setattr(L, name, arr(name, np.uint32).ctypes.data)
    for name in ("gate_s", "gate_b", "up_s", "up_b", "down_s", "down_b"):
        setattr(L, name, arr(name, sbd).ctypes.data)
    if weights.get("shared_gate_q") is not None:
        sgq = arr("shared_gate_q", np.uint32)
        L.I_shared = sgq.shape[1]
        L.sh_gate_q = sgq.ctypes.data
        L.sh_up_q = arr("shared_up_q", np.uint32).ctypes.data
        L.sh_down_q = arr("shared_down_q", np.uint32).ctypes.data
        for name in ("gate_s", "gate_b", "up_s", "up_b", "down_s", "down_b"):
            setattr(L, "sh_" + name, arr("shared_" + name, sbd).ctypes.data)
    else:
        L.I_shared = 0
    seg = arr("shared_expert_gate", np.uint16)
    L.sh_expert_gate = _ptr(seg)
    tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    n = T if tok is None else len(tok)
    out = np.empty((n, H), dtype=np.float64)
    logits = np.empty((T, E), dtype=np.float64) if want_logits else None
    idx = np.empty((T, top_k), dtype=np.int32)
    w = np.empty((T, top_k), dtype=np.float64)
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    ss = np.empty(T * top_k, dtype=np.int32)
    rc = lib().oracle_moe_layer(C.byref(L), n, _ptr(tok), out.ctypes.data, _ptr(logits), idx.ctypes.data,
                                w.ctypes.data, counts.ctypes.data, offsets.ctypes.data, ss.ctypes.data)
    if rc != 0:
        raise MemoryError("oracle_moe_layer could not allocate its working buffers")
    res = dict(out=out, idx=idx, w=w, counts=counts, offsets=offsets, sorted_slot=ss)
    if want_logits:
        res["logits"] = logits
    return res
