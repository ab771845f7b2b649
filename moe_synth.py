"""Seeded synthetic inputs for the 4-bit grouped-expert MoE layer.

This module draws random numbers and lays them out in the byte formats the
layer consumes.  It holds none of the layer's arithmetic: no dequantisation,
no routing, no expert maths.  Both the CPU oracle (``oracle/``) and the HIP
path (``bit_expert_grouped_amd``) receive the very bytes produced here.

Layer shape and weight format follow the pages on Lily (Perplexity's engine
for Qwen3.6-35B-A3B):

* 256 routed experts, 8 picked per token, plus one always-on shared expert
  (aimanavo.com page, section on Qwen3.6's 256 experts and two layer types);
* MLX affine 4-bit weights with group size 64 (aimanavo.com page, section on
  the single supported 4-bit checkpoint; news.mantis.guru page, section
  "Rust drives the model, Metal does the compute").

Byte formats (the MLX convention):

* ``*_q``  uint32 ``[n][N][K/8]``: eight 4-bit codes per word, code for input
  column ``k`` at bits ``[4*(k%8), 4*(k%8)+4)`` of word ``k/8``;
* ``*_s``, ``*_b``  ``[n][N][K/64]``: per-group scale and bias, float32 or
  bfloat16 bit patterns (uint16);
* activations and router weights: bfloat16 bit patterns (uint16).

Distributions (identical for every config): codes uniform over 0..15 (drawn as
uniform uint32 words), scale ~ U(0.005, 0.02), bias ~ U(-0.1, 0.1),
activations ~ N(0, 1), router weights ~ N(0, 0.02).  Real values are drawn in
float64, rounded to float32, and for bfloat16 tensors rounded again to
bfloat16 with round-to-nearest-even.

Every tensor has its own PCG64 stream keyed by
``SeedSequence([seed, layer, kind, expert])``; token row ``t`` of the
activations has the stream ``[seed, KIND_X, t, attempt]`` so that single rows
can be re-drawn (``attempt`` > 0) without touching the others.
"""
from __future__ import annotations

import dataclasses
import json
import os

import numpy as np

# tensor kinds used as the third word of the seed sequence
KIND_ROUTER = 1
KIND_GATE_Q, KIND_GATE_S, KIND_GATE_B = 2, 3, 4
KIND_UP_Q, KIND_UP_S, KIND_UP_B = 5, 6, 7
KIND_DOWN_Q, KIND_DOWN_S, KIND_DOWN_B = 8, 9, 10
KIND_ZIPF_RANK = 11
KIND_SHARED_EXPERT_GATE = 12
KIND_ROUTER_Q8_Q, KIND_ROUTER_Q8_S, KIND_ROUTER_Q8_B = 13, 14, 15
KIND_X = 100
SHARED_EXPERT = 1 << 20  # expert slot used in seed sequences for the shared expert

GROUP = 64
SCALE_RANGE = (0.005, 0.02)
BIAS_RANGE = (-0.1, 0.1)
ROUTER_STD = 0.02
ZIPF_S = 1.1

_HERE = os.path.dirname(os.path.abspath(__file__))
ZIPF_ALPHA_FILE = os.path.join(_HERE, "tests", "golden", "zipf_alpha.json")


@dataclasses.dataclass(frozen=True)
class Shape:
    """Sizes of one MoE layer invocation."""

    T: int          # tokens
    H: int          # hidden size
    E: int          # routed experts
    top_k: int      # experts picked per token
    I: int          # routed expert SwiGLU intermediate size
    I_shared: int   # shared expert intermediate size
    sb_bf16: bool   # scales/biases stored as bfloat16 (else float32)
    group: int = GROUP


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    shape: Shape
    seed: int
    layers: int = 1
    zipf: bool = False
    description: str = ""


_QWEN = dict(H=2048, E=256, top_k=8, I=512, I_shared=512, sb_bf16=True)

CONFIGS = {
    "tiny": Config("tiny", Shape(T=16, H=256, E=16, top_k=2, I=64, I_shared=64, sb_bf16=False),
                   seed=0, description="T=16, H=256, 16 experts top-2 + shared, I=64, fp32 scales"),
    "decode": Config("decode", Shape(T=1, **_QWEN), seed=1,
                     description="decode step, T=1, H=2048, 256 experts top-8 + shared, I=512"),
    "prefill512": Config("prefill512", Shape(T=512, **_QWEN), seed=2,
                         description="prefill T=512 (512-token prompt case)"),
    "prefill4096": Config("prefill4096", Shape(T=4096, **_QWEN), seed=3,
                          description="prefill T=4096"),
    "decode64": Config("decode64", Shape(T=64, **_QWEN), seed=3,
                       description="batched decode T=64, run beside prefill T=4096"),
    "stack40": Config("stack40", Shape(T=4096, **_QWEN), seed=4, layers=40, zipf=True,
                      description="40 stacked layers, T=4096, Zipf(1.1)-skewed routing"),
}
# the batched-decode case draws its activations from a stream apart from T=4096's
_X_STREAM_OFFSET = {"decode64": 1 << 16}


def _rng(*words: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(w) for w in words])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _uniform(rng, lo, hi, size, bf16: bool):
    v = rng.uniform(lo, hi, size=size).astype(np.float32)
    return f32_to_bf16_bits(v) if bf16 else v


def _normal(rng, std, size):
    return f32_to_bf16_bits((rng.standard_normal(size=size) * std).astype(np.float32))


def _words(rng, size):
    return rng.integers(0, 1 << 32, size=size, dtype=np.uint32)


# Centred biases: shifted by -CODE_MIDPOINT * scale, so that the weights average
# to about zero as an affine quantisation of zero-mean weights does (its bias
# is near -7.5 * scale).  The decode stack draws its layers this way: with the
# configs' uncentred biases every weight averages about +0.09, each layer adds a
# large common-mode vector to the residual stream, and after one layer the
# normalised stream drives every gate to saturation.
CODE_MIDPOINT = 7.5


def _matrix(seed, layer, expert, kinds, N, K, sb_bf16, centred=False):
    kq, ks, kb = kinds
    q = _words(_rng(seed, layer, kq, expert), (N, K // 8))
    if not centred:
        s = _uniform(_rng(seed, layer, ks, expert), *SCALE_RANGE, (N, K // GROUP), sb_bf16)
        b = _uniform(_rng(seed, layer, kb, expert), *BIAS_RANGE, (N, K // GROUP), sb_bf16)
        return q, s, b
    s = _rng(seed, layer, ks, expert).uniform(*SCALE_RANGE, size=(N, K // GROUP)).astype(np.float32)
    b = _rng(seed, layer, kb, expert).uniform(*BIAS_RANGE, size=(N, K // GROUP)).astype(np.float32)
    b = (b - np.float32(CODE_MIDPOINT) * s).astype(np.float32)
    if sb_bf16:
        s, b = f32_to_bf16_bits(s), f32_to_bf16_bits(b)
    return q, s, b


def expert_tensors(shape: Shape, seed: int, layer: int, expert: int, intermediate: int, centred: bool = False):
    """gate/up ([I][H/8] words) and down ([H][I/8] words) of one expert."""
    H, I, bf = shape.H, intermediate, shape.sb_bf16
    out = {}
    for name, kinds, N, K in (("gate", (KIND_GATE_Q, KIND_GATE_S, KIND_GATE_B), I, H),
                              ("up", (KIND_UP_Q, KIND_UP_S, KIND_UP_B), I, H),
                              ("down", (KIND_DOWN_Q, KIND_DOWN_S, KIND_DOWN_B), H, I)):
        q, s, b = _matrix(seed, layer, expert, kinds, N, K, bf, centred)
        out[name + "_q"], out[name + "_s"], out[name + "_b"] = q, s, b
    return out


def router_weights(cfg: Config, layer: int = 0) -> np.ndarray:
    """Router matrix [E][H] as bf16 bits."""
    sh = cfg.shape
    return _normal(_rng(cfg.seed, layer, KIND_ROUTER, 0), ROUTER_STD, (sh.E, sh.H))


def shared_expert_gate(cfg: Config, layer: int = 0) -> np.ndarray:
    """Gate vector [H] of the shared expert as bf16 bits, drawn like a router row.

    An optional checkpoint detail the configs do not use; the tests of the
    gated shared expert add it to a layer's weights under "shared_expert_gate".
    """
    return _normal(_rng(cfg.seed, layer, KIND_SHARED_EXPERT_GATE, 0), ROUTER_STD, (cfg.shape.H,))


def router_q8(cfg: Config, layer: int = 0) -> dict:
    """An 8-bit router in the MLX affine layout (4 codes per uint32 word, low
    byte first; a scale and a bias per 64 columns in the config's scale dtype).

    Codes are uniform bytes; scales ~U(1.5e-4, 2.5e-4) and biases near
    -127.5 * scale, so the restored weights spread like the dense router's
    N(0, 0.02).  An optional checkpoint detail the configs do not use.
    """
    sh = cfg.shape
    E, H = sh.E, sh.H
    q = _words(_rng(cfg.seed, layer, KIND_ROUTER_Q8_Q, 0), (E, H // 4))
    s = _rng(cfg.seed, layer, KIND_ROUTER_Q8_S, 0).uniform(1.5e-4, 2.5e-4, size=(E, H // GROUP))
    b = -127.5 * s + _rng(cfg.seed, layer, KIND_ROUTER_Q8_B, 0).uniform(-2e-3, 2e-3, size=(E, H // GROUP))
    s, b = s.astype(np.float32), b.astype(np.float32)
    if sh.sb_bf16:
        s, b = f32_to_bf16_bits(s), f32_to_bf16_bits(b)
    return {"router_q8": q, "router_scale": s, "router_bias": b}


def layer_weights(cfg: Config, layer: int = 0, centred: bool = False) -> dict:
    """All weights of one layer: router, the E routed experts (stacked), the shared expert."""
    sh = cfg.shape
    w = {"router": router_weights(cfg, layer)}
    per = [expert_tensors(sh, cfg.seed, layer, e, sh.I, centred) for e in range(sh.E)]
    for key in per[0]:
        w[key] = np.stack([p[key] for p in per])
    shared = expert_tensors(sh, cfg.seed, layer, SHARED_EXPERT, sh.I_shared, centred)
    for key, v in shared.items():
        w["shared_" + key] = v[None]
    w["logit_bias"] = zipf_bias(cfg, layer) if cfg.zipf else None
    return w


def token_rows(cfg: Config, T: int | None = None, attempts: dict | None = None) -> np.ndarray:
    """Activations [T][H] as bf16 bits; row t re-drawn ``attempts[t]`` times."""
    sh = cfg.shape
    T = sh.T if T is None else T
    attempts = attempts or {}
    off = _X_STREAM_OFFSET.get(cfg.name, 0)
    x = np.empty((T, sh.H), dtype=np.uint16)
    for t in range(T):
        x[t] = _normal(_rng(cfg.seed, KIND_X, off + t, attempts.get(t, 0)), 1.0, (sh.H,))
    return x


def zipf_ranks(cfg: Config, layer: int) -> np.ndarray:
    """A seeded permutation of 1..E: the popularity rank of each expert in this layer."""
    return _rng(cfg.seed, layer, KIND_ZIPF_RANK, 0).permutation(cfg.shape.E) + 1


def zipf_alpha() -> float:
    """Strength of the Zipf offset; calibrated by ``oracle/calibrate_zipf.py``."""
    with open(ZIPF_ALPHA_FILE) as f:
        return float(json.load(f)["alpha"])


def zipf_bias(cfg: Config, layer: int, alpha: float | None = None) -> np.ndarray:
    """Per-expert logit offset ``-alpha * s * ln(rank)`` with s = 1.1, float32."""
    a = zipf_alpha() if alpha is None else alpha
    r = zipf_ranks(cfg, layer).astype(np.float64)
    return (-a * ZIPF_S * np.log(r)).astype(np.float32)


# ---------------------------------------------------------------------------
# device-side generation for timing runs (same distributions, torch's RNG)
# ---------------------------------------------------------------------------

def device_layer(shape: Shape, seed: int, layer: int, device, zipf_alpha_value: float | None = None,
                 centred: bool = False):
    """One layer's weights drawn directly in device memory with torch's generator.

    Used where many distinct weight sets are needed (timing runs that must not
    be served from the 256 MB last-level cache).  Same distributions and byte
    formats as :func:`layer_weights`; different random streams.
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed((seed << 20) ^ (layer * 7919 + 17))
    E, H, I, Is = shape.E, shape.H, shape.I, shape.I_shared

    def words(*size):
        return torch.randint(-(1 << 31), 1 << 31, size, dtype=torch.int32, device=device, generator=g)

    def unif(lo, hi, *size):
        v = torch.rand(size, dtype=torch.float32, device=device, generator=g) * (hi - lo) + lo
        return v.to(torch.bfloat16) if shape.sb_bf16 else v

    def expert_set(n, inter):
        d = {}
        for name, N, K in (("gate", inter, H), ("up", inter, H), ("down", H, inter)):
            d[name + "_q"] = words(n, N, K // 8)
            if centred:
                sv = torch.rand((n, N, K // GROUP), dtype=torch.float32, device=device, generator=g)
                sv = sv * (SCALE_RANGE[1] - SCALE_RANGE[0]) + SCALE_RANGE[0]
                bv = torch.rand((n, N, K // GROUP), dtype=torch.float32, device=device, generator=g)
                bv = bv * (BIAS_RANGE[1] - BIAS_RANGE[0]) + BIAS_RANGE[0] - CODE_MIDPOINT * sv
                dt = torch.bfloat16 if shape.sb_bf16 else torch.float32
                d[name + "_s"], d[name + "_b"] = sv.to(dt), bv.to(dt)
            else:
                d[name + "_s"] = unif(*SCALE_RANGE, n, N, K // GROUP)
                d[name + "_b"] = unif(*BIAS_RANGE, n, N, K // GROUP)
        return d

    w = {"router": (torch.randn(E, H, device=device, generator=g) * ROUTER_STD).to(torch.bfloat16)}
    w.update(expert_set(E, I))
    for k, v in expert_set(1, Is).items():
        w["shared_" + k] = v
    if zipf_alpha_value is not None:
        ranks = torch.randperm(E, device=device, generator=g).to(torch.float64) + 1
        w["logit_bias"] = (-zipf_alpha_value * ZIPF_S * torch.log(ranks)).to(torch.float32)
    else:
        w["logit_bias"] = None
    return w


def device_stack(shape: Shape, seed: int, n_layers: int, device, zipf_alpha_value: float | None = None,
                 centred: bool = True):
    """n_layers layers drawn directly in device memory, every tensor stacked
    with a leading layer dimension ([n_layers][...]), for the multi-layer
    decode kernel.  Layer l holds exactly what :func:`device_layer` draws for
    layer l (centred biases by default: see CODE_MIDPOINT)."""
    import torch

    layers = [device_layer(shape, seed, l, device, zipf_alpha_value, centred) for l in range(n_layers)]
    out = {}
    for key in layers[0]:
        vals = [lw[key] for lw in layers]
        out[key] = None if vals[0] is None else torch.stack(vals)
        for lw in layers:
            lw[key] = None
    return out


def host_stack(cfg: Config, n_layers: int, centred: bool = True) -> dict:
    """n_layers layers of :func:`layer_weights` (host, numpy), stacked with a
    leading layer dimension (centred biases by default: see CODE_MIDPOINT)."""
    layers = [layer_weights(cfg, l, centred) for l in range(n_layers)]
    return {key: (None if layers[0][key] is None else np.stack([lw[key] for lw in layers])) for key in layers[0]}


def device_tokens(shape: Shape, T: int, seed: int, step: int, device):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed((seed << 24) ^ (step * 104729 + 3))
    return torch.randn(T, shape.H, device=device, generator=g).to(torch.bfloat16)


# ---------------------------------------------------------------- decode attention inputs

KIND_ATTN_Q, KIND_ATTN_K, KIND_ATTN_V = 200, 201, 202


@dataclasses.dataclass(frozen=True)
class AttnShape:
    """Decode attention: B sequences of one query token, Hq query heads over Hkv
    KV heads of size D, a cache of S rows per (sequence, KV head)."""
    B: int
    Hq: int
    Hkv: int
    D: int
    S: int


# the model's full-attention layer at 32K context, one sequence (the context the
# pages quote the packing gain at); head size H / Hq
GQA32K = AttnShape(B=1, Hq=16, Hkv=2, D=128, S=32768)


def attn_inputs(shape: AttnShape, seed: int, q_std: float = 1.0):
    """Host bf16 bits: q [B][Hq][D] ~ N(0, q_std^2), k and v [B][Hkv][S][D] ~ N(0, 1)."""
    q = _normal(_rng(seed, KIND_ATTN_Q, 0, 0), q_std, (shape.B, shape.Hq, shape.D))
    k = _normal(_rng(seed, KIND_ATTN_K, 0, 0), 1.0, (shape.B, shape.Hkv, shape.S, shape.D))
    v = _normal(_rng(seed, KIND_ATTN_V, 0, 0), 1.0, (shape.B, shape.Hkv, shape.S, shape.D))
    return q, k, v


def device_attn(shape: AttnShape, seed: int, device, q_std: float = 1.0):
    """The same distributions as :func:`attn_inputs`, drawn in device memory with
    torch's generator (different streams): bf16 tensors q, k, v."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed((seed << 16) ^ 0xA77)
    q = (torch.randn(shape.B, shape.Hq, shape.D, device=device, generator=g) * q_std).to(torch.bfloat16)
    k = torch.randn(shape.B, shape.Hkv, shape.S, shape.D, device=device, generator=g).to(torch.bfloat16)
    v = torch.randn(shape.B, shape.Hkv, shape.S, shape.D, device=device, generator=g).to(torch.bfloat16)
    return q, k, v
