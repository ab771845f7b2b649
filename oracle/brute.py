"""Dense brute-force evaluation of the MoE layer in numpy float64 (tiny shapes only).

TEST INFRASTRUCTURE ONLY.  A second, independent statement of what the layer
computes, used to check the C oracle: it evaluates EVERY expert on EVERY token
and masks the results with the top-k selection,

    y[t] = sum_e M[t,e] * r[t,e] * F_e(x_t) + s_t * F_shared(x_t),

where M is the top-k mask from a full stable sort of the float32-rounded
router logits (larger first, lower index first on equal values) and r is the
softmax over all experts renormalised over the mask; s_t = sigmoid(x_t . g) with
an optional shared-expert gate vector g, else 1.  It shares no code with
``moe_oracle.c``: nibbles are unpacked with numpy shifts, products are numpy
matrix multiplications, selection is a lexicographic sort.

Pages: 256 experts scored, 8 kept, one shared expert added (aimanavo.com page,
section "Qwen3.6's 256 experts and two layer types make the MLX-Lily gap");
MLX affine 4-bit weights, group size 64 (same page, section on the single 4-bit
checkpoint).
"""
from __future__ import annotations

import numpy as np


def _bf16(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _sb(a):
    a = np.asarray(a)
    return _bf16(a) if a.dtype == np.uint16 else a.astype(np.float64)


def dense_matrix(q, s, b, group=64):
    """[N][K/8] words -> [N][K] float64 values, vectorised."""
    q = np.asarray(q, dtype=np.uint32)
    N, W = q.shape
    shifts = (4 * np.arange(8, dtype=np.uint32))[None, None, :]
    codes = ((q[:, :, None] >> shifts) & np.uint32(15)).reshape(N, W * 8).astype(np.float64)
    s = np.repeat(_sb(s), group, axis=1)
    b = np.repeat(_sb(b), group, axis=1)
    return codes * s + b


def ffn(Wg, Wu, Wd, X):
    g = X @ Wg.T
    u = X @ Wu.T
    return ((g / (1.0 + np.exp(-g))) * u) @ Wd.T


def topk_mask(logits, k):
    keys = logits.astype(np.float32)
    T, E = keys.shape
    M = np.zeros((T, E), dtype=bool)
    for t in range(T):
        order = np.lexsort((np.arange(E), -keys[t].astype(np.float64)))
        M[t, order[:k]] = True
    return M


def layer(weights: dict, x_bits, top_k: int, group: int = 64):
    X = _bf16(x_bits)
    R = _bf16(weights["router"])
    logits = X @ R.T
    if weights.get("logit_bias") is not None:
        logits = logits + np.asarray(weights["logit_bias"], dtype=np.float32).astype(np.float64)[None, :]
    M = topk_mask(logits, top_k)
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    r = np.where(M, p, 0.0)
    r = r / r.sum(axis=1, keepdims=True)
    E = R.shape[0]
    y = np.zeros((X.shape[0], X.shape[1]), dtype=np.float64)
    for e in range(E):
        Fe = ffn(dense_matrix(weights["gate_q"][e], weights["gate_s"][e], weights["gate_b"][e], group),
                 dense_matrix(weights["up_q"][e], weights["up_s"][e], weights["up_b"][e], group),
                 dense_matrix(weights["down_q"][e], weights["down_s"][e], weights["down_b"][e], group), X)
        y += r[:, e:e + 1] * Fe
    if weights.get("shared_gate_q") is not None:
        # optional shared-expert gate (a checkpoint detail the pages do not
        # mention): the shared output is scaled by sigmoid(x . g)
        sw = np.ones((X.shape[0], 1))
        if weights.get("shared_expert_gate") is not None:
            z = X @ _bf16(weights["shared_expert_gate"])
            sw = (1.0 / (1.0 + np.exp(-z)))[:, None]
        y += sw * ffn(dense_matrix(weights["shared_gate_q"][0], weights["shared_gate_s"][0], weights["shared_gate_b"][0], group),
                 dense_matrix(weights["shared_up_q"][0], weights["shared_up_s"][0], weights["shared_up_b"][0], group),
                 dense_matrix(weights["shared_down_q"][0], weights["shared_down_s"][0], weights["shared_down_b"][0], group), X)
    return dict(out=y, mask=M, r=r, logits=logits)
