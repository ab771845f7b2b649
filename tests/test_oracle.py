"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: hand-worked
values (tests/golden), closed forms, textbook routines (torch CPU float64),
an independent dense brute force (oracle.brute), or invariants.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import moe_synth
import oracle
from oracle import brute, tie_filter

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _sb_array(vals, kind):
    if kind == "bf16":
        return np.array([[int(v, 16) for v in vals]], dtype=np.uint16)
    return np.array([vals], dtype=np.float32)


def small_cfg(T=8, H=128, E=6, k=2, I=64, Is=64, bf16=True, seed=11):
    return moe_synth.Config("custom", moe_synth.Shape(T=T, H=H, E=E, top_k=k, I=I, I_shared=Is,
                                                      sb_bf16=bf16), seed=seed)


def _zero_sb(w, prefix):
    for m in ("gate", "up", "down"):
        for p in ("_s", "_b"):
            w[prefix + m + p] = np.zeros_like(w[prefix + m + p])


# ---------------------------------------------------------------- dequant


@pytest.mark.parametrize("ex", _load("dequant_examples.json")["examples"], ids=lambda e: e["name"])
def test_dequant_hand_examples(ex):
    if "words_repeat" in ex:
        word, n = ex["words_repeat"]
        words = np.array([[int(word, 16)] * n], dtype=np.uint32)
    else:
        words = np.array([[int(w, 16) for w in ex["words"]]], dtype=np.uint32)
    s = _sb_array(ex["scale"], ex["sb"])
    b = _sb_array(ex["bias"], ex["sb"])
    W = oracle.dequant(words, s, b, group=ex["group"])[0]
    if "values_runs" in ex:
        expect = np.concatenate([np.full(n, v) for v, n in ex["values_runs"]])
    else:
        expect = np.array(ex["values"])
        codes = [oracle.code(words, s, b, 0, k, group=ex["group"]) for k in range(8)]
        assert codes == ex["codes"]
    np.testing.assert_array_equal(W, expect)


def test_code_position_single_nibble():
    """A lone non-zero nibble at bit position 4p of word w is element 8w+p."""
    K = 128
    for w in range(K // 8):
        for p in range(8):
            q = np.zeros((1, K // 8), dtype=np.uint32)
            q[0, w] = np.uint32(9 << (4 * p))
            W = oracle.dequant(q, np.ones((1, 2), np.float32), np.zeros((1, 2), np.float32))
            nz = np.nonzero(W[0])[0]
            assert list(nz) == [8 * w + p] and W[0, 8 * w + p] == 9.0


# ---------------------------------------------------------------- routing


@pytest.mark.parametrize("ex", _load("routing_examples.json")["examples"], ids=str)
def test_routing_hand_examples(ex):
    idx, w = oracle.select(np.array([ex["logits"]]), ex["k"])
    assert list(idx[0]) == ex["idx"]
    np.testing.assert_allclose(w[0], ex["w"], rtol=0, atol=1e-15)


def test_routing_invariants_random():
    rng = np.random.default_rng(5)
    for E, k in ((16, 2), (256, 8), (64, 7), (5, 5)):
        logits = rng.standard_normal((200, E))
        idx, w = oracle.select(logits, k)
        assert np.all(np.abs(w.sum(axis=1) - 1.0) <= k * 2.0 ** -52)
        for t in range(len(idx)):
            sel = idx[t]
            assert len(set(sel.tolist())) == k and sel.min() >= 0 and sel.max() < E
            rest = np.setdiff1d(np.arange(E), sel)
            if len(rest):
                assert logits[t, sel].min() >= logits[t, rest].max()
            assert np.all(np.diff(w[t]) <= 0)
            assert np.all(np.diff(logits[t, sel]) <= 0)


def test_routing_k1_weight_is_one():
    logits = np.random.default_rng(1).standard_normal((50, 16))
    idx, w = oracle.select(logits, 1)
    assert np.all(w == 1.0)
    np.testing.assert_array_equal(idx[:, 0], np.argmax(logits, axis=1))


def test_routing_k_equals_E_is_full_softmax():
    logits = np.random.default_rng(2).standard_normal((20, 9)) * 3
    idx, w = oracle.select(logits, 9)
    sm = torch.softmax(torch.from_numpy(logits), dim=1).numpy()
    for t in range(20):
        np.testing.assert_allclose(w[t], sm[t, idx[t]], rtol=1e-13)
        np.testing.assert_array_equal(np.sort(idx[t]), np.arange(9))


def test_router_logits_against_matmul():
    cfg = small_cfg(T=5, H=256, E=7)
    x = moe_synth.token_rows(cfg)
    R = moe_synth.router_weights(cfg)
    bias = np.linspace(-1, 1, 7).astype(np.float32)
    got = oracle.router_logits(x, R, bias)
    X = torch.from_numpy(moe_synth.bf16_bits_to_f32(x).astype(np.float64))
    Wr = torch.from_numpy(moe_synth.bf16_bits_to_f32(R).astype(np.float64))
    ref = (X @ Wr.T).numpy() + bias.astype(np.float64)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- permute


def test_permute_hand_example():
    ex = _load("permute_example.json")
    counts, offsets, ss = oracle.permute(np.array(ex["idx"]), ex["E"])
    assert counts.tolist() == ex["counts"]
    assert offsets.tolist() == ex["offsets"]
    assert ss.tolist() == ex["sorted_slot"]


def test_permute_invariants():
    rng = np.random.default_rng(3)
    T, k, E = 300, 8, 256
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, offsets, ss = oracle.permute(idx, E)
    assert counts.sum() == T * k and offsets[-1] == T * k
    np.testing.assert_array_equal(np.sort(ss), np.arange(T * k))
    flat = idx.ravel()
    for e in range(E):
        seg = ss[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)


# ---------------------------------------------------------------- expert FFN


def _expert(w, e, prefix=""):
    return tuple((w[prefix + m + "_q"][e], w[prefix + m + "_s"][e], w[prefix + m + "_b"][e])
                 for m in ("gate", "up", "down"))


def test_ffn_one_hot_input_reads_one_column():
    """x = unit vector e_i (bf16 1.0 at i): g[n] = W_gate[n][i] exactly."""
    cfg = small_cfg(H=256, I=64)
    w = moe_synth.layer_weights(cfg)
    gate, up, down = _expert(w, 1)
    Wg = oracle.dequant(*gate)
    Wu = oracle.dequant(*up)
    for i in (0, 7, 8, 63, 64, 200, 255):
        x = np.zeros((1, 256), dtype=np.uint16)
        x[0, i] = 0x3F80  # 1.0
        y, g, u = oracle.expert_ffn(gate, up, down, x, want_gu=True)
        np.testing.assert_array_equal(g[0], Wg[:, i])
        np.testing.assert_array_equal(u[0], Wu[:, i])


def test_ffn_all_codes_zero_closed_form():
    """All codes 0: W = bias per group, so g[n] = sum_g b[n][g] * sum_{h in g} x[h]."""
    cfg = small_cfg(H=256, I=64, bf16=False)
    w = moe_synth.layer_weights(cfg)
    gate, up, down = _expert(w, 0)
    gate = (np.zeros_like(gate[0]),) + gate[1:]
    x = moe_synth.token_rows(cfg)[:3]
    _, g, _ = oracle.expert_ffn(gate, up, down, x, want_gu=True)
    xs = moe_synth.bf16_bits_to_f32(x).astype(np.float64).reshape(3, 4, 64).sum(axis=2)
    expect = xs @ gate[2].astype(np.float64).T
    np.testing.assert_allclose(g, expect, rtol=1e-12, atol=1e-12)


def test_single_expert_is_textbook_swiglu_mlp():
    """E=1, k=1: routing weight 1, so out = SwiGLU(x; expert 0) + SwiGLU(x; shared)."""
    cfg = small_cfg(T=6, H=128, E=1, k=1, I=64, Is=128)
    w = moe_synth.layer_weights(cfg)
    x = moe_synth.token_rows(cfg)
    res = oracle.moe_layer(w, x, 1)
    X = torch.from_numpy(moe_synth.bf16_bits_to_f32(x).astype(np.float64))

    def mlp(prefix, e):
        Wg, Wu, Wd = (torch.from_numpy(oracle.dequant(*m)) for m in _expert(w, e, prefix))
        return torch.nn.functional.linear(torch.nn.functional.silu(X @ Wg.T) * (X @ Wu.T), Wd)

    ref = (mlp("", 0) + mlp("shared_", 0)).numpy()
    np.testing.assert_allclose(res["out"], ref, rtol=1e-11, atol=1e-11)
    assert np.all(res["w"] == 1.0) and np.all(res["idx"] == 0)


def test_k_equals_E_is_dense_softmax_mixture():
    cfg = small_cfg(T=4, H=128, E=5, k=5, I=64)
    w = moe_synth.layer_weights(cfg)
    x = moe_synth.token_rows(cfg)
    res = oracle.moe_layer(w, x, 5, want_logits=True)
    X = torch.from_numpy(moe_synth.bf16_bits_to_f32(x).astype(np.float64))
    p = torch.softmax(torch.from_numpy(res["logits"]), dim=1)

    def mlp(prefix, e):
        Wg, Wu, Wd = (torch.from_numpy(oracle.dequant(*m)) for m in _expert(w, e, prefix))
        return (torch.nn.functional.silu(X @ Wg.T) * (X @ Wu.T)) @ Wd.T

    ref = sum(p[:, e:e + 1] * mlp("", e) for e in range(5)) + mlp("shared_", 0)
    np.testing.assert_allclose(res["out"], ref.numpy(), rtol=1e-11, atol=1e-11)


def test_zeroed_routed_experts_leave_shared_only_and_vice_versa():
    cfg = small_cfg(T=5, E=6, k=2)
    w = moe_synth.layer_weights(cfg)
    x = moe_synth.token_rows(cfg)
    full = oracle.moe_layer(w, x, 2)["out"]
    w_r0 = dict(w)
    _zero_sb(w_r0, "")
    shared_only = oracle.moe_layer(w_r0, x, 2)["out"]
    w_s0 = dict(w)
    _zero_sb(w_s0, "shared_")
    routed_only = oracle.moe_layer(w_s0, x, 2)["out"]
    ys = oracle.expert_ffn(*_expert(w, 0, "shared_"), x)
    np.testing.assert_allclose(shared_only, ys, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(routed_only + shared_only, full, rtol=1e-12, atol=1e-12)
    assert np.abs(routed_only).max() > 0.1 and np.abs(shared_only).max() > 0.1


# ---------------------------------------------------------------- whole layer vs brute force


def _rms(a):
    return float(np.sqrt(np.mean(np.square(a))))


def test_tiny_config_against_brute_force():
    cfg = moe_synth.CONFIGS["tiny"]
    w = moe_synth.layer_weights(cfg)
    x = tie_filter.tokens("tiny")
    res = oracle.moe_layer(w, x, cfg.shape.top_k)
    bf = brute.layer(w, x, cfg.shape.top_k)
    assert np.abs(res["out"] - bf["out"]).max() <= 1e-12 * _rms(bf["out"]) * 1e3
    M = np.zeros_like(bf["mask"])
    np.put_along_axis(M, res["idx"].astype(np.int64), True, axis=1)
    np.testing.assert_array_equal(M, bf["mask"])
    np.testing.assert_allclose(np.take_along_axis(bf["r"], res["idx"].astype(np.int64), 1), res["w"], rtol=1e-13)


@pytest.mark.parametrize("seed", [21, 22, 23, 24])
def test_random_tiny_shapes_against_brute_force(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(1, 12))
    k = int(rng.integers(1, E + 1))
    cfg = small_cfg(T=int(rng.integers(1, 9)), H=64 * int(rng.integers(1, 4)), E=E, k=k,
                    I=64 * int(rng.integers(1, 3)), Is=64 * int(rng.integers(1, 3)),
                    bf16=bool(seed % 2), seed=seed)
    w = moe_synth.layer_weights(cfg)
    x = moe_synth.token_rows(cfg)
    res = oracle.moe_layer(w, x, k)
    bf = brute.layer(w, x, k)
    assert np.abs(res["out"] - bf["out"]).max() <= 1e-9 * _rms(bf["out"])
    M = np.zeros_like(bf["mask"])
    np.put_along_axis(M, res["idx"].astype(np.int64), True, axis=1)
    np.testing.assert_array_equal(M, bf["mask"])


def test_logit_bias_enters_selection_and_softmax():
    cfg = small_cfg(T=6, E=8, k=3)
    w = moe_synth.layer_weights(cfg)
    w["logit_bias"] = np.linspace(2.0, -2.0, 8).astype(np.float32)
    x = moe_synth.token_rows(cfg)
    res = oracle.moe_layer(w, x, 3)
    bf = brute.layer(w, x, 3)
    assert np.abs(res["out"] - bf["out"]).max() <= 1e-9 * _rms(bf["out"])


# ---------------------------------------------------------------- optional shared-expert gate (R14)


def _bf16_bits(vals):
    return (np.asarray(vals, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("ex", _load("shared_gate_examples.json")["examples"], ids=str)
def test_shared_gate_hand_examples(ex):
    x = _bf16_bits(ex["x"])[None, :]
    g = _bf16_bits(ex["g"])
    np.testing.assert_allclose(oracle.shared_gate(x, g), [ex["s"]], rtol=1e-15, atol=0)


def test_zero_shared_gate_halves_the_shared_expert():
    cfg = small_cfg(T=5, E=6, k=2)
    w = moe_synth.layer_weights(cfg)
    x = moe_synth.token_rows(cfg)
    full = oracle.moe_layer(w, x, 2)["out"]
    w_s0 = dict(w)
    _zero_sb(w_s0, "shared_")
    routed_only = oracle.moe_layer(w_s0, x, 2)["out"]
    wg = dict(w)
    wg["shared_expert_gate"] = np.zeros(cfg.shape.H, dtype=np.uint16)  # sigmoid(0) = 1/2 exactly
    gated = oracle.moe_layer(wg, x, 2)["out"]
    np.testing.assert_allclose(gated, (full + routed_only) / 2, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", [31, 32])
def test_shared_gate_against_brute_force(seed):
    cfg = small_cfg(T=7, H=192, E=5, k=2, I=64, Is=128, bf16=bool(seed % 2), seed=seed)
    w = moe_synth.layer_weights(cfg)
    w["shared_expert_gate"] = moe_synth.shared_expert_gate(cfg)
    x = moe_synth.token_rows(cfg)
    res = oracle.moe_layer(w, x, 2)
    bf = brute.layer(w, x, 2)
    assert np.abs(res["out"] - bf["out"]).max() <= 1e-9 * _rms(bf["out"])
    s = oracle.shared_gate(x, w["shared_expert_gate"])
    assert 0.1 < s.min() and s.max() < 0.9 and s.std() > 0.01  # the gate does vary across tokens


# ---------------------------------------------------------------- invariances


def test_token_subset_equals_full_batch():
    cfg = small_cfg(T=8, E=6, k=2)
    w = moe_synth.layer_weights(cfg)
    x = moe_synth.token_rows(cfg)
    full = oracle.moe_layer(w, x, 2)
    sub = oracle.moe_layer(w, x, 2, tokens=[6, 1, 3])
    np.testing.assert_array_equal(sub["out"], full["out"][[6, 1, 3]])
    alone = oracle.moe_layer(w, x[3:4], 2)
    np.testing.assert_allclose(alone["out"][0], full["out"][3], rtol=1e-14, atol=1e-14)


def test_expert_relabelling_invariance():
    cfg = small_cfg(T=8, E=6, k=2)
    w = moe_synth.layer_weights(cfg)
    x = moe_synth.token_rows(cfg)
    perm = np.array([3, 5, 0, 1, 4, 2])
    w2 = dict(w)
    for key in ("router", "gate_q", "gate_s", "gate_b", "up_q", "up_s", "up_b", "down_q", "down_s", "down_b"):
        w2[key] = w[key][perm]
    a = oracle.moe_layer(w, x, 2)
    b = oracle.moe_layer(w2, x, 2)
    np.testing.assert_allclose(a["out"], b["out"], rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(np.sort(a["idx"], 1), np.sort(perm[b["idx"]], 1))


# ---------------------------------------------------------------- inputs


def test_near_ties_removed():
    for name in ("tiny", "decode", "decode64"):
        cfg = moe_synth.CONFIGS[name]
        x = tie_filter.tokens(name)
        l = tie_filter.router_logits_f64(x, moe_synth.router_weights(cfg))
        assert np.all(tie_filter.kth_gap(l, cfg.shape.top_k) >= tie_filter.TAU)


def test_oracle_float32_logit_error_is_far_below_tie_margin():
    """fp32 sums of the router products (pairwise and sequential) stay within TAU/10 of float64."""
    cfg = moe_synth.CONFIGS["decode64"]
    x = tie_filter.tokens("decode64")
    R = moe_synth.router_weights(cfg)
    l64 = tie_filter.router_logits_f64(x, R)
    X = moe_synth.bf16_bits_to_f32(x)
    W = moe_synth.bf16_bits_to_f32(R)
    l32 = X @ W.T
    seq = np.zeros_like(l32)
    for h in range(0, X.shape[1], 16):
        seq += X[:, h:h + 16] @ W[:, h:h + 16].T
    assert np.abs(l32 - l64).max() < tie_filter.TAU / 10
    assert np.abs(seq - l64).max() < tie_filter.TAU / 10


def test_zipf_offset_reaches_half_of_assignments_on_sampled_layers():
    cfg = moe_synth.CONFIGS["stack40"]
    x = moe_synth.token_rows(cfg, 1024)
    shares = []
    for layer in (0, 13, 39):
        l = tie_filter.router_logits_f64(x, moe_synth.router_weights(cfg, layer), moe_synth.zipf_bias(cfg, layer))
        idx, _ = oracle.select(l, cfg.shape.top_k)
        c = np.sort(np.bincount(idx.ravel(), minlength=cfg.shape.E))[::-1]
        shares.append(c[:16].sum() / idx.size)
    assert abs(np.mean(shares) - 0.5) < 0.05


def test_generator_formats():
    cfg = moe_synth.CONFIGS["tiny"]
    w = moe_synth.layer_weights(cfg)
    sh = cfg.shape
    assert w["gate_q"].shape == (sh.E, sh.I, sh.H // 8) and w["gate_q"].dtype == np.uint32
    assert w["down_q"].shape == (sh.E, sh.H, sh.I // 8)
    assert w["gate_s"].shape == (sh.E, sh.I, sh.H // 64) and w["gate_s"].dtype == np.float32
    assert w["shared_down_b"].shape == (1, sh.H, sh.I_shared // 64)
    assert 0.005 <= w["gate_s"].min() and w["gate_s"].max() <= 0.02
    w1 = moe_synth.layer_weights(moe_synth.CONFIGS["tiny"])
    np.testing.assert_array_equal(w1["up_q"], w["up_q"])
    assert math.isclose(moe_synth.bf16_bits_to_f32(np.array([0x3F80], np.uint16))[0], 1.0)


# ---------------------------------------------------------------- 8-bit router (R16)

@pytest.mark.parametrize("ex", _load("router_q8_examples.json")["cases"], ids=lambda e: e["what"][:24])
def test_router_q8_hand_examples(ex):
    codes = np.zeros((1, 16), dtype=np.uint32)  # one row of 64 columns: one group
    codes[0, 0] = ex["word"]
    for bf16_sb in (True, False):
        sc = np.array([[ex["scale"]]], dtype=np.float32)
        bi = np.array([[ex["bias"]]], dtype=np.float32)
        if bf16_sb:
            sc, bi = moe_synth.f32_to_bf16_bits(sc), moe_synth.f32_to_bf16_bits(bi)
        w = moe_synth.bf16_bits_to_f32(oracle.router_dequant_q8(codes, sc, bi))
        np.testing.assert_array_equal(w[0, :4], np.array(ex["weights"], dtype=np.float32))
        np.testing.assert_array_equal(w[0, 4:], np.float32(ex["bias"]))  # code 0 restores the bias


def test_router_q8_against_brute_force():
    """Every byte, scale and bias position: bf16 scales and biases make
    s * q + b exact in float64, so one rounding to float32 is the fused
    multiply-add's, then nearest-even to bfloat16."""
    cfg = small_cfg(T=2, E=5, k=2)
    r = moe_synth.router_q8(cfg, 3)
    got = oracle.router_dequant_q8(r["router_q8"], r["router_scale"], r["router_bias"])
    E, H = got.shape
    q = np.stack([(r["router_q8"] >> (8 * i)) & 0xFF for i in range(4)], axis=-1).reshape(E, H).astype(np.float64)
    s = np.repeat(moe_synth.bf16_bits_to_f32(r["router_scale"]).astype(np.float64), 64, axis=1)
    b = np.repeat(moe_synth.bf16_bits_to_f32(r["router_bias"]).astype(np.float64), 64, axis=1)
    want = moe_synth.f32_to_bf16_bits((s * q + b).astype(np.float32))
    np.testing.assert_array_equal(got, want)
    assert np.abs(moe_synth.bf16_bits_to_f32(got)).max() < 0.06  # spread like the dense router


def test_layer_with_q8_router_uses_the_restored_matrix():
    cfg = small_cfg(T=7, E=6, k=2)
    w = moe_synth.layer_weights(cfg)
    x = moe_synth.token_rows(cfg)
    wq = dict(w)
    wq.update(moe_synth.router_q8(cfg, 0))
    wq["router"] = None
    dense = dict(w)
    dense["router"] = oracle.router_dequant_q8(wq["router_q8"], wq["router_scale"], wq["router_bias"])
    a, b = oracle.moe_layer(wq, x, 2), oracle.moe_layer(dense, x, 2)
    np.testing.assert_array_equal(a["idx"], b["idx"])
    np.testing.assert_array_equal(a["out"], b["out"])


# ------------------------------------------------------------------ RMSNorm of the residual stream (R17)


@pytest.mark.parametrize("ex", _load("rmsnorm_examples.json")["examples"], ids=str)
def test_rmsnorm_hand_examples(ex):
    x = moe_synth.f32_to_bf16_bits(np.array(ex["x"], dtype=np.float32))
    g = None if ex["gamma"] is None else moe_synth.f32_to_bf16_bits(np.array(ex["gamma"], dtype=np.float32))
    y = moe_synth.bf16_bits_to_f32(oracle.rmsnorm(x, g, eps=ex["eps"])[0])
    np.testing.assert_array_equal(y, np.array(ex["y"], dtype=np.float32))


def test_rmsnorm_power_of_two_scale_invariance():
    """eps = 0: scaling the row by 2^k scales mean(x^2) by 4^k and leaves every
    output bit as it was."""
    rng = np.random.default_rng(11)
    x = moe_synth.f32_to_bf16_bits(rng.standard_normal(2048).astype(np.float32))
    base = oracle.rmsnorm(x, eps=0.0)
    for k in (-3, 5, 9):
        xs = moe_synth.f32_to_bf16_bits(moe_synth.bf16_bits_to_f32(x) * np.float32(2.0 ** k))
        np.testing.assert_array_equal(oracle.rmsnorm(xs, eps=0.0), base)


def test_rmsnorm_unit_rms_and_gamma():
    """gamma absent: the output's root mean square is 1 up to bf16 rounding; a
    gamma of 2 doubles every output exactly; a gamma of -1 negates it."""
    rng = np.random.default_rng(12)
    x = moe_synth.f32_to_bf16_bits((rng.standard_normal(2048) * 37.0).astype(np.float32))
    y = moe_synth.bf16_bits_to_f32(oracle.rmsnorm(x, eps=0.0)[0]).astype(np.float64)
    assert abs(np.sqrt(np.mean(y * y)) - 1.0) < 2.0 ** -8
    two = moe_synth.f32_to_bf16_bits(np.full(2048, 2.0, dtype=np.float32))
    y2 = moe_synth.bf16_bits_to_f32(oracle.rmsnorm(x, two, eps=0.0)[0]).astype(np.float64)
    np.testing.assert_array_equal(y2, 2.0 * y)
    neg = moe_synth.f32_to_bf16_bits(np.full(2048, -1.0, dtype=np.float32))
    yn = moe_synth.bf16_bits_to_f32(oracle.rmsnorm(x, neg, eps=0.0)[0]).astype(np.float64)
    np.testing.assert_array_equal(yn, -y)


# ---------------------------------------------------------------- decode attention (R19)


def _bits(a):
    return moe_synth.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def _values(bits):
    return moe_synth.bf16_bits_to_f32(bits).astype(np.float64)


def _gqa_inputs(B, Hq, Hkv, D, S, seed, q_scale=1.0):
    rng = np.random.default_rng(seed)
    q = _bits(rng.standard_normal((B, Hq, D)) * q_scale)
    k = _bits(rng.standard_normal((B, Hkv, S, D)))
    v = _bits(rng.standard_normal((B, Hkv, S, D)))
    return q, k, v


@pytest.mark.parametrize("ex", _load("gqa_examples.json")["examples"], ids=lambda e: e["name"])
def test_gqa_hand_examples(ex):
    out = oracle.gqa_decode(_bits(ex["q"]), _bits(ex["k"]), _bits(ex["v"]), np.array(ex["seq_len"]), ex["scale"])
    np.testing.assert_allclose(out, np.array(ex["out"], dtype=np.float64), rtol=1e-14, atol=1e-14)


def test_gqa_against_torch_attention_with_shared_kv_heads():
    """torch's float64 scaled_dot_product_attention with enable_gqa (the KV heads
    repeated for consecutive query heads), per sequence on its valid rows."""
    B, Hq, Hkv, D, S = 3, 16, 2, 64, 50
    q, k, v = _gqa_inputs(B, Hq, Hkv, D, S, 21, q_scale=2.0)
    lens = np.array([50, 17, 1], dtype=np.int32)
    out = oracle.gqa_decode(q, k, v, lens)
    for b in range(B):
        n = lens[b]
        tq = torch.from_numpy(_values(q[b]))[None, :, None, :]
        tk = torch.from_numpy(_values(k[b, :, :n]))[None]
        tv = torch.from_numpy(_values(v[b, :, :n]))[None]
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, enable_gqa=True)[0, :, 0].numpy()
        np.testing.assert_allclose(out[b], ref, rtol=1e-12, atol=1e-13)


def test_gqa_single_row_returns_its_value_row():
    """One cached row: its softmax weight is 1 and each head returns the value row exactly."""
    q, k, v = _gqa_inputs(2, 8, 2, 32, 5, 22)
    out = oracle.gqa_decode(q, k, v, np.array([1, 1]))
    for h in range(8):
        np.testing.assert_array_equal(out[:, h], _values(v[:, h // 4, 0]))


def test_gqa_zero_query_averages_the_values():
    """q = 0 gives equal scores: the output is the mean of the valid value rows."""
    q, k, v = _gqa_inputs(1, 4, 2, 16, 9, 23)
    q[:] = 0
    out = oracle.gqa_decode(q, k, v, np.array([7]))
    for h in range(4):
        np.testing.assert_allclose(out[0, h], _values(v[0, h // 2, :7]).mean(axis=0), rtol=1e-14, atol=1e-15)


def test_gqa_each_head_reads_its_own_kv_head():
    """Value rows constant per KV head (g + 1): every query head returns the
    constant of KV head h / (Hq / Hkv), whatever the scores."""
    B, Hq, Hkv, D, S = 2, 16, 4, 8, 6
    q, k, v = _gqa_inputs(B, Hq, Hkv, D, S, 24, q_scale=3.0)
    for g in range(Hkv):
        v[:, g] = _bits(np.full((B, S, D), g + 1.0))
    out = oracle.gqa_decode(q, k, v, np.array([6, 3]))
    for h in range(Hq):
        np.testing.assert_allclose(out[:, h], h // (Hq // Hkv) + 1.0, rtol=1e-14)


def test_gqa_row_order_does_not_matter():
    """Permuting the valid rows of K and V together leaves the output unchanged."""
    q, k, v = _gqa_inputs(1, 8, 2, 32, 40, 25, q_scale=2.0)
    perm = np.random.default_rng(26).permutation(33)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, :33] = k[:, :, perm]
    v2[:, :, :33] = v[:, :, perm]
    np.testing.assert_allclose(oracle.gqa_decode(q, k2, v2, np.array([33])), oracle.gqa_decode(q, k, v, np.array([33])),
                               rtol=1e-12, atol=1e-14)


def test_gqa_dominant_key_selects_its_value_row():
    """A key aligned with the query at a scale far above the rest takes all the weight."""
    q, k, v = _gqa_inputs(1, 2, 1, 16, 12, 27)
    k[0, 0, 5] = _bits(64.0 * _values(q[0, 0]))
    out = oracle.gqa_decode(q, k, v, np.array([12]))
    np.testing.assert_allclose(out[0, 0], _values(v[0, 0, 5]), rtol=0, atol=1e-12)


def test_gqa_scale_equals_scaled_query():
    """scale * (q.k) with scale 4 equals the default scale applied to 4 q (exact in bf16)."""
    q, k, v = _gqa_inputs(2, 4, 2, 16, 10, 28)
    q4 = _bits(4.0 * _values(q))
    a = oracle.gqa_decode(q, k, v, np.array([10, 4]), scale=4.0 / np.sqrt(16))
    b = oracle.gqa_decode(q4, k, v, np.array([10, 4]))
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)


def test_gqa_rows_past_the_length_are_not_read():
    """A sequence of n rows in a larger cache equals the same rows in a cache of exactly n."""
    q, k, v = _gqa_inputs(1, 8, 2, 32, 30, 29)
    v[:, :, 20:] = _bits(np.full((1, 2, 10, 32), 1000.0))
    a = oracle.gqa_decode(q, k, v, np.array([20]))
    b = oracle.gqa_decode(q, np.ascontiguousarray(k[:, :, :20]), np.ascontiguousarray(v[:, :, :20]), np.array([20]))
    np.testing.assert_array_equal(a, b)
