"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar (per the layer's contract): expert indices as per-token sets and
per-expert counts bit-exact; routing weights matched by expert index within
1e-5; outputs within max|err| <= 2e-2 * RMS(oracle output).  Several results are
correct for the slot order inside a token and the row order inside an expert
bucket, so those are compared as sets.
"""
import functools

import numpy as np
import pytest

import moe_synth
import oracle
from oracle import tie_filter

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def bem():
    import bit_expert_grouped_amd as m

    m.lib()
    return m


def rms(a):
    return float(np.sqrt(np.mean(np.square(np.asarray(a, dtype=np.float64)))))


def assert_close(gpu, ref, what):
    gpu = np.asarray(gpu, dtype=np.float64)
    err = np.abs(gpu - ref).max()
    bound = TOL * rms(ref)
    print("%s: max|err| = %.3e, 2e-2*RMS = %.3e, ratio %.4f" % (what, err, bound, err / bound))
    assert np.all(np.isfinite(gpu)), what + ": non-finite output"
    assert err <= bound, what


def assert_same_routing(idx_gpu, w_gpu, idx_ref, w_ref):
    idx_gpu = np.asarray(idx_gpu)
    w_gpu = np.asarray(w_gpu, dtype=np.float64)
    assert idx_gpu.shape == idx_ref.shape
    np.testing.assert_array_equal(np.sort(idx_gpu, axis=1), np.sort(idx_ref, axis=1))
    og = np.argsort(idx_gpu, axis=1)
    orf = np.argsort(idx_ref, axis=1)
    wg = np.take_along_axis(w_gpu, og, 1)
    wr = np.take_along_axis(w_ref, orf, 1)
    assert np.abs(wg - wr).max() <= 1e-5
    assert np.abs(w_gpu.sum(axis=1) - 1).max() <= 1e-5


@functools.lru_cache(maxsize=None)
def case(name, layer=0, n_sample=None):
    """Seeded inputs of a config plus the oracle's result (on a token sample when given)."""
    cfg = moe_synth.CONFIGS[name]
    w = moe_synth.layer_weights(cfg, layer)
    x = tie_filter.tokens(name)
    T = x.shape[0]
    tokens = None
    if n_sample is not None and n_sample < T:
        rng = np.random.default_rng(1234 + layer)
        tokens = np.sort(rng.choice(T, n_sample, replace=False)).astype(np.int32)
        tokens[0] = 0
        tokens[-1] = T - 1
    ref = oracle.moe_layer(w, x, cfg.shape.top_k, tokens=tokens)
    return cfg, w, x, tokens, ref


def run_layer(w, x, top_k):
    m = bem()
    lw = m.upload_weights(w)
    xt = m.bf16_tensor(x)
    out, idx, wt, counts = m.moe_layer(xt, lw, top_k, want_routing=True)
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy(), wt.cpu().numpy(), counts.cpu().numpy()


# ------------------------------------------------------------------ whole layer on the configs


@pytest.mark.parametrize("name,n_sample", [("tiny", None), ("decode", None), ("decode64", None),
                                           ("prefill512", 48), ("prefill4096", 32)])
def test_layer_config(name, n_sample):
    cfg, w, x, tokens, ref = case(name, 0, n_sample)
    print("case", name, "T", x.shape[0], flush=True)
    out, idx, wt, counts = run_layer(w, x, cfg.shape.top_k)
    assert_same_routing(idx, wt, ref["idx"], ref["w"])
    np.testing.assert_array_equal(counts, ref["counts"])
    sel = out if tokens is None else out[tokens]
    assert_close(sel, ref["out"], name)


@pytest.mark.parametrize("layer", [0, 23])
def test_layer_stack40_sampled_layers(layer):
    cfg, w, x, tokens, ref = case("stack40", layer, 16)
    print("case stack40 layer", layer, flush=True)
    out, idx, wt, counts = run_layer(w, x, cfg.shape.top_k)
    assert_same_routing(idx, wt, ref["idx"], ref["w"])
    np.testing.assert_array_equal(counts, ref["counts"])
    assert counts.max() > 1000  # skewed: the hottest expert spans many row tiles
    assert_close(out[tokens], ref["out"], "stack40 layer %d" % layer)


def _host(tensors):
    """Device weights in the bench's layout -> numpy arrays in the oracle's formats."""
    out = {}
    for key, v in tensors.items():
        if v is None:
            out[key] = None
        elif v.dtype == torch.int32:
            out[key] = v.cpu().numpy().view(np.uint32)
        elif v.dtype == torch.bfloat16:
            out[key] = v.view(torch.int16).cpu().numpy().view(np.uint16)
        else:
            out[key] = v.cpu().numpy()
    return out


@pytest.mark.parametrize("name,layer,n_sample", [("decode", 0, 1), ("decode", 17, 1), ("decode64", 2, 16),
                                                 ("prefill512", 1, 16), ("stack40", 3, 8)])
def test_bench_inputs_against_oracle(name, layer, n_sample):
    """The weights and tokens that bench.py draws on the device (and times) give
    the oracle's result on sampled tokens.  Tokens whose k-th and (k+1)-th logits
    are closer than 1e-4 are left out (there two correct implementations may pick
    differently; the parity inputs re-draw such rows, the bench's do not)."""
    cfg = moe_synth.CONFIGS[name]
    sh = cfg.shape
    alpha = moe_synth.zipf_alpha() if cfg.zipf else None
    t = moe_synth.device_layer(sh, cfg.seed, layer, "cuda", alpha)
    x = moe_synth.device_tokens(sh, sh.T, cfg.seed, layer, "cuda")
    m = bem()
    out, idx, wt, counts = m.moe_layer(x, m.LayerWeights(t), sh.top_k, want_routing=True)
    torch.cuda.synchronize()
    w = _host(t)
    xb = x.view(torch.int16).cpu().numpy().view(np.uint16)
    lg = oracle.router_logits(xb, w["router"], w.get("logit_bias"))
    srt = -np.sort(-lg.astype(np.float32).astype(np.float64), axis=1)
    clear = np.nonzero(srt[:, sh.top_k - 1] - srt[:, sh.top_k] >= 1e-4)[0]
    if len(clear) == 0:
        pytest.skip("every token of this draw is a near-tie")
    rng = np.random.default_rng(99 + layer)
    tokens = np.sort(rng.choice(clear, min(n_sample, len(clear)), replace=False)).astype(np.int32)
    ref = oracle.moe_layer(w, xb, sh.top_k, tokens=tokens)
    idx = idx.cpu().numpy()
    np.testing.assert_array_equal(np.sort(idx[tokens], 1), np.sort(ref["idx"][tokens], 1))
    if len(clear) == sh.T:
        np.testing.assert_array_equal(counts.cpu().numpy(), ref["counts"])
    assert_close(out.cpu().numpy()[tokens], ref["out"], "bench inputs %s layer %d" % (name, layer))


# ------------------------------------------------------------------ step-by-step ABI


def test_route_step():
    cfg, w, x, _, ref = case("decode64")
    m = bem()
    idx, wt = m.moe_route(m.bf16_tensor(x), m.bf16_tensor(w["router"]), cfg.shape.top_k)
    torch.cuda.synchronize()
    assert_same_routing(idx.cpu().numpy(), wt.cpu().numpy(), ref["idx"], ref["w"])


def test_route_step_with_logit_bias():
    cfg = moe_synth.CONFIGS["stack40"]
    x = tie_filter.tokens("stack40")[:256]
    R = moe_synth.router_weights(cfg, 5)
    b = moe_synth.zipf_bias(cfg, 5)
    l = oracle.router_logits(x, R, b)
    ref_idx, ref_w = oracle.select(l, cfg.shape.top_k)
    m = bem()
    idx, wt = m.moe_route(m.bf16_tensor(x), m.bf16_tensor(R), cfg.shape.top_k,
                          logit_bias=torch.from_numpy(b).cuda())
    torch.cuda.synchronize()
    assert_same_routing(idx.cpu().numpy(), wt.cpu().numpy(), ref_idx, ref_w)


@pytest.mark.parametrize("T,k,E", [(1, 8, 256), (37, 8, 256), (4096, 8, 256), (16, 2, 16), (50, 3, 40), (9, 1, 1)])
def test_permute_step(T, k, E):
    rng = np.random.default_rng(T * 1000 + E)
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    counts_r, offsets_r, ss_r = oracle.permute(idx, E)
    m = bem()
    counts, offsets, ss = m.moe_permute(torch.from_numpy(idx).cuda(), E)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(counts.cpu().numpy(), counts_r)
    np.testing.assert_array_equal(offsets.cpu().numpy(), offsets_r)
    ss = ss.cpu().numpy()[: T * k]
    for e in range(E):
        a, b = offsets_r[e], offsets_r[e + 1]
        np.testing.assert_array_equal(np.sort(ss[a:b]), ss_r[a:b])


def _slot_reference(w, x, idx, slots, k):
    """oracle expert outputs for the given slots (t*k+j)."""
    out = {}
    by_e = {}
    for s in slots:
        by_e.setdefault(int(idx.ravel()[s]), []).append(int(s))
    for e, ss in by_e.items():
        ex = tuple((w[m + "_q"][e], w[m + "_s"][e], w[m + "_b"][e]) for m in ("gate", "up", "down"))
        y = oracle.expert_ffn(*ex, x[[s // k for s in ss]])
        for s, row in zip(ss, y):
            out[s] = row
    return out


@pytest.mark.parametrize("name", ["tiny", "decode64", "prefill512"])
def test_expert_ffn_and_combine_steps(name):
    cfg, w, x, _, ref = case(name, 0, 48 if name == "prefill512" else None)
    k = cfg.shape.top_k
    m = bem()
    lw = m.upload_weights(w)
    xt = m.bf16_tensor(x)
    offsets = torch.from_numpy(ref["offsets"]).cuda()
    ss = torch.from_numpy(ref["sorted_slot"]).cuda()
    y_slot, y_shared = m.moe_expert_ffn(xt, offsets, ss, lw, k)
    torch.cuda.synchronize()
    y_slot = y_slot.cpu().numpy()
    y_shared = y_shared.cpu().numpy()
    rng = np.random.default_rng(7)
    slots = rng.choice(x.shape[0] * k, min(64, x.shape[0] * k), replace=False)
    yr = _slot_reference(w, x, ref["idx"], slots, k)
    assert_close(y_slot[slots], np.stack([yr[s] for s in slots]), name + " y_slot")
    toks = np.unique(slots // k)[:16]
    ex = tuple((w["shared_" + mm + "_q"][0], w["shared_" + mm + "_s"][0], w["shared_" + mm + "_b"][0])
               for mm in ("gate", "up", "down"))
    assert_close(y_shared[toks], oracle.expert_ffn(*ex, x[toks]), name + " y_shared")


def test_combine_step():
    rng = np.random.default_rng(3)
    T, k, H = 37, 8, 2048
    y_slot = rng.standard_normal((T * k, H)).astype(np.float32)
    y_sh = rng.standard_normal((T, H)).astype(np.float32)
    w = rng.random((T, k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    ref = oracle.combine(y_slot.reshape(T, k, H), w, y_sh)
    m = bem()
    out = m.moe_combine(torch.from_numpy(y_slot).cuda(), torch.from_numpy(w).cuda(), torch.from_numpy(y_sh).cuda())
    torch.cuda.synchronize()
    np.testing.assert_allclose(out.cpu().numpy(), ref, rtol=1e-5, atol=1e-5)
    out2 = m.moe_combine(torch.from_numpy(y_slot).cuda(), torch.from_numpy(w).cuda(), None)
    ref2 = oracle.combine(y_slot.reshape(T, k, H), w, None)
    torch.cuda.synchronize()
    np.testing.assert_allclose(out2.cpu().numpy(), ref2, rtol=1e-5, atol=1e-5)


# ------------------------------------------------------------------ edge cases


def _custom(T, H, E, k, I, Is, bf16=True, seed=77, bias=None):
    cfg = moe_synth.Config("custom", moe_synth.Shape(T=T, H=H, E=E, top_k=k, I=I, I_shared=Is, sb_bf16=bf16),
                           seed=seed)
    w = moe_synth.layer_weights(cfg)
    if bias is not None:
        w["logit_bias"] = bias
    x = tie_filter.tokens_for(cfg, w["router"], bias)
    return cfg, w, x


@pytest.mark.parametrize("T,H,E,k,I,bf16", [
    (37, 2048, 256, 8, 512, True),     # ragged token count, real shapes
    (129, 512, 64, 4, 128, False),     # ragged, several row tiles per expert
    (5, 256, 40, 3, 64, True),         # E not a multiple of 32
    (6, 128, 8, 8, 64, True),          # k == E
    (7, 192, 1, 1, 192, False),        # single expert
    # large-batch path (T*k > 32*E): 8-wave gate/up on 128-row tiles, down on the 64-row map
    (600, 384, 16, 2, 192, True),      # ragged H and I: partial column slabs in both products
    (520, 256, 12, 3, 320, False),     # E not a multiple of 32, fp32 scales, I = 256 + 64
    (1200, 256, 8, 2, 128, True),      # ~300 rows per expert: several 128-row tiles each
    # gate/up synchronises once per pair of K stages; a scale block starts on the first stage of a pair
    (1100, 320, 8, 2, 128, False),     # fp32 scales (4 groups per block): 5 stages, a block start at stage 4, which is alone
    (1100, 576, 8, 2, 64, True),       # bf16 scales (8 groups per block): 9 stages, the block start at 8 alone in its pair
    # large-batch router (T >= 2048): LDS-staged 64 x 64 logit tiles with K split S ways
    (2100, 1024, 256, 8, 64, True),    # ragged last token tile, S = 2 (8 chunks of 64 columns)
    (2100, 256, 40, 3, 64, False),     # one 64-expert tile with 24 clamped rows, S = 4 (one chunk)
    (2050, 192, 48, 2, 64, True),      # H = 192: S = 1 with an odd count of 3 chunks; a 2-token last tile
])
def test_edge_shapes(T, H, E, k, I, bf16):
    cfg, w, x = _custom(T, H, E, k, I, I, bf16)
    ref = oracle.moe_layer(w, x, k)
    out, idx, wt, counts = run_layer(w, x, k)
    assert_same_routing(idx, wt, ref["idx"], ref["w"])
    np.testing.assert_array_equal(counts, ref["counts"])
    assert_close(out, ref["out"], "edge T%d H%d E%d k%d I%d" % (T, H, E, k, I))


def _tied(T, H, E, k, I, seed=91, tau=1e-4):
    """Router rows repeated in threes (experts 3i, 3i+1, 3i+2 share a row), so
    every logit is exactly equal to its group's on both sides; with k = 8 the
    k-th boundary splits a group and only the tie rule (the lower expert index
    ranks first) decides which members are kept.  Tokens whose distinct top
    logits come closer than tau (where rounding order could reorder the groups)
    are left out."""
    cfg = moe_synth.Config("tied", moe_synth.Shape(T=T, H=H, E=E, top_k=k, I=I, I_shared=I, sb_bf16=True),
                           seed=seed)
    w = moe_synth.layer_weights(cfg)
    R = w["router"].copy()
    for e in range(0, E - 2, 3):
        R[e + 1] = R[e]
        R[e + 2] = R[e]
    w["router"] = R
    x = moe_synth.token_rows(cfg, 4 * T)
    lg = oracle.router_logits(x, R)
    keep = []
    for t in range(x.shape[0]):
        top = np.unique(lg[t])[::-1][: k + 2]
        if np.min(top[:-1] - top[1:]) >= tau:
            keep.append(t)
    assert len(keep) >= T
    return w, x[np.array(keep[:T])]


# (3, 256, 96) and the E = 128 decode shape below leave whole groups of the
# decode selection's 8 groups of 32 experts empty, so more than 64 candidates
# reach its bound and it falls back to the radix search
@pytest.mark.parametrize("T,H,E", [(3, 256, 48), (3, 256, 96), (64, 256, 48), (1, 2048, 256), (600, 2048, 256)])
def test_exact_logit_ties_go_to_the_lower_index(T, H, E):
    k = 8
    w, x = _tied(T, H, E, k, 64)
    ref = oracle.moe_layer(w, x, k)
    # the boundary group is split in every token: the rule is exercised
    for t in range(T):
        kept = set(ref["idx"][t].tolist())
        groups = {e // 3 for e in kept}
        assert any(sum((g * 3 + j) in kept for j in range(3)) not in (0, 3) for g in groups if g * 3 + 2 < E)
    out, idx, wt, counts = run_layer(w, x, k)
    assert_same_routing(idx, wt, ref["idx"], ref["w"])
    np.testing.assert_array_equal(counts, ref["counts"])
    assert_close(out, ref["out"], "tied logits T%d" % T)
    m = bem()
    ridx, rw = m.moe_route(m.bf16_tensor(x), m.bf16_tensor(w["router"]), k)
    torch.cuda.synchronize()
    assert_same_routing(ridx.cpu().numpy(), rw.cpu().numpy(), ref["idx"], ref["w"])


@pytest.mark.parametrize("T,H,E,k,I,bf16", [
    (16, 256, 16, 2, 64, False),     # tiny shapes, fp32 scales (prefill path)
    (1, 2048, 256, 8, 512, True),    # decode
    (3, 2048, 256, 8, 512, True),    # decode, several tokens
    (64, 2048, 256, 8, 512, True),   # batched decode on the prefill path
    (600, 384, 16, 2, 192, True),    # large-batch path
])
def test_gated_shared_expert(T, H, E, k, I, bf16):
    """The optional shared-expert gate (a checkpoint detail): the shared output
    scaled by sigmoid(x . g) on every path, against the oracle."""
    cfg, w, x = _custom(T, H, E, k, I, I, bf16, seed=500 + T)
    w["shared_expert_gate"] = moe_synth.shared_expert_gate(cfg)
    ref = oracle.moe_layer(w, x, k)
    out, idx, wt, counts = run_layer(w, x, k)
    assert_same_routing(idx, wt, ref["idx"], ref["w"])
    np.testing.assert_array_equal(counts, ref["counts"])
    assert_close(out, ref["out"], "gated shared expert T%d" % T)
    w0 = {key: v for key, v in w.items() if key != "shared_expert_gate"}
    ungated = oracle.moe_layer(w0, x, k)["out"]
    assert np.abs(ungated - ref["out"]).max() > 4 * TOL * rms(ref["out"])  # the gate matters at this tolerance


def test_shared_gate_and_gated_combine_steps():
    cfg, w, x = _custom(37, 2048, 256, 8, 512, 512, True, seed=808)
    g = moe_synth.shared_expert_gate(cfg)
    m = bem()
    s = m.moe_shared_gate(m.bf16_tensor(x), m.bf16_tensor(g))
    torch.cuda.synchronize()
    s_ref = oracle.shared_gate(x, g)
    np.testing.assert_allclose(s.cpu().numpy(), s_ref, rtol=0, atol=2e-5)
    rng = np.random.default_rng(5)
    T, k, H = 37, 8, 2048
    y_slot = rng.standard_normal((T * k, H)).astype(np.float32)
    y_sh = rng.standard_normal((T, H)).astype(np.float32)
    wt = rng.random((T, k)).astype(np.float32)
    wt /= wt.sum(axis=1, keepdims=True)
    sw = s_ref.astype(np.float32)
    out = m.moe_combine(torch.from_numpy(y_slot).cuda(), torch.from_numpy(wt).cuda(), torch.from_numpy(y_sh).cuda(),
                        shared_w=torch.from_numpy(sw).cuda())
    torch.cuda.synchronize()
    ref = oracle.combine(y_slot.reshape(T, k, H), wt, y_sh, shared_w=sw)
    np.testing.assert_allclose(out.cpu().numpy(), ref, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("T,H,E,k,I,bf16,res", [
    (1, 2048, 256, 8, 512, True, "none"),      # decode
    (1, 2048, 256, 8, 512, True, "inplace"),
    (3, 2048, 256, 8, 512, True, "separate"),
    (64, 2048, 256, 8, 512, True, "inplace"),  # prefill path
    (600, 384, 16, 2, 192, True, "separate"),  # large-batch path
    (16, 256, 16, 2, 64, False, "inplace"),    # tiny shapes, fp32 scales
])
def test_layer_into_bf16_residual_stream(T, H, E, k, I, bf16, res):
    """moe_layer_residual: out = bf16(residual + layer).  Bar: the layer's own
    2e-2 * RMS plus one bf16 rounding of the total (2^-8 relative)."""
    cfg, w, x = _custom(T, H, E, k, I, I, bf16, seed=900 + T)
    ref = oracle.moe_layer(w, x, k)["out"]
    rng = np.random.default_rng(T + 7)
    res_bits = moe_synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    total = ref + (moe_synth.bf16_bits_to_f32(res_bits).astype(np.float64) if res != "none" else 0.0)
    m = bem()
    lw = m.upload_weights(w)
    res_t = m.bf16_tensor(res_bits) if res != "none" else None
    out = m.moe_layer_residual(m.bf16_tensor(x), lw, k, residual=res_t, out=res_t if res == "inplace" else None)
    torch.cuda.synchronize()
    if res == "inplace":
        assert out.data_ptr() == res_t.data_ptr()
    got = moe_synth.bf16_bits_to_f32(out.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    err = np.abs(got - total)
    bound = TOL * rms(ref) + 2.0 ** -8 * np.abs(total)
    print("bf16 residual T%d %s: max err/bound %.3f" % (T, res, float((err / bound).max())))
    assert np.all(np.isfinite(got)) and np.all(err <= bound)


@pytest.mark.parametrize("T,H,E,k,I,bf16,n_sample", [
    (40, 2560, 16, 4, 768, True, None),    # small-tile prefill path, H > 2048 and I > 512
    (700, 2304, 16, 2, 1024, False, 24),   # large-batch path, fp32 scales, sampled tokens
])
def test_prefill_wide_shapes(T, H, E, k, I, bf16, n_sample):
    cfg, w, x = _custom(T, H, E, k, I, I, bf16, seed=300 + T)
    tokens = None
    if n_sample is not None:
        rng = np.random.default_rng(T)
        tokens = np.sort(rng.choice(T, n_sample, replace=False)).astype(np.int32)
    ref = oracle.moe_layer(w, x, k, tokens=tokens)
    out, idx, wt, counts = run_layer(w, x, k)
    assert_same_routing(idx, wt, ref["idx"], ref["w"])
    np.testing.assert_array_equal(counts, ref["counts"])
    assert_close(out if tokens is None else out[tokens], ref["out"], "wide prefill T%d H%d I%d" % (T, H, I))


def test_hot_expert_spans_many_tiles():
    bias = np.zeros(32, dtype=np.float32)
    bias[5] = 50.0
    cfg, w, x = _custom(300, 256, 32, 2, 128, 128, True, bias=bias)
    ref = oracle.moe_layer(w, x, 2)
    out, idx, wt, counts = run_layer(w, x, 2)
    assert counts[5] == 300
    assert_same_routing(idx, wt, ref["idx"], ref["w"])
    np.testing.assert_array_equal(counts, ref["counts"])
    assert_close(out, ref["out"], "hot expert")


@pytest.mark.parametrize("k", [4, 5, 6, 7])
def test_every_top_k_width(k):
    """The combine is specialised per k (1..8): the widths the other cases do
    not reach, each with and without the shared expert."""
    cfg, w, x = _custom(45, 256, 24, k, 64, 64, True, seed=900 + k)
    for shared in (True, False):
        wk = w if shared else {key: v for key, v in w.items() if not key.startswith("shared_")}
        ref = oracle.moe_layer(wk, x, k)
        out, idx, wt, counts = run_layer(wk, x, k)
        assert_same_routing(idx, wt, ref["idx"], ref["w"])
        np.testing.assert_array_equal(counts, ref["counts"])
        assert_close(out, ref["out"], "k=%d shared=%s" % (k, shared))


@pytest.mark.parametrize("T", [37, 600, 2100])
def test_prefill_path_is_bitwise_reproducible(T):
    """Slots of one expert land in atomic order, but every row's products run
    in a fixed K order and the combine adds in slot order, so two calls give
    identical bits (the decode kernel's float32 atomics do not promise this)."""
    cfg, w, x = _custom(T, 512, 64, 8, 128, 128, True, seed=950 + T)
    m = bem()
    lw = m.upload_weights(w)
    xt = m.bf16_tensor(x)
    outs = []
    for _ in range(3):
        outs.append(m.moe_layer(xt, lw, 8).cpu().numpy())
    torch.cuda.synchronize()
    for o in outs[1:]:
        np.testing.assert_array_equal(o.view(np.uint32), outs[0].view(np.uint32))


def _custom_q8(T, H, E, k, I, bf16=True, seed=61):
    """A layer whose router is 8-bit (the MLX affine layout); tokens drawn
    away from near-ties of the restored router."""
    cfg = moe_synth.Config("custom", moe_synth.Shape(T=T, H=H, E=E, top_k=k, I=I, I_shared=I, sb_bf16=bf16),
                           seed=seed)
    w = moe_synth.layer_weights(cfg)
    w.update(moe_synth.router_q8(cfg, 0))
    w["router"] = None
    x = tie_filter.tokens_for(cfg, oracle.layer_router(w), None)
    return cfg, w, x


@pytest.mark.parametrize("E,H,bf16", [(256, 2048, True), (40, 192, False), (3, 64, True)])
def test_router_dequant_step(E, H, bf16):
    cfg = moe_synth.Config("custom", moe_synth.Shape(T=1, H=H, E=E, top_k=1, I=64, I_shared=64, sb_bf16=bf16),
                           seed=5 + E)
    r = moe_synth.router_q8(cfg, 2)
    want = oracle.router_dequant_q8(r["router_q8"], r["router_scale"], r["router_bias"])
    m = bem()
    q = torch.from_numpy(r["router_q8"].view(np.int32)).cuda()
    if bf16:
        sc = torch.from_numpy(r["router_scale"].view(np.int16)).cuda().view(torch.bfloat16)
        bi = torch.from_numpy(r["router_bias"].view(np.int16)).cuda().view(torch.bfloat16)
    else:
        sc, bi = torch.from_numpy(r["router_scale"]).cuda(), torch.from_numpy(r["router_bias"]).cuda()
    got = m.moe_router_dequant(q, sc, bi)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.view(torch.int16).cpu().numpy().view(np.uint16), want)


@pytest.mark.parametrize("T,H,E,k,I,bf16", [
    (1, 2048, 256, 8, 512, True),    # decode kernel
    (3, 2048, 256, 8, 512, True),    # decode kernel, several tokens
    (2, 256, 24, 3, 64, False),      # decode kernel, float32 scales and biases
    (64, 2048, 256, 8, 512, True),   # batched decode on the prefill path (restored in the logits kernel)
    (40, 256, 24, 3, 64, False),     # the same with float32 scales and biases
    (600, 512, 64, 8, 128, True),    # large-batch path
    (2100, 1024, 256, 8, 64, True),  # the LDS-staged router (restored into the workspace first)
])
def test_layer_with_q8_router(T, H, E, k, I, bf16):
    cfg, w, x = _custom_q8(T, H, E, k, I, bf16=bf16, seed=70 + T)
    print("case q8 router T", T, flush=True)
    ref = oracle.moe_layer(w, x, k)
    out, idx, wt, counts = run_layer(w, x, k)
    assert_same_routing(idx, wt, ref["idx"], ref["w"])
    np.testing.assert_array_equal(counts, ref["counts"])
    assert_close(out, ref["out"], "q8 router T%d" % T)


def test_large_batch_router_with_logit_bias():
    """The LDS-staged router (T >= 2048) with K split in two: only split 0 adds
    the bias; skewed routing from a Zipf-ranked per-expert offset."""
    shape = moe_synth.Shape(T=2100, H=1024, E=256, top_k=8, I=64, I_shared=64, sb_bf16=True)
    bias = moe_synth.zipf_bias(moe_synth.Config("custom", shape, seed=31), 3)
    cfg, w, x = _custom(2100, 1024, 256, 8, 64, 64, True, seed=31, bias=bias)
    ref = oracle.moe_layer(w, x, 8)
    out, idx, wt, counts = run_layer(w, x, 8)
    assert counts.max() > 4 * counts.mean()  # the offsets skew the routing
    assert_same_routing(idx, wt, ref["idx"], ref["w"])
    np.testing.assert_array_equal(counts, ref["counts"])
    assert_close(out, ref["out"], "large-batch router with bias")


def test_no_shared_expert():
    cfg, w, x = _custom(20, 256, 16, 2, 64, 64, True)
    w = {key: v for key, v in w.items() if not key.startswith("shared_")}
    ref = oracle.moe_layer(w, x, 2)
    m = bem()
    lw = m.upload_weights(w)
    assert lw.I_shared == 0
    out = m.moe_layer(m.bf16_tensor(x), lw, 2)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref["out"], "no shared expert")


def test_empty_batch_is_a_noop():
    import ctypes

    cfg, w, x = _custom(4, 256, 16, 2, 64, 64)
    m = bem()
    lw = m.upload_weights(w)
    out = torch.full((1, 256), 7.0, device="cuda")
    d = lw.dims(0, 2)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    st = m.lib().moe_layer(ctypes.byref(d), ctypes.byref(lw.struct), None, out.data_ptr(), None, None, None,
                           ws.data_ptr(), ws.numel(), m._stream())
    torch.cuda.synchronize()
    assert st == 0
    assert float(out[0, 0]) == 7.0


# ------------------------------------------------------------------ invariances


def test_batch_invariance_and_repeatability():
    cfg, w, x, _, ref = case("decode64")
    k = cfg.shape.top_k
    out, idx, wt, counts = run_layer(w, x, k)
    out2, idx2, _, counts2 = run_layer(w, x, k)
    np.testing.assert_array_equal(idx, idx2)
    np.testing.assert_array_equal(counts, counts2)
    for t in (0, 17, 63):
        o1, i1, _, _ = run_layer(w, x[t:t + 1], k)
        np.testing.assert_array_equal(np.sort(i1[0]), np.sort(idx[t]))
        assert np.abs(o1[0] - out[t]).max() <= 1e-3 * rms(out[t])


# ------------------------------------------------------------------ decode path (T <= 4)


@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_decode_path_real_shapes(T):
    cfg, w, x = _custom(T, 2048, 256, 8, 512, 512, True, seed=500 + T)
    ref = oracle.moe_layer(w, x, 8)
    out, idx, wt, counts = run_layer(w, x, 8)
    assert_same_routing(idx, wt, ref["idx"], ref["w"])
    np.testing.assert_array_equal(counts, ref["counts"])
    assert_close(out, ref["out"], "decode T=%d" % T)


@pytest.mark.parametrize("T,H,E,k,I,bf16,shared", [
    (3, 256, 16, 2, 64, False, True),
    (2, 512, 40, 3, 128, True, True),
    (1, 128, 8, 8, 64, True, False),
    (4, 2560, 64, 4, 192, True, True),
    (2, 256, 128, 8, 64, True, True),
    # a grid of 7 workgroups, padded up to the 32 the decode kernel's arrival count needs
    (1, 64, 2, 1, 64, True, False),
    # down rows too long for LDS (I > 512): the down workgroups read them from memory
    (2, 1024, 16, 2, 1024, False, True),
    # ... and float32 scales and biases of I = 2048 that do not fit beside them either
    (1, 512, 8, 2, 2048, False, True),
    (3, 4096, 16, 4, 4096, True, True),    # the largest intermediate size the library accepts
])
def test_decode_path_other_shapes(T, H, E, k, I, bf16, shared):
    cfg, w, x = _custom(T, H, E, k, I, I, bf16, seed=600 + T + E)
    if not shared:
        w = {key: v for key, v in w.items() if not key.startswith("shared_")}
    ref = oracle.moe_layer(w, x, k)
    out, idx, wt, counts = run_layer(w, x, k)
    assert_same_routing(idx, wt, ref["idx"], ref["w"])
    np.testing.assert_array_equal(counts, ref["counts"])
    assert_close(out, ref["out"], "decode T%d H%d E%d k%d I%d" % (T, H, E, k, I))


def control_words(ws):
    """(decode call counter, timeout flag) of a workspace.  The decode
    workgroups count themselves in on 32 64-bit words (uint32 words 512 + 32 g
    and 513 + 32 g: started workgroups of the running call, calls made), whose
    call counts must agree; word 255 is the timeout flag."""
    words = ws[:8192].view(torch.int32).cpu().numpy()
    calls = {int(words[513 + 32 * g]) for g in range(32)}
    assert len(calls) == 1, calls
    return calls.pop(), int(words[255])


def arrivals(ws):
    """Workgroups of a running decode call that have started, per group: all
    back to zero once a call has run, whatever its grid."""
    words = ws[:8192].view(torch.int32).cpu().numpy()
    return [int(words[512 + 32 * g]) for g in range(32)]


def test_decode_repeated_calls_and_control_words():
    """Successive decode calls on one workspace each match the oracle; the call
    counter advances by one per call and no wait times out."""
    cfg, w, x = _custom(4, 2048, 256, 8, 512, 512, True, seed=700)
    m = bem()
    lw = m.upload_weights(w)
    d = lw.dims(1, 8)
    ws = m.workspace(d)
    for t in range(4):
        ref = oracle.moe_layer(w, x[t:t + 1], 8)
        out = m.moe_layer(m.bf16_tensor(x[t:t + 1]), lw, 8, ws=ws)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), ref["out"], "decode call %d" % t)
        assert control_words(ws) == (t + 1, 0)
        assert arrivals(ws) == [0] * 32


def test_workspace_shared_by_prefill_and_decode():
    """One workspace serves prefill and decode calls of different dims in any
    order: the decode region sits at fixed offsets, so what a prefill call wrote
    can never pass for a published decode value."""
    cfg, w, x = _custom(64, 2048, 256, 8, 512, 512, True, seed=710)
    m = bem()
    lw = m.upload_weights(w)
    ws = m.workspace(lw.dims(64, 8))
    calls = [64, 1, 3, 48, 4, 2, 64, 1]
    for n, T in enumerate(calls):
        xs = x[n % 3:n % 3 + T]
        ref = oracle.moe_layer(w, xs, 8)
        out = m.moe_layer(m.bf16_tensor(xs), lw, 8, ws=ws)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), ref["out"], "call %d T%d" % (n, T))
    assert control_words(ws) == (sum(1 for T in calls if T <= 4), 0)
    assert arrivals(ws) == [0] * 32


# ------------------------------------------------------------------ HIP graph capture


@pytest.mark.parametrize("T", [1, 37, 1100])
def test_graph_replays_match_eager(T):
    """moe_layer captured in a HIP graph: several replays, with new inputs copied in
    eagerly between them, each match an eager call on the same inputs (T=1: the
    decode kernel; 37: 64-row tiles; 1100: 128-row gate/up tiles and the 64-row
    down map)."""
    cfg, w, x = _custom(3 * T, 2048, 256, 8, 512, 512, True, seed=800 + T)
    m = bem()
    lw = m.upload_weights(w)
    d = lw.dims(T, 8)
    ws = m.workspace(d)
    xin = m.bf16_tensor(x[:T])
    out = torch.empty(T, 2048, device="cuda")
    idx = torch.empty(T, 8, dtype=torch.int32, device="cuda")
    wt = torch.empty(T, 8, device="cuda")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        m.moe_layer(xin, lw, 8, out=out, ws=ws, want_routing=True, topk_idx_out=idx, topk_w_out=wt)  # warm-up
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            m.moe_layer(xin, lw, 8, out=out, ws=ws, want_routing=True, topk_idx_out=idx, topk_w_out=wt)
    torch.cuda.synchronize()
    ws_eager = m.workspace(d)
    for rep in range(3):
        xr = m.bf16_tensor(x[rep * T:(rep + 1) * T])
        xin.copy_(xr)                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_e, i_e, w_e, _ = m.moe_layer(xr, lw, 8, ws=ws_eager, want_routing=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(np.sort(idx.cpu().numpy(), 1), np.sort(i_e.cpu().numpy(), 1))
        ref = o_e.cpu().numpy().astype(np.float64)
        assert np.abs(out.cpu().numpy() - ref).max() <= 1e-3 * rms(ref)
        assert control_words(ws)[1] == 0


def test_back_to_back_decode_calls_in_one_graph():
    """Ten decode calls captured into one graph, each with its own input and
    output and no synchronisation between them: every output matches the oracle,
    no wait timed out (word 255) and the call counter (word 0) advanced by the
    number of calls on every replay.  This is how the timed decode steps run."""
    n = 10
    cfg, w, x = _custom(n, 2048, 256, 8, 512, 512, True, seed=1500)
    m = bem()
    lw = m.upload_weights(w)
    d = lw.dims(1, 8)
    ws = m.workspace(d)
    xs = [m.bf16_tensor(x[i:i + 1]) for i in range(n)]
    outs = [torch.full((1, 2048), float("nan"), device="cuda") for _ in range(n)]
    refs = [oracle.moe_layer(w, x[i:i + 1], 8)["out"] for i in range(n)]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(n):
                m.moe_layer(xs[i], lw, 8, out=outs[i], ws=ws)
    torch.cuda.synchronize()
    assert control_words(ws) == (0, 0)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert control_words(ws) == ((rep + 1) * n, 0)
        assert arrivals(ws) == [0] * 32
        for i in range(n):
            assert_close(outs[i].cpu().numpy(), refs[i], "graph replay %d call %d" % (rep, i))
