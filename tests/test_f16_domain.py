"""The float16 range of the expert products, on the GPU.

The expert products take float16 operands with float32 accumulation: the
activations x, the SwiGLU output h = silu(gate)*up and, on the prefill path
(T > 4), each expert's unweighted output row y are rounded to float16 (nearest
even), whose largest finite value is 65504.  The layer's contract for values
beyond that range: a value of magnitude >= 65520 rounds to +-inf, which
reaches every output element computed from it as inf or NaN.  So a finite
output element always meets the layer's accuracy, and a non-finite one marks
a value beyond the float16 range.

Inputs: seeded token rows scaled by powers of two (exact in bf16, and the
router logits scale exactly, so the near-tie filter of the unscaled rows still
holds), so that max|h| runs from a few percent of the limit to ~25 times it.
Each token is classified by the oracle's own h = silu(g)*u and y for its
selected experts and the shared one (float64): in range if every magnitude is
below 0.98 * 65504, beyond if one exceeds 1.02 * 65520 (the GPU's float32
sums differ from the float64 ones by far less than 2 %), else not compared.
In range: the row is finite and within 2e-2 * RMS of the oracle's row (the
layer's bar, per token because the rows' scales differ by ~10^4).  Beyond: the
row holds a non-finite element, and its finite elements meet the same bar.
"""
import numpy as np
import pytest

import moe_synth
import oracle
from oracle import tie_filter

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-2
F16_MAX = 65504.0
F16_INF_FROM = 65520.0  # the smallest magnitude that rounds to inf (nearest even)
T, H, E, K, I = 64, 512, 32, 4, 256


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


def _case():
    cfg = moe_synth.Config("custom", moe_synth.Shape(T=T, H=H, E=E, top_k=K, I=I, I_shared=I, sb_bf16=True),
                           seed=91)
    w = moe_synth.layer_weights(cfg)
    base = tie_filter.tokens_for(cfg, w["router"], None)
    p = np.arange(T) % 8
    x = moe_synth.f32_to_bf16_bits(moe_synth.bf16_bits_to_f32(base) * (2.0 ** p)[:, None].astype(np.float32))
    ref = oracle.moe_layer(w, x, K)
    return w, x, ref


def _magnitudes(w, x, ref):
    """Per token: max |h| and max |y| over its selected experts and the shared one (oracle, float64)."""
    hmax = np.zeros(T)
    ymax = np.zeros(T)

    def one(e, row, pre):
        mat = lambda n: tuple(w[pre + n + s][e] for s in ("_q", "_s", "_b"))
        y, g, u = oracle.expert_ffn(mat("gate"), mat("up"), mat("down"), row[None], want_gu=True)
        with np.errstate(over="ignore"):
            h = g / (1.0 + np.exp(-g)) * u
        return np.abs(h).max(), np.abs(y).max()

    for t in range(T):
        for hm, ym in [one(e, x[t], "") for e in ref["idx"][t]] + [one(0, x[t], "shared_")]:
            hmax[t] = max(hmax[t], hm)
            ymax[t] = max(ymax[t], ym)
    return hmax, ymax


def _check(out, ref, peak, what):
    inside = peak < 0.98 * F16_MAX
    beyond = peak > 1.02 * F16_INF_FROM
    near = inside & (peak >= 0.5 * F16_MAX)
    print("%s: %d tokens in range (%d above half the limit), %d beyond, %d not compared"
          % (what, inside.sum(), near.sum(), beyond.sum(), T - inside.sum() - beyond.sum()), flush=True)
    assert near.sum() >= 2 and beyond.sum() >= 10, "the scale ladder must reach both sides of the limit"
    for t in range(T):
        bound = TOL * rms(ref["out"][t])
        fin = np.isfinite(out[t])
        if inside[t]:
            assert fin.all(), "%s token %d (max %.0f): non-finite output inside the float16 range" % (what, t, peak[t])
        elif beyond[t]:
            assert not fin.all(), "%s token %d (max %.0f): finite output beyond the float16 range" % (what, t, peak[t])
        else:
            continue
        err = np.abs(out[t][fin] - ref["out"][t][fin]).max(initial=0.0)
        assert err <= bound, "%s token %d: max|err| %.3e over finite elements, bound %.3e" % (what, t, err, bound)


def _routing(idx, wt, ref):
    np.testing.assert_array_equal(np.sort(idx, axis=1), np.sort(ref["idx"], axis=1))
    og, orf = np.argsort(idx, axis=1), np.argsort(ref["idx"], axis=1)
    assert np.abs(np.take_along_axis(wt, og, 1) - np.take_along_axis(ref["w"], orf, 1)).max() <= 1e-5


def test_prefill_path_float16_range():
    """T = 64 in one call: x, h and y are float16."""
    w, x, ref = _case()
    hmax, ymax = _magnitudes(w, x, ref)
    m = bem()
    lw = m.upload_weights(w)
    out, idx, wt, _ = m.moe_layer(m.bf16_tensor(x), lw, K, want_routing=True)
    torch.cuda.synchronize()
    _routing(idx.cpu().numpy(), wt.cpu().numpy(), ref)
    _check(out.cpu().numpy().astype(np.float64), ref, np.maximum(hmax, ymax), "prefill")


def test_decode_path_float16_range():
    """The same tokens four at a time (the decode kernel): x and h are float16,
    y stays float32, so only h decides."""
    w, x, ref = _case()
    hmax, _ = _magnitudes(w, x, ref)
    m = bem()
    lw = m.upload_weights(w)
    outs, idxs, wts = [], [], []
    for t0 in range(0, T, 4):
        out, idx, wt, _ = m.moe_layer(m.bf16_tensor(x[t0:t0 + 4]), lw, K, want_routing=True)
        outs.append(out.cpu().numpy())
        idxs.append(idx.cpu().numpy())
        wts.append(wt.cpu().numpy())
    torch.cuda.synchronize()
    _routing(np.concatenate(idxs), np.concatenate(wts), ref)
    _check(np.concatenate(outs).astype(np.float64), ref, hmax, "decode")
