"""GPU parity of moe_gqa_decode (decode attention with grouped-query KV
sharing) against the oracle.

Bar, per (sequence, query head) row, from the arithmetic: the scores are
float32 sums of exact bf16 products, and the softmax weights enter the P V
product rounded to bf16 (relative error <= 2^-9), the normaliser summing the
same rounded weights.  The output is then a weighted mean of the value rows
whose weights are off by at most ~2^-9 relative, so |error| <= 2^-8 *
max|v - out| <= 2^-7 * max|v|; the check is that bound per element, and the
root-mean-square error within 1e-2 of the row's RMS (the expected error of
random roundings is ~1e-3 of it).
"""
import numpy as np
import pytest

import moe_synth
import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def bem():
    import bit_expert_grouped_amd as m

    m.lib()
    return m


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def check(out, ref, v_bits, lens, G, what):
    """out, ref [B][Hq][D]; v_bits [B][Hkv][S][D]."""
    out = np.asarray(out, dtype=np.float64)
    B, Hq, D = ref.shape
    worst = 0.0
    for b in range(B):
        n = max(0, min(int(lens[b]), v_bits.shape[2]))
        for h in range(Hq):
            if n == 0:
                np.testing.assert_array_equal(out[b, h], 0.0)
                continue
            vmax = np.abs(moe_synth.bf16_bits_to_f32(v_bits[b, h // G, :n])).max()
            err = np.abs(out[b, h] - ref[b, h])
            assert np.all(np.isfinite(out[b, h])), "%s: non-finite output at b=%d h=%d" % (what, b, h)
            assert err.max() <= 2.0 ** -7 * vmax + 1e-6, "%s b=%d h=%d: max|err| %.3e > 2^-7 max|v| %.3e" % (
                what, b, h, err.max(), 2.0 ** -7 * vmax)
            r = np.sqrt(np.mean(err ** 2)) / np.sqrt(np.mean(ref[b, h] ** 2))
            assert r <= 1e-2, "%s b=%d h=%d: RMS(err)/RMS(ref) %.3e" % (what, b, h, r)
            worst = max(worst, r)
    print("%s: worst RMS(err)/RMS(ref) %.2e" % (what, worst), flush=True)


def run(shape, lens, seed, q_std=1.0, scale=None):
    q, k, v = moe_synth.attn_inputs(shape, seed, q_std)
    lens = np.asarray(lens, dtype=np.int32)
    ref = oracle.gqa_decode(q, k, v, lens, scale)
    m = bem()
    d = m.gqa_dims(shape.B, shape.Hq, shape.Hkv, shape.D, shape.S)
    ws = m.gqa_workspace(d)
    out = m.gqa_decode(_dev(q), _dev(k), _dev(v), torch.from_numpy(lens).cuda(), scale, ws=ws)
    torch.cuda.synchronize()
    assert not m.gqa_timed_out(ws, d)
    return out.cpu().numpy(), ref, v, lens


@pytest.mark.parametrize("B,Hq,Hkv,D,S,lens,q_std", [
    (1, 16, 2, 128, 1000, [1000], 1.0),          # the model's heads, a ragged last run
    (3, 16, 2, 128, 700, [700, 1, 257], 1.0),    # one row; one row past a run of 256
    (2, 8, 8, 64, 300, [300, 0], 1.0),           # one query head per KV head; an empty sequence
    (1, 32, 2, 256, 600, [600], 1.0),            # 16 query heads per KV head, D = 256 (runs of 128)
    (2, 16, 4, 64, 520, [520, 255], 1.0),        # 4 per KV head, D = 64; a run one row short
    (1, 16, 2, 256, 129, [129], 1.0),            # D = 256: two runs, the second of one row
    (1, 16, 1, 128, 50, [50], 1.0),              # one KV head for all 16
    (2, 16, 2, 128, 3000, [3000, 2049], 8.0),    # peaked softmax (scores ~ N(0, 64))
    (1, 16, 2, 128, 600, [600], 0.0),            # q = 0: the mean of the value rows
])
def test_gqa_small_shapes(B, Hq, Hkv, D, S, lens, q_std):
    shape = moe_synth.AttnShape(B=B, Hq=Hq, Hkv=Hkv, D=D, S=S)
    print("case B=%d Hq=%d Hkv=%d D=%d S=%d lens=%s q_std=%g" % (B, Hq, Hkv, D, S, lens, q_std), flush=True)
    out, ref, v, lens = run(shape, lens, 61, q_std)
    check(out, ref, v, lens, Hq // Hkv, "gqa %s" % (shape,))


def test_gqa_grid_larger_than_the_device():
    """24 sequences of 4096 rows: 768 workgroups, more than the device holds at
    once, so the partials are merged by a second kernel."""
    shape = moe_synth.AttnShape(B=24, Hq=16, Hkv=2, D=128, S=4096)
    assert bem().gqa_decode_kernels(bem().gqa_dims(24, 16, 2, 128, 4096)) == 2
    assert bem().gqa_decode_kernels(bem().gqa_dims(1, 16, 2, 128, 32768)) == 1
    lens = [4096 - 97 * i for i in range(24)]
    out, ref, v, lens = run(shape, lens, 66)
    check(out, ref, v, lens, 8, "two-kernel merge")


def test_gqa_scale_argument():
    shape = moe_synth.AttnShape(B=1, Hq=16, Hkv=2, D=128, S=400)
    out, ref, v, lens = run(shape, [400], 62, 1.0, scale=0.3)
    check(out, ref, v, lens, 8, "scale 0.3")


@pytest.mark.parametrize("q_std", [1.0, 4.0])
def test_gqa_32k_context(q_std):
    """The model's full-attention decode at 32K context (16 query / 2 KV heads, D = 128), every output."""
    print("case 32K context q_std=%g" % q_std, flush=True)
    out, ref, v, lens = run(moe_synth.GQA32K, [moe_synth.GQA32K.S], 63, q_std)
    check(out, ref, v, lens, 8, "32K q_std %g" % q_std)


def test_gqa_lengths_below_the_cache_and_repeats():
    """Sequences shorter than the cache read only their rows; repeated calls
    give the same bits (no atomics); a captured graph replays them exactly."""
    shape = moe_synth.AttnShape(B=4, Hq=16, Hkv=2, D=128, S=5000)
    q, k, v = moe_synth.attn_inputs(shape, 64)
    lens = np.array([5000, 4097, 13, 2500], dtype=np.int32)
    ref = oracle.gqa_decode(q, k, v, lens)
    m = bem()
    tq, tk, tv = _dev(q), _dev(k), _dev(v)
    tl = torch.from_numpy(lens).cuda()
    # rows past each length hold NaN: never read
    for b in range(4):
        tk[b, :, lens[b]:] = float("nan")
        tv[b, :, lens[b]:] = float("nan")
    a = m.gqa_decode(tq, tk, tv, tl)
    b2 = m.gqa_decode(tq, tk, tv, tl)
    torch.cuda.synchronize()
    check(a.cpu().numpy(), ref, v, lens, 8, "lengths below the cache")
    assert torch.equal(a, b2)
    out = torch.empty_like(a)
    ws = m.gqa_workspace(m.gqa_dims(4, 16, 2, 128, 5000))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            m.gqa_decode(tq, tk, tv, tl, out=out, ws=ws)
    torch.cuda.synchronize()
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, a)


def test_gqa_events_variant_matches():
    """moe_gqa_decode_events: the same bits as moe_gqa_decode, with its three
    events recorded in order."""
    shape = moe_synth.AttnShape(B=2, Hq=16, Hkv=2, D=128, S=900)
    q, k, v = moe_synth.attn_inputs(shape, 65)
    m = bem()
    tq, tk, tv = _dev(q), _dev(k), _dev(v)
    tl = torch.tensor([900, 333], dtype=torch.int32, device="cuda")
    a = m.gqa_decode(tq, tk, tv, tl)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    b = m.gqa_decode(tq, tk, tv, tl, events=ev)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert ev[0].elapsed_time(ev[1]) > 0 and ev[1].elapsed_time(ev[2]) > 0


def test_gqa_back_to_back_calls_share_a_workspace():
    """Four calls on different caches, one workspace, launched back to back with
    no host sync between them (then replayed as a graph): each output matches
    its own oracle, so nothing a call leaves in the workspace or in a cache is
    read by the next."""
    shape = moe_synth.AttnShape(B=1, Hq=16, Hkv=2, D=128, S=8192)
    m = bem()
    d = m.gqa_dims(1, 16, 2, 128, 8192)
    ws = m.gqa_workspace(d)
    lens = np.array([8192 - 300 * i for i in range(4)], dtype=np.int32)
    cases = []
    for i in range(4):
        q, k, v = moe_synth.attn_inputs(shape, 70 + i)
        ref = oracle.gqa_decode(q, k, v, lens[i:i + 1])
        cases.append((_dev(q), _dev(k), _dev(v), torch.from_numpy(lens[i:i + 1]).cuda(), ref, v))
    outs = [torch.empty(1, 16, 128, dtype=torch.float32, device="cuda") for _ in range(4)]
    for (tq, tk, tv, tl, _, _), o in zip(cases, outs):
        m.gqa_decode(tq, tk, tv, tl, out=o, ws=ws)
    torch.cuda.synchronize()
    assert not m.gqa_timed_out(ws, d)
    for (_, _, _, _, ref, v), o, i in zip(cases, outs, range(4)):
        check(o.cpu().numpy(), ref, v, lens[i:i + 1], 8, "back to back call %d" % i)
    eager = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for (tq, tk, tv, tl, _, _), o in zip(cases, outs):
                m.gqa_decode(tq, tk, tv, tl, out=o, ws=ws)
    torch.cuda.synchronize()
    for _ in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e)
    assert not m.gqa_timed_out(ws, d)
