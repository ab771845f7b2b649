"""moe_layer_no_alloc: the layer on the library's static per-device scratch,
for callers that cannot allocate.  Through the C ABI, two calls in a row (the
second on a smaller batch) must give what moe_layer gives on a workspace of its
own: expert indices and counts bit-exact, outputs within 2e-2 * RMS (and the
oracle's result to the same bar).  Run last: the scratch keeps what earlier
calls left, which is part of what is tested."""
import ctypes

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


def rms(a):
    return float(np.sqrt(np.mean(np.square(np.asarray(a, dtype=np.float64)))))


def _layer(T, H, E, k, I, bf16, seed):
    cfg = moe_synth.Config("custom", moe_synth.Shape(T=T, H=H, E=E, top_k=k, I=I, I_shared=I, sb_bf16=bf16),
                           seed=seed)
    w = moe_synth.layer_weights(cfg)
    x = tie_filter.tokens_for(cfg, w["router"], None)
    return w, x


def _no_alloc_call(m, lw, x, k):
    """One moe_layer_no_alloc call through the C entry point."""
    T, H = x.shape
    d = lw.dims(T, k)
    out = torch.full((T, H), float("nan"), device="cuda")
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    wt = torch.empty(T, k, dtype=torch.float32, device="cuda")
    counts = torch.empty(lw.E, dtype=torch.int32, device="cuda")
    st = m.lib().moe_layer_no_alloc(ctypes.byref(d), ctypes.byref(lw.struct), x.data_ptr(), out.data_ptr(),
                                    idx.data_ptr(), wt.data_ptr(), counts.data_ptr(), m._stream())
    assert st == 0, m.status_string(st)
    return out, idx, wt, counts


@pytest.mark.parametrize("T1,T2,H,E,k,I,bf16", [
    (300, 37, 2048, 256, 8, 512, True),   # prefill path, then a smaller prefill batch
    (3, 1, 2048, 256, 8, 512, True),      # decode kernel, then a single token
    (64, 2, 256, 16, 2, 64, False),       # prefill, then decode, fp32 scales
])
def test_no_alloc_matches_moe_layer(T1, T2, H, E, k, I, bf16):
    import bit_expert_grouped_amd as m

    w, x = _layer(T1, H, E, k, I, bf16, seed=1700 + T1)
    lw = m.upload_weights(w)
    for T in (T1, T2):
        print("case no_alloc T", T, flush=True)
        xs = x[:T]
        xt = m.bf16_tensor(xs)
        got = _no_alloc_call(m, lw, xt, k)
        ref_out, ref_idx, ref_w, ref_counts = m.moe_layer(xt, lw, k, want_routing=True)
        torch.cuda.synchronize()
        got = [a.cpu().numpy() for a in got]
        np.testing.assert_array_equal(np.sort(got[1], 1), np.sort(ref_idx.cpu().numpy(), 1))
        np.testing.assert_array_equal(got[3], ref_counts.cpu().numpy())
        ref = ref_out.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(got[0]))
        assert np.abs(got[0] - ref).max() <= TOL * rms(ref)
        orc = oracle.moe_layer(w, xs, k)
        np.testing.assert_array_equal(np.sort(got[1], 1), np.sort(orc["idx"], 1))
        assert np.abs(got[0] - orc["out"]).max() <= TOL * rms(orc["out"])


def test_no_alloc_in_a_captured_graph():
    """Captured into a graph and replayed (after an eager call has prepared the
    device's scratch), the entry point still matches moe_layer."""
    import bit_expert_grouped_amd as m

    w, x = _layer(8, 2048, 256, 8, 512, True, seed=1801)
    lw = m.upload_weights(w)
    xin = m.bf16_tensor(x[:1])
    m.moe_layer_no_alloc(xin, lw, 8)
    torch.cuda.synchronize()
    out = torch.empty(1, 2048, device="cuda")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            m.moe_layer_no_alloc(xin, lw, 8, out=out)
    torch.cuda.synchronize()
    for rep in range(3):
        xin.copy_(m.bf16_tensor(x[rep + 1:rep + 2]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = m.moe_layer(xin, lw, 8).cpu().numpy().astype(np.float64)
        torch.cuda.synchronize()
        assert np.abs(out.cpu().numpy() - ref).max() <= TOL * rms(ref)


def test_no_alloc_refuses_dims_beyond_its_scratch():
    import bit_expert_grouped_amd as m

    d = m.dims(1024, 2048, 256, 8, 512, 512)
    assert m.moe_workspace_size(d) > m.NO_ALLOC_SCRATCH_BYTES
    fake = 0x10000
    q = m.QMat(fake, fake, fake)
    f = m.Ffn(q, q, q)
    wts = m.Weights(fake, None, f, f)
    st = m.lib().moe_layer_no_alloc(ctypes.byref(d), ctypes.byref(wts), fake, fake, None, None, None, None)
    assert st == -5
