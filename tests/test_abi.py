"""The C ABI without a GPU: the library loads, exports every entry point that
include/moe.h declares, sizes its workspace, and rejects bad arguments on the
host before anything is enqueued (no call here reaches a kernel launch)."""
import ctypes as C
import os
import re

import pytest

import bit_expert_grouped_amd as bem

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

FAKE = 0x10000  # a 256-byte aligned non-NULL address; never dereferenced by these calls


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bem.LIB_PATH):
        from bit_expert_grouped_amd import build

        build.build()
    return bem.lib()


def declared_functions():
    text = open(HEADER).read()
    # declarations start in column 0 with their return type
    return sorted(set(re.findall(r"^(?:const\s+)?[a-z_][a-z_0-9]*\s*\**\s*(moe_[a-z_]+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(bem.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def qwen_dims(tokens=512, **kw):
    d = bem.dims(tokens, 2048, 256, 8, 512, 512)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_workspace_size(lib):
    d = qwen_dims(4096)
    n = bem.moe_workspace_size(d)
    # float16 activations, h rows and expert output rows (routed + shared) dominate
    big = 4096 * 2048 * 2 + (4096 * 8 + 4096) * 512 * 2 + (4096 * 8 + 4096) * 2048 * 2
    # plus the small regions: routing, tile maps, logit partials and the fixed
    # decode and stack exchange regions (about 2 MB)
    assert big <= n < big + (12 << 20)
    assert bem.moe_workspace_size(qwen_dims(1)) > 0
    assert bem.moe_workspace_size(qwen_dims(0)) > 0
    assert bem.moe_workspace_size(qwen_dims(4096)) > bem.moe_workspace_size(qwen_dims(512))


@pytest.mark.parametrize("field,value,status", [
    ("H", 100, -2), ("I", 96, -2), ("top_k", 0, -2), ("top_k", 300, -2), ("T", -1, -2), ("E", 0, -2),
    ("group", 32, -3), ("E", 512, -3), ("top_k", 9, -3), ("H", 32768, -3), ("I_shared", 1024, -3),
    ("out_dtype", 5, -2), ("sb_dtype", 7, -2),
])
def test_invalid_dims(lib, field, value, status):
    d = qwen_dims(8, **{field: value})
    assert bem.moe_workspace_size(d) == 0
    ws = FAKE
    st = lib.moe_permute(C.byref(d), FAKE, FAKE, FAKE, FAKE, ws, 1 << 30, None)
    assert st == status
    st = lib.moe_route(C.byref(d), FAKE, FAKE, None, FAKE, FAKE, None)
    assert st == status


def _weights(ptr=FAKE, shared=True):
    q = bem.QMat(ptr, ptr, ptr)
    f = bem.Ffn(q, q, q)
    return bem.Weights(ptr, None, f, f if shared else bem.Ffn())


def test_layer_argument_checks(lib):
    d = qwen_dims(8)
    need = bem.moe_workspace_size(d)
    w = _weights()
    assert lib.moe_layer(C.byref(d), None, FAKE, FAKE, None, None, None, FAKE, need, None) == -1
    assert lib.moe_layer(C.byref(d), C.byref(w), None, FAKE, None, None, None, FAKE, need, None) == -1
    assert lib.moe_layer(C.byref(d), C.byref(w), FAKE + 2, FAKE, None, None, None, FAKE, need, None) == -4
    assert lib.moe_layer(C.byref(d), C.byref(w), FAKE, FAKE, None, None, None, FAKE + 16, need, None) == -4
    assert lib.moe_layer(C.byref(d), C.byref(w), FAKE, FAKE, None, None, None, FAKE, need - 1, None) == -5
    assert lib.moe_layer(C.byref(d), C.byref(w), FAKE, FAKE, None, None, None, None, need, None) == -1
    bad = _weights()
    bad.experts.down.scale = None
    assert lib.moe_layer(C.byref(d), C.byref(bad), FAKE, FAKE, None, None, None, FAKE, need, None) == -1
    bad = _weights()
    bad.experts.up.q = FAKE + 4
    assert lib.moe_layer(C.byref(d), C.byref(bad), FAKE, FAKE, None, None, None, FAKE, need, None) == -4
    noshared = _weights(shared=False)
    assert lib.moe_layer(C.byref(d), C.byref(noshared), FAKE, FAKE, None, None, None, FAKE, need, None) == -1
    d0 = qwen_dims(8, I_shared=0)
    assert lib.moe_layer(C.byref(d0), C.byref(w), FAKE, FAKE, None, None, None, FAKE, need, None) == -2
    assert lib.moe_layer(None, C.byref(w), FAKE, FAKE, None, None, None, FAKE, need, None) == -1


def test_shared_expert_gate_checks(lib):
    d = qwen_dims(8)
    need = bem.moe_workspace_size(d)
    w = _weights()
    w.shared_expert_gate = FAKE + 2  # misaligned
    assert lib.moe_layer(C.byref(d), C.byref(w), FAKE, FAKE, None, None, None, FAKE, need, None) == -4
    noshared = _weights(shared=False)
    noshared.shared_expert_gate = FAKE  # a gate without a shared expert
    d0 = qwen_dims(8, I_shared=0)
    assert lib.moe_layer(C.byref(d0), C.byref(noshared), FAKE, FAKE, None, None, None, FAKE, need, None) == -2
    assert lib.moe_shared_gate(C.byref(d), FAKE, None, FAKE, None) == -1
    assert lib.moe_shared_gate(C.byref(d), FAKE, FAKE + 2, FAKE, None) == -4
    assert lib.moe_combine_gated(C.byref(d), FAKE, FAKE, FAKE, FAKE + 4, FAKE, None) == -4
    assert lib.moe_combine_gated(C.byref(d), None, FAKE, None, None, FAKE, None) == -1
    e = qwen_dims(0)
    assert lib.moe_shared_gate(C.byref(e), None, None, None, None) == 0
    assert lib.moe_combine_gated(C.byref(e), None, None, None, None, None, None) == 0


def test_q8_router_checks(lib):
    d = qwen_dims(8)
    need = bem.moe_workspace_size(d)
    w = _weights()
    w.router_q8, w.router_scale, w.router_bias = FAKE, FAKE, FAKE
    assert lib.moe_layer(C.byref(d), C.byref(w), FAKE, FAKE, None, None, None, FAKE, need, None) == -2  # both routers
    w.router = None
    w.router_scale = None
    assert lib.moe_layer(C.byref(d), C.byref(w), FAKE, FAKE, None, None, None, FAKE, need, None) == -1
    w.router_scale = FAKE + 4
    assert lib.moe_layer(C.byref(d), C.byref(w), FAKE, FAKE, None, None, None, FAKE, need, None) == -4
    w.router_q8 = None
    w.router_scale = FAKE
    assert lib.moe_layer(C.byref(d), C.byref(w), FAKE, FAKE, None, None, None, FAKE, need, None) == -1  # no router
    assert lib.moe_router_dequant(C.byref(d), FAKE, FAKE, None, FAKE, None) == -1
    assert lib.moe_router_dequant(C.byref(d), FAKE + 8, FAKE, FAKE, FAKE, None) == -4
    bad = qwen_dims(8, H=100)
    assert lib.moe_router_dequant(C.byref(bad), FAKE, FAKE, FAKE, FAKE, None) == -2


def test_output_dtype_per_entry_point(lib):
    """moe_layer writes float32 only; moe_layer_residual writes the bf16 residual stream only."""
    w = _weights()
    d32 = qwen_dims(8)
    d16 = qwen_dims(8, out_dtype=bem.MOE_BF16)
    need = bem.moe_workspace_size(d16)
    assert need > 0 and bem.moe_workspace_size(d32) > 0
    assert lib.moe_layer(C.byref(d16), C.byref(w), FAKE, FAKE, None, None, None, FAKE, need, None) == -3
    assert lib.moe_layer_residual(C.byref(d32), C.byref(w), FAKE, None, FAKE, FAKE, need, None) == -3
    assert lib.moe_layer_residual(C.byref(d16), C.byref(w), FAKE, None, None, FAKE, need, None) == -1
    assert lib.moe_layer_residual(C.byref(d16), C.byref(w), FAKE, FAKE + 2, FAKE, FAKE, need, None) == -4
    assert lib.moe_layer_residual(C.byref(d16), C.byref(w), FAKE, None, FAKE, FAKE, need - 1, None) == -5
    e = qwen_dims(0, out_dtype=bem.MOE_BF16)
    assert lib.moe_layer_residual(C.byref(e), None, None, None, None, None, 0, None) == 0


def test_empty_call_enqueues_nothing(lib):
    d = qwen_dims(0)
    assert lib.moe_layer(C.byref(d), None, None, None, None, None, None, None, 0, None) == 0
    assert lib.moe_route(C.byref(d), None, None, None, None, None, None) == 0
    assert lib.moe_combine(C.byref(d), None, None, None, None, None) == 0


def test_other_calls_check_arguments(lib):
    d = qwen_dims(8)
    need = bem.moe_workspace_size(d)
    f = bem.Ffn(bem.QMat(FAKE, FAKE, FAKE), bem.QMat(FAKE, FAKE, FAKE), bem.QMat(FAKE, FAKE, FAKE))
    assert lib.moe_route(C.byref(d), FAKE, FAKE, FAKE + 8, FAKE, FAKE, None) == -4
    assert lib.moe_route(C.byref(d), FAKE, None, None, FAKE, FAKE, None) == -1
    assert lib.moe_permute(C.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, need - 256, None) == -5
    assert lib.moe_expert_ffn(C.byref(d), FAKE, FAKE, FAKE, None, None, FAKE, None, FAKE, need, None) == -1
    assert lib.moe_expert_ffn(C.byref(d), FAKE, FAKE, FAKE, C.byref(f), None, None, None, FAKE, need, None) == -1
    assert lib.moe_combine(C.byref(d), FAKE, FAKE, FAKE + 4, FAKE, None) == -4
    assert lib.moe_combine(C.byref(d), FAKE, None, None, FAKE, None) == -1


def test_permute_slot_limit(lib):
    """moe_permute sorts at most 2^22 slots (T * top_k) in one call."""
    big = qwen_dims(1 << 20, top_k=4)  # exactly 2^22 slots: within the limit
    need = bem.moe_workspace_size(big)
    assert need > 0
    # within the limit the call reaches the workspace check (a too-small size is refused)
    assert lib.moe_permute(C.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, need - 256, None) == -5
    over = qwen_dims(1 << 20, top_k=5)  # 5 * 2^20 slots
    assert lib.moe_permute(C.byref(over), FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == -3


def test_no_alloc_checks(lib):
    """moe_layer_no_alloc: dims beyond its static scratch and bad arguments are
    refused on the host, before any device call."""
    big = qwen_dims(1024)
    assert bem.moe_workspace_size(big) > bem.NO_ALLOC_SCRATCH_BYTES
    w = _weights()
    assert lib.moe_layer_no_alloc(C.byref(big), C.byref(w), FAKE, FAKE, None, None, None, None) == -5
    assert lib.moe_layer_no_alloc(C.byref(qwen_dims(8, out_dtype=bem.MOE_BF16)), C.byref(w), FAKE, FAKE,
                                  None, None, None, None) == -3
    assert lib.moe_layer_no_alloc(C.byref(qwen_dims(8, H=100)), C.byref(w), FAKE, FAKE, None, None, None,
                                  None) == -2
    e = qwen_dims(0)
    assert lib.moe_layer_no_alloc(C.byref(e), None, None, None, None, None, None, None) == 0


def test_decode_stack_checks(lib):
    """moe_decode_stack refuses, on the host, what it does not support."""
    w = _weights()
    d = qwen_dims(1, out_dtype=bem.MOE_BF16)
    need = bem.moe_workspace_size(d)

    def call(dims, weights=w, strides=None, n=4, x=FAKE, ws=FAKE, ws_bytes=need):
        return lib.moe_decode_stack(C.byref(dims), C.byref(weights) if weights is not None else None, None,
                                    C.byref(strides) if strides is not None else None, n, x, FAKE, None, None,
                                    None, None, None, ws, ws_bytes, None)

    assert call(qwen_dims(0, out_dtype=bem.MOE_BF16)) == 0          # nothing to do
    assert call(d, n=0) == -2
    assert call(qwen_dims(2, out_dtype=bem.MOE_BF16)) == -3          # one token only
    assert call(qwen_dims(1)) == -3                                  # the residual stream is bf16
    assert call(qwen_dims(1, H=4096, out_dtype=bem.MOE_BF16)) == -3
    assert call(qwen_dims(1, I=1024, I_shared=1024, out_dtype=bem.MOE_BF16)) == -3
    assert call(d, weights=None) == -1
    assert call(d, x=None) == -1
    assert call(d, x=FAKE + 8) == -4
    q8 = _weights()
    q8.router_q8 = FAKE
    assert call(d, weights=q8) == -3
    gated = _weights()
    gated.shared_expert_gate = FAKE
    assert call(d, weights=gated) == -3
    st = bem.LayerStrides()
    st.experts.down.q = 24  # not a multiple of 16
    assert call(d, strides=st) == -4
    st = bem.LayerStrides()
    st.logit_bias = 6
    assert call(d, strides=st) == -4
    st = bem.LayerStrides()
    st.norm_weight = 8
    assert call(d, strides=st) == -4
    assert lib.moe_decode_stack(C.byref(d), C.byref(w), FAKE + 2, None, 4, FAKE, FAKE, None, None, None, None,
                                None, FAKE, need, None) == -4  # misaligned norm weight
    assert call(d, ws=FAKE + 16) == -4
    assert call(d, ws_bytes=need - 1) == -5


def test_gqa_workspace_and_checks(lib):
    """moe_gqa_workspace_size and moe_gqa_decode's host-side checks."""
    d = bem.gqa_dims(1, 16, 2, 128, 32768)
    n = lib.moe_gqa_workspace_size(C.byref(d))
    # 128 runs of 256 rows per KV head, each partial a 128-byte flag line and 6 bytes per
    # (head, column); 256 bytes of control words per (sequence, KV head); 256 for the timeout word
    assert n == 2 * 128 * (128 + 6 * 8 * 128) + 2 * 256 + 256
    assert lib.moe_gqa_workspace_size(C.byref(bem.gqa_dims(1, 16, 2, 256, 32768))) == \
        2 * 256 * (128 + 6 * 8 * 256) + 2 * 256 + 256
    assert lib.moe_gqa_workspace_size(C.byref(bem.gqa_dims(3, 16, 2, 128, 100))) == \
        (3 * 2 * 1 * (128 + 6 * 8 * 128) + 255) // 256 * 256 + 6 * 256 + 256
    assert lib.moe_gqa_workspace_size(C.byref(bem.gqa_dims(1, 16, 3, 128, 10))) == 0

    def call(dims, q=FAKE, k=FAKE, v=FAKE, lens=FAKE, scale=0.088, out=FAKE, ws=FAKE, ws_bytes=n):
        return lib.moe_gqa_decode(C.byref(dims), q, k, v, lens, scale, out, ws, ws_bytes, None)

    assert call(bem.gqa_dims(0, 16, 2, 128, 32768), q=None) == 0       # nothing to do
    assert call(bem.gqa_dims(1, 16, 3, 128, 64)) == -2                 # heads not a multiple
    assert call(bem.gqa_dims(1, 16, 2, 128, 0)) == -2
    assert call(bem.gqa_dims(-1, 16, 2, 128, 64)) == -2
    assert call(bem.gqa_dims(1, 16, 2, 96, 64)) == -3                  # head size
    assert call(bem.gqa_dims(1, 34, 2, 128, 64)) == -3                 # 17 query heads per KV head
    assert call(bem.gqa_dims(1, 16, 2, 128, (1 << 24) + 1)) == -3
    assert call(d, scale=float("nan")) == -2
    assert call(d, scale=float("inf")) == -2
    assert call(d, scale=3e38) == -2                                   # infinite in log2 units
    assert call(d, q=None) == -1
    assert call(d, lens=None) == -1
    assert call(d, v=FAKE + 8) == -4
    assert call(d, lens=FAKE + 2) == -4
    assert call(d, ws=None) == -1
    assert call(d, ws=FAKE + 16) == -4
    assert call(d, ws_bytes=n - 1) == -5
    assert lib.moe_gqa_decode_kernels(C.byref(bem.gqa_dims(0, 16, 2, 128, 64))) == 0
    assert lib.moe_gqa_decode_kernels(C.byref(bem.gqa_dims(1, 16, 3, 128, 64))) == 0
    ev = (C.c_void_p * 3)(FAKE, FAKE, FAKE)
    assert lib.moe_gqa_decode_events(C.byref(d), FAKE, FAKE, FAKE, FAKE, 0.088, FAKE, FAKE, n, None, None, 3) == -1
    assert lib.moe_gqa_decode_events(C.byref(d), FAKE, FAKE, FAKE, FAKE, 0.088, FAKE, FAKE, n, None, ev, 2) == -2
    assert lib.moe_gqa_decode_events(C.byref(d), None, FAKE, FAKE, FAKE, 0.088, FAKE, FAKE, n, None, ev, 3) == -1


def test_status_strings(lib):
    for code in bem.STATUS:
        assert len(bem.status_string(code)) >= 2
    assert "workspace" in bem.status_string(-5)
