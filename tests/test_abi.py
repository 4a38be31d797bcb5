"""The C ABI library on the host: it loads, exports every entry point include/moe.h declares, and
rejects invalid arguments before touching the device (no GPU needed: every call here fails its
host-side checks or is a pure host query)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "moe_layer_softmax_amd", "libmoe.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libmoe.so not built")


def _declared():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    names = _declared()
    assert {"moe_route", "moe_permute", "moe_grouped_gemm", "moe_combine", "moe_layer",
            "moe_quantize", "moe_shared_gate", "moe_routing_blob_plane"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    import moe_layer_softmax_amd as m
    lib = m.lib()
    for s in range(5):
        assert lib.moe_status_str(s)
    assert lib.moe_status_str(m.MOE_ERR_WORKSPACE) == b"workspace too small"


def _desc(**kw):
    import moe_layer_softmax_amd as m
    base = dict(T=64, H=256, E=8, e0=0, E_loc=8, I=128, k=2, I_s=0, scoring=0, renormalize=1,
                io_dtype=m.MOE_F32, expert_dtype=m.MOE_F32)
    base.update(kw)
    return m.make_desc(**base)


def test_workspace_queries():
    import moe_layer_softmax_amd as m
    d = _desc()
    ws = m.moe_layer_workspace_bytes(d)
    assert ws > 64 * 8 * 4                      # holds at least the logits
    big = _desc(T=16384, H=4096, E=128, E_loc=32, I=1536, k=8, io_dtype=m.MOE_BF16,
                expert_dtype=m.MOE_BF16)
    assert m.moe_layer_workspace_bytes(big) > 16384 * 8 * 4096 * 2     # holds y
    assert m.moe_permute_workspace_bytes(big) > 0
    assert m.moe_layer_workspace_bytes(_desc(k=0)) == 0                 # invalid desc -> 0
    # the router's K-split partial sums: a decode-sized bf16 router needs them, a prefill-sized
    # one and the fp32 router do not
    dec = _desc(T=64, H=4096, E=128, E_loc=32, I=1536, k=8, io_dtype=m.MOE_BF16,
                expert_dtype=m.MOE_BF16)
    r = m.moe_route_workspace_bytes(dec)
    assert r > 0 and r % (64 * 128 * 4) == 0
    assert m.moe_layer_workspace_bytes(dec) >= r
    assert m.moe_route_workspace_bytes(big) == 0
    assert m.moe_route_workspace_bytes(d) == 0


def test_route_workspace_too_small():
    import moe_layer_softmax_amd as m
    lib = m.lib()
    ok = ctypes.c_void_p(4096)
    dec = _desc(T=64, H=4096, E=128, E_loc=32, I=1536, k=8, io_dtype=m.MOE_BF16,
                expert_dtype=m.MOE_BF16)
    need = m.moe_route_workspace_bytes(dec)
    assert lib.moe_route(ctypes.byref(dec), ok, ok, None, ok, ok, ok, None, 0, None) == m.MOE_ERR_WORKSPACE
    assert lib.moe_route(ctypes.byref(dec), ok, ok, None, ok, ok, ok, ok, need - 4, None) == m.MOE_ERR_WORKSPACE


@pytest.mark.parametrize("bad", [dict(k=0), dict(k=17), dict(E=0), dict(E=2000), dict(T=-1),
                                 dict(e0=4, E_loc=8), dict(H=100), dict(scoring=5),
                                 dict(io_dtype=7), dict(renormalize=2), dict(out_dtype=3)])
def test_route_rejects_bad_descriptors(bad):
    import moe_layer_softmax_amd as m
    d = _desc(**bad)
    fake = ctypes.c_void_p(256)
    st = m.lib().moe_route(ctypes.byref(d), fake, fake, None, fake, fake, fake, None, 0, None)
    assert st == m.MOE_ERR_INVALID_ARG


def test_null_and_misaligned_pointers_are_rejected():
    import moe_layer_softmax_amd as m
    d = _desc()
    ok = ctypes.c_void_p(4096)
    bad = ctypes.c_void_p(4100)
    lib = m.lib()
    assert lib.moe_route(ctypes.byref(d), ok, ok, None, None, ok, ok, None, 0, None) == m.MOE_ERR_INVALID_ARG
    assert lib.moe_route(ctypes.byref(d), bad, ok, None, ok, ok, ok, None, 0, None) == m.MOE_ERR_INVALID_ARG
    assert lib.moe_route(ctypes.byref(d), ok, ok, None, ok, ok, ok, bad, 64, None) == m.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(ctypes.byref(d), m.MOE_F32, ok, ok, ok, None, None, bad, None) == m.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(ctypes.byref(d), 9, ok, ok, ok, None, None, ok, None) == m.MOE_ERR_INVALID_ARG
    # a gate for shared rows that are not there
    assert lib.moe_combine(ctypes.byref(d), m.MOE_F32, ok, ok, ok, None, ok, ok, None) == m.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(ctypes.byref(d), m.MOE_F32, ok, ok, ok, ok, bad, ok, None) == m.MOE_ERR_INVALID_ARG
    assert lib.moe_shared_gate(ctypes.byref(d), ok, None, ok, None) == m.MOE_ERR_INVALID_ARG
    assert lib.moe_shared_gate(ctypes.byref(d), ok, ok, bad, None) == m.MOE_ERR_INVALID_ARG
    g = m.moe_gemm_desc(2, 64, 256, 128, m.MOE_BF16, m.MOE_EPI_SWIGLU, m.MOE_BF16, 1, 1)
    # SWIGLU needs B2
    assert lib.moe_grouped_gemm(ctypes.byref(g), ok, None, None, ok, None, None, None, ok, ok,
                                None, None) == m.MOE_ERR_INVALID_ARG
    g.K = 100                                              # K not a multiple of 64
    assert lib.moe_grouped_gemm(ctypes.byref(g), ok, None, None, ok, None, ok, None, ok, ok,
                                None, None) == m.MOE_ERR_INVALID_ARG


def test_workspace_too_small_and_unsupported():
    import moe_layer_softmax_amd as m
    lib = m.lib()
    ok = ctypes.c_void_p(4096)
    d = _desc(T=4096, k=8, E=64, E_loc=16)                 # 32768 slots: needs the scan workspace
    st = lib.moe_permute(ctypes.byref(d), ok, None, None, ok, ok, ok, ok, None, None, ok, 16, None)
    assert st == m.MOE_ERR_WORKSPACE
    w = m.moe_weights(*([4096] * 14))
    d2 = _desc()
    st = lib.moe_layer(ctypes.byref(d2), ctypes.byref(w), ok, None, ok, None, None, None, ok, 10,
                       None)
    assert st == m.MOE_ERR_WORKSPACE
    d3 = _desc(io_dtype=m.MOE_F32, expert_dtype=m.MOE_BF16)   # bf16 experts need bf16 io
    st = lib.moe_layer(ctypes.byref(d3), ctypes.byref(w), ok, None, ok, None, None, None, ok,
                       1 << 40, None)
    assert st == m.MOE_ERR_UNSUPPORTED
    d4 = _desc(I_s=96)                                     # shared size off the 64-column grid
    st = lib.moe_layer(ctypes.byref(d4), ctypes.byref(w), ok, None, ok, None, None, None, ok,
                       1 << 40, None)
    assert st == m.MOE_ERR_INVALID_ARG


def test_f16_scaled_rules():
    """MOE_F16_SCALED: rows of 2 * cols bytes of fp16 values then cols / 64 fp32 scales, padded to
    16 bytes; an output of bf16 STORE GEMMs and an input of the combine (H % 64 == 0) only."""
    import moe_layer_softmax_amd as m
    lib = m.lib()
    ok = ctypes.c_void_p(4096)
    assert [m.moe_f16_scaled_row_bytes(c) for c in (64, 192, 4096, 7168)] == [144, 400, 8448, 14784]
    d = _desc(H=272, io_dtype=m.MOE_F32, expert_dtype=m.MOE_F32)   # H % 64 != 0
    assert lib.moe_combine(ctypes.byref(d), m.MOE_F16_SCALED, ok, ok, ok, None, None, ok, None) == m.MOE_ERR_INVALID_ARG
    for dt, epi in ((m.MOE_BF16, m.MOE_EPI_SWIGLU), (m.MOE_F32, m.MOE_EPI_STORE),
                    (m.MOE_FP8_E4M3, m.MOE_EPI_STORE), (m.MOE_MXFP4, m.MOE_EPI_STORE),
                    (m.MOE_MXFP8, m.MOE_EPI_STORE), (m.MOE_NVFP4, m.MOE_EPI_STORE)):
        g = m.moe_gemm_desc(2, 64, 512, 256, dt, epi, m.MOE_F16_SCALED, 1, 1)
        st = lib.moe_grouped_gemm(ctypes.byref(g), ok, ok, None, ok, ok, ok, ok, ok, ok, ok, None)
        assert st == m.MOE_ERR_UNSUPPORTED, (dt, epi)


def test_zero_tokens_is_a_no_op():
    import moe_layer_softmax_amd as m
    lib = m.lib()
    d = _desc(T=0)
    w = m.moe_weights(*([4096] * 14))
    assert lib.moe_route(ctypes.byref(d), None, None, None, None, None, None, None, 0, None) == m.MOE_OK
    assert lib.moe_combine(ctypes.byref(d), m.MOE_F32, None, None, None, None, None, None, None) == m.MOE_OK
    assert lib.moe_shared_gate(ctypes.byref(d), None, None, None, None) == m.MOE_OK
    assert lib.moe_layer(ctypes.byref(d), ctypes.byref(w), None, None, None, None, None, None,
                         None, 0, None) == m.MOE_OK


def test_routing_blob_plane():
    import moe_layer_softmax_amd as m
    for T, k, P in ((1, 8, 8), (3, 2, 8), (5, 3, 16), (0, 4, 0), (16384, 8, 131072), (7, 10, 72)):
        assert m.moe_routing_blob_plane(_desc(T=T, k=k, E=16, E_loc=16)) == P
    assert m.moe_routing_blob_plane(_desc(T=-1)) == 0
