"""Python binding of libmoe.so (the gfx950 MoE layer library declared in include/moe.h).

Argument marshalling only: every function forwards torch tensors' device pointers and the current
HIP stream to the C entry point of the same name and raises MoeError on a non-OK status. There is
no fallback path: if libmoe.so is missing or cannot be loaded, importing this package fails.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

# enums of include/moe.h
MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_MXFP4, MOE_MXFP8, MOE_NVFP4, MOE_F16_SCALED = range(7)
MOE_SOFTMAX, MOE_SIGMOID = 0, 1
MOE_EPI_STORE, MOE_EPI_SWIGLU = 0, 1

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run moe_layer_softmax_amd/build.py "
                      "(or __graft_entry__.build()) first")
_lib = ctypes.CDLL(LIB_PATH)


class MoeError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _lib.moe_status_str(status).decode()
        if status == MOE_ERR_HIP:
            msg += f" (hipError {_lib.moe_last_hip_error()})"
        super().__init__(f"{where}: {msg}")


class moe_desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "H", "E", "e0", "E_loc", "I", "k", "I_s", "scoring", "renormalize",
                 "io_dtype", "out_dtype", "expert_dtype")]


class moe_gemm_desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("G", "max_rows", "K", "N", "dtype", "epilogue", "out_dtype", "a_row_div",
                 "a_scale_rows")]


class moe_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_router", "w_gate", "w_gate_scales", "w_up", "w_up_scales", "w_down",
                 "w_down_scales", "sh_gate", "sh_gate_scales", "sh_up", "sh_up_scales",
                 "sh_down", "sh_down_scales", "w_shared_gate")]


_P = ctypes.c_void_p
_D = ctypes.POINTER(moe_desc)
_lib.moe_status_str.restype = ctypes.c_char_p
_lib.moe_status_str.argtypes = [ctypes.c_int]
_lib.moe_last_hip_error.restype = ctypes.c_int32
_lib.moe_route.argtypes = [_D, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
_lib.moe_route_workspace_bytes.argtypes = [_D]
_lib.moe_route_workspace_bytes.restype = ctypes.c_size_t
_lib.moe_permute.argtypes = [_D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
_lib.moe_permute_workspace_bytes.argtypes = [_D]
_lib.moe_permute_workspace_bytes.restype = ctypes.c_size_t
_lib.moe_grouped_gemm.argtypes = [ctypes.POINTER(moe_gemm_desc), _P, _P, _P, _P, _P, _P, _P, _P,
                                  _P, _P, _P]
_lib.moe_combine.argtypes = [_D, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P]
_lib.moe_shared_gate.argtypes = [_D, _P, _P, _P, _P]
_lib.moe_routing_blob_plane.argtypes = [_D]
_lib.moe_routing_blob_plane.restype = ctypes.c_int64
_lib.moe_quantize.argtypes = [ctypes.c_int32] * 6 + [_P, _P, _P, _P]
_lib.moe_layer.argtypes = [_D, ctypes.POINTER(moe_weights), _P, _P, _P, _P, _P, _P, _P,
                           ctypes.c_size_t, _P]
_lib.moe_layer_noalloc.argtypes = [_D, ctypes.POINTER(moe_weights), _P, _P, _P, _P, _P, _P, _P]
_lib.moe_layer_workspace_bytes.argtypes = [_D]
_lib.moe_layer_workspace_bytes.restype = ctypes.c_size_t
for _f in ("moe_route", "moe_permute", "moe_grouped_gemm", "moe_combine", "moe_shared_gate",
           "moe_quantize", "moe_layer"):
    getattr(_lib, _f).restype = ctypes.c_int


def lib():
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status, where):
    if status != MOE_OK:
        raise MoeError(status, where)


def make_desc(T, H, E, e0, E_loc, I, k, I_s=0, scoring=MOE_SOFTMAX, renormalize=1,
              io_dtype=MOE_BF16, expert_dtype=MOE_BF16, out_dtype=MOE_F32):
    return moe_desc(T, H, E, e0, E_loc, I, k, I_s, scoring, renormalize, io_dtype, out_dtype,
                    expert_dtype)


def moe_route_workspace_bytes(d):
    return _lib.moe_route_workspace_bytes(ctypes.byref(d))


def moe_route(d, x, w_router, bias, logits, topk_ids, topk_w, stream=None, ws=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.moe_route(ctypes.byref(d), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(logits),
                          _ptr(topk_ids), _ptr(topk_w), _ptr(ws), nbytes, _stream(stream)),
           "moe_route")


def moe_permute_workspace_bytes(d):
    return _lib.moe_permute_workspace_bytes(ctypes.byref(d))


def moe_permute(d, topk_ids, a_in, a_in_scales, counts, offsets, slot_to_row, row_to_flat,
                a_perm, a_perm_scales, ws, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.moe_permute(ctypes.byref(d), _ptr(topk_ids), _ptr(a_in), _ptr(a_in_scales),
                            _ptr(counts), _ptr(offsets), _ptr(slot_to_row), _ptr(row_to_flat),
                            _ptr(a_perm), _ptr(a_perm_scales), _ptr(ws), nbytes,
                            _stream(stream)), "moe_permute")


def moe_grouped_gemm(g, A, A_scales, a_rows, B, B_scales, B2, B2_scales, group_offsets, C,
                     C_scales, stream=None):
    _check(_lib.moe_grouped_gemm(ctypes.byref(g), _ptr(A), _ptr(A_scales), _ptr(a_rows), _ptr(B),
                                 _ptr(B_scales), _ptr(B2), _ptr(B2_scales), _ptr(group_offsets),
                                 _ptr(C), _ptr(C_scales), _stream(stream)), "moe_grouped_gemm")


def moe_f16_scaled_row_bytes(cols):
    """Bytes of one MOE_F16_SCALED row (the header's inline function of the same name)."""
    return 2 * cols + (cols // 64 * 4 + 15) // 16 * 16


def moe_combine(d, y_dtype, y, topk_w, slot_to_row, shared, out, stream=None, shared_w=None):
    _check(_lib.moe_combine(ctypes.byref(d), y_dtype, _ptr(y), _ptr(topk_w), _ptr(slot_to_row),
                            _ptr(shared), _ptr(shared_w), _ptr(out), _stream(stream)),
           "moe_combine")


def moe_routing_blob_plane(d):
    return _lib.moe_routing_blob_plane(ctypes.byref(d))


def moe_shared_gate(d, x, w_shared_gate, shared_w, stream=None):
    _check(_lib.moe_shared_gate(ctypes.byref(d), _ptr(x), _ptr(w_shared_gate), _ptr(shared_w),
                                _stream(stream)), "moe_shared_gate")


def moe_quantize(dst_dtype, src_dtype, batch, rows, cols, block_rows, src, codes, scales,
                 stream=None):
    _check(_lib.moe_quantize(dst_dtype, src_dtype, batch, rows, cols, block_rows, _ptr(src),
                             _ptr(codes), _ptr(scales), _stream(stream)), "moe_quantize")


def make_weights(w_router, w_gate, w_up, w_down, scales=(None, None, None), shared=None,
                 shared_scales=(None, None, None), shared_gate=None):
    sh = shared if shared is not None else (None, None, None)
    keep = [w_router, w_gate, w_up, w_down, *scales, *sh, *shared_scales, shared_gate]
    w = moe_weights(*(_p.value if _p is not None else None for _p in (
        _ptr(w_router), _ptr(w_gate), _ptr(scales[0]), _ptr(w_up), _ptr(scales[1]), _ptr(w_down),
        _ptr(scales[2]), _ptr(sh[0]), _ptr(shared_scales[0]), _ptr(sh[1]),
        _ptr(shared_scales[1]), _ptr(sh[2]), _ptr(shared_scales[2]), _ptr(shared_gate))))
    w._keep = keep          # keep the tensors alive as long as the struct
    return w


def moe_layer_workspace_bytes(d):
    return _lib.moe_layer_workspace_bytes(ctypes.byref(d))


def moe_layer(d, weights, x, bias, out, logits, topk_ids, topk_w, ws, stream=None):
    nbytes = ws.numel() * ws.element_size()
    _check(_lib.moe_layer(ctypes.byref(d), ctypes.byref(weights), _ptr(x), _ptr(bias), _ptr(out),
                          _ptr(logits), _ptr(topk_ids), _ptr(topk_w), _ptr(ws), nbytes,
                          _stream(stream)), "moe_layer")


# bytes of the library's per-GPU scratch array behind moe_layer_noalloc (MOE_NOALLOC_SCRATCH_BYTES)
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20


def moe_layer_noalloc(d, weights, x, bias, out, logits, topk_ids, topk_w, stream=None):
    _check(_lib.moe_layer_noalloc(ctypes.byref(d), ctypes.byref(weights), _ptr(x), _ptr(bias),
                                  _ptr(out), _ptr(logits), _ptr(topk_ids), _ptr(topk_w),
                                  _stream(stream)), "moe_layer_noalloc")
