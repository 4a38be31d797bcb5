"""CPU oracle of the MoE FFN layer (numpy front end over liboracle.so).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the benchmark's
CPU-baseline leg. The GPU library and its Python binding never import it.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16, FP8, MX4, MX8, NV4 = 0, 1, 2, 3, 4, 5
SOFTMAX, SIGMOID = 0, 1


def build(force=True):
    """Compile liboracle.so with gcc (OpenMP, no fast-math, no FP contraction)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.check_call(cmd, cwd=_HERE)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


class _Mat(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int), ("G", ctypes.c_int), ("N", ctypes.c_int),
                ("K", ctypes.c_int), ("bn", ctypes.c_int), ("bk", ctypes.c_int),
                ("q", ctypes.c_void_p), ("s", ctypes.c_void_p), ("r", ctypes.c_void_p)]


class _Desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in
                ("T", "H", "E", "e0", "E_loc", "I", "k", "I_s", "scoring", "renormalize",
                 "act_fmt")]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        L.oracle_e4m3_value.restype = ctypes.c_double
        L.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e2m1_value.restype = ctypes.c_double
        L.oracle_e2m1_value.argtypes = [ctypes.c_uint8]
        L.oracle_e2m1_encode.restype = ctypes.c_uint8
        L.oracle_e2m1_encode.argtypes = [ctypes.c_float]
        L.oracle_bf16_round.restype = ctypes.c_float
        L.oracle_bf16_round.argtypes = [ctypes.c_float]
        L.oracle_e8m0_value.restype = ctypes.c_double
        L.oracle_e8m0_value.argtypes = [ctypes.c_uint8]
        L.oracle_mat_at.restype = ctypes.c_double
        L.oracle_permute.restype = ctypes.c_int
        L.oracle_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# ---- number formats ------------------------------------------------------------------------

def e4m3_value(code):
    return lib().oracle_e4m3_value(int(code))


def e4m3_encode(v):
    return lib().oracle_e4m3_encode(float(v))


def e2m1_value(code):
    return lib().oracle_e2m1_value(int(code))


def e2m1_encode(v):
    return lib().oracle_e2m1_encode(float(v))


def bf16_round(v):
    return lib().oracle_bf16_round(float(v))


def e8m0_value(code):
    return lib().oracle_e8m0_value(int(code))


def quant_fp8(src, bn=128, bk=128):
    """e4m3 codes [rows, cols] and fp32 block scales [ceil(rows/bn), ceil(cols/bk)]."""
    src = _c(src, np.float32)
    rows, cols = src.shape
    codes = np.empty((rows, cols), np.uint8)
    scales = np.empty(((rows + bn - 1) // bn, (cols + bk - 1) // bk), np.float32)
    lib().oracle_quant_fp8(rows, cols, bn, bk, _p(src), _p(codes), _p(scales))
    return codes, scales


def quant_mx4(src):
    """packed e2m1 [rows, cols/2] and E8M0 scales [rows, cols/32]."""
    src = _c(src, np.float32)
    rows, cols = src.shape
    packed = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 32), np.uint8)
    lib().oracle_quant_mx4(rows, cols, _p(src), _p(packed), _p(scales))
    return packed, scales


def quant_mx8(src):
    """e4m3 codes [rows, cols] and E8M0 scales [rows, cols/32] (MXFP8)."""
    src = _c(src, np.float32)
    rows, cols = src.shape
    codes = np.empty((rows, cols), np.uint8)
    scales = np.empty((rows, cols // 32), np.uint8)
    lib().oracle_quant_mx8(rows, cols, _p(src), _p(codes), _p(scales))
    return codes, scales


def quant_nv4(src):
    """NVFP4: packed e2m1 [rows, cols/2], e4m3 block scales [rows, cols/16] (one per 16
    elements), fp32 row scales [rows]."""
    src = _c(src, np.float32)
    rows, cols = src.shape
    packed = np.empty((rows, cols // 2), np.uint8)
    bscales = np.empty((rows, cols // 16), np.uint8)
    rscales = np.empty(rows, np.float32)
    lib().oracle_quant_nv4(rows, cols, _p(src), _p(packed), _p(bscales), _p(rscales))
    return packed, bscales, rscales


class Mat:
    """A stack of G [N, K] matrices in one of the formats F32 / FP8 / MX4 / MX8 / NV4 (keeps its
    arrays). NV4 takes its fp32 row scales [G, N] as r."""

    def __init__(self, fmt, q, s=None, bn=128, bk=128, r=None):
        self.fmt = fmt
        if fmt == F32:
            q = _c(q, np.float32)
        else:
            q = _c(q, np.uint8)
        if q.ndim == 2:
            q = q[None]
        self.q = q
        self.s = None if s is None else np.ascontiguousarray(s)
        self.r = None if r is None else _c(r, np.float32)
        if fmt == NV4 and self.r is None:
            raise ValueError("NV4 needs its row scales")
        G, N, Kq = q.shape
        K = Kq * 2 if fmt in (MX4, NV4) else Kq
        self.G, self.N, self.K, self.bn, self.bk = G, N, K, bn, bk
        self._c = _Mat(fmt, G, N, K, bn, bk, _p(self.q), _p(self.s), _p(self.r))

    @property
    def ref(self):
        return ctypes.byref(self._c)

    def dequant(self):
        out = np.empty((self.G, self.N, self.K), np.float64)
        lib().oracle_mat_dequant(self.ref, _p(out))
        return out

    def at(self, g, n, k):
        return lib().oracle_mat_at(self.ref, g, n, k)


def quantise_stack(fmt, w):
    """Quantise a float32 stack [G, N, K] with the oracle's own quantiser into a Mat."""
    w = _c(w, np.float32)
    if w.ndim == 2:
        w = w[None]
    if fmt == F32:
        return Mat(F32, w)
    G, N, K = w.shape
    if fmt == FP8:
        qs, ss = zip(*(quant_fp8(w[g]) for g in range(G)))
        return Mat(FP8, np.stack(qs), np.stack(ss))
    if fmt == MX4:
        qs, ss = zip(*(quant_mx4(w[g]) for g in range(G)))
        return Mat(MX4, np.stack(qs), np.stack(ss))
    if fmt == NV4:
        qs, ss, rs = zip(*(quant_nv4(w[g]) for g in range(G)))
        return Mat(NV4, np.stack(qs), np.stack(ss), r=np.stack(rs))
    if fmt == MX8:
        qs, ss = zip(*(quant_mx8(w[g]) for g in range(G)))
        return Mat(MX8, np.stack(qs), np.stack(ss))
    raise ValueError(fmt)


# ---- routing and dispatch ---------------------------------------------------------------

def logits(x, w_r, bias=None, tok=None):
    """(logits float64 [n, E], absdot float64 [n, E]) for all tokens or a subset."""
    x = _c(x, np.float32)
    w_r = _c(w_r, np.float32)
    T, H = x.shape
    E = w_r.shape[0]
    b = None if bias is None else _c(bias, np.float32)
    t = None if tok is None else _c(tok, np.int32)
    n = T if t is None else len(t)
    L = np.empty((n, E), np.float64)
    A = np.empty((n, E), np.float64)
    lib().oracle_logits(T, H, E, _p(x), _p(w_r), _p(b), n, _p(t), _p(L), _p(A))
    return L, A


def topk(logits32, k, scoring=SOFTMAX, renormalize=1):
    L = _c(logits32, np.float32)
    T, E = L.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    lib().oracle_topk(T, E, k, _p(L), scoring, renormalize, _p(ids), _p(w))
    return ids, w


def permute(ids, e0, E_loc):
    """(counts [E_loc], offsets [E_loc+1], slot_to_row [T,k], row_to_flat [R]) ."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    counts = np.empty(E_loc, np.int32)
    offsets = np.empty(E_loc + 1, np.int32)
    s2r = np.empty((T, k), np.int32)
    r2f = np.empty(max(T * k, 1), np.int32)
    R = lib().oracle_permute(T, k, e0, E_loc, _p(ids), _p(counts), _p(offsets), _p(s2r), _p(r2f))
    return counts, offsets, s2r, r2f[:R].copy()


# ---- grouped GEMM and combine on their own ------------------------------------------------

def grouped_gemm(offsets, A, B, B2=None, a_rows=None, a_row_div=1, bias=None):
    """A: Mat [1, rows_a, K]; B, B2: Mat [G, N, K]. Returns float64 [offsets[-1], N]."""
    off = _c(offsets, np.int32)
    G = len(off) - 1
    ar = None if a_rows is None else _c(a_rows, np.int32)
    b = None if bias is None else _c(bias, np.float32)
    out = np.empty((int(off[-1]), B.N), np.float64)
    null = ctypes.c_void_p(None)
    lib().oracle_grouped_gemm(G, _p(off), A.ref, _p(ar), int(a_row_div), B.ref,
                              B2.ref if B2 is not None else null, _p(b), _p(out))
    return out


def combine(y, w, slot_to_row, shared=None, shared_w=None):
    y = _c(y, np.float32)
    w = _c(w, np.float32)
    s2r = _c(slot_to_row, np.int32)
    T, k = s2r.shape
    H = y.shape[1]
    sh = None if shared is None else _c(shared, np.float32)
    sw = None if shared_w is None else _c(shared_w, np.float32)
    out = np.empty((T, H), np.float64)
    lib().oracle_combine(T, H, k, _p(y), _p(w), _p(s2r), _p(sh), _p(sw), _p(out))
    return out


def shared_gate(x, w_sg, tok=None):
    """Gate of the shared expert per token: 1 / (1 + exp(-(x_t . w_sg))), double [n]."""
    x = _c(x, np.float32)
    g_w = _c(w_sg, np.float32)
    T, H = x.shape
    t = None if tok is None else _c(tok, np.int32)
    n = T if t is None else len(t)
    g = np.empty(n, np.float64)
    lib().oracle_shared_gate(T, H, _p(x), _p(g_w), n, _p(t), _p(g))
    return g


# ---- the layer -------------------------------------------------------------------------

def ffn_row(a, gate, up, down, g=0, act_fmt=F32):
    a = _c(a, np.float64)
    I = gate.N
    d = _Desc(0, len(a), 0, 0, 0, I, 0, 0, 0, 0, act_fmt)
    y = np.empty(len(a), np.float64)
    lib().oracle_ffn_row(ctypes.byref(d), I, _p(a), gate.ref, up.ref, down.ref, g, _p(y))
    return y


def moe_layer(desc, x, w_r, bias, xa, gate, up, down, shared=None, tok=None, shared_gate=None):
    """Run the layer for all tokens (tok None) or a subset of token indices.

    desc: dict with T, H, E, e0, E_loc, I, k, I_s, scoring, renormalize, act_fmt.
    x: float32 [T, H] unquantised input (router and shared-gate input); xa: Mat [1, T, H] fed to
    the experts; shared_gate: float32 [H] gate vector of the shared expert, or None (ungated).
    Returns dict(out, logits64, logits32, ids, w)."""
    x = _c(x, np.float32)
    w_r = _c(w_r, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    t = None if tok is None else _c(tok, np.int32)
    n = desc["T"] if t is None else len(t)
    E, k, H = desc["E"], desc["k"], desc["H"]
    d = _Desc(*(int(desc[f]) for f in ("T", "H", "E", "e0", "E_loc", "I", "k", "I_s",
                                       "scoring", "renormalize", "act_fmt")))
    out = np.empty((n, H), np.float64)
    L64 = np.empty((n, E), np.float64)
    L32 = np.empty((n, E), np.float32)
    ids = np.empty((n, k), np.int32)
    w = np.empty((n, k), np.float64)
    null = ctypes.c_void_p(None)
    sg, su, sd = (shared if shared is not None else (None, None, None))
    gv = None if shared_gate is None else _c(shared_gate, np.float32)
    lib().oracle_moe_layer(ctypes.byref(d), _p(x), _p(w_r), _p(b), xa.ref, gate.ref, up.ref,
                           down.ref, sg.ref if sg else null, su.ref if su else null,
                           sd.ref if sd else null, _p(gv), n, _p(t), _p(out), _p(L64), _p(L32),
                           _p(ids), _p(w))
    return dict(out=out, logits64=L64, logits32=L32, ids=ids, w=w)


def moe_layer_routed(desc, x, xa, gate, up, down, shared, tok, ids, w, shared_gate=None):
    """The expert part of the layer for given routing: tokens tok (int32 [n]) with chosen experts
    ids [n, k] and fp32 weights w [n, k]. Returns float64 out [n, H]."""
    x = _c(x, np.float32)
    t = _c(tok, np.int32)
    i = _c(ids, np.int32)
    wf = _c(w, np.float32)
    H = desc["H"]
    d = _Desc(*(int(desc[f]) for f in ("T", "H", "E", "e0", "E_loc", "I", "k", "I_s",
                                       "scoring", "renormalize", "act_fmt")))
    out = np.empty((len(t), H), np.float64)
    null = ctypes.c_void_p(None)
    sg, su, sd = (shared if shared is not None else (None, None, None))
    gv = None if shared_gate is None else _c(shared_gate, np.float32)
    lib().oracle_moe_layer_routed(ctypes.byref(d), _p(x), xa.ref, gate.ref, up.ref, down.ref,
                                  sg.ref if sg else null, su.ref if su else null,
                                  sd.ref if sd else null, _p(gv), len(t), _p(t), _p(i), _p(wf),
                                  _p(out))
    return out


def num_threads():
    return lib().oracle_num_threads()
