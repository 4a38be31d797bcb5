"""Helpers of the GPU tests: device upload, the layer run through the C ABI, and the comparisons
(tolerances and the routing checks)."""
import numpy as np
import torch

import moe_inputs as mi
import moe_layer_softmax_amd as moe
import oracle
from moe_inputs import gen

DEV = "cuda"

U32 = 2.0 ** -23     # unit roundoff used for the logit bound (covers truncating accumulation)


def to_dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(dtype)


def io_torch(fmt):
    return torch.float32 if fmt == mi.FMT_F32 else torch.bfloat16


def gamma(n):
    return n * U32 / (1 - n * U32)


def topk_numpy(L, k):
    """top-k by a full stable sort on (value desc, index asc) -- the selection rule, in numpy."""
    T, E = L.shape
    out = np.empty((T, k), np.int32)
    idx = np.arange(E)
    for t in range(T):
        out[t] = np.lexsort((idx, -L[t].astype(np.float64)))[:k]
    return out


def routing_consistent(ids_gpu, L64, bound):
    """True if the GPU's ranked choice is a valid top-k for some logits inside [L64 - b, L64 + b]."""
    k = len(ids_gpu)
    lo, hi = L64 - bound, L64 + bound
    for a in range(k - 1):
        if hi[ids_gpu[a]] < lo[ids_gpu[a + 1]]:
            return False
    rest = np.setdiff1d(np.arange(len(L64)), ids_gpu)
    return len(rest) == 0 or hi[ids_gpu[-1]] >= lo[rest].max()


def rel_err(gpu, ref):
    rms = float(np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
    err = float(np.abs(gpu.astype(np.float64) - ref).max()) if gpu.size else 0.0
    return err / rms if rms > 0 else err, rms


def tol_for(fmt):
    return 6e-2 if fmt in (mi.FMT_FP8, mi.FMT_MX4, mi.FMT_MX8, mi.FMT_NV4) else 2e-2


# ---- scaled fp16 rows (MOE_F16_SCALED) -----------------------------------------------------

def f16s_split(buf, cols):
    """Rows of MOE_F16_SCALED bytes [rows, pitch] -> (fp16 values as float64 [rows, cols], fp32
    scales as float64 [rows, cols / 64]): each row is its fp16 values, then one fp32 scale per 64
    columns."""
    buf = np.ascontiguousarray(buf)
    vals = np.ascontiguousarray(buf[:, :2 * cols]).view(np.float16).astype(np.float64)
    sc = np.ascontiguousarray(buf[:, 2 * cols:2 * cols + cols // 64 * 4]).view(np.float32).astype(np.float64)
    return vals, sc


def f16s_decode(buf, cols):
    """The values of MOE_F16_SCALED rows: fp16 value times its 64-column block's scale."""
    vals, sc = f16s_split(buf, cols)
    return vals * np.repeat(sc, 64, axis=1)


def f16s_pack(vals16, sc):
    """MOE_F16_SCALED bytes [rows, pitch] from fp16 values [rows, cols] and fp32 scales
    [rows, cols / 64] (the combine's inputs; the padding bytes after the scales are zero)."""
    rows, cols = vals16.shape
    buf = np.zeros((rows, moe.moe_f16_scaled_row_bytes(cols)), np.uint8)
    buf[:, :2 * cols] = np.ascontiguousarray(vals16.astype(np.float16)).view(np.uint8).reshape(rows, 2 * cols)
    buf[:, 2 * cols:2 * cols + cols // 64 * 4] = (
        np.ascontiguousarray(sc.astype(np.float32)).view(np.uint8).reshape(rows, cols // 64 * 4))
    return buf


def check_f16s_format(vals, sc):
    """Invariants of the rows the GEMM writes: every scale a power of two in normal fp32 range;
    a block with a nonzero maximum m stores m / scale in [2^14, 2^15] unless its scale sits at the
    2^-126 floor; an all-zero block has the scale 2^-15."""
    mant, _ = np.frexp(sc)
    assert np.all(mant == 0.5), "scales are powers of two"
    assert np.all(sc >= 2.0 ** -126)
    bmax = np.abs(vals).reshape(vals.shape[0], -1, 64).max(axis=2)
    nz = bmax > 0
    free = nz & (sc > 2.0 ** -126)
    assert np.all((bmax[free] >= 2.0 ** 14) & (bmax[free] <= 2.0 ** 15))
    assert np.all(sc[~nz] == 2.0 ** -15)


# ---- quantised formats ------------------------------------------------------------------

FMTS = {"fp8": (moe.MOE_FP8_E4M3, oracle.FP8), "mx4": (moe.MOE_MXFP4, oracle.MX4),
        "mx8": (moe.MOE_MXFP8, oracle.MX8), "nv4": (moe.MOE_NVFP4, oracle.NV4)}
E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6])


def gpu_quant(fmt, a, block_rows):
    """Quantise float32 [G, R, C] on the GPU: (codes, scales) device tensors."""
    a = np.ascontiguousarray(a, np.float32)
    if a.ndim == 2:
        a = a[None]
    G, R, C = a.shape
    src = to_dev(a, torch.float32)
    if fmt == moe.MOE_FP8_E4M3:
        codes = torch.empty((G, R, C), dtype=torch.uint8, device="cuda")
        scales = torch.empty((G, (R + block_rows - 1) // block_rows, C // 128), dtype=torch.float32,
                             device="cuda")
    elif fmt == moe.MOE_MXFP8:
        codes = torch.empty((G, R, C), dtype=torch.uint8, device="cuda")
        scales = torch.empty((G, R, C // 32), dtype=torch.uint8, device="cuda")
    elif fmt == moe.MOE_NVFP4:
        # one scale record per matrix: e4m3 block scales [R, C/16], then fp32 row scales [R]
        codes = torch.empty((G, R, C // 2), dtype=torch.uint8, device="cuda")
        scales = torch.empty((G, R * (C // 16) + 4 * R), dtype=torch.uint8, device="cuda")
    else:
        codes = torch.empty((G, R, C // 2), dtype=torch.uint8, device="cuda")
        scales = torch.empty((G, R, C // 32), dtype=torch.uint8, device="cuda")
    moe.moe_quantize(fmt, moe.MOE_F32, G, R, C, block_rows, src, codes, scales)
    return codes, scales


def oracle_quant(ofmt, a, block_rows):
    a = np.ascontiguousarray(a, np.float32)
    if a.ndim == 2:
        a = a[None]
    if ofmt == oracle.FP8:
        qs = [oracle.quant_fp8(a[g], block_rows, 128) for g in range(a.shape[0])]
        return oracle.Mat(oracle.FP8, np.stack([q[0] for q in qs]), np.stack([q[1] for q in qs]),
                          bn=block_rows, bk=128)
    if ofmt == oracle.MX8:
        qs = [oracle.quant_mx8(a[g]) for g in range(a.shape[0])]
        return oracle.Mat(oracle.MX8, np.stack([q[0] for q in qs]), np.stack([q[1] for q in qs]))
    if ofmt == oracle.NV4:
        qs = [oracle.quant_nv4(a[g]) for g in range(a.shape[0])]
        return oracle.Mat(oracle.NV4, np.stack([q[0] for q in qs]), np.stack([q[1] for q in qs]),
                          r=np.stack([q[2] for q in qs]))
    qs = [oracle.quant_mx4(a[g]) for g in range(a.shape[0])]
    return oracle.Mat(oracle.MX4, np.stack([q[0] for q in qs]), np.stack([q[1] for q in qs]))


def nv4_split(scales, rows, cols):
    """An NVFP4 scale record per matrix ([G, rows*cols/16 + 4*rows] bytes, host or device) as
    (e4m3 block-scale bytes [G, rows, cols/16], fp32 row scales [G, rows]) numpy arrays."""
    s = scales.cpu().numpy() if hasattr(scales, "cpu") else np.asarray(scales)
    s = s.reshape(-1, rows * (cols // 16) + 4 * rows)
    nb = rows * (cols // 16)
    return (s[:, :nb].reshape(-1, rows, cols // 16).copy(),
            np.ascontiguousarray(s[:, nb:]).view(np.float32).reshape(-1, rows).copy())


def nv4_block_values(codes, bscales):
    """e2m1 code * e4m3 block scale (numpy table and torch's e4m3 decoding), float64 [..., cols]."""
    codes = codes.cpu().numpy() if hasattr(codes, "cpu") else np.asarray(codes)
    lo, hi = codes & 15, codes >> 4
    v = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,))
    v[..., 0::2] = E2M1[lo]
    v[..., 1::2] = E2M1[hi]
    s = torch.from_numpy(np.ascontiguousarray(bscales, np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    return v * np.repeat(s, 16, axis=-1)


def decode(fmt, codes, scales, cols):
    """Dequantise GPU-written h (numpy / torch decoders, independent of both sides' code)."""
    codes = codes.cpu().numpy()
    scales = scales.cpu().numpy()
    if fmt == moe.MOE_FP8_E4M3:
        v = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
        return v * np.repeat(scales.astype(np.float64), 128, axis=1)[:, :cols]
    if fmt == moe.MOE_MXFP8:
        v = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
        return v * np.repeat(2.0 ** (scales.astype(np.int64) - 127), 32, axis=1)[:, :cols]
    lo, hi = codes & 15, codes >> 4
    v = np.empty((codes.shape[0], cols))
    v[:, 0::2] = E2M1[lo]
    v[:, 1::2] = E2M1[hi]
    return v * np.repeat(2.0 ** (scales.astype(np.int64) - 127), 32, axis=1)[:, :cols]




# ---- re-quantised h near a code boundary ------------------------------------------------
#
# The GPU forms h = silu(g) * u from fp32 accumulations (|dg| <= gamma_K sum|a b|, likewise u) and
# the oracle from exact sums, so an element of h whose exact value lies within that bound of a
# rounding boundary of the fp8 / MX re-quantisation may legitimately get the neighbouring code (and
# a group whose amax lies that close to a power of two, or fp8's amax / 448 scale, the neighbouring
# scale). At the small intermediate sizes of the edge-case layers one such code moves an output by
# several % of the output RMS. `h_flip_allowance` bounds, per output column of one expert row, how
# far any GPU h inside those intervals can move y from the oracle's y; the layer check adds it
# (weighted like the row) to the bar for the tokens that exceed the bar alone.

def _e2m1_rne(q):
    a = np.minimum(np.abs(q), 6.0)
    r = np.where(a < 2, np.round(a * 2) / 2, np.where(a < 4, np.round(a), np.round(a / 2) * 2))
    return np.copysign(np.minimum(r, 6.0), q)


def _e4m3_rne(q):
    q = np.clip(q, -448.0, 448.0).astype(np.float32)
    return torch.from_numpy(q).to(torch.float8_e4m3fn).float().numpy().astype(np.float64)


def _mx_exp(amax, emax):
    amax = np.asarray(amax, np.float64)
    e = np.frexp(np.where(amax > 0, amax, 1.0))[1] - 1 - emax
    return np.where(amax > 0, np.clip(e, -127, 127), -127)


def _quant_groups(h, fmt, e_or_s):
    """dequantised h [G, 32|128] for given per-group MX exponents (or fp8 scales)"""
    if fmt == moe.MOE_FP8_E4M3:
        s = e_or_s[:, None]
        return _e4m3_rne((h / s).astype(np.float32)) * s
    mul = 2.0 ** e_or_s[:, None]
    q = (h * 2.0 ** -e_or_s[:, None]).astype(np.float32).astype(np.float64)
    return (_e2m1_rne(q) if fmt == moe.MOE_MXFP4 else _e4m3_rne(q)) * mul


def h_flip_allowance(fmt, a, wg, wu, wd):
    """a [K] float64 (dequantised activation row); wg, wu [I, K], wd [H, I] float64 (dequantised).
    Returns (allowance [H], y_oracle_like [H]): a bound on |y_gpu - y_oracle| from h codes that
    the fp32 accumulation may put one step (or one group scale) away, plus the fp32 accumulation
    of the down projection itself."""
    K = len(a)
    g, u = wg @ a, wu @ a
    sg, su = np.abs(wg) @ np.abs(a), np.abs(wu) @ np.abs(a)
    silu = g / (1.0 + np.exp(-g))
    h = silu * u
    dh = 1.1 * gamma(K) * sg * np.abs(u) + np.abs(silu) * gamma(K) * su + 8 * U32 * np.abs(h)
    grp = 128 if fmt == moe.MOE_FP8_E4M3 else 32
    I = len(h)
    hg, dg_ = h.reshape(I // grp, grp), dh.reshape(I // grp, grp)
    amax = np.abs(hg.astype(np.float32)).max(1).astype(np.float64)
    amax_lo = np.maximum(np.abs(hg) - dg_, 0).max(1)
    amax_hi = (np.abs(hg) + dg_).max(1)
    if fmt == moe.MOE_FP8_E4M3:
        sc = lambda m: np.where(m > 0, (m.astype(np.float32) / np.float32(448.0)).astype(np.float64), 1.0)
        ref_s, cands = sc(amax), [sc(amax_lo), sc(amax_hi)]
    else:
        emax = 2 if fmt == moe.MOE_MXFP4 else 8
        ref_s, cands = _mx_exp(amax, emax), [_mx_exp(amax_lo, emax), _mx_exp(amax_hi, emax)]
    hq = _quant_groups(hg.astype(np.float32).astype(np.float64), fmt, ref_s)
    allow = np.zeros_like(hg)
    for c in cands:
        for sgn in (-1.0, 1.0):
            allow = np.maximum(allow, np.abs(_quant_groups(hg + sgn * dg_, fmt, c) - hq))
    if fmt == moe.MOE_FP8_E4M3:   # the same code at a scale moved with amax
        allow += (amax_hi - amax_lo)[:, None]
    allow = allow.reshape(I)
    hq = hq.reshape(I)
    y = wd @ hq
    return np.abs(wd) @ allow + gamma(I) * (np.abs(wd) @ np.abs(hq)) + 2.0 ** -8 * np.abs(y), y
