"""Pins of the CPU oracle against what the pages, the format specifications and the mathematics
fix, independently of the oracle's own code (library routines, closed forms, brute force, worked
numbers). CPU only."""
import os

import numpy as np
import pytest
import torch
from scipy.special import expit, softmax

import oracle
from moe_inputs import gen

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read_pairs(name):
    out = []
    for line in open(os.path.join(GOLD, name)):
        line = line.split("#")[0].strip()
        if line:
            a, b = line.split()
            out.append((int(a, 0), float(b)))
    return out


# ------------------------------------------------------------------------------------------
# number formats
# ------------------------------------------------------------------------------------------

def test_e4m3_spec_points():
    for code, val in _read_pairs("ocp_e4m3_points.txt"):
        assert oracle.e4m3_value(code) == val
        if code != 0x80:
            assert oracle.e4m3_encode(val) == code
    assert np.isnan(oracle.e4m3_value(0x7F)) and np.isnan(oracle.e4m3_value(0xFF))


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    ours = np.array([oracle.e4m3_value(c) for c in codes])
    both_nan = np.isnan(ref) & np.isnan(ours)
    assert np.all(both_nan | (ref == ours))


def test_e4m3_encode_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 50,
        rng.standard_normal(5000).astype(np.float32) * 0.01,      # subnormal range
        np.float32(2.0) ** np.arange(-12, 9, dtype=np.float32),   # powers of two
        # exact midpoints between neighbouring codes (ties)
        np.array([(oracle.e4m3_value(c) + oracle.e4m3_value(c + 1)) / 2 for c in range(0, 0x7E)],
                 np.float32),
    ]).astype(np.float32)
    v = np.clip(v, -448, 448).astype(np.float32)
    ours = np.array([oracle.e4m3_encode(a) for a in v], np.uint8)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    # saturation (torch's cast does not saturate, the quantiser's definition does)
    assert oracle.e4m3_encode(1e6) == 0x7E and oracle.e4m3_encode(-470.0) == 0xFE


def _e2m1_rne_numpy(v):
    """RNE onto the E2M1 grid written binade by binade with numpy's rint (ties to even)."""
    a = abs(float(v))
    if a < 2.0:
        q = np.rint(a * 2.0) / 2.0          # step 0.5 on [0, 2)
    elif a < 4.0:
        q = np.rint(a)                      # step 1 on [2, 4)
    else:
        q = min(2.0 * np.rint(a / 2.0), 6.0)  # step 2 on [4, 6], saturate
    return -q if np.signbit(v) else q


def test_e2m1_spec_points_and_rne():
    for code, val in _read_pairs("ocp_e2m1_points.txt"):
        assert oracle.e2m1_value(code) == val
    grid = np.concatenate([np.arange(-8, 8.0001, 0.0625), [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]])
    for v in grid.astype(np.float32):
        assert oracle.e2m1_value(oracle.e2m1_encode(v)) == _e2m1_rne_numpy(v), v


def test_e8m0_values():
    assert oracle.e8m0_value(127) == 1.0
    assert oracle.e8m0_value(0) == 2.0 ** -127
    assert oracle.e8m0_value(254) == 2.0 ** 127
    assert np.isnan(oracle.e8m0_value(255))


def test_mx4_hand_example():
    lines = {}
    for line in open(os.path.join(GOLD, "mx4_packing_example.txt")):
        if line.startswith("#") or ":" not in line:
            continue
        key, val = line.split(":", 1)
        lines[key.strip()] = val.split()
    vals = np.array([float(v) for v in lines["values"]], np.float32)[None]
    packed, scales = oracle.quant_mx4(vals)
    assert scales[0, 0] == int(lines["scale"][0])
    assert [int(b) for b in packed[0]] == [int(b, 0) for b in lines["bytes"]]


def test_mx4_scale_rule_and_roundtrip():
    rng = np.random.default_rng(2)
    for e in range(-20, 20):
        # amax in [2^(e+2), 2^(e+3)) must give shared exponent e
        amax = np.float32(2.0 ** (e + 2) * (1 + rng.random() * 0.999))
        v = (rng.random(32).astype(np.float32) * 2 - 1) * amax
        v[rng.integers(32)] = amax
        _, s = oracle.quant_mx4(v[None].astype(np.float32))
        assert int(s[0, 0]) == e + 127
    # values on the grid (E2M1 value x 2^e, amax hitting 6 * 2^e) survive exactly
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    for e in (-8, -1, 0, 3):
        v = rng.choice(mags, size=(4, 64)) * rng.choice([-1, 1], size=(4, 64))
        v[:, 0] = 6.0
        v[:, 32] = 6.0
        v = (v * 2.0 ** e).astype(np.float32)
        p, s = oracle.quant_mx4(v)
        m = oracle.Mat(oracle.MX4, p[None], s[None])
        assert np.array_equal(m.dequant()[0], v.astype(np.float64))
    # an all-zero group gets the smallest scale and zero codes
    p, s = oracle.quant_mx4(np.zeros((1, 32), np.float32))
    assert s[0, 0] == 0 and not p.any()
    # error: at most half the top grid step (2^e) inside the E2M1 range, and below 2 * 2^e where
    # values between 6 * 2^e and amax < 8 * 2^e saturate
    v = rng.standard_normal((16, 256)).astype(np.float32)
    p, s = oracle.quant_mx4(v)
    dq = oracle.Mat(oracle.MX4, p[None], s[None]).dequant()[0]
    unit = np.repeat(2.0 ** (s.astype(np.int32) - 127), 32, axis=1)
    inside = np.abs(v) <= 6 * unit
    err = np.abs(dq - v)
    assert np.all(err[inside] <= unit[inside]) and np.all(err[~inside] < 2 * unit[~inside])
    assert np.all(np.abs(dq[~inside]) == 6 * unit[~inside])


def _golden_kv(name):
    lines = {}
    for line in open(os.path.join(GOLD, name)):
        if line.startswith("#") or ":" not in line:
            continue
        key, val = line.split(":", 1)
        lines[key.strip()] = val.split()
    return lines


def test_mx8_hand_example():
    lines = _golden_kv("mx8_block_example.txt")
    vals = np.array([float(v) for v in lines["values"]], np.float32)[None]
    codes, scales = oracle.quant_mx8(vals)
    assert [int(s) for s in scales[0]] == [int(s) for s in lines["scales"]]
    assert [int(c) for c in codes[0]] == [int(c, 0) for c in lines["codes"]]


def test_mx8_scale_rule_and_codes_match_torch_cast():
    """Shared exponent: amax in [2^(e+8), 2^(e+9)) gives e. Codes: torch's round-to-nearest-even
    e4m3 cast of v * 2^-e after clamping to +-448 (torch's cast does not saturate)."""
    rng = np.random.default_rng(21)
    for e in range(-30, 30):
        amax = np.float32(2.0 ** (e + 8) * (1 + rng.random() * 0.999))
        v = ((rng.random((3, 32)) * 2 - 1) * amax).astype(np.float32)
        v[1, :8] *= np.float32(1e-3)                 # small elements go subnormal in e4m3
        v[:, 8 + rng.integers(24)] = amax
        c, s = oracle.quant_mx8(v)
        assert np.all(s == e + 127)
        q = np.clip(v * np.float32(2.0 ** -e), -448, 448).astype(np.float32)
        ref = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(c, ref), e
    c, s = oracle.quant_mx8(np.zeros((2, 64), np.float32))
    assert np.all(s == 0) and not c.any()


def test_mx8_roundtrip_and_error_bound():
    rng = np.random.default_rng(22)
    # E4M3 grid values times 2^e, with 448 * 2^e present in every group, survive exactly
    grid = np.array([oracle.e4m3_value(c) for c in range(0x7F)], np.float64)
    for e in (-9, -1, 0, 4):
        v = rng.choice(grid, size=(3, 64)) * rng.choice([-1, 1], size=(3, 64))
        v[:, 0] = 448.0
        v[:, 40] = -448.0
        v = (v * 2.0 ** e).astype(np.float32)
        c, s = oracle.quant_mx8(v)
        assert np.all(s == e + 127)
        m = oracle.Mat(oracle.MX8, c[None], s[None])
        assert np.array_equal(m.dequant()[0], v.astype(np.float64))
    # error: within the normal E4M3 range at most half a step (2^-4 relative), below the
    # subnormal threshold at most 2^-10 * 2^e; values above 448 * 2^e saturate
    v = rng.standard_normal((16, 256)).astype(np.float32) * np.float32(3.0)
    c, s = oracle.quant_mx8(v)
    dq = oracle.Mat(oracle.MX8, c[None], s[None]).dequant()[0]
    unit = np.repeat(2.0 ** (s.astype(np.int32) - 127), 32, axis=1)
    a = np.abs(v.astype(np.float64))
    err = np.abs(dq - v)
    normal = (a >= 2.0 ** -6 * unit) & (a <= 448 * unit)
    sub = a < 2.0 ** -6 * unit
    sat = a > 448 * unit
    assert np.all(err[normal] <= a[normal] * 2.0 ** -4)
    assert np.all(err[sub] <= 2.0 ** -10 * unit[sub])
    assert np.all(np.abs(dq[sat]) == 448 * unit[sat]) and np.all(err[sat] < 64 * unit[sat])


def test_ffn_quantised_activations_mx8():
    """h quantised to MXFP8 (1x32 groups along I): equals the dense FFN with h passed through the
    independent scale rule and torch's e4m3 cast of the clamped quotient."""
    rng = np.random.default_rng(23)
    H, I = 64, 128
    a = rng.standard_normal(H)
    wg, wu = (rng.standard_normal((I, H)) * 0.1 for _ in range(2))
    wd = rng.standard_normal((H, I)) * 0.1
    M = oracle.Mat
    y = oracle.ffn_row(a, M(oracle.F32, wg.astype(np.float32)), M(oracle.F32, wu.astype(np.float32)),
                       M(oracle.F32, wd.astype(np.float32)), act_fmt=oracle.MX8)
    wg32, wu32, wd32 = (w.astype(np.float32).astype(np.float64) for w in (wg, wu, wd))
    gg, uu = a @ wg32.T, a @ wu32.T
    h = (gg * expit(gg) * uu).astype(np.float32)
    hq = np.empty(I)
    for b in range(0, I, 32):
        blk = h[b:b + 32]
        e = int(np.floor(np.log2(np.abs(blk).max()))) - 8
        q = np.clip(blk * np.float32(2.0 ** -e), -448, 448).astype(np.float32)
        c = torch.from_numpy(q).to(torch.float8_e4m3fn).float().numpy()
        hq[b:b + 32] = c.astype(np.float64) * 2.0 ** e
    assert np.allclose(y, hq @ wd32.T, rtol=1e-12, atol=1e-12)


def _e2m1_rne_numpy(q):
    """Nearest E2M1 magnitude with ties to the even code, saturating at 6, sign kept: the
    grid has steps of 0.5 below 2, 1 in [2, 4) and 2 in [4, 6], and ties-to-even on the code
    is half-to-even on the step count (numpy's rounding)."""
    a = np.minimum(np.abs(q.astype(np.float64)), 6.0)
    r = np.where(a < 2, np.round(a * 2) / 2, np.where(a < 4, np.round(a), np.round(a / 2) * 2))
    return np.copysign(np.minimum(r, 6.0), q)


def test_ffn_quantised_activations_mx4():
    """h re-quantised to MXFP4 (1x32 groups along I, OCP MX v1.0): equals the dense FFN with h
    passed through the scale rule floor(log2 amax) - 2 and round-to-nearest-even on the E2M1
    grid, restated here in numpy. The gate rows get a magnitude per 32-column group (1e-3 .. 30)
    so that a wrong group orientation changes the scales; a few h values are set on exact ties."""
    rng = np.random.default_rng(25)
    H, I = 64, 160
    a = rng.standard_normal(H)
    mag = np.repeat(np.array([1e-3, 30.0, 1.0, 0.07, 5.0]), 32)[:, None]
    wg = (rng.standard_normal((I, H)) * 0.1 * mag).astype(np.float32)
    wu = (rng.standard_normal((I, H)) * 0.1).astype(np.float32)
    wd = (rng.standard_normal((H, I)) * 0.1).astype(np.float32)
    M = oracle.Mat
    y = oracle.ffn_row(a, M(oracle.F32, wg), M(oracle.F32, wu), M(oracle.F32, wd), act_fmt=oracle.MX4)
    wg64, wu64, wd64 = (w.astype(np.float64) for w in (wg, wu, wd))
    gg, uu = a @ wg64.T, a @ wu64.T
    h = (gg * expit(gg) * uu).astype(np.float32)
    hq = np.empty(I)
    for b in range(0, I, 32):
        blk = h[b:b + 32]
        amax = float(np.abs(blk).max())
        e = -127 if amax == 0 else int(np.clip(np.frexp(amax)[1] - 1 - 2, -127, 127))
        q = (blk * np.float32(2.0 ** -e)).astype(np.float32)
        hq[b:b + 32] = _e2m1_rne_numpy(q) * 2.0 ** e
    assert np.allclose(y, hq @ wd64.T, rtol=1e-12, atol=1e-12)
    # the restated rounding on the ties and neighbours of the grid (the oracle's own encoder)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 5.9, 6.5, 100.0, 0.2, -0.25, -2.5,
                     -5.0, -0.0], np.float32)
    ref = _e2m1_rne_numpy(ties)
    ours = np.array([oracle.e2m1_value(oracle.e2m1_encode(v)) for v in ties])
    assert np.array_equal(np.abs(ours), np.abs(ref)) and np.array_equal(np.signbit(ours), np.signbit(ref))


def test_grouped_gemm_mx8_equals_dequantised_matmul():
    rng = np.random.default_rng(24)
    K, N, T = 256, 96, 40
    x = rng.standard_normal((T, K)).astype(np.float32)
    w = (rng.standard_normal((2, N, K)) * 0.02).astype(np.float32)
    xc, xs = oracle.quant_mx8(x)
    xa = oracle.Mat(oracle.MX8, xc[None], xs[None])
    wm = oracle.quantise_stack(oracle.MX8, w)
    assert wm.q.shape == (2, N, K) and wm.s.shape == (2, N, K // 32)
    off = np.array([0, 15, T], np.int32)
    out = oracle.grouped_gemm(off, xa, wm)
    xd, wd = xa.dequant()[0], wm.dequant()
    for g in range(2):
        ref = xd[off[g]:off[g + 1]] @ wd[g].T
        assert np.allclose(out[off[g]:off[g + 1]], ref, rtol=0, atol=1e-12)


def test_fp8_block_quantiser():
    rng = np.random.default_rng(3)
    w = rng.standard_normal((256, 384)).astype(np.float32) * 0.02
    w[5, 7] = 0.5                                   # block (0,0) amax
    codes, scales = oracle.quant_fp8(w)
    assert scales.shape == (2, 3)
    assert scales[0, 0] == np.float32(0.5) / np.float32(448.0)
    # the block's largest magnitude maps exactly onto 448
    assert codes[5, 7] == 0x7E
    # the codes are torch's round-to-nearest-even cast of the fp32 quotient
    q = w / np.repeat(np.repeat(scales, 128, 0), 128, 1)
    ref = torch.from_numpy(q.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    # ragged shapes: partial blocks use their own amax
    codes2, scales2 = oracle.quant_fp8(w[:200, :300])
    assert scales2.shape == (2, 3)
    z, zs = oracle.quant_fp8(np.zeros((128, 128), np.float32))
    assert zs[0, 0] == 1.0 and not z.any()
    # dequantised values within half an e4m3 step (relative 2^-4) of the input
    m = oracle.Mat(oracle.FP8, codes[None], scales[None])
    dq = m.dequant()[0]
    assert np.all(np.abs(dq - w) <= np.abs(w) * 2.0 ** -4 + 2.0 ** -10 * scales.max())


# ------------------------------------------------------------------------------------------
# routing
# ------------------------------------------------------------------------------------------

def test_logits_match_numpy_matmul():
    rng = np.random.default_rng(4)
    x = gen.bf16_round(rng.standard_normal((37, 96)).astype(np.float32))
    w = gen.bf16_round(rng.standard_normal((20, 96)).astype(np.float32) * 0.02)
    b = rng.standard_normal(20).astype(np.float32)
    L, A = oracle.logits(x, w, b)
    ref = x.astype(np.float64) @ w.astype(np.float64).T + b.astype(np.float64)
    assert np.allclose(L, ref, rtol=0, atol=1e-12)
    assert np.allclose(A, np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T
                       + np.abs(b), rtol=1e-12)
    Ls, _ = oracle.logits(x, w, b, tok=np.array([5, 0, 36]))
    assert np.array_equal(Ls, L[[5, 0, 36]])


def _topk_bruteforce(L, k):
    T, E = L.shape
    ids = np.empty((T, k), np.int32)
    for t in range(T):
        # full stable sort by (value descending, index ascending); -0.0 == +0.0 in numpy
        order = np.lexsort((np.arange(E), -L[t].astype(np.float64)))
        ids[t] = order[:k]
    return ids


@pytest.mark.parametrize("E,k", [(8, 2), (128, 8), (512, 10), (256, 8), (16, 16), (5, 1)])
def test_topk_matches_full_sort(E, k):
    L = gen.tie_heavy_logits(64, E, seed=E + k)
    ids, w = oracle.topk(L, k)
    assert np.array_equal(ids, _topk_bruteforce(L, k))
    L2 = gen.random_logits(64, E, seed=E)
    ids2, _ = oracle.topk(L2, k)
    assert np.array_equal(ids2, _topk_bruteforce(L2, k))


def test_topk_special_cases():
    L = np.full((3, 16), 0.75, np.float32)
    ids, w = oracle.topk(L, 4)
    assert np.array_equal(ids, np.tile(np.arange(4), (3, 1)))        # all equal -> 0..k-1
    assert np.allclose(w, 0.25, atol=1e-15)
    Lz = np.zeros((1, 8), np.float32)
    Lz[0, ::2] = -0.0                                                  # -0 equals +0
    ids, _ = oracle.topk(Lz, 3)
    assert list(ids[0]) == [0, 1, 2]
    L = gen.random_logits(4, 12, seed=9)
    ids, _ = oracle.topk(L, 12)                                        # k = E: full order
    assert np.array_equal(ids, _topk_bruteforce(L, 12))


def test_softmax_weights():
    L = gen.random_logits(50, 128, seed=5, scale=2.0)
    ids, w = oracle.topk(L, 8, oracle.SOFTMAX, 1)
    sel = np.take_along_axis(L.astype(np.float64), ids, 1)
    assert np.allclose(w, softmax(sel, axis=1), rtol=0, atol=1e-14)
    assert np.allclose(w.sum(1), 1.0, atol=1e-14)
    assert np.all(np.diff(w, axis=1) <= 0)                             # rank order
    # without renormalisation: the full softmax at the chosen experts
    ids0, w0 = oracle.topk(L, 8, oracle.SOFTMAX, 0)
    full = softmax(L.astype(np.float64), axis=1)
    assert np.allclose(w0, np.take_along_axis(full, ids0, 1), rtol=0, atol=1e-14)


def test_sigmoid_weights():
    L = gen.random_logits(50, 256, seed=6, scale=3.0)
    ids, w = oracle.topk(L, 8, oracle.SIGMOID, 1)
    p = expit(np.take_along_axis(L.astype(np.float64), ids, 1))
    assert np.allclose(w, p / p.sum(1, keepdims=True), rtol=0, atol=1e-14)
    ids0, w0 = oracle.topk(L, 8, oracle.SIGMOID, 0)
    assert np.allclose(w0, p, rtol=0, atol=1e-15)


# ------------------------------------------------------------------------------------------
# dispatch
# ------------------------------------------------------------------------------------------

def _check_perm(ids, e0, E_loc):
    T, k = ids.shape
    counts, offsets, s2r, r2f = oracle.permute(ids, e0, E_loc)
    flat = ids.reshape(-1)
    local = (flat >= e0) & (flat < e0 + E_loc)
    R = int(local.sum())
    assert offsets[-1] == R == len(r2f)
    assert np.array_equal(counts, np.bincount(flat[local] - e0, minlength=E_loc))
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    # brute force: stable sort of the local flat indices by local expert
    fl = np.nonzero(local)[0]
    order = fl[np.argsort(flat[fl], kind="stable")]
    assert np.array_equal(r2f, order)
    s = s2r.reshape(-1)
    assert np.all(s[~local] == -1)
    assert np.array_equal(r2f[s[local]], np.nonzero(local)[0])          # exact inverse
    assert np.array_equal(np.sort(s[local]), np.arange(R))              # bijection onto [0,R)
    return counts


@pytest.mark.parametrize("T,E,k,e0,E_loc", [(64, 8, 2, 0, 8), (333, 128, 8, 0, 32),
                                             (200, 512, 10, 64, 64), (1, 16, 4, 12, 4),
                                             (50, 8, 8, 0, 8)])
def test_permute_bruteforce(T, E, k, e0, E_loc):
    ids = gen.random_topk_ids(T, E, k, seed=T, hot=[e0], hot_frac=0.3)
    _check_perm(ids, e0, E_loc)


def test_permute_no_local_rows():
    ids = gen.random_topk_ids(40, 64, 4, seed=1)
    ids = np.where(ids < 8, ids + 8, ids)                                # nothing in [0, 8)
    counts, offsets, s2r, r2f = oracle.permute(ids, 0, 8)
    assert offsets[-1] == 0 and not counts.any() and np.all(s2r == -1) and len(r2f) == 0


def test_worked_example_tokens_per_expert():
    """Hosting Qwen on Blackwell, section "Prefillers": 6000 tokens, top-8, 128 experts give
    6000 * 8 / 128 = 375 tokens per expert on average."""
    vals = {}
    for line in open(os.path.join(GOLD, "prefillers_tokens_per_expert.txt")):
        if not line.startswith("#") and line.strip():
            key, v = line.split()
            vals[key] = int(v)
    T, k, E = vals["T"], vals["k"], vals["E"]
    ids = gen.random_topk_ids(T, E, k, seed=0)
    counts = _check_perm(ids, 0, E)
    assert counts.sum() / E == vals["mean_tokens_per_expert"]


# ------------------------------------------------------------------------------------------
# expert FFN and the layer
# ------------------------------------------------------------------------------------------

def _dense_swiglu(a, wg, wu, wd):
    g = a @ wg.T
    u = a @ wu.T
    return (g * expit(g) * u) @ wd.T


def _tiny(T=12, H=64, E=4, I=32, k=2, e0=0, E_loc=4, I_s=0, scoring=0, seed=0, same=False):
    rng = np.random.default_rng([seed, 77])
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (rng.standard_normal((E, H)) * 0.3).astype(np.float32)
    if same:
        one = [(rng.standard_normal((I, H)) * 0.1).astype(np.float32) for _ in range(2)]
        d1 = (rng.standard_normal((H, I)) * 0.1).astype(np.float32)
        g = np.stack([one[0]] * E_loc)
        u = np.stack([one[1]] * E_loc)
        d = np.stack([d1] * E_loc)
    else:
        g = (rng.standard_normal((E_loc, I, H)) * 0.1).astype(np.float32)
        u = (rng.standard_normal((E_loc, I, H)) * 0.1).astype(np.float32)
        d = (rng.standard_normal((E_loc, H, I)) * 0.1).astype(np.float32)
    sh = None
    if I_s:
        sh = [(rng.standard_normal(s) * 0.1).astype(np.float32)
              for s in ((I_s, H), (I_s, H), (H, I_s))]
    desc = dict(T=T, H=H, E=E, e0=e0, E_loc=E_loc, I=I, k=k, I_s=I_s, scoring=scoring,
                renormalize=1, act_fmt=oracle.F32)
    return desc, x, wr, g, u, d, sh


def _run(desc, x, wr, g, u, d, sh, bias=None, tok=None, shared_gate=None):
    M = oracle.Mat
    shared = None if sh is None else tuple(M(oracle.F32, s) for s in sh)
    return oracle.moe_layer(desc, x, wr, bias, M(oracle.F32, x), M(oracle.F32, g), M(oracle.F32, u),
                            M(oracle.F32, d), shared, tok, shared_gate=shared_gate)


def test_single_expert_is_dense_ffn():
    desc, x, wr, g, u, d, _ = _tiny(E=1, E_loc=1, k=1)
    r = _run(desc, x, wr, g, u, d, None)
    ref = _dense_swiglu(x.astype(np.float64), g[0].astype(np.float64), u[0].astype(np.float64),
                        d[0].astype(np.float64))
    assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(r["w"], 1.0)


def test_identical_experts_equal_dense_ffn():
    desc, x, wr, g, u, d, _ = _tiny(E=6, E_loc=6, k=3, same=True)
    r = _run(desc, x, wr, g, u, d, None)
    ref = _dense_swiglu(x.astype(np.float64), g[0].astype(np.float64), u[0].astype(np.float64),
                        d[0].astype(np.float64))
    assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-12)


def test_combine_equals_dense_per_token_loop():
    for scoring in (oracle.SOFTMAX, oracle.SIGMOID):
        desc, x, wr, g, u, d, sh = _tiny(T=10, E=8, E_loc=4, e0=2, k=3, I_s=16, scoring=scoring)
        bias = np.linspace(-1, 1, 8).astype(np.float32)
        r = _run(desc, x, wr, g, u, d, sh, bias=bias)
        L = x.astype(np.float64) @ wr.astype(np.float64).T + bias
        L32 = L.astype(np.float32)
        ids = _topk_bruteforce(L32, 3)
        sel = np.take_along_axis(L32.astype(np.float64), ids, 1)
        if scoring == oracle.SOFTMAX:
            w = softmax(sel, axis=1)
        else:
            w = expit(sel) / expit(sel).sum(1, keepdims=True)
        x64 = x.astype(np.float64)
        ref = np.zeros((10, desc["H"]))
        for t in range(10):
            for j in range(3):
                el = ids[t, j] - 2
                if 0 <= el < 4:
                    ref[t] += w[t, j] * _dense_swiglu(x64[t:t + 1], g[el].astype(np.float64),
                                                      u[el].astype(np.float64),
                                                      d[el].astype(np.float64))[0]
            ref[t] += _dense_swiglu(x64[t:t + 1], *(s.astype(np.float64) for s in sh))[0]
        assert np.array_equal(r["ids"], ids)
        assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-12)


def test_zero_down_projection_leaves_shared_only():
    desc, x, wr, g, u, d, sh = _tiny(I_s=16)
    r = _run(desc, x, wr, g, u, np.zeros_like(d), sh)
    ref = _dense_swiglu(x.astype(np.float64), *(s.astype(np.float64) for s in sh))
    assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-12)
    r0 = _run(desc, np.zeros_like(x), wr, g, u, d, sh)                 # silu(0) * 0 = 0
    assert not np.any(r0["out"])


def test_layer_token_subset_and_permutation_equivariance():
    desc, x, wr, g, u, d, sh = _tiny(T=16, I_s=8)
    full = _run(desc, x, wr, g, u, d, sh)
    tok = np.array([7, 3, 15, 0], np.int32)
    sub = _run(desc, x, wr, g, u, d, sh, tok=tok)
    assert np.array_equal(sub["out"], full["out"][tok])
    perm = np.random.default_rng(0).permutation(16)
    px = _run(desc, x[perm], wr, g, u, d, sh)
    assert np.allclose(px["out"], full["out"][perm], rtol=0, atol=1e-13)


def test_layer_with_given_routing_equals_dense_loop():
    """oracle_moe_layer_routed: the expert part for a routing handed in (arbitrary chosen experts,
    some not local, arbitrary fp32 weights) equals the dense per-token loop in numpy; handed the
    oracle's own routing it reproduces the layer up to the fp32 rounding of the weights."""
    desc, x, wr, g, u, d, sh = _tiny(T=9, E=8, E_loc=4, e0=2, k=3, I_s=16)
    M = oracle.Mat
    mats = [M(oracle.F32, a) for a in (g, u, d)]
    shared = tuple(M(oracle.F32, s) for s in sh)
    rng = np.random.default_rng(5)
    tok = np.array([8, 0, 4, 4], np.int32)
    ids = np.stack([rng.permutation(8)[:3] for _ in tok]).astype(np.int32)
    w = rng.random((len(tok), 3)).astype(np.float32)
    out = oracle.moe_layer_routed(desc, x, M(oracle.F32, x), *mats, shared, tok, ids, w)
    x64 = x.astype(np.float64)
    for i, t in enumerate(tok):
        ref = _dense_swiglu(x64[t:t + 1], *(s.astype(np.float64) for s in sh))[0]
        for j in range(3):
            el = ids[i, j] - 2
            if 0 <= el < 4:
                ref = ref + np.float64(w[i, j]) * _dense_swiglu(
                    x64[t:t + 1], g[el].astype(np.float64), u[el].astype(np.float64),
                    d[el].astype(np.float64))[0]
        assert np.allclose(out[i], ref, rtol=1e-12, atol=1e-12)
    full = _run(desc, x, wr, g, u, d, sh)
    allt = np.arange(9, dtype=np.int32)
    again = oracle.moe_layer_routed(desc, x, M(oracle.F32, x), *mats, shared, allt, full["ids"],
                                    full["w"].astype(np.float32))
    assert np.allclose(again, full["out"], rtol=1e-6, atol=1e-6 * np.abs(full["out"]).max())


def test_ffn_quantised_activations_fp8():
    """h quantised to e4m3 with 1x128 scales: equals the dense FFN with h passed through torch's
    e4m3 cast at scale amax/448 per 128 columns."""
    rng = np.random.default_rng(8)
    H, I = 128, 256
    a = rng.standard_normal(H)
    wg, wu = (rng.standard_normal((I, H)) * 0.1 for _ in range(2))
    wd = rng.standard_normal((H, I)) * 0.1
    M = oracle.Mat
    y = oracle.ffn_row(a, M(oracle.F32, wg.astype(np.float32)), M(oracle.F32, wu.astype(np.float32)),
                       M(oracle.F32, wd.astype(np.float32)), act_fmt=oracle.FP8)
    wg32, wu32, wd32 = (w.astype(np.float32).astype(np.float64) for w in (wg, wu, wd))
    gg, uu = a @ wg32.T, a @ wu32.T
    h = (gg * expit(gg) * uu).astype(np.float32)
    hq = np.empty(I)
    for b in range(0, I, 128):
        blk = h[b:b + 128]
        s = np.float32(np.abs(blk).max()) / np.float32(448.0)
        c = torch.from_numpy((blk / s).astype(np.float32)).to(torch.float8_e4m3fn).float().numpy()
        hq[b:b + 128] = c.astype(np.float64) * np.float64(s)
    assert np.allclose(y, hq @ wd32.T, rtol=1e-12, atol=1e-12)


def test_quantised_weight_stack_dequantises_blockwise():
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((2, 256, 256)) * 0.02).astype(np.float32)
    m = oracle.quantise_stack(oracle.FP8, w)
    assert m.s.shape == (2, 2, 2)
    dq = m.dequant()
    assert np.abs(dq - w).max() <= np.abs(w).max() * 2.0 ** -4
    assert m.at(1, 130, 7) == dq[1, 130, 7]
    m4 = oracle.quantise_stack(oracle.MX4, w)
    assert m4.q.shape == (2, 256, 128) and m4.s.shape == (2, 256, 8)


# ------------------------------------------------------------------------------------------
# grouped GEMM and combine as separate steps
# ------------------------------------------------------------------------------------------

def test_grouped_gemm_matches_numpy_per_group():
    rng = np.random.default_rng(11)
    G, N, K = 3, 48, 64
    counts = np.array([5, 0, 9])
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = 7
    x = rng.standard_normal((T, K)).astype(np.float32)
    a_rows = rng.integers(0, T * 2, size=off[-1]).astype(np.int32)   # flat slots, k = 2
    B = (rng.standard_normal((G, N, K)) * 0.1).astype(np.float32)
    B2 = (rng.standard_normal((G, N, K)) * 0.1).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    M = oracle.Mat
    st = oracle.grouped_gemm(off, M(oracle.F32, x), M(oracle.F32, B), a_rows=a_rows, a_row_div=2,
                             bias=bias)
    sw = oracle.grouped_gemm(off, M(oracle.F32, x), M(oracle.F32, B), M(oracle.F32, B2),
                             a_rows=a_rows, a_row_div=2)
    x64 = x.astype(np.float64)
    for g in range(G):
        rows = slice(off[g], off[g + 1])
        a = x64[a_rows[rows] // 2]
        d = a @ B[g].astype(np.float64).T
        assert np.allclose(st[rows], d + bias, rtol=0, atol=1e-12)
        u = a @ B2[g].astype(np.float64).T
        assert np.allclose(sw[rows], d * expit(d) * u, rtol=0, atol=1e-12)


def test_grouped_gemm_fp8_blocks_equal_dequantised_matmul():
    rng = np.random.default_rng(12)
    K, N, T = 256, 128, 200
    x = rng.standard_normal((T, K)).astype(np.float32)
    w = (rng.standard_normal((1, N, K)) * 0.02).astype(np.float32)
    xc, xs = oracle.quant_fp8(x, 128, 128)                 # 128-token x 128-channel blocks
    xa = oracle.Mat(oracle.FP8, xc[None], xs[None], bn=128, bk=128)
    wm = oracle.quantise_stack(oracle.FP8, w)
    off = np.array([0, T], np.int32)
    out = oracle.grouped_gemm(off, xa, wm)
    ref = xa.dequant()[0] @ wm.dequant()[0].T
    assert np.allclose(out, ref, rtol=0, atol=1e-12)
    # the codes of x are torch's e4m3 cast of x / s with s = amax / 448 over each 128 x 128 block
    s = np.abs(x[:128, :128]).max() / np.float32(448.0)
    assert xs[0, 0] == np.float32(s)
    ref_codes = torch.from_numpy((x[:128, :128] / xs[0, 0]).astype(np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(xc[:128, :128], ref_codes)


def test_combine_matches_gather_formula_and_layer():
    rng = np.random.default_rng(13)
    T, k, H, R = 9, 3, 16, 20
    y = rng.standard_normal((R, H)).astype(np.float32)
    w = rng.random((T, k)).astype(np.float32)
    s2r = rng.integers(-1, R, size=(T, k)).astype(np.int32)
    sh = rng.standard_normal((T, H)).astype(np.float32)
    out = oracle.combine(y, w, s2r, sh)
    wm = np.where(s2r >= 0, w.astype(np.float64), 0.0)
    ref = np.einsum("tj,tjh->th", wm, y.astype(np.float64)[np.maximum(s2r, 0)]) + sh
    assert np.allclose(out, ref, rtol=0, atol=1e-12)
    assert np.allclose(oracle.combine(y, np.zeros_like(w), s2r, sh), sh)
    # the layer's output is the combine of per-slot FFN rows placed by the permutation
    desc, x, wr, g, u, d, shw = _tiny(T=8, E=6, E_loc=3, e0=1, k=2, I_s=8)
    full = _run(desc, x, wr, g, u, d, shw)
    counts, offsets, s2r, r2f = oracle.permute(full["ids"], 1, 3)
    M = oracle.Mat
    ys = np.zeros((max(len(r2f), 1), desc["H"]), np.float32)
    for r, f in enumerate(r2f):
        t, j = divmod(int(f), 2)
        ys[r] = oracle.ffn_row(x[t], M(oracle.F32, g), M(oracle.F32, u), M(oracle.F32, d),
                               g=int(full["ids"][t, j]) - 1)
    shy = np.stack([oracle.ffn_row(x[t], *(M(oracle.F32, s) for s in shw)) for t in range(8)])
    comb = oracle.combine(ys, full["w"].astype(np.float32), s2r, shy.astype(np.float32))
    assert np.allclose(comb, full["out"], rtol=1e-5, atol=1e-5)


def test_shared_gate_closed_forms():
    # logistic function at z = +-ln 3 (3/4 and 1/4) and z = 0 (1/2), reached through one-hot rows
    H = 16
    x = np.zeros((4, H), np.float32)
    x[0, 3], x[1, 3], x[3, 5] = 1.0, -1.0, 2.0
    w = np.zeros(H, np.float32)
    w[3] = np.float32(np.log(3.0))
    w[5] = np.float32(-np.log(3.0) / 2)
    g = oracle.shared_gate(x, w)
    assert np.allclose(g, [0.75, 0.25, 0.5, 0.25], rtol=0, atol=1e-7)
    # a zero gate vector halves the shared expert for every token, exactly
    rng = np.random.default_rng(21)
    xr = rng.standard_normal((7, 40)).astype(np.float32)
    assert np.array_equal(oracle.shared_gate(xr, np.zeros(40, np.float32)), np.full(7, 0.5))
    # g(x) + g(-x) = 1, strictly increasing in the logit, subset of tokens = rows of the full call
    wr = (rng.standard_normal(40) * 0.3).astype(np.float32)
    gp, gm = oracle.shared_gate(xr, wr), oracle.shared_gate(-xr, wr)
    assert np.allclose(gp + gm, 1.0, rtol=0, atol=1e-15)
    z = xr.astype(np.float64) @ wr.astype(np.float64)
    assert np.all(np.diff(gp[np.argsort(z)]) > 0)
    tok = np.array([6, 0, 3], np.int32)
    assert np.array_equal(oracle.shared_gate(xr, wr, tok), gp[tok])


def test_gated_shared_expert_scales_only_the_shared_term():
    desc, x, wr, g, u, d, sh = _tiny(T=9, E=6, E_loc=3, e0=2, k=2, I_s=8)
    routed = _run(dict(desc, I_s=0), x, wr, g, u, d, None)["out"]
    ungated = _run(desc, x, wr, g, u, d, sh)["out"]
    # zero gate vector: exactly half of the shared expert's output is added to the routed sum
    half = _run(desc, x, wr, g, u, d, sh, shared_gate=np.zeros(desc["H"], np.float32))["out"]
    assert np.allclose(half, routed + 0.5 * (ungated - routed), rtol=0, atol=1e-12)
    # any gate vector: per token, a single factor in (0, 1) on the shared term, equal to the gate
    gv = (np.random.default_rng(22).standard_normal(desc["H"]) * 0.5).astype(np.float32)
    gated = _run(desc, x, wr, g, u, d, sh, shared_gate=gv)["out"]
    sh_term = ungated - routed
    ratio = (gated - routed) / sh_term
    gt = oracle.shared_gate(x, gv)
    assert np.all((gt > 0) & (gt < 1)) and gt.std() > 0.05
    assert np.allclose(ratio, gt[:, None], rtol=0, atol=1e-9)
    # the combine step applies the same per-token factor to the shared rows
    rng = np.random.default_rng(23)
    T, k, H, R = 5, 2, 8, 7
    y = rng.standard_normal((R, H)).astype(np.float32)
    w = rng.random((T, k)).astype(np.float32)
    s2r = rng.integers(-1, R, size=(T, k)).astype(np.int32)
    shr = rng.standard_normal((T, H)).astype(np.float32)
    sw = rng.random(T).astype(np.float32)
    wm = np.where(s2r >= 0, w.astype(np.float64), 0.0)
    ref = (np.einsum("tj,tjh->th", wm, y.astype(np.float64)[np.maximum(s2r, 0)])
           + sw.astype(np.float64)[:, None] * shr)
    assert np.allclose(oracle.combine(y, w, s2r, shr, sw), ref, rtol=0, atol=1e-12)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(14)
    v = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 3,
                        rng.standard_normal(2000).astype(np.float32) * 1e-30,
                        # exact midpoints between neighbouring bf16 values (ties)
                        (np.arange(1, 3000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)]
                       ).astype(np.float32)
    ours = np.array([oracle.bf16_round(a) for a in v], np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).float().numpy()
    assert np.array_equal(ours, ref)


def test_ffn_bf16_activation_rounds_h():
    rng = np.random.default_rng(15)
    H, I = 64, 96
    a = rng.standard_normal(H)
    wg, wu = ((rng.standard_normal((I, H)) * 0.2).astype(np.float32) for _ in range(2))
    wd = (rng.standard_normal((H, I)) * 0.2).astype(np.float32)
    M = oracle.Mat
    y = oracle.ffn_row(a, M(oracle.F32, wg), M(oracle.F32, wu), M(oracle.F32, wd), act_fmt=oracle.BF16)
    gg, uu = a @ wg.astype(np.float64).T, a @ wu.astype(np.float64).T
    h = torch.from_numpy((gg * expit(gg) * uu).astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.allclose(y, h @ wd.astype(np.float64).T, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------------------------------
# NVFP4: e2m1 elements, e4m3 scale per 16 along K, fp32 row scale
# ------------------------------------------------------------------------------------------

_E2M1_MAG = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)


def _e2m1_decode_numpy(nib):
    nib = nib.astype(np.int64)
    return np.where(nib & 8, -1.0, 1.0) * _E2M1_MAG[nib & 7]


def _e4m3_decode_torch(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def _nv4_decode_numpy(packed, bscales, rscales):
    """Element values e2m1 * s * g from the stored codes, with a numpy nibble table and torch's
    e4m3 decoding (no oracle code involved)."""
    lo, hi = packed & 15, packed >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], packed.shape[-1] * 2)
    s = np.repeat(_e4m3_decode_torch(bscales), 16, axis=-1)
    return _e2m1_decode_numpy(nib) * s * rscales.astype(np.float64)[..., None]


def test_nv4_hand_example():
    lines = _golden_kv("nv4_block_example.txt")
    for r in (0, 1):
        v = np.array([float(a) for a in lines[f"values{r}"]], np.float32)[None]
        p, b, rs = oracle.quant_nv4(v)
        assert rs[0] == np.float32(float(lines[f"rscale{r}"][0]))
        assert [int(c) for c in b[0]] == [int(c, 0) for c in lines[f"scales{r}"]]
        assert [int(c) for c in p[0]] == [int(c, 0) for c in lines[f"bytes{r}"]]
    rows = [np.array([float(a) for a in lines[f"values{r}"]], np.float32) for r in (0, 1)]
    p, b, rs = oracle.quant_nv4(np.stack(rows))
    m = oracle.Mat(oracle.NV4, p[None], b[None], r=rs[None])
    deq = lines["deq"]
    for i in range(0, len(deq), 3):
        assert m.at(0, int(deq[i]), int(deq[i + 1])) == float(deq[i + 2])


def test_nv4_scale_rules_and_codes_restated():
    """Row scale g = amax / 2688 (fp32), block scale code = e4m3 (torch's nearest-even cast of
    the clamped fp32 quotient bamax / (6 g)), element = nearest-even e2m1 of v / (s g), all
    restated in numpy/torch. Blocks get magnitudes from 1e-6 to 1e3 so the block scales cover
    e4m3's subnormal and normal ranges and the 16-element grouping matters."""
    rng = np.random.default_rng(41)
    rows, cols = 24, 256
    mag = 10.0 ** rng.uniform(-6, 3, size=(rows, cols // 16))
    v = (rng.standard_normal((rows, cols)) * np.repeat(mag, 16, axis=1)).astype(np.float32)
    v[3] = 0.0
    v[5, :16] = 0.0
    p, b, rs = oracle.quant_nv4(v)
    amax = np.abs(v).max(axis=1)
    g = np.where(amax > 0, amax / np.float32(2688), np.float32(1)).astype(np.float32)
    assert np.array_equal(rs, g)
    d6 = (np.float32(6) * g).astype(np.float32)
    bamax = np.abs(v).reshape(rows, cols // 16, 16).max(axis=2)
    q = np.minimum((bamax / d6[:, None]).astype(np.float32), np.float32(448))
    ref_b = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(b, ref_b)
    s = _e4m3_decode_torch(b).astype(np.float32)
    d = np.repeat((s * g[:, None]).astype(np.float32), 16, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        ref = np.where(d > 0, _e2m1_rne_numpy((v / np.where(d > 0, d, 1)).astype(np.float32)), 0.0)
    lo, hi = p & 15, p >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(rows, cols)
    ours = _e2m1_decode_numpy(nib)
    assert np.array_equal(ours, ref)
    assert np.array_equal(np.signbit(ours), np.signbit(v))     # zeros keep the element's sign


def test_nv4_roundtrip_and_error_bound():
    rng = np.random.default_rng(42)
    # values on the grid: g = 2^-k (row amax 2688 * 2^-k), block maxima 6 * s * g with s on the
    # e4m3 grid, elements e2m1 * s * g: quantise and decode without loss
    e4 = np.array([oracle.e4m3_value(c) for c in range(1, 0x7F)], np.float64)
    for k in (0, 5, 12):
        g = 2.0 ** -k
        v = np.empty((3, 128))
        for r in range(3):
            top = rng.integers(8)                               # the block holding 6 * 448 * g
            for blk in range(8):
                sb = 448.0 if blk == top else rng.choice(e4)
                el = rng.choice(_E2M1_MAG, 16) * rng.choice([-1, 1], 16)
                el[rng.integers(16)] = 6.0
                v[r, blk * 16:(blk + 1) * 16] = el * sb * g
        v = v.astype(np.float32)
        assert np.array_equal(v.astype(np.float64), v)          # exact in fp32
        p, b, rs = oracle.quant_nv4(v)
        m = oracle.Mat(oracle.NV4, p[None], b[None], r=rs[None])
        assert np.all(rs == np.float32(g))
        assert np.array_equal(m.dequant()[0], v.astype(np.float64))
    # random rows: the decoded value equals the numpy decode of the stored codes; inside the e2m1
    # range the error is at most half the grid step (0.25, 0.5, 1 times d below 2, 4, 6); above
    # it (the block scale rounded down by up to 2^-4) the value saturates at 6 d
    v = (rng.standard_normal((32, 512)) * 0.05).astype(np.float32)
    p, b, rs = oracle.quant_nv4(v)
    m = oracle.Mat(oracle.NV4, p[None], b[None], r=rs[None])
    dq = m.dequant()[0]
    assert np.array_equal(dq, _nv4_decode_numpy(p, b, rs))
    d = np.repeat(_e4m3_decode_torch(b), 16, axis=1) * rs.astype(np.float64)[:, None]
    a = np.abs(v.astype(np.float64)) / d
    err = np.abs(dq - v) / d
    half = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0))
    inside = a <= 6
    assert np.all(err[inside] <= half[inside] * (1 + 1e-6))
    assert np.all(np.abs(dq[~inside]) == 6 * d[~inside]) and np.all(a[~inside] <= 6 * (1 + 2.0 ** -4) * (1 + 1e-6))
    # per block the error stays below d <= (bamax / 6)(1 + 2^-4) (block scales in e4m3's
    # normal range here, where its rounding is within 2^-4)
    blk_err = np.abs(dq - v).reshape(32, 32, 16).max(axis=2)
    bamax = np.abs(v.astype(np.float64)).reshape(32, 32, 16).max(axis=2)
    assert np.all(_e4m3_decode_torch(b) >= 2.0 ** -6)
    assert np.all(blk_err <= bamax / 6 * (1 + 2.0 ** -4) * (1 + 1e-6))


def test_grouped_gemm_nv4_equals_dequantised_matmul():
    """NVFP4 weights and activations in the oracle's grouped GEMM: the numpy product of the
    independently decoded operands."""
    rng = np.random.default_rng(43)
    K, N, T = 256, 96, 40
    x = rng.standard_normal((T, K)).astype(np.float32)
    w = (rng.standard_normal((2, N, K)) * 0.02).astype(np.float32)
    xp, xb, xr = oracle.quant_nv4(x)
    xa = oracle.Mat(oracle.NV4, xp[None], xb[None], r=xr[None])
    wm = oracle.quantise_stack(oracle.NV4, w)
    assert wm.q.shape == (2, N, K // 2) and wm.s.shape == (2, N, K // 16) and wm.r.shape == (2, N)
    off = np.array([0, 15, T], np.int32)
    out = oracle.grouped_gemm(off, xa, wm)
    xd = _nv4_decode_numpy(xp, xb, xr)
    wd = _nv4_decode_numpy(wm.q, wm.s, wm.r)
    for g in range(2):
        ref = xd[off[g]:off[g + 1]] @ wd[g].T
        assert np.allclose(out[off[g]:off[g + 1]], ref, rtol=0, atol=1e-12)


def test_ffn_nv4_rounds_h_to_bf16():
    """An NVFP4 layer keeps h in bf16: the FFN with act_fmt NV4 equals the dense FFN with h
    rounded by torch's bf16 cast."""
    rng = np.random.default_rng(44)
    H, I = 64, 96
    a = rng.standard_normal(H)
    wg, wu = ((rng.standard_normal((I, H)) * 0.2).astype(np.float32) for _ in range(2))
    wd = (rng.standard_normal((H, I)) * 0.2).astype(np.float32)
    M = oracle.Mat
    y = oracle.ffn_row(a, M(oracle.F32, wg), M(oracle.F32, wu), M(oracle.F32, wd), act_fmt=oracle.NV4)
    gg, uu = a @ wg.astype(np.float64).T, a @ wu.astype(np.float64).T
    h = torch.from_numpy((gg * expit(gg) * uu).astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.allclose(y, h @ wd.astype(np.float64).T, rtol=1e-12, atol=1e-12)


def test_layer_nv4_equals_dense_loop_on_decoded_operands():
    """The NVFP4 layer for a given routing: per token, the weighted sum over its local experts of
    the dense SwiGLU FFN on the numpy-decoded x row and weights, with h rounded to bf16."""
    rng = np.random.default_rng(45)
    T, H, I, E_loc, k = 6, 64, 48, 3, 2
    x = rng.standard_normal((T, H)).astype(np.float32)
    g, u = ((rng.standard_normal((E_loc, I, H)) * 0.15).astype(np.float32) for _ in range(2))
    d = (rng.standard_normal((E_loc, H, I)) * 0.15).astype(np.float32)
    mats = [oracle.quantise_stack(oracle.NV4, w) for w in (g, u, d)]
    xp, xb, xr = oracle.quant_nv4(x)
    xa = oracle.Mat(oracle.NV4, xp[None], xb[None], r=xr[None])
    desc = dict(T=T, H=H, E=5, e0=1, E_loc=E_loc, I=I, k=k, I_s=0, scoring=0, renormalize=1,
                act_fmt=oracle.NV4)
    tok = np.arange(T, dtype=np.int32)
    ids = np.array([[1, 2], [3, 0], [4, 1], [2, 3], [0, 4], [3, 3]], np.int32)
    w = rng.random((T, k)).astype(np.float32)
    out = oracle.moe_layer_routed(desc, x, xa, *mats, None, tok, ids, w)
    xd = _nv4_decode_numpy(xp, xb, xr)
    gd, ud, dd = (_nv4_decode_numpy(m.q, m.s, m.r) for m in mats)
    for t in range(T):
        ref = np.zeros(H)
        for j in range(k):
            el = ids[t, j] - 1
            if 0 <= el < E_loc:
                gg, uu = gd[el] @ xd[t], ud[el] @ xd[t]
                h = torch.from_numpy((gg * expit(gg) * uu).astype(np.float32)).to(torch.bfloat16).double().numpy()
                ref += np.float64(w[t, j]) * (dd[el] @ h)
        assert np.allclose(out[t], ref, rtol=1e-12, atol=1e-12)
