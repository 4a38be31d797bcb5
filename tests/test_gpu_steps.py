"""Per-step parity of the HIP path against the oracle, through the C ABI: quantisers, routing,
dispatch, grouped GEMM and combine. Integer results bit-exact; floating results within the stated
tolerances."""
import numpy as np
import pytest
import torch

import moe_layer_softmax_amd as moe
import oracle
from moe_inputs import gen

from gpu_util import (check_f16s_format, f16s_pack, f16s_split, gamma, gpu_quant, rel_err,
                      routing_consistent, to_dev, topk_numpy)

pytestmark = pytest.mark.gpu


def _sync():
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------------------------
# quantisers: codes and scales bit-exact
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("rows,cols,block_rows,src", [(256, 384, 128, "f32"), (200, 256, 128, "bf16"),
                                                       (37, 1024, 1, "f32"), (128, 7168, 128, "bf16")])
def test_quantize_fp8_bitexact(rows, cols, block_rows, src):
    rng = np.random.default_rng(rows + cols)
    a = (rng.standard_normal((2, rows, cols)) * rng.choice([0.02, 1.0, 30.0])).astype(np.float32)
    a[0, :7, :] = 0.0                               # an all-zero region
    if src == "bf16":
        a = gen.bf16_round(a)
    t = to_dev(a, torch.float32 if src == "f32" else torch.bfloat16)
    nbr = (rows + block_rows - 1) // block_rows
    codes = torch.empty((2, rows, cols), dtype=torch.uint8, device="cuda")
    scales = torch.empty((2, nbr, cols // 128), dtype=torch.float32, device="cuda")
    moe.moe_quantize(moe.MOE_FP8_E4M3, moe.MOE_F32 if src == "f32" else moe.MOE_BF16, 2, rows,
                     cols, block_rows, t, codes, scales)
    _sync()
    for b in range(2):
        c_ref, s_ref = oracle.quant_fp8(a[b], block_rows, 128)
        assert np.array_equal(scales[b].cpu().numpy(), s_ref)
        assert np.array_equal(codes[b].cpu().numpy(), c_ref)


@pytest.mark.parametrize("rows,cols,src", [(64, 256, "f32"), (333, 7168, "bf16"), (5, 2048, "f32")])
def test_quantize_mx4_bitexact(rows, cols, src):
    rng = np.random.default_rng(rows * cols)
    a = rng.standard_normal((3, rows, cols)).astype(np.float32)
    a[1] *= 1e-3
    a[2, :, :32] = 0.0
    a[2, 0, 40:72] = np.array([0.25, -0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0] * 4, np.float32)
    if src == "bf16":
        a = gen.bf16_round(a)
    t = to_dev(a, torch.float32 if src == "f32" else torch.bfloat16)
    packed = torch.empty((3, rows, cols // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((3, rows, cols // 32), dtype=torch.uint8, device="cuda")
    moe.moe_quantize(moe.MOE_MXFP4, moe.MOE_F32 if src == "f32" else moe.MOE_BF16, 3, rows, cols, 1,
                     t, packed, scales)
    _sync()
    for b in range(3):
        p_ref, s_ref = oracle.quant_mx4(a[b])
        assert np.array_equal(scales[b].cpu().numpy(), s_ref)
        assert np.array_equal(packed[b].cpu().numpy(), p_ref)


@pytest.mark.parametrize("rows,cols,src", [(64, 256, "f32"), (333, 4096, "bf16"), (5, 1536, "f32")])
def test_quantize_mx8_bitexact(rows, cols, src):
    rng = np.random.default_rng(rows + 7 * cols)
    a = rng.standard_normal((3, rows, cols)).astype(np.float32)
    a[1] *= 1e-3
    a[2, :, :32] = 0.0
    a[2, 0, 40:72] = np.array([300.0, -1.0, 0.5, 3.0, -250.0, 17.0, -0.0, 0.001] * 4, np.float32)
    a[2, 1, 64:96] = np.float32(7.5)                 # scaled values saturate at 448
    if src == "bf16":
        a = gen.bf16_round(a)
    t = to_dev(a, torch.float32 if src == "f32" else torch.bfloat16)
    codes = torch.empty((3, rows, cols), dtype=torch.uint8, device="cuda")
    scales = torch.empty((3, rows, cols // 32), dtype=torch.uint8, device="cuda")
    moe.moe_quantize(moe.MOE_MXFP8, moe.MOE_F32 if src == "f32" else moe.MOE_BF16, 3, rows, cols, 1,
                     t, codes, scales)
    _sync()
    for b in range(3):
        c_ref, s_ref = oracle.quant_mx8(a[b])
        assert np.array_equal(scales[b].cpu().numpy(), s_ref)
        assert np.array_equal(codes[b].cpu().numpy(), c_ref)


def _edge_values(grid):
    """Every grid value with both signs, the midpoints of neighbouring grid values (exact ties),
    the fp32 neighbours of each midpoint and of each grid value, and +-0."""
    g = np.unique(np.concatenate([grid, -grid])).astype(np.float32)
    mids = ((g[1:].astype(np.float64) + g[:-1]) / 2).astype(np.float32)
    vals = [g, mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(-np.inf)),
            np.nextafter(g, np.float32(np.inf)), np.nextafter(g, np.float32(-np.inf)),
            np.array([0.0, -0.0], np.float32)]
    return np.concatenate(vals).astype(np.float32)


def _pack_groups(vals, group, anchor):
    """Rows of `group`-element blocks, each block led by `anchor` (which fixes a unit scale) and
    filled with test values; the last block is padded with zeros."""
    per = group - 1
    n = (len(vals) + per - 1) // per
    v = np.zeros(n * per, np.float32)
    v[:len(vals)] = vals
    blocks = np.concatenate([np.full((n, 1), anchor, np.float32), v.reshape(n, per)], axis=1)
    return blocks.reshape(-1)


# The quantisers on the values where rounding decisions are made: every e4m3 / e2m1 grid value,
# every tie between neighbours, their fp32 neighbours, subnormals, +-0 and the saturation range
# 440..620. Blocks are led by the value that makes the scale exactly 1 (448 for fp8's amax / 448
# and for MXFP8's floor(log2 amax) - 8; 6 for MXFP4's floor(log2 amax) - 2), so every test value
# is itself the quotient that is rounded; a second set runs with the natural scales.
@pytest.mark.parametrize("fmt", ["fp8", "mx8", "mx4"])
def test_quantize_edge_values_bitexact(fmt):
    if fmt == "mx4":
        grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
        anchor, group, cols = 6.0, 32, 256
    else:
        codes = np.arange(0x7F, dtype=np.uint8)                  # every finite non-negative e4m3
        grid = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
        anchor, group, cols = 448.0, (128 if fmt == "fp8" else 32), 256
    vals = _edge_values(grid)
    sat = np.linspace(440.0, 620.0, 361, dtype=np.float32)      # around and beyond the maximum
    if fmt == "mx4":
        sat = sat / np.float32(448.0 / 6.0)
    vals = np.concatenate([vals, sat, -sat])
    flat = _pack_groups(vals, group, anchor)
    flat = np.concatenate([flat, np.zeros((-len(flat)) % cols, np.float32)])
    a_unit = flat.reshape(-1, cols)
    # the same values without the anchors: block scales follow from each block's own maximum
    free = np.concatenate([vals, np.zeros((-len(vals)) % cols, np.float32)]).reshape(-1, cols)
    dfmt = {"fp8": moe.MOE_FP8_E4M3, "mx8": moe.MOE_MXFP8, "mx4": moe.MOE_MXFP4}[fmt]
    for a in (a_unit, free):
        rows = a.shape[0]
        block_rows = 1
        q, sc = gpu_quant(dfmt, a, block_rows)
        if fmt == "fp8":
            c_ref, s_ref = oracle.quant_fp8(a, block_rows, 128)
        elif fmt == "mx8":
            c_ref, s_ref = oracle.quant_mx8(a)
        else:
            c_ref, s_ref = oracle.quant_mx4(a)
        assert np.array_equal(sc[0].cpu().numpy(), s_ref), rows
        assert np.array_equal(q[0].cpu().numpy(), c_ref), rows


# ---------------------------------------------------------------------------------------------
# routing
# ---------------------------------------------------------------------------------------------

def _route_given_logits(L, k, scoring, renorm, e0=0, E_loc=None):
    T, E = L.shape
    d = moe.make_desc(T, 64, E, e0, E_loc or E, 64, k, 0, scoring, renorm)
    lt = to_dev(L, torch.float32)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.moe_route(d, None, None, None, lt, ids, w)
    _sync()
    return ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("E,k", [(8, 2), (128, 8), (512, 10), (256, 8), (16, 16), (1024, 16),
                                 (5, 1), (70, 3)])
@pytest.mark.parametrize("scoring,renorm", [(0, 1), (1, 1), (0, 0), (1, 0)])
def test_topk_bitexact(E, k, scoring, renorm):
    for T, L in ((333, gen.tie_heavy_logits(333, E, seed=E)),
                 (1000, gen.random_logits(1000, E, seed=k, scale=2.0)),
                 (257, gen.random_logits(257, E, seed=1, scale=1.0,
                                         bias=gen.router_bias(_zipf_wl(E))))):
        ids, w = _route_given_logits(L, k, scoring, renorm)
        ids_ref, w_ref = oracle.topk(L, k, scoring, renorm)
        assert np.array_equal(ids, ids_ref)
        assert np.abs(w - w_ref).max() <= 1e-6


def _zipf_wl(E):
    from moe_inputs.workloads import Workload
    return Workload("z", 1, 64, E, 0, E, 64, 1, 0, 0, 1, 1, 1, 1.1)


# Router shapes: few tokens (K-split partial sums finished by the top-k kernel), more tokens
# (64-token waves, split or not), enough tokens for each tile shape of the router GEMM (32, 64 and
# 128 tokens per tile, ragged last tiles),
# an expert count that is not a multiple of 16 (grouped-GEMM router) and the fp32 router.
@pytest.mark.parametrize("T,H,E,k,zipf,scoring", [(300, 4096, 128, 8, 1.1, 0), (64, 7168, 256, 8, 1.2, 1),
                                                  (40, 4096, 512, 10, 0.0, 0), (33, 256, 8, 2, 0.0, 0),
                                                  (64, 4096, 128, 8, 1.1, 0), (1, 4096, 128, 8, 1.1, 0),
                                                  (1500, 4096, 256, 8, 0.0, 1), (4096, 4096, 128, 8, 1.1, 0),
                                                  (100, 4096, 72, 4, 0.0, 0), (17, 1024, 16, 16, 0.0, 0),
                                                  (8200, 4096, 512, 10, 0.0, 0), (16400, 4096, 128, 8, 1.1, 0)])
def test_route_from_x(T, H, E, k, zipf, scoring):
    from moe_inputs.workloads import Workload
    io = 0 if H == 256 else 1
    wl = Workload("r", T, H, E, 0, E, 64, k, 0, scoring, 1, io, io, zipf)
    x, wr, bias = gen.tokens(wl), gen.router_weight(wl), gen.router_bias(wl)
    dt = torch.float32 if io == 0 else torch.bfloat16
    d = moe.make_desc(T, H, E, 0, E, 64, k, 0, scoring, 1, io, io)
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    rws = torch.empty(max(moe.moe_route_workspace_bytes(d), 16), dtype=torch.uint8, device="cuda")
    moe.moe_route(d, to_dev(x, dt), to_dev(wr, dt), None if bias is None else to_dev(bias, torch.float32),
                  lg, ids, w, ws=rws)
    _sync()
    lg, ids, w = lg.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()
    L64, absdot = oracle.logits(x, wr, bias)
    bound = gamma(H + 1) * absdot
    assert np.all(np.abs(lg.astype(np.float64) - L64) <= bound)
    # the GPU chose from exactly the fp32 logits it wrote (selection rule checked in numpy)
    assert np.array_equal(ids, topk_numpy(lg, k))
    # against the oracle's own routing: equal, or a valid choice inside the logit bound
    ids_ref, w_ref = oracle.topk(L64.astype(np.float32), k, scoring, 1)
    diff = np.nonzero((ids != ids_ref).any(1))[0]
    assert len(diff) <= max(1, T // 100)
    for t in diff:
        assert routing_consistent(ids[t], L64[t], bound[t])
    same = np.setdiff1d(np.arange(T), diff)
    assert np.abs(w[same] - w_ref[same]).max() <= 1e-4


# ---------------------------------------------------------------------------------------------
# dispatch
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("T,E,k,e0,E_loc,hot", [(64, 8, 2, 0, 8, 0.0), (333, 128, 8, 0, 32, 0.3),
                                                (2048, 512, 10, 64, 64, 0.0), (1, 16, 4, 12, 4, 0.0),
                                                (16384, 128, 8, 0, 32, 0.5), (3000, 256, 8, 96, 32, 0.2),
                                                (2047, 1024, 16, 0, 1024, 0.0), (50, 8, 8, 0, 8, 0.0),
                                                (3000, 72, 7, 3, 45, 0.1), (2500, 512, 8, 100, 300, 0.0),
                                                (8192, 512, 10, 64, 64, 0.0)])
def test_permute_bitexact(T, E, k, e0, E_loc, hot):
    ids_np = gen.random_topk_ids(T, E, k, seed=T + E, hot=[e0, e0 + 1], hot_frac=hot)
    H = 128
    rng = np.random.default_rng(T)
    x = gen.bf16_round(rng.standard_normal((T, H)).astype(np.float32))
    d = moe.make_desc(T, H, E, e0, E_loc, 64, k)
    ws = torch.empty(moe.moe_permute_workspace_bytes(d), dtype=torch.uint8, device="cuda")
    counts = torch.empty(E_loc, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E_loc + 1, dtype=torch.int32, device="cuda")
    s2r = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    r2f = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
    a_perm = torch.zeros((T * k, H), dtype=torch.bfloat16, device="cuda")
    moe.moe_permute(d, to_dev(ids_np, torch.int32), to_dev(x, torch.bfloat16), None, counts,
                    offsets, s2r, r2f, a_perm, None, ws)
    _sync()
    c_ref, o_ref, s_ref, r_ref = oracle.permute(ids_np, e0, E_loc)
    R = len(r_ref)
    assert np.array_equal(counts.cpu().numpy(), c_ref)
    assert np.array_equal(offsets.cpu().numpy(), o_ref)
    assert np.array_equal(s2r.cpu().numpy(), s_ref)
    r2f_g = r2f.cpu().numpy()
    assert np.array_equal(r2f_g[:R], r_ref)
    assert np.all(r2f_g[R:] == -7)                      # rows >= R untouched
    ap = a_perm.float().cpu().numpy()
    assert np.array_equal(ap[:R], x[r_ref // k])         # bytes of the gathered rows


# the quantised row copy of the dispatch: codes and scales of x (quantised in token order) moved to
# expert-contiguous rows. fp8 carries the 128x128 block scale row of each token (T not a multiple
# of 128: a partial last block), MXFP4 / MXFP8 the E8M0 row of the token. Tables up to 16384 slots
# take the one-workgroup dispatch, larger ones the split count / scan / scatter kernels. The
# permuted rows then feed the grouped GEMM (per-row scales, no gather), which must give the same
# bytes as the GEMM gathering the rows of x itself.
@pytest.mark.parametrize("fmt", ["fp8", "mx4", "mx8"])
@pytest.mark.parametrize("T,E,k,E_loc", [(333, 64, 8, 16), (2500, 128, 8, 32)])
def test_permute_quantised_rows(fmt, T, E, k, E_loc):
    from gpu_util import FMTS, oracle_quant
    dfmt, ofmt = FMTS[fmt]
    H = 512
    rng = np.random.default_rng([T, E, dfmt])
    x = gen.bf16_round(rng.standard_normal((T, H)).astype(np.float32))
    x[:, 64:128] *= 40.0                                   # distinct block / group scales
    ids_np = gen.random_topk_ids(T, E, k, seed=T, hot=[0, 1], hot_frac=0.3)
    blk = 128 if fmt == "fp8" else 1
    xq, xs = gpu_quant(dfmt, x, blk)
    xq, xs = xq[0], xs[0]
    ref_q = oracle_quant(ofmt, x, blk)
    assert np.array_equal(xq.cpu().numpy(), ref_q.q[0]) and np.array_equal(xs.cpu().numpy(), ref_q.s[0])
    d = moe.make_desc(T, H, E, 0, E_loc, 256, k, 0, 1, 1, moe.MOE_BF16, dfmt)
    ws = torch.empty(max(moe.moe_permute_workspace_bytes(d), 16), dtype=torch.uint8, device="cuda")
    counts = torch.empty(E_loc, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E_loc + 1, dtype=torch.int32, device="cuda")
    s2r = torch.empty((T, k), dtype=torch.int32, device="cuda")
    r2f = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
    rb = H // 2 if fmt == "mx4" else H
    a_perm = torch.full((T * k, rb), 0xA5, dtype=torch.uint8, device="cuda")
    if fmt == "fp8":
        a_ps = torch.full((T * k, H // 128), -3.0, dtype=torch.float32, device="cuda")
    else:
        a_ps = torch.full((T * k, H // 32), 0xA5, dtype=torch.uint8, device="cuda")
    moe.moe_permute(d, to_dev(ids_np, torch.int32), xq, xs, counts, offsets, s2r, r2f, a_perm,
                    a_ps, ws)
    _sync()
    c_ref, o_ref, s_ref, r_ref = oracle.permute(ids_np, 0, E_loc)
    R = len(r_ref)
    assert np.array_equal(offsets.cpu().numpy(), o_ref)
    assert np.array_equal(r2f.cpu().numpy()[:R], r_ref)
    tok_of_row = r_ref // k
    ap, ps = a_perm.cpu().numpy(), a_ps.cpu().numpy()
    assert np.array_equal(ap[:R], ref_q.q[0][tok_of_row])
    if fmt == "fp8":
        assert np.array_equal(ps[:R], ref_q.s[0][tok_of_row // 128])
    else:
        assert np.array_equal(ps[:R], ref_q.s[0][tok_of_row])
    assert np.all(ap[R:] == 0xA5)                           # rows past R untouched
    # the permuted rows as the GEMM input (one scale row per row) against the gathering GEMM
    N = 256
    B = (rng.standard_normal((E_loc, N, H)) * 0.05).astype(np.float32)
    bq, bs = gpu_quant(dfmt, B, 128)
    outs = []
    for gather in (False, True):
        g = moe.moe_gemm_desc(E_loc, T * k, H, N, dfmt, moe.MOE_EPI_STORE, moe.MOE_F32,
                              k if gather else 1, blk if gather else 1)
        C = torch.full((T * k, N), 1024.0, dtype=torch.float32, device="cuda")
        if gather:
            moe.moe_grouped_gemm(g, xq, xs, r2f, bq, bs, None, None, offsets, C, None)
        else:
            moe.moe_grouped_gemm(g, a_perm, a_ps, None, bq, bs, None, None, offsets, C, None)
        _sync()
        outs.append(C.cpu().numpy())
    assert np.array_equal(outs[0][:R], outs[1][:R])
    ref = oracle.grouped_gemm(o_ref, ref_q, oracle_quant(ofmt, B, 128), a_rows=r_ref, a_row_div=k)
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.abs(outs[0][:R] - ref).max() <= 2e-3 * rms


def test_permute_no_local_rows():
    T, E, k = 100, 64, 4
    ids_np = gen.random_topk_ids(T, E, k, seed=3)
    ids_np = np.where(ids_np < 8, ids_np + 8, ids_np).astype(np.int32)
    d = moe.make_desc(T, 128, E, 0, 8, 64, k)
    ws = torch.empty(moe.moe_permute_workspace_bytes(d), dtype=torch.uint8, device="cuda")
    counts = torch.full((8,), 5, dtype=torch.int32, device="cuda")
    offsets = torch.full((9,), 5, dtype=torch.int32, device="cuda")
    s2r = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    r2f = torch.zeros((T * k,), dtype=torch.int32, device="cuda")
    moe.moe_permute(d, to_dev(ids_np, torch.int32), None, None, counts, offsets, s2r, r2f, None,
                    None, ws)
    _sync()
    assert not counts.cpu().numpy().any() and not offsets.cpu().numpy().any()
    assert np.all(s2r.cpu().numpy() == -1)


# ---------------------------------------------------------------------------------------------
# grouped GEMM
# ---------------------------------------------------------------------------------------------

def _gemm_case(counts, K, N, swiglu, gather, out_f32, dtype_in="bf16", seed=0, f16s=False):
    """The grouped GEMM through the C ABI against the oracle. f16s: C in MOE_F16_SCALED rows (A's
    rows spread over eight decades, A's first row zero); returns C's bytes and also the oracle's
    sum of |a| |b| per entry (the accumulation error bound's scale)."""
    rng = np.random.default_rng([seed, K, N, len(counts)])
    G = len(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(off[-1])
    max_rows = R + 17
    f32 = dtype_in == "f32"
    rnd = (lambda a: a) if f32 else gen.bf16_round
    tdt = torch.float32 if f32 else torch.bfloat16
    if gather:
        T, kk = max(R // 3, 1), 4
        A = rnd(rng.standard_normal((T, K)).astype(np.float32))
        a_rows = rng.integers(0, T * kk, size=max_rows).astype(np.int32)
    else:
        kk = 1
        A = rnd(rng.standard_normal((max_rows, K)).astype(np.float32))
        a_rows = None
    if f16s:
        A = rnd(A * (10.0 ** rng.uniform(-4, 4, size=(A.shape[0], 1))).astype(np.float32))
        A[0] = 0.0
    B = rnd((rng.standard_normal((G, N, K)) * 0.05).astype(np.float32))
    B2 = rnd((rng.standard_normal((G, N, K)) * 0.05).astype(np.float32)) if swiglu else None
    out_dt = moe.MOE_F16_SCALED if f16s else moe.MOE_F32 if out_f32 else moe.MOE_BF16
    g = moe.moe_gemm_desc(G, max_rows, K, N, moe.MOE_F32 if f32 else moe.MOE_BF16,
                          moe.MOE_EPI_SWIGLU if swiglu else moe.MOE_EPI_STORE, out_dt, kk, 1)
    if f16s:
        C = torch.full((max_rows, moe.moe_f16_scaled_row_bytes(N)), 0xAB, dtype=torch.uint8, device="cuda")
    else:
        C = torch.full((max_rows, N), 1024.0, dtype=torch.float32 if out_f32 else torch.bfloat16,
                       device="cuda")
    moe.moe_grouped_gemm(g, to_dev(A, tdt), None, None if a_rows is None else to_dev(a_rows, torch.int32),
                         to_dev(B, tdt), None, None if B2 is None else to_dev(B2, tdt), None,
                         to_dev(off, torch.int32), C, None)
    _sync()
    M = oracle.Mat
    ref = oracle.grouped_gemm(off, M(oracle.F32, A), M(oracle.F32, B),
                              None if B2 is None else M(oracle.F32, B2), a_rows=a_rows, a_row_div=kk)
    if f16s:
        absref = oracle.grouped_gemm(off, M(oracle.F32, np.abs(A)), M(oracle.F32, np.abs(B)),
                                     a_rows=a_rows, a_row_div=kk)
        return C.cpu().numpy(), ref, R, absref
    Cg = C.float().cpu().numpy()
    return Cg, ref, R


@pytest.mark.parametrize("counts", [[0, 37, 130, 1, 9], [700, 1200, 0, 513], [150, 97, 200, 0, 101]])
@pytest.mark.parametrize("swiglu", [False, True])
@pytest.mark.parametrize("gather", [False, True])
def test_grouped_gemm_bf16(counts, swiglu, gather):
    Cg, ref, R = _gemm_case(counts, K=512, N=256, swiglu=swiglu, gather=gather, out_f32=False)
    err = np.abs(Cg[:R] - ref)
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.all(err <= 2 ** -8 * np.abs(ref) + 1e-3 * rms), err.max() / rms
    assert np.all(Cg[R:] == 1024.0)                      # rows outside every group untouched


# decode-sized groups (the weight-streaming kernel): groups of 0, 1, 63, 64 and 65 rows (a second
# 64-row tile), K of one 64-wide step, an odd number of steps (the 2-deep register ring), and a
# long K whose 65 steps are split over four waves (16, 16, 16 and 17 steps)
@pytest.mark.parametrize("K", [64, 320, 1536, 4160])
@pytest.mark.parametrize("swiglu", [False, True])
@pytest.mark.parametrize("gather", [False, True])
def test_grouped_gemm_bf16_decode_groups(K, swiglu, gather):
    counts = [5, 0, 64, 65, 1, 12, 63, 2, 0, 30]
    Cg, ref, R = _gemm_case(counts, K=K, N=192, swiglu=swiglu, gather=gather, out_f32=not swiglu)
    rms = np.sqrt(np.mean(ref ** 2))
    if swiglu:
        assert np.all(np.abs(Cg[:R] - ref) <= 2 ** -8 * np.abs(ref) + 1e-3 * rms)
    else:
        assert np.abs(Cg[:R] - ref).max() <= 1e-4 * rms * np.sqrt(K / 256)
    assert np.all(Cg[R:] == 1024.0)


@pytest.mark.parametrize("swiglu", [False, True])
@pytest.mark.parametrize("N", [320, 384])
def test_grouped_gemm_bf16_large_tiles_ragged_n(swiglu, N):
    # enough rows per group for the 256 x 256 tiles; N leaves a partial last n-tile
    Cg, ref, R = _gemm_case([1500, 300, 0, 701], K=1024, N=N, swiglu=swiglu, gather=swiglu,
                            out_f32=False)
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.all(np.abs(Cg[:R] - ref) <= 2 ** -8 * np.abs(ref) + 1e-3 * rms)
    assert np.all(Cg[R:] == 1024.0)


@pytest.mark.parametrize("counts,K,N", [([3, 70, 0, 5], 4096, 128), ([600, 40], 256, 1536),
                                        ([1500, 300, 0, 701], 1536, 4096)])
def test_grouped_gemm_bf16_f32_out(counts, K, N):
    Cg, ref, R = _gemm_case(counts, K=K, N=N, swiglu=False, gather=False, out_f32=True)
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.abs(Cg[:R] - ref).max() <= 1e-4 * rms * np.sqrt(K / 256)


# more 256 x 256 tiles (459, the last n-tile partial) than CUs: the down projection's persistent
# kernel gives each workgroup several tiles, priming each next tile's loads behind the stores
@pytest.mark.parametrize("out_f32", [False, True])
def test_grouped_gemm_bf16_persistent_tiles(out_f32):
    Cg, ref, R = _gemm_case([1500, 1300, 0, 2701, 900], K=128, N=4160, swiglu=False, gather=False,
                            out_f32=out_f32)
    rms = np.sqrt(np.mean(ref ** 2))
    if out_f32:
        assert np.abs(Cg[:R] - ref).max() <= 1e-4 * rms
    else:
        assert np.all(np.abs(Cg[:R] - ref) <= 2 ** -8 * np.abs(ref) + 1e-3 * rms)
    assert np.all(Cg[R:] == 1024.0)


# more 256 x 256 tiles than CUs, no row gather, several K lengths (2 to 48 K-steps of 32) and a
# partial last n-tile: each persistent workgroup runs several tiles, issuing a tile's first
# K-steps before the previous tile's stores and leaving those stores in flight
@pytest.mark.parametrize("K,out_f32", [(1536, True), (1536, False), (192, True), (448, False),
                                       (64, True)])
def test_grouped_gemm_bf16_many_tiles(K, out_f32):
    Cg, ref, R = _gemm_case([1500, 1300, 0, 2701, 900, 5], K=K, N=4160, swiglu=False, gather=False,
                            out_f32=out_f32, seed=K)
    rms = np.sqrt(np.mean(ref ** 2))
    if out_f32:
        assert np.abs(Cg[:R] - ref).max() <= 1e-4 * rms * np.sqrt(K / 256)
    else:
        assert np.all(np.abs(Cg[:R] - ref) <= 2 ** -8 * np.abs(ref) + 1e-3 * rms)
    assert np.all(Cg[R:] == 1024.0)


# groups of ~150-200 rows (routed rows per group 163 = max_rows / G: the ping-pong kernel's 192-row
# tiles, whose second wave group loads one A slice less per step): an empty group, a one-row
# group, one of 400 rows (three tiles, the last ragged); N = 320 leaves a partial n-tile
@pytest.mark.parametrize("swiglu,gather,out", [(False, False, "bf16"), (False, True, "f32"),
                                               (True, True, "bf16"), (True, False, "f32"),
                                               (False, False, "f16s")])
@pytest.mark.parametrize("K", [256, 1536])
def test_grouped_gemm_bf16_192_row_tiles(swiglu, gather, out, K):
    counts = [150, 0, 400, 1, 191, 180, 170, 200]
    N = 192 if swiglu else 320
    if out == "f16s":
        N = 256
        Cb, ref, R, absref = _gemm_case(counts, K=K, N=N, swiglu=False, gather=gather, out_f32=False,
                                        f16s=True, seed=192)
        vals, sc = f16s_split(Cb[:R], N)
        check_f16s_format(vals, sc)
        scale = np.repeat(sc, 64, axis=1)
        assert np.all(np.abs(vals * scale - ref) <= gamma(K) * absref + 8 * scale)
        assert np.all(Cb[R:] == 0xAB)
        return
    Cg, ref, R = _gemm_case(counts, K=K, N=N, swiglu=swiglu, gather=gather, out_f32=out == "f32",
                            seed=192)
    rms = np.sqrt(np.mean(ref ** 2))
    if out == "f32" and not swiglu:
        assert np.abs(Cg[:R] - ref).max() <= 1e-4 * rms * np.sqrt(K / 256)
    else:
        assert np.all(np.abs(Cg[:R] - ref) <= 2 ** -8 * np.abs(ref) + 1e-3 * rms)
    assert np.all(Cg[R:] == 1024.0)


# MOE_F16_SCALED output rows (the layer's y for bf16 experts) from each bf16 kernel: decode-sized
# groups (weight streaming; K = 4160 splits its steps over four waves), mid-sized groups (128 x 128
# tiles) and large ones (the persistent 256 x 256 ping-pong tiles; N = 4160 leaves an n-tile whose
# last three waves lie past N). Error bar per entry: fp32 accumulation, gamma_K * sum |a| |b|,
# plus fp16 rounding of the scaled value, at most 8 (half an fp16 ulp below 2^15) times the
# block's scale.
@pytest.mark.parametrize("counts,K,N,gather", [
    ([5, 0, 64, 65, 1, 12, 63, 2, 0, 30], 1536, 192, False),
    ([5, 0, 64, 65, 1, 12, 63, 2, 0, 30], 4160, 256, True),
    ([150, 97, 200, 0, 101], 512, 320, True),
    ([1500, 1300, 0, 2701, 900, 5], 1536, 4160, False),
    ([1500, 300, 0, 701], 128, 4096, True)])
def test_grouped_gemm_bf16_f16_scaled_out(counts, K, N, gather):
    Cb, ref, R, absref = _gemm_case(counts, K=K, N=N, swiglu=False, gather=gather, out_f32=False,
                                    f16s=True)
    vals, sc = f16s_split(Cb[:R], N)
    check_f16s_format(vals, sc)
    scale = np.repeat(sc, 64, axis=1)
    err = np.abs(vals * scale - ref)
    assert np.all(err <= gamma(K) * absref + 8 * scale), (err / (gamma(K) * absref + 8 * scale)).max()
    if not gather:
        assert np.all(vals[0] == 0) and np.all(sc[0] == 2.0 ** -15)   # A's zero row
    assert np.all(Cb[R:] == 0xAB)                         # rows outside every group untouched


def test_grouped_gemm_f16_scaled_out_rules():
    """MOE_F16_SCALED is an output of bf16 STORE GEMMs only."""
    g = moe.moe_gemm_desc(1, 64, 256, 256, moe.MOE_BF16, moe.MOE_EPI_SWIGLU, moe.MOE_F16_SCALED, 1, 1)
    a = torch.zeros((64, 256), dtype=torch.bfloat16, device="cuda")
    c = torch.zeros((64, moe.moe_f16_scaled_row_bytes(256)), dtype=torch.uint8, device="cuda")
    off = torch.tensor([0, 64], dtype=torch.int32, device="cuda")
    with pytest.raises(moe.MoeError):
        moe.moe_grouped_gemm(g, a, None, None, a, None, a, None, off, c, None)


@pytest.mark.parametrize("swiglu", [False, True])
def test_grouped_gemm_f32(swiglu):
    Cg, ref, R = _gemm_case([20, 0, 65, 7], K=256, N=128, swiglu=swiglu, gather=True, out_f32=True,
                            dtype_in="f32")
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.abs(Cg[:R] - ref).max() <= 1e-5 * rms


# The decode microbenchmark of "Hosting Qwen on Blackwell" (section "MoE GEMM"): every local
# expert activated by exactly one token. Qwen3-235B expert shape (hidden 4096, intermediate 1536,
# top-8 of 128), E_loc / 8 tokens with token t routed to local experts 8t .. 8t+7, run through the
# public steps (dispatch maps, gate/up GEMM gathering x, down GEMM, combine) and compared with the
# oracle's dense per-token loop over the chosen experts (h rounded to bf16, as the layer does).
@pytest.mark.parametrize("E_loc", [8, 16, 32, 64])
def test_one_token_per_expert_decode(E_loc):
    H, I, E, k = 4096, 1536, 128, 8
    T = E_loc // k
    rng = np.random.default_rng(E_loc)
    x = gen.bf16_round(rng.standard_normal((T, H)).astype(np.float32))
    wg, wu = (gen.bf16_round((rng.standard_normal((E_loc, I, H)) * 0.02).astype(np.float32))
              for _ in range(2))
    wd = gen.bf16_round((rng.standard_normal((E_loc, H, I)) * 0.02).astype(np.float32))
    ids_np = (np.arange(T)[:, None] * k + np.arange(k)[None, :]).astype(np.int32)
    w_np = rng.random((T, k)).astype(np.float32) + 0.1
    w_np /= w_np.sum(1, keepdims=True)
    d = moe.make_desc(T, H, E, 0, E_loc, I, k)
    ws = torch.empty(max(moe.moe_permute_workspace_bytes(d), 16), dtype=torch.uint8, device="cuda")
    counts = torch.empty(E_loc, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E_loc + 1, dtype=torch.int32, device="cuda")
    s2r = torch.empty((T, k), dtype=torch.int32, device="cuda")
    r2f = torch.empty(T * k, dtype=torch.int32, device="cuda")
    moe.moe_permute(d, to_dev(ids_np, torch.int32), None, None, counts, offsets, s2r, r2f, None,
                    None, ws)
    h = torch.empty((T * k, I), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((T * k, H), dtype=torch.float32, device="cuda")
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    g_up = moe.moe_gemm_desc(E_loc, T * k, H, I, moe.MOE_BF16, moe.MOE_EPI_SWIGLU, moe.MOE_BF16, k, 1)
    g_dn = moe.moe_gemm_desc(E_loc, T * k, I, H, moe.MOE_BF16, moe.MOE_EPI_STORE, moe.MOE_F32, 1, 1)
    moe.moe_grouped_gemm(g_up, to_dev(x, torch.bfloat16), None, r2f, to_dev(wg, torch.bfloat16),
                         None, to_dev(wu, torch.bfloat16), None, offsets, h, None)
    moe.moe_grouped_gemm(g_dn, h, None, None, to_dev(wd, torch.bfloat16), None, None, None, offsets,
                         y, None)
    moe.moe_combine(d, moe.MOE_F32, y, to_dev(w_np, torch.float32), s2r, None, out)
    _sync()
    c_ref, off_ref, s2r_ref, r2f_ref = oracle.permute(ids_np, 0, E_loc)
    assert np.array_equal(counts.cpu().numpy(), np.ones(E_loc, np.int32))
    assert np.array_equal(offsets.cpu().numpy(), off_ref)
    assert np.array_equal(s2r.cpu().numpy(), s2r_ref)
    assert np.array_equal(r2f.cpu().numpy()[:E_loc], r2f_ref)
    M = oracle.Mat
    ref = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            e = ids_np[t, j]
            ref[t] += np.float64(w_np[t, j]) * oracle.ffn_row(
                x[t], M(oracle.F32, wg[e]), M(oracle.F32, wu[e]), M(oracle.F32, wd[e]),
                act_fmt=oracle.BF16)
    err, rms = rel_err(out.cpu().numpy(), ref)
    # the bar of bf16 layers; in fact only fp32 accumulation (and a rare bf16 rounding of h that
    # the fp32 and fp64 sums put on different sides of a rounding boundary) differs here
    assert err <= 2e-2, err
    assert err <= 2e-3, err


# ---------------------------------------------------------------------------------------------
# combine
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("T,k,H,shared,io,out_bf16,gated", [(64, 2, 256, False, "f32", False, False),
                                                            (300, 8, 4096, False, "bf16", False, False),
                                                            (77, 10, 1024, True, "bf16", True, False),
                                                            (5, 16, 7168, True, "f32", True, False),
                                                            (77, 10, 1024, True, "bf16", False, True),
                                                            (33, 8, 7168, True, "f32", True, True),
                                                            (300, 8, 4096, True, "f16s", True, True),
                                                            (64, 2, 256, False, "f16s", False, False),
                                                            (5, 16, 7168, True, "f16s", False, False)])
def test_combine(T, k, H, shared, io, out_bf16, gated):
    rng = np.random.default_rng(T * k)
    R = T * k

    def rows(n):
        """n rows of y in the test's format: (values, device tensor)"""
        if io == "f16s":                                  # fp16 values, scales over 2^-30 .. 2^-2
            v16 = rng.uniform(-2.0 ** 15, 2.0 ** 15, size=(n, H)).astype(np.float16)
            sc = 2.0 ** rng.integers(-30, -1, size=(n, H // 64))
            vals = (v16.astype(np.float64) * np.repeat(sc, 64, axis=1)).astype(np.float32)
            return vals, to_dev(f16s_pack(v16, sc), torch.uint8)
        v = rng.standard_normal((n, H)).astype(np.float32)
        if io == "f32":
            return v, to_dev(v, torch.float32)
        v = gen.bf16_round(v)
        return v, to_dev(v, torch.bfloat16)

    y, y_dev = rows(R)
    w = rng.random((T, k)).astype(np.float32)
    s2r = rng.permutation(R).reshape(T, k).astype(np.int32)
    s2r[rng.random((T, k)) < 0.3] = -1
    s2r[0, :] = -1                                        # a token with no local expert
    sh, sh_dev = rows(T) if shared else (None, None)
    sw = rng.random(T).astype(np.float32) if gated else None
    ydt = {"f32": moe.MOE_F32, "bf16": moe.MOE_BF16, "f16s": moe.MOE_F16_SCALED}[io]
    iodt = moe.MOE_F32 if io == "f32" else moe.MOE_BF16
    d = moe.make_desc(T, H, 64, 0, 8, 64, k, 0, 0, 1, iodt, iodt,
                      out_dtype=moe.MOE_BF16 if out_bf16 else moe.MOE_F32)
    out = torch.empty((T, H), dtype=torch.bfloat16 if out_bf16 else torch.float32, device="cuda")
    moe.moe_combine(d, ydt, y_dev, to_dev(w, torch.float32), to_dev(s2r, torch.int32), sh_dev, out,
                    shared_w=None if sw is None else to_dev(sw, torch.float32))
    _sync()
    ref = oracle.combine(y, w, s2r, sh, sw)
    og = out.float().cpu().numpy()
    rms = np.sqrt(np.mean(ref ** 2))
    if not out_bf16:
        assert np.abs(og - ref).max() <= 1e-5 * rms
    else:
        assert np.all(np.abs(og - ref) <= 2 ** -8 * np.abs(ref) + 1e-5 * rms)
    if not shared:
        assert not og[0].any()


# shared-expert gate: bf16 and fp32 tokens, hidden sizes of the workloads and a ragged one (H not a
# multiple of the 512 columns a wave covers per step), 1 to 4099 tokens (a partial last workgroup)
@pytest.mark.parametrize("T,H,io", [(1, 4096, "bf16"), (5, 7168, "bf16"), (4099, 4096, "bf16"),
                                    (3, 4160, "bf16"), (130, 272, "f32"), (7, 7168, "f32")])
def test_shared_gate(T, H, io):
    rng = np.random.default_rng([T, H])
    rnd = (lambda a: a) if io == "f32" else gen.bf16_round
    tdt = torch.float32 if io == "f32" else torch.bfloat16
    x = rnd(rng.standard_normal((T, H)).astype(np.float32))
    wg = rnd((rng.standard_normal(H) * 0.02).astype(np.float32))
    d = moe.make_desc(T, H, 64, 0, 8, 64, 2, 64, 0, 1, moe.MOE_F32 if io == "f32" else moe.MOE_BF16)
    g = torch.full((T,), -1.0, dtype=torch.float32, device="cuda")
    moe.moe_shared_gate(d, to_dev(x, tdt), to_dev(wg, tdt), g)
    _sync()
    ref = oracle.shared_gate(x, wg)
    # fp32 accumulation of H products (bounded by gamma_H * sum |x w|), then the logistic
    # function, whose slope is at most 1/4, plus a few ulps of the fp32 exponential and division
    absdot = np.abs(x.astype(np.float64)) @ np.abs(wg.astype(np.float64))
    bound = 0.25 * gamma(H) * absdot + 4e-7
    assert np.all(np.abs(g.cpu().numpy() - ref) <= bound)
