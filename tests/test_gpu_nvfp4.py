"""NVFP4 (e2m1 + e4m3 scale per 16 along K + fp32 row scale) through the C ABI against the oracle:
the quantiser bit for bit, the dispatch copy (which dequantises to the bf16 block values) bit for
bit, and the grouped GEMM on both kernels (weight streaming for decode-sized groups, LDS tiles for
larger ones) within the fp32-accumulation bar of the other formats."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import moe_layer_softmax_amd as moe
import oracle

from gpu_util import E2M1, gpu_quant, nv4_block_values, nv4_split, oracle_quant, to_dev

pytestmark = pytest.mark.gpu


def _edge_rows(rng, cols):
    """Rows whose row scale is a power of two (g = 2^-k: the row holds 2688 * 2^-k), with blocks
    of every kind: e4m3-grid block scales with elements on the e2m1 grid and on its midpoints (exact
    ties of v / d), a zero block with signed zeros, a block far below the row maximum (a zero or
    subnormal block scale), and values just around the ties."""
    e4 = np.array([oracle.e4m3_value(c) for c in range(1, 0x7F)])
    mid = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    rows = []
    for k in (0, 3, 9):
        g = 2.0 ** -k
        for r in range(4):
            v = np.zeros(cols)
            for b in range(cols // 16):
                kind = (b + r) % 5
                blk = v[b * 16:(b + 1) * 16]
                if kind == 0:                           # the row maximum's block
                    blk[:] = rng.choice(E2M1, 16) * 448 * g
                    blk[0] = 6 * 448 * g
                elif kind == 1:                         # grid scale, ties
                    s = rng.choice(e4)
                    blk[:] = rng.choice(mid, 16) * rng.choice([-1, 1], 16) * s * g
                    blk[1] = 6 * s * g
                elif kind == 2:
                    blk[:] = 0.0
                    blk[::3] = -0.0
                elif kind == 3:                         # tiny block
                    blk[:] = rng.standard_normal(16) * 1e-7 * g
                else:                                   # near ties
                    s = rng.choice(e4)
                    blk[:] = rng.choice(mid, 16) * s * g * (1 + rng.choice([-1, 1], 16) * 2.0 ** -20)
                    blk[2] = 6 * s * g
            rows.append(v)
    return np.array(rows, np.float32)


@pytest.mark.parametrize("src", ["f32", "bf16"])
def test_quantize_nv4_bitexact(src):
    rng = np.random.default_rng(51)
    cols = 320
    a = (rng.standard_normal((3, 40, cols)) * 10.0 ** rng.uniform(-4, 3, size=(3, 40, 1))).astype(np.float32)
    a[0, 5] = 0.0                                       # an all-zero row: g = 1, zero codes
    a[1, :12] = _edge_rows(rng, cols)
    if src == "bf16":
        a = torch.from_numpy(a).to(torch.bfloat16).float().numpy()
    G, R, C = a.shape
    dev = to_dev(a, torch.float32 if src == "f32" else torch.bfloat16)
    codes = torch.empty((G, R, C // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((G, R * (C // 16) + 4 * R), dtype=torch.uint8, device="cuda")
    moe.moe_quantize(moe.MOE_NVFP4, moe.MOE_F32 if src == "f32" else moe.MOE_BF16, G, R, C, 1, dev,
                     codes, scales)
    torch.cuda.synchronize()
    bs, rs = nv4_split(scales, R, C)
    for g in range(G):
        p, b, r = oracle.quant_nv4(a[g])
        assert np.array_equal(rs[g].view(np.uint32), r.view(np.uint32)), g
        assert np.array_equal(bs[g], b), g
        assert np.array_equal(codes[g].cpu().numpy(), p), g


def test_quantize_nv4_rejects_bad_shapes():
    x = torch.zeros((4, 96), dtype=torch.float32, device="cuda")
    c = torch.zeros((4, 48), dtype=torch.uint8, device="cuda")
    s = torch.zeros(4 * 6 + 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(moe.MoeError):
        moe.moe_quantize(moe.MOE_NVFP4, moe.MOE_F32, 1, 4, 96, 1, x, c, s)   # cols % 64 != 0


@pytest.mark.parametrize("T,E,k,e0,E_loc", [(37, 16, 4, 4, 8), (300, 8, 2, 0, 8)])
def test_permute_nv4_dequantises_rows(T, E, k, e0, E_loc):
    """The dispatch copy of NVFP4 rows writes each routed row's block values q * s as bf16 (exact)
    and its row scale; rows past R stay untouched."""
    rng = np.random.default_rng([T, E])
    H = 448
    x = (rng.standard_normal((T, H)) * 3).astype(np.float32)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    desc = moe.make_desc(T, H, E, e0, E_loc, 256, k, 0, mi.SOFTMAX, 1, moe.MOE_BF16, moe.MOE_NVFP4)
    codes, scales = gpu_quant(moe.MOE_NVFP4, x, 1)
    counts = torch.empty(E_loc, dtype=torch.int32, device="cuda")
    offs = torch.empty(E_loc + 1, dtype=torch.int32, device="cuda")
    s2r = torch.empty((T, k), dtype=torch.int32, device="cuda")
    r2f = torch.empty(T * k, dtype=torch.int32, device="cuda")
    a_perm = torch.full((T * k, H), -7.0, dtype=torch.bfloat16, device="cuda")
    a_sc = torch.full((T * k,), -7.0, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(moe.moe_permute_workspace_bytes(desc), 16), dtype=torch.uint8, device="cuda")
    moe.moe_permute(desc, to_dev(ids, torch.int32), codes[0], scales[0], counts, offs, s2r, r2f,
                    a_perm, a_sc, ws)
    torch.cuda.synchronize()
    c_ref, o_ref, s_ref, r_ref = oracle.permute(ids, e0, E_loc)
    R = int(o_ref[-1])
    assert np.array_equal(offs.cpu().numpy(), o_ref) and np.array_equal(r2f[:R].cpu().numpy(), r_ref)
    p, b, r = oracle.quant_nv4(x)
    vals = nv4_block_values(p, b)                        # the oracle's codes decoded in numpy
    ap = a_perm.float().cpu().numpy().astype(np.float64)
    src = r_ref // k
    assert np.array_equal(ap[:R], vals[src])
    assert np.array_equal(a_sc[:R].cpu().numpy(), r[src])
    assert np.all(ap[R:] == -7.0) and np.all(a_sc[R:].cpu().numpy() == -7.0)


def _nv4_case(epi, counts, K, N, with_a_scales=True, seed=0):
    rng = np.random.default_rng([seed, len(counts), sum(counts), K])
    swiglu = epi.startswith("swiglu")
    G = len(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(off[-1])
    max_rows = R + 9
    T, kk = max(R // 3, 5), 4
    x = (rng.standard_normal((T, K)) * 10.0 ** rng.uniform(-1, 1, size=(T, 1))).astype(np.float32)
    a_rows = rng.integers(0, T * kk, size=max_rows).astype(np.int32)
    B = (rng.standard_normal((G, N, K)) * 0.05).astype(np.float32)
    B2 = (rng.standard_normal((G, N, K)) * 0.05).astype(np.float32)
    # GPU side: weights by moe_quantize; activations as the bf16 block values of the GPU's own
    # codes (decoded in numpy) with their row scales, or (down-projection style) a plain bf16 A
    bq, bs = gpu_quant(moe.MOE_NVFP4, B, 1)
    b2q, b2s = gpu_quant(moe.MOE_NVFP4, B2, 1)
    if with_a_scales:
        xq, xsc = gpu_quant(moe.MOE_NVFP4, x, 1)
        xb, xr = nv4_split(xsc, T, K)
        a_vals = nv4_block_values(xq[0], xb[0])
        A_dev = to_dev(a_vals.astype(np.float32), torch.bfloat16)
        A_sc = to_dev(xr[0], torch.float32)
        A_or = oracle_quant(oracle.NV4, x, 1)
    else:
        xbf = torch.from_numpy(x).to(torch.bfloat16)
        A_dev = xbf.cuda()
        A_sc = None
        A_or = oracle.Mat(oracle.F32, xbf.float().numpy())
    out_dt = moe.MOE_F32 if epi.endswith("f32") else moe.MOE_BF16
    g = moe.moe_gemm_desc(G, max_rows, K, N, moe.MOE_NVFP4,
                          moe.MOE_EPI_SWIGLU if swiglu else moe.MOE_EPI_STORE, out_dt, kk, 1)
    C = torch.full((max_rows, N), 1024.0, dtype=torch.float32 if out_dt == moe.MOE_F32 else torch.bfloat16,
                   device="cuda")
    print(f"[nv4 gemm] epi={epi} counts={counts} K={K} N={N} a_scales={with_a_scales}", flush=True)
    moe.moe_grouped_gemm(g, A_dev, A_sc, to_dev(a_rows, torch.int32), bq, bs,
                         b2q if swiglu else None, b2s if swiglu else None,
                         to_dev(off, torch.int32), C, None)
    torch.cuda.synchronize()
    ref = oracle.grouped_gemm(off, A_or, oracle_quant(oracle.NV4, B, 1),
                              oracle_quant(oracle.NV4, B2, 1) if swiglu else None,
                              a_rows=a_rows, a_row_div=kk)
    rms = np.sqrt(np.mean(ref ** 2)) if R else 1.0
    Cg = C.float().cpu().numpy()
    err = np.abs(Cg[:R] - ref)
    if out_dt == moe.MOE_F32 and not swiglu:
        # fp32 accumulation of exact products: gamma_K * sum|a b| is ~1e-3 rms at these K
        assert err.max() <= 2e-3 * rms, err.max() / rms
    else:
        assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 2e-3 * rms), err.max() / rms
    assert np.all(Cg[R:] == 1024.0)


# decode-sized groups (the streaming kernel): empty groups, 1..33 rows, one group of 40 (three
# 16-row tiles); K of 3 and 17 chunks (one wave per workgroup / K split over four waves)
@pytest.mark.parametrize("epi", ["store_f32", "store_bf16", "swiglu_bf16", "swiglu_f32"])
@pytest.mark.parametrize("K", [768, 4352])
def test_grouped_gemm_nv4_decode(epi, K):
    _nv4_case(epi, [3, 0, 17, 40, 1, 8, 33, 2], K, 256)


# prefill-sized groups (the tile kernel): an empty group, a one-row group and ragged m-tiles;
# 4 and 24 K-steps; a partial last 128-column tile for the stores (N = 384)
@pytest.mark.parametrize("epi", ["store_f32", "store_bf16", "swiglu_bf16", "swiglu_f32"])
@pytest.mark.parametrize("K", [256, 1536])
def test_grouped_gemm_nv4_prefill(epi, K):
    _nv4_case(epi, [700, 0, 1, 513, 300], K, 384 if epi.startswith("store") else 256)


# the down projection's form: A a plain bf16 tensor without row scales
@pytest.mark.parametrize("counts", [[5, 0, 31, 2], [200, 90, 0, 313]])
def test_grouped_gemm_nv4_without_a_scales(counts):
    _nv4_case("store_bf16", counts, 512, 256, with_a_scales=False)


# groups of 33-255 rows on average (the 128 x 128 tiles): ragged groups, an empty one, one of 300
@pytest.mark.parametrize("epi", ["store_bf16", "swiglu_bf16"])
def test_grouped_gemm_nv4_mid_groups(epi):
    _nv4_case(epi, [100, 150, 0, 60, 300, 7], 512, 384 if epi.startswith("store") else 256)
