"""Block-scaled fp8 (e4m3, 128x128 fp32 scales), MXFP4 (e2m1 + E8M0 per 32) and MXFP8 (e4m3 + E8M0
per 32) grouped GEMMs against the oracle. Each side quantises the same float32 inputs with its own quantiser (the codes
are checked equal in test_gpu_steps); the GPU GEMM runs on its own codes, the oracle dequantises
its own."""
import numpy as np
import pytest
import torch

import moe_layer_softmax_amd as moe
import oracle
from moe_inputs import gen

from gpu_util import FMTS, decode, gamma, gpu_quant, oracle_quant, to_dev

pytestmark = pytest.mark.gpu

@pytest.mark.parametrize("fmt", ["fp8", "mx4", "mx8"])
@pytest.mark.parametrize("epi", ["store_f32", "store_bf16", "swiglu_bf16", "swiglu_q"])
@pytest.mark.parametrize("counts", [[0, 37, 130, 1, 9], [300, 140, 0, 513]])
def test_grouped_gemm_quant(fmt, epi, counts):
    _quant_case(fmt, epi, counts, 512)


# decode-sized groups (the weight-streaming kernel): empty groups, groups of 1-33 rows and one of
# 40 (a second 32-row tile), and an odd number of 128-byte K-pairs per row
@pytest.mark.parametrize("fmt", ["fp8", "mx4", "mx8"])
@pytest.mark.parametrize("epi", ["store_f32", "store_bf16", "swiglu_bf16", "swiglu_q"])
def test_grouped_gemm_quant_decode(fmt, epi):
    _quant_case(fmt, epi, [3, 0, 17, 40, 1, 8, 33, 2], 768 if fmt == "mx4" else 640)


# prefill-sized groups (256 rows or more per group on average): the 256 x 256 tiles of the MX formats
# (fp8 keeps the 128-row tiles), with an empty group, a one-row group, ragged last m-tiles and, for
# the stores, a partial last 256-column tile; 2 to 12 K-steps
@pytest.mark.parametrize("fmt", ["fp8", "mx4", "mx8"])
@pytest.mark.parametrize("epi", ["store_f32", "store_bf16", "swiglu_bf16", "swiglu_q"])
@pytest.mark.parametrize("K", [512, 1536])
def test_grouped_gemm_quant_prefill_groups(fmt, epi, K):
    _quant_case(fmt, epi, [700, 0, 1, 513, 300], K)


# decode-sized groups with fewer 128-byte K-pairs than the streaming kernel's four K-split waves
# (K = 256: two of the four waves get no K-pair and contribute zeros)
@pytest.mark.parametrize("fmt", ["fp8", "mx8"])
@pytest.mark.parametrize("epi", ["store_f32", "store_bf16", "swiglu_bf16", "swiglu_q"])
def test_grouped_gemm_quant_decode_short_k(fmt, epi):
    _quant_case(fmt, epi, [5, 0, 31, 2], 256)


# narrow and short shapes: 128 h-columns (fewer than one 256-row B tile of gate + up) on the wide
# MX tiles (one group of 700 rows), the 128-row tiles (groups of ~175) and the streaming kernel;
# stores with one and two K-steps on the 128-row tiles
@pytest.mark.parametrize("fmt", ["fp8", "mx4", "mx8"])
@pytest.mark.parametrize("epi,counts,K,N", [("swiglu_q", [700], 512, 128),
                                            ("swiglu_bf16", [700], 512, 128),
                                            ("swiglu_q", [175, 170, 180, 176], 512, 128),
                                            ("swiglu_q", [5, 30, 1], 512, 128),
                                            ("store_bf16", [700], 128, 512),
                                            ("store_bf16", [175, 170, 180, 176], 256, 512),
                                            ("store_f32", [700], 128, 512)])
def test_grouped_gemm_quant_narrow_shapes(fmt, epi, counts, K, N):
    if fmt == "mx4" and K % 256:
        pytest.skip("MXFP4 K-steps are 256 elements")
    _quant_case(fmt, epi, counts, K, N)


def _quant_case(fmt, epi, counts, K, N=None):
    dfmt, ofmt = FMTS[fmt]
    rng = np.random.default_rng([len(counts), sum(counts)])
    swiglu = epi.startswith("swiglu")
    if N is None:
        N = 256 if swiglu else 384             # 384: a partial 256-column tile
    G = len(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(off[-1])
    max_rows = R + 9
    T, kk = max(R // 3, 5), 4
    x = gen.bf16_round(rng.standard_normal((T, K)).astype(np.float32))
    a_rows = rng.integers(0, T * kk, size=max_rows).astype(np.int32)
    B = (rng.standard_normal((G, N, K)) * 0.05).astype(np.float32)
    B2 = (rng.standard_normal((G, N, K)) * 0.05).astype(np.float32)
    a_block = 128 if fmt == "fp8" else 1
    xq, xs = gpu_quant(dfmt, x, a_block)
    bq, bs = gpu_quant(dfmt, B, 128)
    b2q, b2s = gpu_quant(dfmt, B2, 128)
    out_dt = {"store_f32": moe.MOE_F32, "store_bf16": moe.MOE_BF16, "swiglu_bf16": moe.MOE_BF16,
              "swiglu_q": dfmt}[epi]
    g = moe.moe_gemm_desc(G, max_rows, K, N, dfmt, moe.MOE_EPI_SWIGLU if swiglu else moe.MOE_EPI_STORE,
                          out_dt, kk, a_block)
    C_scales = None
    if epi == "swiglu_q":
        C = torch.zeros((max_rows, N // 2 if fmt == "mx4" else N), dtype=torch.uint8, device="cuda")
        C_scales = torch.zeros((max_rows, N // 128) if fmt == "fp8" else (max_rows, N // 32),
                               dtype=torch.float32 if fmt == "fp8" else torch.uint8, device="cuda")
    else:
        C = torch.full((max_rows, N), 1024.0,
                       dtype=torch.float32 if out_dt == moe.MOE_F32 else torch.bfloat16, device="cuda")
    moe.moe_grouped_gemm(g, xq[0], xs[0], to_dev(a_rows, torch.int32), bq, bs,
                         b2q if swiglu else None, b2s if swiglu else None,
                         to_dev(off, torch.int32), C, C_scales)
    torch.cuda.synchronize()
    A = oracle_quant(ofmt, x, a_block)
    ref = oracle.grouped_gemm(off, A, oracle_quant(ofmt, B, 128),
                              oracle_quant(ofmt, B2, 128) if swiglu else None,
                              a_rows=a_rows, a_row_div=kk)
    rms = np.sqrt(np.mean(ref ** 2)) if R else 1.0
    if epi == "swiglu_q":
        h = decode(dfmt, C[:R], C_scales[:R], N)
        # h itself comes from fp32 accumulations: |dg|, |du| <= gamma_K sum|a b| (the bound used
        # for the router logits), so |dh| <= |silu'(g)| |dg| |u| + |silu(g)| |du| with |silu'| < 1.1;
        # a code is then within the quantisation bounds below of the fp32 h, not of the exact one
        Ad = np.abs(A.dequant()[0])
        g_ref = oracle.grouped_gemm(off, A, oracle_quant(ofmt, B, 128), None, a_rows=a_rows, a_row_div=kk)
        u_ref = oracle.grouped_gemm(off, A, oracle_quant(ofmt, B2, 128), None, a_rows=a_rows, a_row_div=kk)
        Bd, B2d = np.abs(oracle_quant(ofmt, B, 128).dequant()), np.abs(oracle_quant(ofmt, B2, 128).dequant())
        dg = np.zeros_like(ref)
        du = np.zeros_like(ref)
        for gi in range(G):
            rows = slice(int(off[gi]), int(off[gi + 1]))
            Ar = Ad[a_rows[rows] // kk]
            dg[rows] = gamma(K) * (Ar @ Bd[gi].T)
            du[rows] = gamma(K) * (Ar @ B2d[gi].T)
        silu = g_ref / (1.0 + np.exp(-g_ref))
        dh = 1.1 * dg * np.abs(u_ref) + np.abs(silu) * du
        ref_abs = np.abs(ref) + dh
        if fmt == "fp8":
            # within one e4m3 step of the block's scale grid (fp32 vs fp64 h may round differently)
            s = np.repeat(C_scales[:R].cpu().numpy().astype(np.float64), 128, axis=1)
            assert np.all(np.abs(h - ref) <= 2.0 ** -3 * ref_abs + s * 2.0 ** -8 + dh)
        elif fmt == "mx8":
            # within one e4m3 step (relative 2^-3, saturation above 448 * 2^e included) or one
            # subnormal step 2^(e-9) of the group's scale
            unit = np.repeat(2.0 ** (C_scales[:R].cpu().numpy().astype(np.int64) - 127), 32, axis=1)
            assert np.all(np.abs(h - ref) <= 2.0 ** -3 * ref_abs + unit * 2.0 ** -8 + dh)
        else:
            unit = np.repeat(2.0 ** (C_scales[:R].cpu().numpy().astype(np.int64) - 127), 32, axis=1)
            assert np.all(np.abs(h - ref) <= 2.0 * unit + dh + 1e-30)
    else:
        Cg = C.float().cpu().numpy()
        err = np.abs(Cg[:R] - ref)
        if out_dt == moe.MOE_F32:
            # fp32 accumulation bound gamma_K * sum|a b| with u = 2^-23 is ~1e-3 rms at K = 512
            assert err.max() <= 2e-3 * rms, err.max() / rms
        else:
            assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-3 * rms), err.max() / rms
        assert np.all(Cg[R:] == 1024.0)
