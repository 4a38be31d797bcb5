"""Grouped GEMMs at the workloads' full shapes (gate/up with K = H = 4096 / 7168 and the SwiGLU
epilogue, down with K = I and N = H), for every expert format, with prefill-sized groups (the tile
kernels) and decode-sized groups (the weight-streaming kernels). The GPU computes every row; the
oracle computes a sample of rows (every group's first and last rows plus random ones): a row of
C depends only on its A row and its group's weights, so the oracle runs on the sampled rows as a
grouped GEMM of its own."""
import numpy as np
import pytest
import torch

import moe_layer_softmax_amd as moe
import oracle

from gpu_util import FMTS, gpu_quant, nv4_block_values, nv4_split, oracle_quant, to_dev

pytestmark = pytest.mark.gpu

PREFILL = {"bf16": [3000, 1500, 0, 700, 257], "fp8": [900, 300, 0, 2100], "mx4": [2000, 0, 900],
           "mx8": [3000, 700], "nv4": [2000, 0, 900]}
DECODE = [3, 17, 0, 40, 1]
SHAPE = {"bf16": (4096, 1536), "mx8": (4096, 1536), "fp8": (7168, 2048), "mx4": (7168, 2048),
         "nv4": (7168, 2048)}     # (H, I) of the workload the format runs in


def _sample_rows(off, rng, n_rand=64):
    rows = set()
    for g in range(len(off) - 1):
        a, b = int(off[g]), int(off[g + 1])
        rows.update(r for r in (a, a + 1, b - 2, b - 1) if a <= r < b)
    R = int(off[-1])
    rows.update(int(r) for r in rng.choice(R, min(n_rand, R), replace=False))
    return np.array(sorted(rows), np.int64)


def _case(fmt, proj, counts):
    H, I = SHAPE[fmt]
    swiglu = proj == "gate_up"
    K, N = (H, I) if swiglu else (I, H)
    rng = np.random.default_rng([len(counts), sum(counts), K, N])
    G = len(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(off[-1])
    max_rows = R + 5
    kk = 8
    T = max(R // 3, 8)
    x = rng.standard_normal((T, K)).astype(np.float32)
    a_rows = rng.integers(0, T * kk, size=max_rows).astype(np.int32)
    B = (rng.standard_normal((G, N, K)) * 0.02).astype(np.float32)
    B2 = (rng.standard_normal((G, N, K)) * 0.02).astype(np.float32) if swiglu else None
    print(f"[full-shape gemm] fmt={fmt} proj={proj} counts={counts} K={K} N={N}", flush=True)
    out_dt = moe.MOE_BF16
    epi = moe.MOE_EPI_SWIGLU if swiglu else moe.MOE_EPI_STORE
    if fmt == "bf16":
        xb = torch.from_numpy(x).to(torch.bfloat16)
        Bb = torch.from_numpy(B).to(torch.bfloat16)
        B2b = None if B2 is None else torch.from_numpy(B2).to(torch.bfloat16)
        A_dev, A_sc, bq, bs, b2q, b2s = xb.cuda(), None, Bb.cuda(), None, None if B2b is None else B2b.cuda(), None
        A_or = oracle.Mat(oracle.F32, xb.float().numpy())
        B_or = oracle.Mat(oracle.F32, Bb.float().numpy())
        B2_or = None if B2b is None else oracle.Mat(oracle.F32, B2b.float().numpy())
        dt, a_block = moe.MOE_BF16, 1
        if not swiglu:
            out_dt = moe.MOE_F32
    else:
        dt, ofmt = FMTS[fmt]
        a_block = 128 if fmt == "fp8" else 1
        bq, bs = gpu_quant(dt, B, 128)
        b2q, b2s = (None, None) if B2 is None else gpu_quant(dt, B2, 128)
        B_or = oracle_quant(ofmt, B, 128)
        B2_or = None if B2 is None else oracle_quant(ofmt, B2, 128)
        A_or = oracle_quant(ofmt, x, a_block)
        if fmt == "nv4":
            xq, xsc = gpu_quant(dt, x, 1)
            xb_, xr = nv4_split(xsc, T, K)
            A_dev = to_dev(nv4_block_values(xq[0], xb_[0]).astype(np.float32), torch.bfloat16)
            A_sc = to_dev(xr[0], torch.float32)
        else:
            xq, xsc = gpu_quant(dt, x, a_block)
            A_dev, A_sc = xq[0], xsc[0]
    g = moe.moe_gemm_desc(G, max_rows, K, N, dt, epi, out_dt, kk, a_block)
    C = torch.full((max_rows, N), 1024.0, dtype=torch.float32 if out_dt == moe.MOE_F32 else torch.bfloat16,
                   device="cuda")
    moe.moe_grouped_gemm(g, A_dev, A_sc, to_dev(a_rows, torch.int32), bq, bs, b2q, b2s,
                         to_dev(off, torch.int32), C, None)
    torch.cuda.synchronize()
    Cg = C.float().cpu().numpy()
    assert np.all(Cg[R:] == 1024.0)
    # the oracle on the sampled rows: per group, the sampled rows in order
    S = _sample_rows(off, rng)
    grp = np.searchsorted(off, S, side="right") - 1
    sub_off = np.concatenate([[0], np.cumsum(np.bincount(grp, minlength=G))]).astype(np.int32)
    ref = oracle.grouped_gemm(sub_off, A_or, B_or, B2_or, a_rows=a_rows[S], a_row_div=kk)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = np.abs(Cg[S] - ref)
    if out_dt == moe.MOE_F32:
        assert err.max() <= 2e-3 * rms, err.max() / rms
    else:
        assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 2e-3 * rms), err.max() / rms


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mx4", "mx8", "nv4"])
@pytest.mark.parametrize("proj", ["gate_up", "down"])
def test_grouped_gemm_full_shape_prefill_groups(fmt, proj):
    _case(fmt, proj, PREFILL[fmt])


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mx4", "mx8", "nv4"])
@pytest.mark.parametrize("proj", ["gate_up", "down"])
def test_grouped_gemm_full_shape_decode_groups(fmt, proj):
    _case(fmt, proj, DECODE)
