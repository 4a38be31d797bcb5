"""The whole layer (moe_layer through the C ABI) against the oracle on the workloads, at full size
(sampled tokens where the oracle cannot do all of them in seconds), plus edge cases."""
import json
import os
from dataclasses import replace

import numpy as np
import pytest
import torch

import moe_inputs as mi
import moe_layer_softmax_amd as moe
import oracle
from moe_inputs import gen

from gpu_util import (gamma, gpu_quant, h_flip_allowance, io_torch, oracle_quant, rel_err,
                      routing_consistent, to_dev, tol_for, topk_numpy)

pytestmark = pytest.mark.gpu

_FMT = {mi.FMT_F32: moe.MOE_F32, mi.FMT_BF16: moe.MOE_BF16, mi.FMT_FP8: moe.MOE_FP8_E4M3,
        mi.FMT_MX4: moe.MOE_MXFP4, mi.FMT_MX8: moe.MOE_MXFP8, mi.FMT_NV4: moe.MOE_NVFP4}
_QUANT = (mi.FMT_FP8, mi.FMT_MX4, mi.FMT_MX8, mi.FMT_NV4)
_H_QUANT = (mi.FMT_FP8, mi.FMT_MX4, mi.FMT_MX8)      # h re-quantised to the expert format


def make_inputs(wl, bias_override=None):
    x, wr = gen.tokens(wl), gen.router_weight(wl)
    bias = gen.router_bias(wl) if bias_override is None else bias_override
    g, u, d = gen.expert_weights(wl)
    sh = gen.shared_weights(wl)
    return x, wr, bias, (g, u, d), sh


def gpu_layer(wl, x, wr, bias, experts, sh, sgate=None):
    dt = io_torch(wl.io_fmt)
    desc = moe.make_desc(wl.T, wl.H, wl.E, wl.e0, wl.E_loc, wl.I, wl.k, wl.I_s, wl.scoring,
                         wl.renormalize, _FMT[wl.io_fmt], _FMT[wl.fmt])
    if wl.fmt in _QUANT:
        # expert weights quantised on the GPU (128 x 128 fp8 blocks / MX groups of 32)
        f = _FMT[wl.fmt]
        eq = [gpu_quant(f, a, 128) for a in experts]
        shq = None if sh is None else [gpu_quant(f, a, 128) for a in sh]
        weights = moe.make_weights(to_dev(wr, dt), *(c for c, _ in eq),
                                   scales=tuple(s for _, s in eq),
                                   shared=None if shq is None else tuple(c for c, _ in shq),
                                   shared_scales=(None, None, None) if shq is None
                                   else tuple(s for _, s in shq),
                                   shared_gate=None if sgate is None else to_dev(sgate, dt))
    else:
        ew = [to_dev(a, dt) for a in experts]
        shw = None if sh is None else [to_dev(a, dt) for a in sh]
        weights = moe.make_weights(to_dev(wr, dt), *ew, shared=shw,
                                   shared_gate=None if sgate is None else to_dev(sgate, dt))
    out = torch.empty((wl.T, wl.H), dtype=torch.float32, device="cuda")
    logits = torch.empty((wl.T, wl.E), dtype=torch.float32, device="cuda")
    ids = torch.empty((wl.T, wl.k), dtype=torch.int32, device="cuda")
    w = torch.empty((wl.T, wl.k), dtype=torch.float32, device="cuda")
    ws = torch.empty(moe.moe_layer_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    xb = to_dev(x, dt)
    bt = None if bias is None else to_dev(bias, torch.float32)
    moe.moe_layer(desc, weights, xb, bt, out, logits, ids, w, ws)
    torch.cuda.synchronize()
    return (out.float().cpu().numpy(), logits.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy(),
            (desc, weights, xb, bt, out, logits, ids, w, ws))


def _act_fmt(wl, unrounded=False):
    # h enters the down projection in the expert format (bf16 / fp8 1x128 / MXFP4 / MXFP8; bf16 for
    # NVFP4, whose oracle format code also selects the NVFP4 quantiser for x and the weights); with
    # unrounded=True a bf16 layer's oracle keeps h exact (fp64) instead
    if unrounded:
        return oracle.F32
    return {mi.FMT_F32: oracle.F32, mi.FMT_BF16: oracle.BF16, mi.FMT_FP8: oracle.FP8,
            mi.FMT_MX4: oracle.MX4, mi.FMT_MX8: oracle.MX8, mi.FMT_NV4: oracle.NV4}[wl.fmt]


def _oracle_operands(wl, x, experts, sh):
    act = _act_fmt(wl)
    M = oracle.Mat
    if wl.fmt in _QUANT:
        # the oracle quantises x (fp8: 128-token x 128-channel blocks; MX: 1 x 32; NVFP4: per token
        # row) and the weights with its own quantisers
        xa = oracle_quant(act, x, 128)
        mats = [oracle_quant(act, a, 128) for a in experts]
        shared = None if sh is None else tuple(oracle_quant(act, a, 128) for a in sh)
    else:
        xa = M(oracle.F32, x)
        mats = [M(oracle.F32, a) for a in experts]
        shared = None if sh is None else tuple(M(oracle.F32, a) for a in sh)
    return xa, mats, shared


def _odesc(wl, unrounded=False):
    return dict(T=wl.T, H=wl.H, E=wl.E, e0=wl.e0, E_loc=wl.E_loc, I=wl.I, k=wl.k, I_s=wl.I_s,
                scoring=wl.scoring, renormalize=wl.renormalize,
                act_fmt=_act_fmt(wl, unrounded))


def oracle_layer(wl, x, wr, bias, experts, sh, tok, sgate=None, operands=None, unrounded=False):
    xa, mats, shared = operands or _oracle_operands(wl, x, experts, sh)
    return oracle.moe_layer(_odesc(wl, unrounded), x, wr, bias, xa, *mats, shared, tok,
                            shared_gate=sgate)


def _record(entry):
    """Append one parity result to the JSON-lines file named by MOE_PARITY_RECORD (if set)."""
    path = os.environ.get("MOE_PARITY_RECORD")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(entry) + "\n")


def check_layer(wl, n_sample=None, bias_override=None, seed=0, gated=None, unrounded=False):
    gated = bool(wl.gated) if gated is None else gated
    print(f"[layer] {wl.name} T={wl.T} H={wl.H} E={wl.E} E_loc={wl.E_loc} I={wl.I} k={wl.k} "
          f"I_s={wl.I_s} gated={gated}", flush=True)
    x, wr, bias, experts, sh = make_inputs(wl, bias_override)
    sgate = gen.shared_gate_vector(wl) if gated else None
    out, lg, ids, w, _ = gpu_layer(wl, x, wr, bias, experts, sh, sgate)
    T = wl.T
    if n_sample is None or n_sample >= T:
        tok = np.arange(T, dtype=np.int32)
    else:
        rng = np.random.default_rng([seed, T])
        tok = np.unique(np.concatenate([[0, T - 1], rng.choice(T, n_sample, replace=False)]))
        tok = tok.astype(np.int32)
    ops = _oracle_operands(wl, x, experts, sh)
    ref = oracle_layer(wl, x, wr, bias, experts, sh, tok, sgate, operands=ops)
    # logits inside the fp32 accumulation bound
    L64, absdot = oracle.logits(x, wr, bias, tok=tok)
    bound = gamma(wl.H + 1) * absdot
    assert np.all(np.abs(lg[tok].astype(np.float64) - L64) <= bound)
    # the selection was made on exactly the logits written (every token, numpy brute force)
    assert np.array_equal(ids, topk_numpy(lg, wl.k))
    # against the oracle's own routing: equal, or a valid choice within the bound
    diff = np.nonzero((ids[tok] != ref["ids"]).any(1))[0]
    assert len(diff) <= max(1, len(tok) // 50), len(diff)
    for i in diff:
        assert routing_consistent(ids[tok[i]], L64[i], bound[i])
    keep = np.setdiff1d(np.arange(len(tok)), diff)
    if len(keep):
        assert np.abs(w[tok[keep]] - ref["w"][keep]).max() <= 1e-4
    # every sampled token's output is checked: tokens routed like the oracle against the oracle's
    # layer, near-tie tokens against the oracle's expert sum under the GPU's own routing
    want = ref["out"].copy()
    if len(diff):
        want[diff] = oracle.moe_layer_routed(_odesc(wl), x, *ops[:1], *ops[1], ops[2], tok[diff],
                                             ids[tok[diff]], w[tok[diff]], shared_gate=sgate)
    err, rms = rel_err(out[tok], want)
    entry = dict(workload=wl.name, T=T, fmt=wl.fmt, tokens=int(len(tok)), flips=int(len(diff)),
                 max_err_over_rms=err, rms=rms, bar=tol_for(wl.fmt))
    msg = (f"[layer] {wl.name}: max|err|/rms = {err:.3e} (rms {rms:.3e}), tokens {len(tok)}, "
           f"near-tie flips {len(diff)}")
    if unrounded and wl.fmt == mi.FMT_BF16:
        # the same tokens against the layer with h left unrounded (the exact SwiGLU FFN)
        ref_u = oracle_layer(wl, x, wr, bias, experts, sh, tok, sgate, operands=ops, unrounded=True)
        want_u = ref_u["out"].copy()
        if len(diff):
            want_u[diff] = oracle.moe_layer_routed(_odesc(wl, True), x, *ops[:1], *ops[1], ops[2],
                                                   tok[diff], ids[tok[diff]], w[tok[diff]],
                                                   shared_gate=sgate)
        err_u, _ = rel_err(out[tok], want_u)
        entry["max_err_over_rms_unrounded_h"] = err_u
        msg += f", against unrounded h {err_u:.3e}"
        assert err_u <= tol_for(wl.fmt), err_u
    bar = tol_for(wl.fmt)
    if err > bar and wl.fmt in _H_QUANT:
        # tokens above the bar: allowed only what re-quantised h codes next to a rounding boundary
        # (within the fp32 accumulation bound of the exact h) can move the output
        n_allow = _check_with_flip_allowance(wl, out, want, tok, ids, w, ops, bar * rms, sgate, x)
        entry["tokens_within_h_code_allowance"] = n_allow
        msg += f", {n_allow} token(s) within the h code-boundary allowance"
        err = bar
    print(msg, flush=True)
    _record(entry)
    assert err <= bar
    return out


def _sub_mat(m, g):
    """expert g of a weight stack as its own one-matrix Mat"""
    return oracle.Mat(m.fmt, m.q[g], None if m.s is None else m.s[g], bn=m.bn, bk=m.bk)


def _check_with_flip_allowance(wl, out, want, tok, ids, w, ops, abs_bar, sgate, x):
    fmt = _FMT[wl.fmt]
    xa, (G, U, D), shared = ops
    err = np.abs(out[tok] - want)
    over = np.nonzero(err.max(1) > abs_bar)[0]
    cache = {}

    def dq(key, m, g):
        if key not in cache:
            cache[key] = _sub_mat(m, g).dequant()[0]
        return cache[key]

    for i in over:
        t = int(tok[i])
        if wl.fmt == mi.FMT_FP8:
            row = oracle.Mat(xa.fmt, xa.q[0][t:t + 1], xa.s[0][t // 128:t // 128 + 1], bn=128, bk=128)
        else:
            row = oracle.Mat(xa.fmt, xa.q[0][t:t + 1], xa.s[0][t:t + 1])
        a = row.dequant()[0, 0]
        allow = np.zeros(wl.H)
        for j in range(wl.k):
            e = int(ids[t, j]) - wl.e0
            if not 0 <= e < wl.E_loc:
                continue
            al, _ = h_flip_allowance(fmt, a, dq(("g", e), G, e), dq(("u", e), U, e),
                                     dq(("d", e), D, e))
            allow += float(w[t, j]) * al
        if wl.I_s:
            gs = 1.0 if sgate is None else float(oracle.shared_gate(x, sgate, tok=np.array([t], np.int32))[0])
            al, _ = h_flip_allowance(fmt, a, dq("sg", shared[0], 0), dq("su", shared[1], 0),
                                     dq("sd", shared[2], 0))
            allow += gs * al
        assert np.all(err[i] <= abs_bar + allow), (t, float((err[i] - abs_bar - allow).max()))
    return len(over)


@pytest.mark.parametrize("name,n_sample", [("C1", None), ("C2d", None), ("C3a", 96),
                                           ("C2p", 48), ("C3b", 64), ("C4d", 64), ("C4p", 48),
                                           ("C5d", None), ("C5p", 48), ("C2d_mx8", None),
                                           ("C2p_mx8", 48), ("C5d_nv4", None), ("C5p_nv4", 48)])
def test_layer_workloads(name, n_sample):
    check_layer(mi.WORKLOADS[name], n_sample, unrounded=True)


# the shared expert scaled by its per-token logistic gate: bf16 (Qwen3.5-397B slice), fp8 and MXFP4
# (DeepSeek-V3 slice), at a prefill and a decode size
@pytest.mark.parametrize("name,n_sample", [("C3a_g", 96), ("C3b_g", 48), ("C4p", 48),
                                           ("C5d", None), ("C5d_nv4", None)])
def test_layer_gated_shared_expert(name, n_sample):
    check_layer(mi.WORKLOADS[name], n_sample, gated=True)


def _small(**kw):
    base = mi.Workload("edge", 64, 512, 16, 0, 8, 256, 4, 0, mi.SOFTMAX, 1, mi.FMT_BF16,
                       mi.FMT_BF16, 0.0)
    return replace(base, **kw)


def test_layer_single_token_full_shape():
    check_layer(mi.WORKLOADS["C2p"].with_tokens(1))


def test_layer_no_local_rows():
    wl = _small(e0=8)
    bias = np.zeros(16, np.float32)
    bias[8:] = -100.0                                    # nobody routes to the local slice
    out = check_layer(wl, bias_override=bias)
    assert not out.any()


def test_layer_no_local_rows_with_shared():
    wl = _small(e0=8, I_s=256)
    bias = np.zeros(16, np.float32)
    bias[8:] = -100.0
    check_layer(wl, bias_override=bias)


def test_layer_all_tokens_one_expert():
    wl = _small(T=700)
    bias = np.zeros(16, np.float32)
    bias[3] = 30.0
    check_layer(wl, bias_override=bias)


def test_layer_k_equals_E_sigmoid_ragged():
    check_layer(_small(T=37, E=16, k=16, e0=8, E_loc=8, scoring=mi.SIGMOID))
    check_layer(_small(T=37, E=16, k=3, e0=4, E_loc=12, I_s=256))


def test_layer_mx8_single_token_full_shape():
    # one token at the full MXFP8 shape: one row per chosen expert (weight streaming)
    check_layer(mi.WORKLOADS["C2p_mx8"].with_tokens(1))


@pytest.mark.parametrize("fmt", [mi.FMT_FP8, mi.FMT_MX4, mi.FMT_MX8, mi.FMT_NV4])
def test_layer_quantised_single_token_with_shared(fmt):
    # one token, sigmoid routing, shared expert as a one-row extra group
    check_layer(_small(T=1, fmt=fmt, H=512, I=256, I_s=256, scoring=mi.SIGMOID))


@pytest.mark.parametrize("fmt", [mi.FMT_FP8, mi.FMT_MX4, mi.FMT_MX8, mi.FMT_NV4])
def test_layer_quantised_all_tokens_one_expert(fmt):
    # every token's top choice is expert 3 (one large group on the tile kernels, the rest small)
    wl = _small(T=700, fmt=fmt, H=512, I=256)
    bias = np.zeros(16, np.float32)
    bias[3] = 30.0
    check_layer(wl, bias_override=bias)


@pytest.mark.parametrize("fmt", [mi.FMT_FP8, mi.FMT_MX4, mi.FMT_MX8, mi.FMT_NV4])
def test_layer_quantised_no_local_rows_with_shared(fmt):
    wl = _small(e0=8, I_s=256, fmt=fmt, H=512, I=256)
    bias = np.zeros(16, np.float32)
    bias[8:] = -100.0
    check_layer(wl, bias_override=bias)


def test_layer_deterministic():
    wl = mi.WORKLOADS["C3a"]
    x, wr, bias, experts, sh = make_inputs(wl)
    a = gpu_layer(wl, x, wr, bias, experts, sh)[0]
    b = gpu_layer(wl, x, wr, bias, experts, sh)[0]
    assert np.array_equal(a, b)


# the routing result as one stacked 32-bit blob: ids in plane 0, weight bits in plane 1 (T * k = 21 is
# not a multiple of 4, so plane 1 starts at the padded offset); the layer writes the same ids and
# weight bits into the blob as into separate arrays, and permute / combine read the planes
def test_layer_routing_blob():
    wl = _small(T=7, k=3, I_s=256)
    x, wr, bias, experts, sh = make_inputs(wl)
    out, lg, ids, w, (desc, weights, xb, bt, o_dev, l_dev, i_dev, w_dev, ws) = gpu_layer(
        wl, x, wr, bias, experts, sh)
    P = moe.moe_routing_blob_plane(desc)
    assert P == 24
    blob = torch.full((2 * P,), -7, dtype=torch.int32, device="cuda")
    out2 = torch.empty_like(o_dev)
    moe.moe_layer(desc, weights, xb, bt, out2, None, blob[:P], blob[P:].view(torch.float32), ws)
    torch.cuda.synchronize()
    b = blob.cpu().numpy()
    assert np.array_equal(b[:wl.T * wl.k].reshape(wl.T, wl.k), ids)
    assert np.array_equal(b[P:P + wl.T * wl.k].view(np.float32).reshape(wl.T, wl.k), w)
    assert np.all(b[wl.T * wl.k:P] == -7)                       # padding untouched
    assert np.array_equal(out2.cpu().numpy(), out)
    # permute and combine from the planes: the same maps and the same combine as from the arrays
    k, T, H = wl.k, wl.T, wl.H
    counts = torch.empty(wl.E_loc, dtype=torch.int32, device="cuda")
    offs = torch.empty(wl.E_loc + 1, dtype=torch.int32, device="cuda")
    s2r = torch.empty((T, k), dtype=torch.int32, device="cuda")
    r2f = torch.empty(T * k, dtype=torch.int32, device="cuda")
    pws = torch.empty(max(moe.moe_permute_workspace_bytes(desc), 16), dtype=torch.uint8, device="cuda")
    moe.moe_permute(desc, blob[:P], None, None, counts, offs, s2r, r2f, None, None, pws)
    ref = oracle.permute(ids, wl.e0, wl.E_loc)
    torch.cuda.synchronize()
    assert np.array_equal(s2r.cpu().numpy(), ref[2])
    y = torch.randn((T * k, H), device="cuda")
    c1 = torch.empty((T, H), device="cuda")
    c2 = torch.empty((T, H), device="cuda")
    moe.moe_combine(desc, moe.MOE_F32, y, blob[P:].view(torch.float32), s2r, None, c1)
    moe.moe_combine(desc, moe.MOE_F32, y, w_dev, s2r, None, c2)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)


# a shared expert whose intermediate size differs from the routed experts' (its own GEMM launches,
# its h in a separate buffer): larger and smaller than I, every expert format, a decode and a
# prefill token count, and the Qwen3.5-397B-shaped slice with a shared expert twice as wide
@pytest.mark.parametrize("fmt,I,I_s", [(mi.FMT_BF16, 256, 512), (mi.FMT_BF16, 256, 128),
                                       (mi.FMT_FP8, 256, 384), (mi.FMT_MX4, 256, 512),
                                       (mi.FMT_MX8, 256, 128), (mi.FMT_NV4, 256, 512)])
@pytest.mark.parametrize("T", [5, 700])
def test_layer_shared_expert_other_width(fmt, I, I_s, T):
    check_layer(_small(T=T, fmt=fmt, H=512, I=I, I_s=I_s,
                       scoring=mi.SIGMOID if fmt != mi.FMT_BF16 else mi.SOFTMAX))


def test_layer_shared_expert_wider_full_shape():
    wl = replace(mi.WORKLOADS["C3a"], name="C3a_Is2048", I_s=2048)
    check_layer(wl, 48)
    check_layer(replace(wl, name="C3a_Is2048_gated", gated=1).with_tokens(64))
