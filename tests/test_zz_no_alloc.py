"""moe_layer_noalloc (the layer with the library's per-GPU scratch array as its workspace) against
moe_layer with a caller workspace, through the C ABI: identical outputs on two calls in a row, the
second with fewer tokens, and the size limit refused before any launch."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import moe_inputs as mi
import moe_layer_softmax_amd as moe
from moe_inputs import gen

from gpu_util import gpu_quant, io_torch, to_dev

pytestmark = pytest.mark.gpu

_FMT = {mi.FMT_BF16: moe.MOE_BF16, mi.FMT_MX4: moe.MOE_MXFP4}


def _weights(wl):
    dt = io_torch(wl.io_fmt)
    wr = to_dev(gen.router_weight(wl), dt)
    experts = gen.expert_weights(wl)
    sh = gen.shared_weights(wl)
    if wl.fmt == mi.FMT_BF16:
        return moe.make_weights(wr, *(to_dev(a, dt) for a in experts),
                                shared=None if sh is None else [to_dev(a, dt) for a in sh])
    eq = [gpu_quant(_FMT[wl.fmt], a, 128) for a in experts]
    shq = None if sh is None else [gpu_quant(_FMT[wl.fmt], a, 128) for a in sh]
    return moe.make_weights(wr, *(c for c, _ in eq), scales=tuple(s for _, s in eq),
                            shared=None if shq is None else tuple(c for c, _ in shq),
                            shared_scales=(None, None, None) if shq is None
                            else tuple(s for _, s in shq))


def _run(wl, weights, noalloc):
    dt = io_torch(wl.io_fmt)
    desc = moe.make_desc(wl.T, wl.H, wl.E, wl.e0, wl.E_loc, wl.I, wl.k, wl.I_s, wl.scoring,
                         wl.renormalize, _FMT[wl.io_fmt], _FMT[wl.fmt])
    x = to_dev(gen.tokens(wl), dt)
    b = gen.router_bias(wl)
    bias = None if b is None else to_dev(b, torch.float32)
    out = torch.full((wl.T, wl.H), 7.0, dtype=torch.float32, device="cuda")
    ids = torch.full((wl.T, wl.k), -3, dtype=torch.int32, device="cuda")
    w = torch.full((wl.T, wl.k), 7.0, dtype=torch.float32, device="cuda")
    if noalloc:
        moe.moe_layer_noalloc(desc, weights, x, bias, out, None, ids, w)
    else:
        ws = torch.empty(moe.moe_layer_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
        moe.moe_layer(desc, weights, x, bias, out, None, ids, w, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()


# the 64-token Qwen3-235B slice (bf16) and then 17 tokens of it; a small MXFP4 layer with a shared
# expert of another width (its own GEMM launches) at 40 and then 9 tokens
@pytest.mark.parametrize("base,tokens", [
    (mi.WORKLOADS["C2d"], (64, 17)),
    (replace(mi.WORKLOADS["C5d"], name="mx4_small", H=512, E=16, E_loc=8, I=256, I_s=512), (40, 9)),
])
def test_noalloc_matches_layer_with_workspace(base, tokens):
    weights = _weights(base)
    for T in tokens:
        wl = base.with_tokens(T)
        print(f"[noalloc] {wl.name} T={T}", flush=True)
        ref = _run(wl, weights, noalloc=False)
        got = _run(wl, weights, noalloc=True)
        for a, b in zip(got, ref):
            assert np.array_equal(a, b)


def test_noalloc_refuses_layers_beyond_the_scratch():
    wl = mi.WORKLOADS["C2p"]
    desc = moe.make_desc(wl.T, wl.H, wl.E, wl.e0, wl.E_loc, wl.I, wl.k, wl.I_s, wl.scoring,
                         wl.renormalize)
    assert moe.moe_layer_workspace_bytes(desc) > moe.MOE_NOALLOC_SCRATCH_BYTES
    dummy = torch.empty(64, dtype=torch.float32, device="cuda")
    weights = moe.make_weights(dummy, dummy, dummy, dummy)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_layer_noalloc(desc, weights, dummy, None, dummy, None, None, None)
    assert e.value.status == moe.MOE_ERR_WORKSPACE
