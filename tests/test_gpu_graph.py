"""The whole layer captured once into a HIP graph (torch.cuda.CUDAGraph on the capture stream) and
replayed: moe_layer allocates nothing, synchronises with nothing on the host and records no memset
(its tile schedulers read the group offsets on the device), so a captured call is the same launch
sequence as an eager one. Every replay, with new tokens copied into the captured input and eager
layer calls and host synchronisations between replays, must equal the eager output bit for bit."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import moe_layer_softmax_amd as moe
from moe_inputs import gen

from gpu_util import to_dev
from test_gpu_layer import _small, gpu_layer, make_inputs

pytestmark = pytest.mark.gpu

_CASES = {
    # the 64-token Qwen3-235B-shaped decode slice: K-split router, one-kernel dispatch, the
    # weight-streaming GEMMs
    "decode_bf16": lambda: mi.WORKLOADS["C2d"],
    # 2048 tokens, 512 rows per expert: the persistent 256 x 256 GEMMs
    "prefill_bf16": lambda: _small(T=2048),
    # MXFP4 experts with a gated shared expert: the activation quantiser, the quantised GEMMs and the
    # shared expert's gate
    "mx4_shared_gated": lambda: _small(T=300, I_s=256, fmt=mi.FMT_MX4, gated=1),
}


@pytest.mark.parametrize("case", list(_CASES))
def test_layer_graph_replay(case):
    wl = _CASES[case]()
    print(f"[graph] {case}: T={wl.T} H={wl.H} E={wl.E} E_loc={wl.E_loc} I={wl.I} k={wl.k} "
          f"I_s={wl.I_s} fmt={wl.fmt}", flush=True)
    x, wr, bias, experts, sh = make_inputs(wl)
    sgate = gen.shared_gate_vector(wl) if wl.gated else None
    _, _, _, _, (desc, weights, xb, bt, out, _, _, _, ws) = gpu_layer(wl, x, wr, bias, experts, sh,
                                                                       sgate)
    rng = np.random.default_rng([11, wl.T])
    xs = [to_dev(gen.bf16_round(rng.standard_normal(x.shape).astype(np.float32)), xb.dtype)
          for _ in range(3)]
    refs = []
    for xi in xs:
        o = torch.empty_like(out)
        moe.moe_layer(desc, weights, xi, bt, o, None, None, None, ws)
        refs.append(o)
    torch.cuda.synchronize()

    x_static = xs[0].clone()
    out_static = torch.full_like(out, float("nan"))
    ws_g = torch.empty_like(ws)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        moe.moe_layer(desc, weights, x_static, bt, out_static, None, None, None, ws_g)
    torch.cuda.synchronize()
    for rep in range(2):
        for i in range(3):
            x_static.copy_(xs[i])
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out_static, refs[i]), (case, rep, i)
            j = (i + 1) % 3                             # eager work between replays
            moe.moe_layer(desc, weights, xs[j], bt, out, None, None, None, ws)
            torch.cuda.synchronize()
            assert torch.equal(out, refs[j]), (case, rep, j)
    print(f"[graph] {case}: 6 replays equal to the eager layer", flush=True)
