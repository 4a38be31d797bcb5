"""Helpers of the GPU tests: device upload, the layer run through the C ABI, and the comparisons
(tolerances and the routing checks)."""
import numpy as np
import torch

import moe_inputs as mi
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
    return 6e-2 if fmt in (mi.FMT_FP8, mi.FMT_MX4) else 2e-2
