"""Seeded synthetic inputs for the MoE FFN layer.

This module is shared by the oracle side and the GPU side and therefore holds none of the layer's
arithmetic: it only draws random numbers and rounds them to the stored input format.

Recipe (every draw is float32 from numpy's PCG64 `default_rng`, seeded by a tuple):
  * router weight   W_r [E, H]           rng([seed, 0])           N(0, 1) * 0.02
  * local expert e  W_gate [I, H]        rng([seed, 1, e, 0])     N(0, 1) * 0.02
                    W_up   [I, H]        rng([seed, 1, e, 1])     N(0, 1) * 0.02
                    W_down [H, I]        rng([seed, 1, e, 2])     N(0, 1) * 0.02
  * shared expert   same three shapes    rng([seed, 2, 0, m])
  * shared gate     w_sg [H]             rng([seed, 2, 1, 0])     N(0, 1) * 0.02 (gated workloads)
  * tokens          x [T, H]             rng([seed, 3, T])        N(0, 1)
  * router bias     log of the Zipf(s) pmf over experts (expert e has rank e + 1), or none.

Weights are stored as [out_features, in_features] (K contiguous). For bf16 workloads x, W_r and the
expert weights are rounded to bf16 (round to nearest even) and kept as float32 arrays holding
bf16-representable values; for the fp8 / MXFP4 workloads the expert weights stay float32 (each side
quantises them itself) while x and W_r are bf16.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .workloads import FMT_F32, Workload


def bf16_round(a):
    """Round float32 values to the nearest bf16 (ties to even); returns float32 holding them."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(a.shape)


def to_bf16_bits(a):
    """bf16 bit patterns (uint16) of float32 values that are already bf16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _normal(seed_seq, shape, scale=1.0):
    rng = np.random.default_rng(list(seed_seq))
    out = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        out *= np.float32(scale)
    return out


def _io_round(wl, a):
    return a if wl.io_fmt == FMT_F32 else bf16_round(a)


def _expert_round(wl, a):
    # bf16 / fp32 workloads store the expert weights in the io format; quantised workloads keep the
    # float32 draws, which each side quantises with its own quantiser.
    from .workloads import FMT_BF16
    return bf16_round(a) if wl.fmt == FMT_BF16 else a


def router_weight(wl: Workload):
    return _io_round(wl, _normal((wl.seed, 0), (wl.E, wl.H), 0.02))


def router_bias(wl: Workload):
    """log p_e of a Zipf(s) law over the E experts, expert e having rank e + 1; None if s = 0."""
    if wl.zipf_s == 0.0:
        return None
    ranks = np.arange(1, wl.E + 1, dtype=np.float64)
    p = ranks ** (-wl.zipf_s)
    p /= p.sum()
    return np.log(p).astype(np.float32)


def expert_weight(wl: Workload, e_local: int, which: int):
    """which: 0 = gate [I, H], 1 = up [I, H], 2 = down [H, I]."""
    shape = (wl.I, wl.H) if which < 2 else (wl.H, wl.I)
    return _expert_round(wl, _normal((wl.seed, 1, e_local, which), shape, 0.02))


def shared_weight(wl: Workload, which: int):
    shape = (wl.I_s, wl.H) if which < 2 else (wl.H, wl.I_s)
    return _expert_round(wl, _normal((wl.seed, 2, 0, which), shape, 0.02))


def expert_weights(wl: Workload, threads: int = 8):
    """Stacked local expert weights: gate [E_loc, I, H], up [E_loc, I, H], down [E_loc, H, I]."""
    gate = np.empty((wl.E_loc, wl.I, wl.H), np.float32)
    up = np.empty((wl.E_loc, wl.I, wl.H), np.float32)
    down = np.empty((wl.E_loc, wl.H, wl.I), np.float32)
    dst = (gate, up, down)

    def fill(job):
        e, which = job
        dst[which][e] = expert_weight(wl, e, which)

    jobs = [(e, w) for e in range(wl.E_loc) for w in range(3)]
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(fill, jobs))
    return gate, up, down


def shared_weights(wl: Workload):
    if wl.I_s == 0:
        return None
    return tuple(shared_weight(wl, w) for w in range(3))


def shared_gate_vector(wl: Workload):
    """Gate vector of the shared expert [H], in the io format (same rounding as the router)."""
    return _io_round(wl, _normal((wl.seed, 2, 1, 0), (wl.H,), 0.02))


def tokens(wl: Workload):
    return _io_round(wl, _normal((wl.seed, 3, wl.T), (wl.T, wl.H)))


# ---------------------------------------------------------------------------------------------
# Fixtures for the routing and permutation steps on their own (drawn data, no layer arithmetic)
# ---------------------------------------------------------------------------------------------

def tie_heavy_logits(T, E, seed=0):
    """fp32 logits on a coarse grid (multiples of 0.25 in [-2, 2]) so that equal values are common,
    with some all-equal rows and rows mixing +0.0 and -0.0."""
    rng = np.random.default_rng([seed, 10, T, E])
    L = (rng.integers(-8, 9, size=(T, E)) * 0.25).astype(np.float32)
    if T >= 4:
        L[0, :] = 1.5                        # all equal
        L[1, :] = 0.0                        # +0 / -0 mixture
        L[1, rng.random(E) < 0.5] = -0.0
        L[2, :] = -0.0
        L[3, ::2] = 3.0                      # many ties at the top
    return L


def random_logits(T, E, seed=0, scale=1.0, bias=None):
    rng = np.random.default_rng([seed, 11, T, E])
    L = rng.standard_normal((T, E), dtype=np.float32) * np.float32(scale)
    if bias is not None:
        L = L + bias[None, :].astype(np.float32)
    return L.astype(np.float32)


def random_topk_ids(T, E, k, seed=0, hot=None, hot_frac=0.0):
    """int32 [T, k] of distinct expert ids per token, uniform or with a share of slots forced onto
    the experts listed in `hot`."""
    rng = np.random.default_rng([seed, 12, T, E, k])
    keys = rng.random((T, E))
    if hot is not None and hot_frac > 0:
        boost = rng.random((T, len(hot))) < hot_frac
        keys[:, hot] += boost * 2.0
    ids = np.argsort(-keys, axis=1, kind="stable")[:, :k]
    return ids.astype(np.int32)
