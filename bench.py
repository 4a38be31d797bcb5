"""Benchmark of the MoE FFN layer on one MI355X.

Workload: the Qwen3-235B-shaped layer slice (experts 0..31 of 128 on this GPU, hidden 4096,
intermediate 1536, softmax top-8 with renormalisation, Zipf(1.1) router bias), 16384 tokens, bf16
inputs and weights, seeded synthetic data. One step = one full moe_layer call (router, top-k,
dispatch, gate/up GEMM + SwiGLU, down GEMM, combine) with every input already resident in HBM.

Prints one JSON line (rank 0) with the headline throughput, the roofline of the dominant kernel
(the gate/up grouped GEMM, timed with HIP events on its launch stream), a decode-size (64 tokens)
measurement of the same layer against HBM bandwidth, and the CPU oracle's rate on a token sample.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6    # MI355X dense bf16 MFMA (2.5 PFLOP/s class, 2.4 GHz)
PEAK_HBM_GBPS = 8000.0       # MI355X HBM3E


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="C2p")
    p.add_argument("--decode-workload", default="C2d")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target CPU time of the oracle baseline sample (0 disables it)")
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--profile-only", action="store_true",
                   help="only the timed moe_layer steps (for profilers)")
    p.add_argument("--flush", action="store_true",
                   help="with --profile-only: read a 1 GiB buffer before every step (cold caches)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only copy a 1 GiB buffer three times (reference kernel for HBM counters)")
    p.add_argument("--stream-ceiling", action="store_true",
                   help="only time the HBM read probe (libmoe_probe.so) on a 1 GiB row-major matrix")
    p.add_argument("--all-workloads", action="store_true",
                   help="(default) add every workload's layer time and both roofline fractions")
    p.add_argument("--no-workloads", action="store_true",
                   help="skip the table of every workload's layer time and roofline fractions")
    p.add_argument("--workloads", default=None,
                   help="comma-separated names: the workload table for these only")
    p.add_argument("--no-ep-sweep", action="store_true",
                   help="skip the decode MoE-GEMM sweep over local expert counts")
    p.add_argument("--table-one", default=None,
                   help="one line of the workload table, measured in this process and printed "
                        "as JSON (the table runs each workload this way, in a child process)")
    return p.parse_args()


# NVFP4 runs its products (exact in bf16) on the bf16 MFMA, so its MFMA roofline is bf16's
PEAK_TFLOPS = {"bf16": PEAK_BF16_TFLOPS, "fp8": 5033.2, "mxfp8": 5033.2, "mxfp4": 10066.3,
               "nvfp4": PEAK_BF16_TFLOPS}


class TableLayer:
    """One workload's layer call for the workload table and the profiler runs: tokens, router
    weight and bias are the seeded inputs; expert weights are seeded device draws of the same
    shapes (their values do not change the work), quantised by the library for the fp8 / MXFP4 /
    MXFP8 / NVFP4 layers."""

    def __init__(self, wl, stream):
        import torch
        import moe_inputs as mi
        import moe_layer_softmax_amd as moe
        from moe_inputs import gen
        fmt_of = {mi.FMT_BF16: ("bf16", moe.MOE_BF16), mi.FMT_FP8: ("fp8", moe.MOE_FP8_E4M3),
                  mi.FMT_MX4: ("mxfp4", moe.MOE_MXFP4), mi.FMT_MX8: ("mxfp8", moe.MOE_MXFP8),
                  mi.FMT_NV4: ("nvfp4", moe.MOE_NVFP4)}
        self.wl = wl
        fname, fcode = fmt_of[wl.fmt]
        self.fname = fname
        bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(torch.bfloat16)
        x, wr = bf(gen.tokens(wl)), bf(gen.router_weight(wl))
        b = gen.router_bias(wl)
        bias = None if b is None else torch.from_numpy(b).to("cuda")
        gen_t = torch.Generator(device="cuda")
        gen_t.manual_seed(1)
        shapes = [(wl.E_loc, wl.I, wl.H), (wl.E_loc, wl.I, wl.H), (wl.E_loc, wl.H, wl.I)]
        if wl.I_s:
            shapes += [(1, wl.I_s, wl.H), (1, wl.I_s, wl.H), (1, wl.H, wl.I_s)]
        # The weights' own buffers are allocated first and filled one expert at a time (fp32 draws
        # of one matrix, then cast or quantised), as a serving process loads its weights: built
        # from whole fp32 stacks, freed afterwards, the same decode layers measured ~2% slower when
        # other workloads had run in the process before them.
        def buffers(G, R, C):
            if fname == "bf16":
                return torch.empty((G, R, C), dtype=torch.bfloat16, device="cuda"), None
            if fname == "fp8":
                return (torch.empty((G, R, C), dtype=torch.uint8, device="cuda"),
                        torch.empty((G, R // 128, C // 128), dtype=torch.float32, device="cuda"))
            if fname == "mxfp8":
                return (torch.empty((G, R, C), dtype=torch.uint8, device="cuda"),
                        torch.empty((G, R, C // 32), dtype=torch.uint8, device="cuda"))
            if fname == "nvfp4":
                # per matrix: e4m3 block scales [R, C/16], then fp32 row scales [R]
                return (torch.empty((G, R, C // 2), dtype=torch.uint8, device="cuda"),
                        torch.empty((G, R * (C // 16) + 4 * R), dtype=torch.uint8, device="cuda"))
            return (torch.empty((G, R, C // 2), dtype=torch.uint8, device="cuda"),
                    torch.empty((G, R, C // 32), dtype=torch.uint8, device="cuda"))
        bufs = [buffers(*s) for s in shapes]
        mats, scales = [b[0] for b in bufs], [b[1] for b in bufs]
        for (G, R, C), m, sc in zip(shapes, mats, scales):
            for g in range(G):
                src = torch.randn((R, C), generator=gen_t, device="cuda") * 0.02
                if fname == "bf16":
                    m[g].copy_(src)
                else:
                    moe.moe_quantize(fcode, moe.MOE_F32, 1, R, C, 128, src, m[g], sc[g])
                del src
        if fname == "bf16":
            self.wbytes_expert = 3 * wl.I * wl.H * 2
        else:
            self.wbytes_expert = sum(int(m[0].numel() * m.element_size()) +
                                     int(s[0].numel() * s.element_size())
                                     for m, s in zip(mats[:3], scales[:3]))
        torch.cuda.synchronize()
        sgate = (torch.randn(wl.H, generator=gen_t, device="cuda") * 0.02).to(torch.bfloat16) \
            if wl.gated else None
        W = moe.make_weights(wr, *mats[:3], scales=tuple(scales[:3]),
                             shared=tuple(mats[3:]) if wl.I_s else None,
                             shared_scales=tuple(scales[3:]) if wl.I_s else (None, None, None),
                             shared_gate=sgate)
        d = moe.make_desc(wl.T, wl.H, wl.E, wl.e0, wl.E_loc, wl.I, wl.k, wl.I_s, wl.scoring,
                          wl.renormalize, moe.MOE_BF16, fcode, moe.MOE_F32)
        o = torch.empty((wl.T, wl.H), dtype=torch.float32, device="cuda")
        self.ids = torch.empty((wl.T, wl.k), dtype=torch.int32, device="cuda")
        ws = torch.empty(moe.moe_layer_workspace_bytes(d), dtype=torch.uint8, device="cuda")
        self._keep = (mats, scales, W, x, wr, bias, o, ws)
        self.call = lambda: moe.moe_layer(d, W, x, bias, o, None, self.ids, None, ws, stream)


TABLE_WORKLOADS = ("C2p", "C2d", "C3a", "C3b", "C3a_g", "C3b_g", "C4p", "C4d", "C5p", "C5d",
                   "C2p_mx8", "C2d_mx8", "C5p_nv4", "C5d_nv4")


def table_line(name, stream, steps):
    """One workload's layer time (one moe_layer call per step, caches evicted with a 1 GiB read
    before each), with the algorithmic MFMA and HBM roofline fractions."""
    import torch
    import moe_inputs as mi
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    wl = mi.WORKLOADS[name]
    tl = TableLayer(wl, stream)
    fname, wbytes_expert, ids, call = tl.fname, tl.wbytes_expert, tl.ids, tl.call
    with torch.cuda.stream(stream):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    with torch.cuda.stream(stream):
        for a, e in ev:
            flush.sum()
            a.record(stream)
            call()
            e.record(stream)
    torch.cuda.synchronize()
    call_ms = np.array([a.elapsed_time(e) for a, e in ev])
    ms = float(np.median(call_ms))
    loc = ids[(ids >= wl.e0) & (ids < wl.e0 + wl.E_loc)]
    R = int(loc.numel())
    active = int(torch.unique(loc).numel())
    router_fl = 2.0 * wl.T * wl.H * wl.E
    expert_fl = 6.0 * R * wl.H * wl.I + 6.0 * wl.T * wl.H * wl.I_s
    t_mfma = router_fl / PEAK_BF16_TFLOPS / 1e12 + expert_fl / PEAK_TFLOPS[fname] / 1e12
    nbytes = (active * wbytes_expert + (wbytes_expert * wl.I_s // wl.I if wl.I_s else 0)
              + wl.E * wl.H * 2 + wl.T * wl.H * 2 + wl.T * wl.H * 4 + wl.T * wl.k * 8)
    t_hbm = nbytes / (PEAK_HBM_GBPS * 1e9)
    t = ms * 1e-3
    return {"T": wl.T, "format": fname, "ms": round(ms, 4),
            "ms_p10": round(float(np.percentile(call_ms, 10)), 4),
            "ms_p90": round(float(np.percentile(call_ms, 90)), 4),
            "tokens_per_s": round(wl.T / t, 1), "local_rows_R": R, "active_experts": active,
            "tflops": round((router_fl + expert_fl) / t / 1e12, 1),
            "frac_mfma": round(t_mfma / t, 4), "compulsory_bytes": nbytes,
            "hbm_gbps": round(nbytes / t / 1e9, 1), "frac_hbm": round(t_hbm / t, 4),
            "bound": "mfma" if t_mfma > t_hbm else "hbm"}


def workload_table(steps, names=None):
    """table_line of every workload, each in a child process of its own: the decode-sized layers
    stream their weights at rates that depend on where the allocator placed them, and inside one
    process that placement depends on the layers measured before (the same 1024-token layer took
    0.417-0.424 ms after other single workloads and 0.454 ms after most of the table)."""
    import subprocess
    out = {}
    for name in names or TABLE_WORKLOADS:
        r = subprocess.run([sys.executable, "-u", os.path.abspath(__file__), "--table-one", name,
                            "--steps", str(steps), "--cpu-seconds", "0"],
                           capture_output=True, text=True, timeout=600)
        if r.returncode != 0:
            raise RuntimeError(f"workload table line {name}: exit status {r.returncode}\n"
                               f"{r.stderr[-3000:]}")
        out[name] = json.loads(r.stdout.strip().splitlines()[-1])
        print(f"workload {name}: {out[name]['ms']} ms", file=sys.stderr, flush=True)
    return out


def ep_sweep(stream, steps):
    """The decode MoE-GEMM microbenchmark of "Hosting Qwen on Blackwell" (section "MoE GEMM"):
    every local expert activated by exactly one token, at the Qwen3-235B expert shape (hidden 4096,
    intermediate 1536, top-8 of 128) for local slices of 8, 16, 32 and 64 experts (expert-parallel
    degrees 16, 8, 4, 2). E_loc / 8 tokens, token t routed to local experts 8t .. 8t+7. Per slice:
    the MoE GEMM time (gate/up + down, weights streamed from HBM: caches evicted by a 1 GiB read
    before each step) and the whole step (dispatch maps, both GEMMs, combine; routing excluded, the
    routing table is given). Weights are seeded device draws; their values do not change the work."""
    import torch
    import moe_layer_softmax_amd as moe
    H, I, E, k = 4096, 1536, 128, 8
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    out = {}
    for E_loc in (8, 16, 32, 64):
        T = E_loc // k
        gen_t = torch.Generator(device="cuda")
        gen_t.manual_seed(E_loc)
        bf = lambda shape: (torch.randn(shape, generator=gen_t, device="cuda") * 0.02).to(torch.bfloat16)
        wg, wu, wd = bf((E_loc, I, H)), bf((E_loc, I, H)), bf((E_loc, H, I))
        x = torch.randn((T, H), generator=gen_t, device="cuda").to(torch.bfloat16)
        ids = (torch.arange(T, device="cuda")[:, None] * k +
               torch.arange(k, device="cuda")[None, :]).to(torch.int32).contiguous()
        tw = torch.full((T, k), 1.0 / k, dtype=torch.float32, device="cuda")
        d = moe.make_desc(T, H, E, 0, E_loc, I, k)
        ws = torch.empty(max(moe.moe_permute_workspace_bytes(d), 16), dtype=torch.uint8, device="cuda")
        counts = torch.empty(E_loc, dtype=torch.int32, device="cuda")
        offsets = torch.empty(E_loc + 1, dtype=torch.int32, device="cuda")
        s2r = torch.empty((T, k), dtype=torch.int32, device="cuda")
        r2f = torch.empty(T * k, dtype=torch.int32, device="cuda")
        h = torch.empty((T * k, I), dtype=torch.bfloat16, device="cuda")
        y = torch.empty((T * k, moe.moe_f16_scaled_row_bytes(H)), dtype=torch.uint8, device="cuda")
        o = torch.empty((T, H), dtype=torch.float32, device="cuda")
        g_up = moe.moe_gemm_desc(E_loc, T * k, H, I, moe.MOE_BF16, moe.MOE_EPI_SWIGLU, moe.MOE_BF16, k, 1)
        g_dn = moe.moe_gemm_desc(E_loc, T * k, I, H, moe.MOE_BF16, moe.MOE_EPI_STORE,
                                 moe.MOE_F16_SCALED, 1, 1)
        perm = lambda: moe.moe_permute(d, ids, None, None, counts, offsets, s2r, r2f, None, None, ws,
                                       stream)
        gemms = lambda: (moe.moe_grouped_gemm(g_up, x, None, r2f, wg, None, wu, None, offsets, h,
                                              None, stream),
                         moe.moe_grouped_gemm(g_dn, h, None, None, wd, None, None, None, offsets, y,
                                              None, stream))
        comb = lambda: moe.moe_combine(d, moe.MOE_F16_SCALED, y, tw, s2r, None, o, stream)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        with torch.cuda.stream(stream):
            perm(); gemms(); comb()
            for e in ev:
                flush.sum()
                e[0].record(stream)
                perm()
                e[1].record(stream)
                gemms()
                e[2].record(stream)
                comb()
                e[3].record(stream)
        torch.cuda.synchronize()
        gemm_us = float(np.median([e[1].elapsed_time(e[2]) for e in ev])) * 1e3
        step_us = float(np.median([e[0].elapsed_time(e[3]) for e in ev])) * 1e3
        wbytes = E_loc * 3 * I * H * 2
        out[f"E_loc={E_loc}"] = {"ep_degree": E // E_loc, "tokens": T, "moe_gemm_us": round(gemm_us, 1),
                                 "step_us": round(step_us, 1), "weight_bytes": wbytes,
                                 "hbm_gbps": round(wbytes / (gemm_us * 1e-6) / 1e9, 1),
                                 "frac_hbm": round(wbytes / (gemm_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)}
        del wg, wu, wd, x, h, y, o
        torch.cuda.empty_cache()
    return out


# Source files that define the bf16 grouped GEMM kernels' device code; HBM counters taken on an
# older version of them are not reported.
GEMM_SOURCES = ["moe_layer_softmax_amd/csrc/gemm.hip", "moe_layer_softmax_amd/csrc/gemm_common.hpp",
                "moe_layer_softmax_amd/csrc/common.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gate_up_traffic.json")


def gemm_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the gate/up kernel from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by the factor that maps the same counter
    on a copy of known size to its true bytes), or None if the kernel sources changed since."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("gemm_source_sha256") != gemm_source_hash():
        return None
    rd = t["fetch_kib_per_dispatch"] * 1024.0 * t["fetch_factor"]
    wr = t["write_kib_per_dispatch"] * 1024.0 * t["write_factor"]
    return rd, wr


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": 3}), flush=True)


def stream_ceiling(steps):
    """Read rate of a 1 GiB matrix of 8 KB rows with the decode kernels' weight-stream pattern (8 rows
    x 128 bytes per load, 16 rows per wave, 8 loads in flight), with 1 KB of one row per load, and
    with the weight-stream pattern in fewer, longer streams (64 rows per wave, 16 loads in flight),
    non-temporal, each read after a 1 GiB read of another buffer (cold caches); HIP events on the
    probe's stream, median of `steps`."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "moe_layer_softmax_amd", "libmoe_probe.so"))
    lib.moe_probe_read_rows.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_void_p]
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    flush = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    out = torch.empty(n // (64 * 8192) * 256, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    res = {}
    names = {0: "8_rows_per_load", 1: "1_rows_per_load", 2: "8_rows_per_load_64_rows_per_wave_16_in_flight"}
    for pattern in (0, 1, 2):
        ms = []
        for _ in range(steps + 1):
            with torch.cuda.stream(stream):
                flush.sum()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                rc = lib.moe_probe_read_rows(src.data_ptr(), n, pattern, out.data_ptr(),
                                             ctypes.c_void_p(stream.cuda_stream))
                b.record(stream)
            if rc != 0:
                raise RuntimeError(f"probe launch failed: hipError {rc}")
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        t = float(np.median(ms[1:]))
        res[names[pattern]] = {"ms": round(t, 4), "TB_per_s": round(n / (t * 1e-3) / 1e12, 3)}
    print(json.dumps({"hbm_read_ceiling": res, "bytes": n, "row_bytes": 8192, "steps": steps}), flush=True)


class Layer:
    """Device-resident inputs, weights, outputs and workspace of one workload."""

    def __init__(self, wl, weights=None):
        import torch
        import moe_layer_softmax_amd as moe
        from moe_inputs import gen
        self.wl = wl
        dt = torch.bfloat16
        dev = "cuda"
        t = lambda a, d=dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(d)
        self.x_np = gen.tokens(wl)
        self.bias_np = gen.router_bias(wl)
        if weights is None:
            self.wr_np = gen.router_weight(wl)
            self.experts_np = gen.expert_weights(wl)
            self.w_dev = [t(self.wr_np)] + [t(a) for a in self.experts_np]
        else:
            self.wr_np, self.experts_np, self.w_dev = weights
        self.x = t(self.x_np)
        self.bias = None if self.bias_np is None else t(self.bias_np, torch.float32)
        self.desc = moe.make_desc(wl.T, wl.H, wl.E, wl.e0, wl.E_loc, wl.I, wl.k, wl.I_s, wl.scoring,
                                  wl.renormalize, moe.MOE_BF16, moe.MOE_BF16, moe.MOE_F32)
        self.weights = moe.make_weights(*self.w_dev)
        self.out = torch.empty((wl.T, wl.H), dtype=torch.float32, device=dev)
        self.logits = torch.empty((wl.T, wl.E), dtype=torch.float32, device=dev)
        self.ids = torch.empty((wl.T, wl.k), dtype=torch.int32, device=dev)
        self.w = torch.empty((wl.T, wl.k), dtype=torch.float32, device=dev)
        self.ws = torch.empty(moe.moe_layer_workspace_bytes(self.desc), dtype=torch.uint8,
                              device=dev)
        self.rws = torch.empty(max(moe.moe_route_workspace_bytes(self.desc), 16),
                               dtype=torch.uint8, device=dev)
        self.moe = moe

    def shared_weights(self):
        return self.wr_np, self.experts_np, self.w_dev

    def step(self, stream):
        self.moe.moe_layer(self.desc, self.weights, self.x, self.bias, self.out, self.logits,
                           self.ids, self.w, self.ws, stream)


def step_breakdown(L, stream, iters):
    """The layer's steps through the public entry points, each bracketed by HIP events recorded on
    the launch stream. Returns per-step mean ms and the local row count R."""
    import torch
    moe = L.moe
    wl = L.wl
    d = L.desc
    dev = "cuda"
    slots = wl.T * wl.k
    counts = torch.empty(wl.E_loc, dtype=torch.int32, device=dev)
    offsets = torch.empty(wl.E_loc + 1, dtype=torch.int32, device=dev)
    s2r = torch.empty((wl.T, wl.k), dtype=torch.int32, device=dev)
    r2f = torch.empty(slots, dtype=torch.int32, device=dev)
    pws = torch.empty(max(moe.moe_permute_workspace_bytes(d), 16), dtype=torch.uint8, device=dev)
    h = torch.empty((slots, wl.I), dtype=torch.bfloat16, device=dev)
    y = torch.empty((slots, moe.moe_f16_scaled_row_bytes(wl.H)), dtype=torch.uint8, device=dev)
    g_up = moe.moe_gemm_desc(wl.E_loc, slots, wl.H, wl.I, moe.MOE_BF16, moe.MOE_EPI_SWIGLU,
                             moe.MOE_BF16, wl.k, 1)
    g_dn = moe.moe_gemm_desc(wl.E_loc, slots, wl.I, wl.H, moe.MOE_BF16, moe.MOE_EPI_STORE,
                             moe.MOE_F16_SCALED, 1, 1)
    _, wg, wu, wd = L.w_dev
    names = ["route", "permute", "gemm_gate_up", "gemm_down", "combine"]
    calls = [
        lambda: moe.moe_route(d, L.x, L.w_dev[0], L.bias, L.logits, L.ids, L.w, stream, L.rws),
        lambda: moe.moe_permute(d, L.ids, None, None, counts, offsets, s2r, r2f, None, None, pws,
                                stream),
        lambda: moe.moe_grouped_gemm(g_up, L.x, None, r2f, wg, None, wu, None, offsets, h, None,
                                     stream),
        lambda: moe.moe_grouped_gemm(g_dn, h, None, None, wd, None, None, None, offsets, y, None,
                                     stream),
        lambda: moe.moe_combine(d, moe.MOE_F16_SCALED, y, L.w, s2r, None, L.out, stream),
    ]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
          for _ in range(iters)]
    with torch.cuda.stream(stream):
        for c in calls:                       # warm
            c()
        torch.cuda.synchronize()
        for it in range(iters):
            ev[it][0].record(stream)
            for i, c in enumerate(calls):
                c()
                ev[it][i + 1].record(stream)
        torch.cuda.synchronize()
    ms = {n: float(np.mean([ev[it][i].elapsed_time(ev[it][i + 1]) for it in range(iters)]))
          for i, n in enumerate(names)}
    R = int(offsets[-1].item())
    cnt = counts.cpu().numpy()
    return ms, R, cnt


def compulsory_bytes(wl, counts):
    """Weights of the local experts with at least one row, router weight, x read once, out (fp32)
    written once, routing arrays."""
    active = int((counts > 0).sum())
    w = active * 3 * wl.I * wl.H * 2 + wl.E * wl.H * 2
    return w + wl.T * wl.H * 2 + wl.T * wl.H * 4 + wl.T * wl.k * 8


def layer_flops(wl, R):
    return 2.0 * wl.T * wl.H * wl.E + 6.0 * R * wl.H * wl.I + 6.0 * wl.T * wl.H * wl.I_s


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(L, target_s):
    import oracle
    wl = L.wl
    g, u, d = L.experts_np
    M = oracle.Mat
    desc = dict(T=wl.T, H=wl.H, E=wl.E, e0=wl.e0, E_loc=wl.E_loc, I=wl.I, k=wl.k, I_s=wl.I_s,
                scoring=wl.scoring, renormalize=wl.renormalize, act_fmt=oracle.BF16)
    mats = (M(oracle.F32, L.x_np), M(oracle.F32, g), M(oracle.F32, u), M(oracle.F32, d))
    rng = np.random.default_rng(123)
    n = 4
    while True:
        tok = np.sort(rng.choice(wl.T, n, replace=False)).astype(np.int32)
        t0 = time.perf_counter()
        oracle.moe_layer(desc, L.x_np, L.wr_np, L.bias_np, *mats, None, tok)
        dt = time.perf_counter() - t0
        if dt >= target_s * 0.5 or n >= wl.T:
            break
        n = int(min(wl.T, max(n * 2, n * target_s / max(dt, 1e-3) * 0.9)))
    return dict(value=n / dt, unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
                cpu_model=cpu_model(),
                sample=f"{n} random tokens of the same {wl.T}-token layer (routing, all local "
                       f"experts of each token, combine), fp64, {dt:.1f} s")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the layer is one GPU's "
              "expert slice and has no multi-GPU path; the whole-job value for N=1 is the one-GPU "
              "throughput.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.stream_ceiling:
        stream_ceiling(args.steps)
        return
    # the workload table first: its lines run in child processes, started before this process
    # touches the GPU
    table = None
    if not args.profile_only and not args.table_one and (not args.no_workloads or args.workloads):
        names = args.workloads.split(",") if args.workloads else None
        table = workload_table(max(5, min(args.steps, 20)), names)
    import torch
    import moe_inputs as mi

    stream = torch.cuda.Stream()
    if args.table_one:
        print(json.dumps(table_line(args.table_one, stream, args.steps)), flush=True)
        return
    wl = mi.WORKLOADS[args.workload]
    if args.profile_only and (wl.fmt != mi.FMT_BF16 or wl.I_s or wl.gated):
        # quantised layers and layers with a shared expert: the workload table's set-up, the same
        # calls as in the table
        tl = TableLayer(wl, stream)
        flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda") if args.flush else None
        with torch.cuda.stream(stream):
            for _ in range(args.warmup):
                tl.call()
            for _ in range(args.steps):
                if flush is not None:
                    flush.sum()
                tl.call()
        torch.cuda.synchronize()
        print(json.dumps({"workload": wl.name, "steps": args.steps, "flushed": bool(args.flush)}))
        return
    L = Layer(wl)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        L.step(stream)
    torch.cuda.synchronize()
    if args.profile_only and args.flush:
        flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        with torch.cuda.stream(stream):
            for _ in range(args.steps):
                flush.sum()
                L.step(stream)
        torch.cuda.synchronize()
        print(json.dumps({"workload": wl.name, "steps": args.steps, "flushed": True}))
        return
    t0 = time.perf_counter()
    for _ in range(args.steps):
        L.step(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    tokens_per_s = wl.T / (ms_per_step / 1e3)
    if args.profile_only:
        print(json.dumps({"workload": wl.name, "ms_per_step": ms_per_step}))
        return

    # per-call spread of the same layer (HIP events around each call on its stream), outside the
    # timed region above
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(max(5, min(args.steps, 50)))]
    with torch.cuda.stream(stream):
        for a, b in ev:
            a.record(stream)
            L.step(stream)
            b.record(stream)
    torch.cuda.synchronize()
    call_ms = np.array([a.elapsed_time(b) for a, b in ev])

    steps_ms, R, counts = step_breakdown(L, stream, max(5, min(args.steps, 20)))
    flops_gu = 4.0 * R * wl.H * wl.I
    achieved = flops_gu / (steps_ms["gemm_gate_up"] * 1e-3) / 1e12
    layer_tf = layer_flops(wl, R) / (ms_per_step * 1e-3) / 1e12
    traffic = measured_traffic() if args.workload == "C2p" else None

    result = {
        "metric": "MoE-layer tokens/s + % of MFMA peak (prefill) / % HBM BW (decode), 1 MI355X",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) tokens, N(0,0.02) weights, Zipf(1.1) router bias)",
        "config": {"workload": "Qwen3-235B-shaped MoE layer, EP=4 slice (experts 0-31 of 128), "
                               "prefill", "T": wl.T, "H": wl.H, "E": wl.E, "E_loc": wl.E_loc,
                   "I": wl.I, "k": wl.k, "router": "softmax top-8, renormalised",
                   "local_rows_R": R, "parallelism": "single GPU expert slice"},
        "layer_tflops": round(layer_tf, 1),
        "layer_frac_mfma": round(layer_tf / PEAK_BF16_TFLOPS, 4),
        "roofline": {"kernel": "grouped GEMM gate/up + SwiGLU (moe_grouped_gemm)",
                     "bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None if traffic is None else round(sum(traffic)),
                     "traffic_read_bytes": None if traffic is None else round(traffic[0]),
                     "traffic_write_bytes": None if traffic is None else round(traffic[1]),
                     "traffic_source": "committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary "
                                       "(profiles/gate_up_traffic.json) of the same kernel "
                                       "sources, not this run",
                     "flops_per_launch": flops_gu,
                     "avg_launch_ms": round(steps_ms["gemm_gate_up"], 4)},
        "steps_ms": {k: round(v, 4) for k, v in steps_ms.items()},
        "layer_call_ms": {"p10": round(float(np.percentile(call_ms, 10)), 4),
                          "median": round(float(np.median(call_ms)), 4),
                          "p90": round(float(np.percentile(call_ms, 90)), 4), "calls": len(call_ms)},
    }
    if not args.no_decode:
        dwl = mi.WORKLOADS[args.decode_workload]
        D = Layer(dwl, weights=L.shared_weights())
        flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        with torch.cuda.stream(stream):
            for _ in range(3):
                D.step(stream)
            for a, b in ev:
                flush.sum()                  # evict the weights from the caches between steps
                                             # (a read: written lines would be written back
                                             # during the measured step)
                a.record(stream)
                D.step(stream)
                b.record(stream)
        torch.cuda.synchronize()
        dcall = np.array([a.elapsed_time(b) for a, b in ev])
        dms = float(np.median(dcall))
        # the same call captured once into a HIP graph and replayed (same cache eviction between
        # replays): the launch sequence without host-side launch work
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            D.step(stream)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for a, b in ev:
                flush.sum()
                a.record(stream)
                graph.replay()
                b.record(stream)
        torch.cuda.synchronize()
        gcall = np.array([a.elapsed_time(b) for a, b in ev])
        del graph
        _, dR, dcounts = step_breakdown(D, stream, 5)
        dbytes = compulsory_bytes(dwl, dcounts)
        result["decode"] = {"workload": f"same layer, {dwl.T} tokens", "ms": round(dms, 4),
                            "tokens_per_s": round(dwl.T / (dms * 1e-3), 1), "local_rows_R": dR,
                            "compulsory_bytes": dbytes,
                            "hbm_gbps": round(dbytes / (dms * 1e-3) / 1e9, 1),
                            "frac_hbm": round(dbytes / (dms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                            "caches": "1 GiB read between steps",
                            "ms_p10": round(float(np.percentile(dcall, 10)), 4),
                            "ms_p90": round(float(np.percentile(dcall, 90)), 4),
                            "graph_replay_ms": round(float(np.median(gcall)), 4)}
        del D, flush
    if table is not None:
        result["workloads"] = table
    if not args.no_ep_sweep:
        result["decode_one_token_per_expert"] = ep_sweep(stream, max(5, min(args.steps, 20)))
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(L, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
