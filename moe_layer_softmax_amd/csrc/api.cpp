// api.cpp -- the C ABI of the MoE layer library: argument checks, workspace layout and the order
// of kernel launches. Nothing here synchronises the host with the device.
//
// Step order of the layer follows the pages: route, dispatch (count / index / copy), MoE GEMM,
// weighted combine ("Hosting Qwen on Blackwell", sections "MoE dispatch and combine" and
// "Expert parallel"; "CuTeDSL at Perplexity", section "MoE dispatch and combine"). The dispatch
// variant (one workgroup for small routing tables, split count/scan/scatter kernels for large
// ones) is chosen on the host from the table size, as the pages choose their decode and prefill
// dispatch kernels ("CuTeDSL at Perplexity", section on grid synchronisation).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>

#include "../../include/moe.h"
#include "kernels.hpp"

using namespace moe;

namespace {

thread_local int32_t g_last_hip_error = 0;

moe_status hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip_error = static_cast<int32_t>(e);
  return MOE_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool ok_ptr(const void* p) { return p != nullptr && aligned16(p); }
bool ok_opt(const void* p) { return p == nullptr || aligned16(p); }

size_t round_up(size_t v, size_t a = 256) { return (v + a - 1) / a * a; }

int io_bytes(int dt) { return dt == MOE_F32 ? 4 : 2; }

// block-scaled 8-bit / 4-bit formats (quantised codes + scales)
bool quantised(int dt) {
  return dt == MOE_FP8_E4M3 || dt == MOE_MXFP4 || dt == MOE_MXFP8 || dt == MOE_NVFP4;
}
// MX formats: one E8M0 scale byte per 32 elements along K
bool mx_format(int dt) { return dt == MOE_MXFP4 || dt == MOE_MXFP8; }
// formats whose layer re-quantises h into the expert format (NVFP4 keeps h in bf16)
bool h_quantised(int dt) { return dt == MOE_FP8_E4M3 || mx_format(dt); }
// bytes of one row of `cols` elements of a GEMM's A operand: NVFP4 activations enter the GEMM as
// their bf16 block values
long long a_row_bytes(int dt, long long cols);

// format of the per-slot expert outputs y inside moe_layer: fp32 for fp32 experts; scaled fp16
// rows for bf16 experts (a token's output sums up to k weighted rows plus the shared expert's,
// which partly cancel: rounding each row to bf16 measured ~2e-2 of the output RMS on the
// Qwen3.5-397B-shaped slices, while fp16 with a power-of-two scale per 64 columns keeps 2^-11 of
// each block's maximum at half the bytes of fp32); bf16 for the block-scaled formats
int y_dtype_of(const moe_desc* d) {
  if (d->expert_dtype == MOE_F32) return MOE_F32;
  return d->expert_dtype == MOE_BF16 ? MOE_F16_SCALED : MOE_BF16;
}
// bytes of one row of y (`cols` values) in format ydt
long long y_row_bytes(int ydt, long long cols) {
  if (ydt == MOE_F16_SCALED) return moe_f16_scaled_row_bytes(cols);
  return cols * (ydt == MOE_F32 ? 4 : 2);
}

// bytes of one activation row of `cols` elements in expert format dt
long long row_bytes(int dt, long long cols) {
  switch (dt) {
    case MOE_F32: return cols * 4;
    case MOE_BF16: return cols * 2;
    case MOE_FP8_E4M3: return cols;
    case MOE_MXFP4: return cols / 2;
    case MOE_MXFP8: return cols;
    case MOE_NVFP4: return cols / 2;
    default: return 0;
  }
}

long long a_row_bytes(int dt, long long cols) { return dt == MOE_NVFP4 ? cols * 2 : row_bytes(dt, cols); }

bool valid_io(int dt) { return dt == MOE_F32 || dt == MOE_BF16; }
bool valid_expert(int dt) {
  return dt == MOE_F32 || dt == MOE_BF16 || quantised(dt);
}

moe_status check_desc(const moe_desc* d) {
  if (!d) return MOE_ERR_INVALID_ARG;
  if (d->T < 0 || d->H <= 0 || d->E < 1 || d->E > 1024 || d->k < 1 || d->k > 16 || d->k > d->E)
    return MOE_ERR_INVALID_ARG;
  if (d->e0 < 0 || d->E_loc < 1 || d->e0 + d->E_loc > d->E) return MOE_ERR_INVALID_ARG;
  if (d->I <= 0 || d->I_s < 0) return MOE_ERR_INVALID_ARG;
  if (d->scoring != MOE_SOFTMAX && d->scoring != MOE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (d->renormalize != 0 && d->renormalize != 1) return MOE_ERR_INVALID_ARG;
  if (!valid_io(d->io_dtype) || !valid_io(d->out_dtype) || !valid_expert(d->expert_dtype))
    return MOE_ERR_INVALID_ARG;
  if ((long long)d->T * d->k >= (1ll << 31)) return MOE_ERR_INVALID_ARG;
  // the router and the expert GEMMs read 128-byte row slices
  const int kalign = d->io_dtype == MOE_F32 ? 16 : 64;
  if (d->H % kalign) return MOE_ERR_INVALID_ARG;
  if (d->H % 8) return MOE_ERR_INVALID_ARG;                 // combine: 4-column vectors
  return MOE_OK;
}

// K (and N) granularity of the expert GEMMs: one K-step row slice is 128 bytes for bf16 / fp8 /
// MXFP8 / MXFP4 (64 / 128 / 128 / 256 elements), 16 elements for fp32
int k_align(int dt) {
  switch (dt) {
    case MOE_F32: return 16;
    case MOE_BF16: return 64;
    case MOE_FP8_E4M3: return 128;
    case MOE_MXFP8: return 128;
    default: return 256;
  }
}

moe_status check_expert_shapes(const moe_desc* d) {
  const int dt = d->expert_dtype;
  if (dt == MOE_F32 && d->io_dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (dt != MOE_F32 && d->io_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  const int align = k_align(dt);
  if (d->H % align || d->I % align || (d->I_s && d->I_s % align)) return MOE_ERR_INVALID_ARG;
  if (d->I % 64 || d->H % 64 || d->I_s % 64) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// bytes between consecutive experts' scale arrays of an [N, K] weight matrix (NVFP4: the record of
// e4m3 block scales [N, K/16] followed by fp32 row scales [N])
long long scale_bytes(int dt, long long N, long long K) {
  if (dt == MOE_FP8_E4M3) return (N / 128) * (K / 128) * 4;
  if (mx_format(dt)) return N * (K / 32);
  if (dt == MOE_NVFP4) return N * (K / 16) + N * 4;
  return 0;
}

// The router of many bf16 tokens runs as a tiled GEMM (32 or 64 tokens x 128 experts per
// workgroup) once that gives at least half a workgroup per CU; fewer tokens use the K-split router
// kernel (widths in multiples of 16 experts); the fp32 router and other widths run as a grouped
// GEMM with one extra group.
bool router_tiled(const moe_desc* d) {
  return d->io_dtype == MOE_BF16 && (long long)((d->T + 31) / 32) * ((d->E + 127) / 128) >= 128;
}
bool router_fast(const moe_desc* d) {
  return d->io_dtype == MOE_BF16 && d->E % 16 == 0 && !router_tiled(d);
}
int route_splits(const moe_desc* d) { return router_fast(d) ? router_splits(d->T, d->H, d->E) : 1; }
size_t route_ws(const moe_desc* d) { return router_fast(d) ? router_ws_bytes(d->T, d->H, d->E) : 0; }

// ---- layer workspace layout (identical in the size query and in moe_layer) ----------------------
struct LayerWs {
  size_t logits, ids, w, rpart, counts, offsets, s2r, r2f, perm, xq, xs, h, hs, hsh, hshs, y, sw,
      total;
};

// The shared expert runs as an extra group inside the routed experts' GEMM launches when its
// intermediate size equals theirs (one N for all groups); otherwise in launches of its own, with
// its h in a separate [T, I_s] buffer.
bool shared_fused(const moe_desc* d) { return d->I_s > 0 && d->I_s == d->I; }
bool shared_apart(const moe_desc* d) { return d->I_s > 0 && d->I_s != d->I; }

LayerWs layer_ws(const moe_desc* d) {
  LayerWs L{};
  const size_t T = d->T, k = d->k, E = d->E, H = d->H, I = d->I;
  const size_t slots = T * k;
  const size_t rows = slots + (shared_fused(d) ? T : 0);
  const size_t Is = shared_apart(d) ? d->I_s : 0;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o += round_up(bytes); return at; };
  L.logits = take(T * E * 4);
  L.ids = take(slots * 4);
  L.w = take(slots * 4);
  L.rpart = take(route_ws(d));
  L.counts = take(d->E_loc * 4);
  L.offsets = take((d->E_loc + 1) * 4);
  L.s2r = take(slots * 4);
  L.r2f = take(slots * 4);
  L.perm = take(permute_ws_bytes(slots, d->E_loc));
  const int dt = d->expert_dtype;
  if (dt == MOE_FP8_E4M3) {
    L.xq = take(T * H);
    L.xs = take((T + 127) / 128 * (H / 128) * 4);
    L.h = take(rows * I);
    L.hs = take(rows * (I / 128) * 4);
    L.hsh = take(T * Is);
    L.hshs = take(T * (Is / 128) * 4);
  } else if (mx_format(dt)) {
    L.xq = take(row_bytes(dt, H) * T);
    L.xs = take(T * (H / 32));
    L.h = take(row_bytes(dt, I) * rows);
    L.hs = take(rows * (I / 32));
    L.hsh = take(row_bytes(dt, Is) * T);
    L.hshs = take(T * (Is / 32));
  } else if (dt == MOE_NVFP4) {
    // x as its bf16 block values and fp32 row scales; h in bf16
    L.xq = take(T * H * 2);
    L.xs = take(T * 4);
    L.h = take(rows * I * 2);
    L.hsh = take(T * Is * 2);
  } else {
    L.h = take(rows * I * io_bytes(d->io_dtype));
    L.hsh = take(T * Is * io_bytes(d->io_dtype));
  }
  // y: routed rows, then (with a shared expert) its T rows
  L.y = take((slots + (d->I_s ? T : 0)) * y_row_bytes(y_dtype_of(d), H));
  L.sw = take(d->I_s ? T * 4 : 0);
  L.total = o;
  return L;
}

// Router logits (+ top-k): logits = x . w_router^T + bias, then the top-k selection and weights.
// `partial` holds route_ws(d) bytes (the K-split partial sums of a few-token router).
moe_status run_route(const moe_desc* d, const void* x, const void* w_router, const float* bias,
                     float* logits, float* partial, int32_t* ids, float* w, hipStream_t s);

// logits = x . w_router^T + bias, as one extra-group GEMM with no routed groups
moe_status run_router(const moe_desc* d, const void* x, const void* w_router, const float* bias,
                      float* logits, hipStream_t s) {
  GemmArgs a{};
  a.dtype = d->io_dtype;
  a.epilogue = MOE_EPI_STORE;
  a.out_dtype = MOE_F32;
  a.K = d->H;
  a.N = d->E;
  a.A = x;
  a.a_pitch = (long long)d->H * io_bytes(d->io_dtype);
  a.a_row_div = 1;
  a.a_scale_rows = 1;
  a.G = 0;
  a.x_rows = d->T;
  a.x_row0 = 0;
  a.x_a_off = 0;
  a.xB = w_router;
  a.bias = bias;
  a.C = logits;
  a.c_pitch = (long long)d->E * 4;
  return hip_status(router_tiled(d) ? launch_gemm_router(a, s) : launch_gemm(a, s));
}

moe_status run_route(const moe_desc* d, const void* x, const void* w_router, const float* bias,
                     float* logits, float* partial, int32_t* ids, float* w, hipStream_t s) {
  int ns = 1;
  if (x) {
    if (router_fast(d)) {
      ns = route_splits(d);
      moe_status st = hip_status(launch_router(d->T, d->H, d->E, x, w_router, bias, logits, partial,
                                               ns, s));
      if (st != MOE_OK) return st;
    } else {
      moe_status st = run_router(d, x, w_router, bias, logits, s);
      if (st != MOE_OK) return st;
    }
  }
  return hip_status(launch_topk(d->T, d->E, d->k, d->scoring, d->renormalize, logits, partial, ns,
                                ns > 1 ? bias : nullptr, ids, w, s));
}

// Device scratch of the allocation-free layer entry point: one array per GPU the library runs on,
// kept until the process ends. Its name in host code is only a stand-in for the device symbol;
// host code uses the device address obtained once per device with hipGetSymbolAddress.
__device__ __align__(256) static unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// device address of the current device's scratch array (looked up on the device's first call)
moe_status scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (!ptr) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported combination";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int32_t moe_last_hip_error(void) { return g_last_hip_error; }

size_t moe_route_workspace_bytes(const moe_desc* d) {
  if (check_desc(d) != MOE_OK) return 0;
  return route_ws(d);
}

moe_status moe_route(const moe_desc* d, const void* x, const void* w_router, const float* bias,
                     float* logits, int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (!ok_ptr(logits) || !ok_ptr(topk_ids) || !ok_ptr(topk_w) || !ok_opt(x) || !ok_opt(bias) ||
      !ok_opt(ws))
    return d->T == 0 ? MOE_OK : MOE_ERR_INVALID_ARG;
  if (x && !ok_ptr(w_router)) return MOE_ERR_INVALID_ARG;
  if (d->T == 0) return MOE_OK;
  const size_t need = x ? route_ws(d) : 0;
  if (need && (!ws || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  return run_route(d, x, w_router, bias, logits, static_cast<float*>(ws), topk_ids, topk_w, stream);
}

size_t moe_permute_workspace_bytes(const moe_desc* d) {
  if (check_desc(d) != MOE_OK) return 0;
  return permute_ws_bytes((long long)d->T * d->k, d->E_loc);
}

moe_status moe_permute(const moe_desc* d, const int32_t* topk_ids, const void* a_in,
                       const void* a_in_scales, int32_t* counts, int32_t* offsets,
                       int32_t* slot_to_row, int32_t* row_to_flat, void* a_perm,
                       void* a_perm_scales, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (!ok_ptr(counts) || !ok_ptr(offsets)) return MOE_ERR_INVALID_ARG;
  const long long slots = (long long)d->T * d->k;
  if (slots > 0 && (!ok_ptr(topk_ids) || !ok_ptr(slot_to_row) || !ok_ptr(row_to_flat)))
    return MOE_ERR_INVALID_ARG;
  if (!ok_opt(a_perm) || !ok_opt(a_perm_scales) || !ok_opt(ws)) return MOE_ERR_INVALID_ARG;
  const int dt = d->expert_dtype;
  const bool quant = quantised(dt);
  if (a_perm) {
    if (!ok_ptr(a_in)) return MOE_ERR_INVALID_ARG;
    if (quant && (!ok_ptr(a_in_scales) || !ok_ptr(a_perm_scales))) return MOE_ERR_INVALID_ARG;
    if (quant && d->H % (dt == MOE_NVFP4 ? 64 : 128)) return MOE_ERR_INVALID_ARG;
    if (dt == MOE_F32 && d->io_dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
  }
  if (ws_bytes < permute_ws_bytes(slots, d->E_loc) || (slots > 16 * 1024 && !ws))
    return MOE_ERR_WORKSPACE;
  // (with no slots the maps kernel still writes zero counts and offsets)
  hipError_t e = launch_permute_maps(d->T, d->k, d->e0, d->E_loc, topk_ids, counts, offsets,
                                     slot_to_row, row_to_flat, ws, stream);
  if (e != hipSuccess || !a_perm) return hip_status(e);
  if (dt == MOE_NVFP4)
    return hip_status(launch_gather_nv4(slots, d->k, d->T, d->H, offsets + d->E_loc, row_to_flat,
                                        static_cast<const uint8_t*>(a_in),
                                        static_cast<const uint8_t*>(a_in_scales),
                                        static_cast<uint16_t*>(a_perm),
                                        static_cast<float*>(a_perm_scales), stream));
  long long sbytes = 0;
  int sblock = 1;
  if (dt == MOE_FP8_E4M3) { sbytes = (long long)(d->H / 128) * 4; sblock = 128; }
  if (mx_format(dt)) sbytes = d->H / 32;
  e = launch_gather_rows(slots, d->k, offsets + d->E_loc, row_to_flat, a_in, row_bytes(dt, d->H),
                         a_perm, quant ? a_in_scales : nullptr, sbytes, sblock,
                         quant ? a_perm_scales : nullptr, stream);
  return hip_status(e);
}

moe_status moe_grouped_gemm(const moe_gemm_desc* g, const void* A, const void* A_scales,
                            const int32_t* a_rows, const void* B, const void* B_scales,
                            const void* B2, const void* B2_scales, const int32_t* group_offsets,
                            void* C, void* C_scales, hipStream_t stream) {
  if (!g || g->G < 0 || g->max_rows < 0 || g->K <= 0 || g->N <= 0 || g->a_row_div < 1)
    return MOE_ERR_INVALID_ARG;
  if (!valid_expert(g->dtype)) return MOE_ERR_INVALID_ARG;
  if (g->epilogue != MOE_EPI_STORE && g->epilogue != MOE_EPI_SWIGLU) return MOE_ERR_INVALID_ARG;
  if (g->G == 0 || g->max_rows == 0) return MOE_OK;
  if (!ok_ptr(A) || !ok_ptr(B) || !ok_ptr(C) || !ok_ptr(group_offsets) || !ok_opt(a_rows))
    return MOE_ERR_INVALID_ARG;
  if (g->epilogue == MOE_EPI_SWIGLU && !ok_ptr(B2)) return MOE_ERR_INVALID_ARG;
  if (g->K % k_align(g->dtype) || g->N % 64) return MOE_ERR_INVALID_ARG;
  const bool quant = quantised(g->dtype);
  if (g->dtype == MOE_F32 && g->out_dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (g->dtype == MOE_NVFP4) {
    if (!ok_opt(A_scales) || !ok_ptr(B_scales)) return MOE_ERR_INVALID_ARG;
    if (g->epilogue == MOE_EPI_SWIGLU && !ok_ptr(B2_scales)) return MOE_ERR_INVALID_ARG;
    if (g->N % 128) return MOE_ERR_INVALID_ARG;
    if (g->out_dtype != MOE_F32 && g->out_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  } else if (quant) {
    if (!ok_ptr(A_scales) || !ok_ptr(B_scales)) return MOE_ERR_INVALID_ARG;
    if (g->epilogue == MOE_EPI_SWIGLU && !ok_ptr(B2_scales)) return MOE_ERR_INVALID_ARG;
    if (g->N % 128) return MOE_ERR_INVALID_ARG;
    if (g->dtype == MOE_FP8_E4M3 && g->a_scale_rows != 1 && g->a_scale_rows != 128)
      return MOE_ERR_INVALID_ARG;
    const bool requant = g->epilogue == MOE_EPI_SWIGLU && g->out_dtype == g->dtype;
    if (requant && !ok_ptr(C_scales)) return MOE_ERR_INVALID_ARG;
    if (!requant && g->out_dtype != MOE_BF16 && !(g->epilogue == MOE_EPI_STORE && g->out_dtype == MOE_F32))
      return MOE_ERR_UNSUPPORTED;
  } else if (g->out_dtype == MOE_F16_SCALED) {
    if (g->dtype != MOE_BF16 || g->epilogue != MOE_EPI_STORE) return MOE_ERR_UNSUPPORTED;
  } else if (g->out_dtype != MOE_F32 && g->out_dtype != MOE_BF16) {
    return MOE_ERR_UNSUPPORTED;
  }
  GemmArgs a{};
  a.dtype = g->dtype;
  a.epilogue = g->epilogue;
  a.out_dtype = g->out_dtype;
  a.K = g->K;
  a.N = g->N;
  a.A = A;
  a.A_scales = A_scales;
  a.a_pitch = a_row_bytes(g->dtype, g->K);
  a.a_scale_rows = g->a_scale_rows;
  a.a_rows = a_rows;
  a.a_row_div = g->a_row_div;
  a.G = g->G;
  a.offsets = group_offsets;
  a.max_rows = g->max_rows;
  a.B = B;
  a.Bs = B_scales;
  a.B2 = B2;
  a.B2s = B2_scales;
  a.b_stride = row_bytes(g->dtype, g->K) * (long long)g->N;
  a.bs_stride = scale_bytes(g->dtype, g->N, g->K);
  a.C = C;
  a.C_scales = C_scales;
  a.c_pitch = g->out_dtype == g->dtype && quant ? row_bytes(g->dtype, g->N) : y_row_bytes(g->out_dtype, g->N);
  return hip_status(launch_gemm(a, stream));
}

moe_status moe_combine(const moe_desc* d, int32_t y_dtype, const void* y, const float* topk_w,
                       const int32_t* slot_to_row, const void* shared, const float* shared_w,
                       void* out, hipStream_t stream) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (!valid_io(y_dtype) && y_dtype != MOE_F16_SCALED) return MOE_ERR_INVALID_ARG;
  if (y_dtype == MOE_F16_SCALED && d->H % 64) return MOE_ERR_INVALID_ARG;
  if (shared_w && !shared) return MOE_ERR_INVALID_ARG;
  if (d->T == 0) return MOE_OK;
  if (!ok_ptr(y) || !ok_ptr(topk_w) || !ok_ptr(slot_to_row) || !ok_ptr(out) || !ok_opt(shared) ||
      !ok_opt(shared_w))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine(d->T, d->H, d->k, y_dtype, d->out_dtype, y, topk_w, slot_to_row,
                                   shared, shared_w, out, stream));
}

int64_t moe_routing_blob_plane(const moe_desc* d) {
  if (check_desc(d) != MOE_OK) return 0;
  return ((int64_t)d->T * d->k + 3) / 4 * 4;
}

moe_status moe_shared_gate(const moe_desc* d, const void* x, const void* w_shared_gate,
                           float* shared_w, hipStream_t stream) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;
  if (!ok_ptr(x) || !ok_ptr(w_shared_gate) || !ok_ptr(shared_w)) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_shared_gate(d->T, d->H, d->io_dtype, x, w_shared_gate, shared_w,
                                       stream));
}

moe_status moe_quantize(int32_t dst_dtype, int32_t src_dtype, int32_t batch, int32_t rows,
                        int32_t cols, int32_t block_rows, const void* src, void* codes,
                        void* scales, hipStream_t stream) {
  if (batch < 0 || rows < 0 || cols <= 0) return MOE_ERR_INVALID_ARG;
  if (src_dtype != MOE_F32 && src_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (batch == 0 || rows == 0) return MOE_OK;
  if (!ok_ptr(src) || !ok_ptr(codes) || !ok_ptr(scales)) return MOE_ERR_INVALID_ARG;
  if (dst_dtype == MOE_FP8_E4M3) {
    if (cols % 128 || (block_rows != 1 && block_rows != 128)) return MOE_ERR_INVALID_ARG;
    return hip_status(launch_quant_fp8(src_dtype, batch, rows, cols, block_rows, src,
                                       static_cast<uint8_t*>(codes), static_cast<float*>(scales),
                                       stream));
  }
  if (dst_dtype == MOE_MXFP4) {
    if (cols % 32) return MOE_ERR_INVALID_ARG;
    return hip_status(launch_quant_mx4(src_dtype, batch, rows, cols, src,
                                       static_cast<uint8_t*>(codes), static_cast<uint8_t*>(scales),
                                       stream));
  }
  if (dst_dtype == MOE_MXFP8) {
    if (cols % 32) return MOE_ERR_INVALID_ARG;
    return hip_status(launch_quant_mx8(src_dtype, batch, rows, cols, src,
                                       static_cast<uint8_t*>(codes), static_cast<uint8_t*>(scales),
                                       stream));
  }
  if (dst_dtype == MOE_NVFP4) {
    if (cols % 64) return MOE_ERR_INVALID_ARG;
    return hip_status(launch_quant_nv4(src_dtype, batch, rows, cols, src,
                                       static_cast<uint8_t*>(codes), static_cast<uint8_t*>(scales),
                                       nullptr, kNv4Packed, stream));
  }
  return MOE_ERR_INVALID_ARG;
}

size_t moe_layer_workspace_bytes(const moe_desc* d) {
  if (check_desc(d) != MOE_OK) return 0;
  return layer_ws(d).total;
}

moe_status moe_layer(const moe_desc* d, const moe_weights* w, const void* x, const float* bias,
                     void* out, float* logits, int32_t* topk_ids, float* topk_w, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (!w) return MOE_ERR_INVALID_ARG;
  st = check_expert_shapes(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;
  const bool quant = quantised(d->expert_dtype);
  if (!ok_ptr(x) || !ok_ptr(out) || !ok_ptr(w->w_router) || !ok_ptr(w->w_gate) ||
      !ok_ptr(w->w_up) || !ok_ptr(w->w_down) || !ok_opt(bias) || !ok_opt(logits) ||
      !ok_opt(topk_ids) || !ok_opt(topk_w) || !ok_ptr(ws))
    return MOE_ERR_INVALID_ARG;
  if (quant && (!ok_ptr(w->w_gate_scales) || !ok_ptr(w->w_up_scales) ||
                !ok_ptr(w->w_down_scales)))
    return MOE_ERR_INVALID_ARG;
  if (d->I_s && (!ok_ptr(w->sh_gate) || !ok_ptr(w->sh_up) || !ok_ptr(w->sh_down) ||
                 !ok_opt(w->w_shared_gate)))
    return MOE_ERR_INVALID_ARG;
  if (d->I_s && quant && (!ok_ptr(w->sh_gate_scales) || !ok_ptr(w->sh_up_scales) ||
                          !ok_ptr(w->sh_down_scales)))
    return MOE_ERR_INVALID_ARG;
  const LayerWs L = layer_ws(d);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  char* base = static_cast<char*>(ws);
  float* lg = logits ? logits : reinterpret_cast<float*>(base + L.logits);
  int32_t* ids = topk_ids ? topk_ids : reinterpret_cast<int32_t*>(base + L.ids);
  float* tw = topk_w ? topk_w : reinterpret_cast<float*>(base + L.w);
  int32_t* counts = reinterpret_cast<int32_t*>(base + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + L.offsets);
  int32_t* s2r = reinterpret_cast<int32_t*>(base + L.s2r);
  int32_t* r2f = reinterpret_cast<int32_t*>(base + L.r2f);
  const int T = d->T, k = d->k, H = d->H, I = d->I;
  const int slots = T * k;
  const int io = d->io_dtype, dt = d->expert_dtype;
  const bool hq = h_quantised(dt);

  // 1. route
  st = run_route(d, x, w->w_router, bias, lg, reinterpret_cast<float*>(base + L.rpart), ids, tw,
                 stream);
  if (st != MOE_OK) return st;
  // 2. dispatch maps (the rows themselves are gathered inside the gate/up GEMM)
  st = hip_status(launch_permute_maps(T, k, d->e0, d->E_loc, ids, counts, offsets, s2r, r2f,
                                      base + L.perm, stream));
  if (st != MOE_OK) return st;

  // 3. activations for the expert GEMMs: x itself, or x quantised once in token order (fp8 with
  //    128-token x 128-channel blocks, MXFP4 / MXFP8 with 1 x 32 groups) before the rows are
  //    dispatched
  const void* xa = x;
  const void* xs = nullptr;
  if (dt == MOE_FP8_E4M3) {
    st = hip_status(launch_quant_fp8(io, 1, T, H, 128, x, reinterpret_cast<uint8_t*>(base + L.xq),
                                     reinterpret_cast<float*>(base + L.xs), stream));
    xa = base + L.xq;
    xs = base + L.xs;
  } else if (dt == MOE_MXFP4) {
    st = hip_status(launch_quant_mx4(io, 1, T, H, x, reinterpret_cast<uint8_t*>(base + L.xq),
                                     reinterpret_cast<uint8_t*>(base + L.xs), stream));
    xa = base + L.xq;
    xs = base + L.xs;
  } else if (dt == MOE_MXFP8) {
    st = hip_status(launch_quant_mx8(io, 1, T, H, x, reinterpret_cast<uint8_t*>(base + L.xq),
                                     reinterpret_cast<uint8_t*>(base + L.xs), stream));
    xa = base + L.xq;
    xs = base + L.xs;
  } else if (dt == MOE_NVFP4) {
    // NVFP4 per token, kept as the fp16 block values the gate/up GEMM consumes (exact; its weights
    // are then dequantised to fp16 too, one packed multiply per two elements) plus the row scales
    st = hip_status(launch_quant_nv4(io, 1, T, H, x, reinterpret_cast<uint8_t*>(base + L.xq),
                                     nullptr, reinterpret_cast<float*>(base + L.xs), kNv4ValuesF16,
                                     stream));
    xa = base + L.xq;
    xs = base + L.xs;
  }
  if (st != MOE_OK) return st;

  // 4. gate/up GEMM with the SwiGLU epilogue; routed rows gather the activations through
  //    row_to_flat / k, shared-expert rows (C rows slots..slots+T) read them in token order. h
  //    leaves in the down projection's input format (bf16 / fp32, or re-quantised fp8 / MXFP4 /
  //    MXFP8; bf16 for NVFP4).
  GemmArgs a{};
  a.dtype = dt;
  a.epilogue = MOE_EPI_SWIGLU;
  a.out_dtype = hq ? dt : (dt == MOE_F32 ? MOE_F32 : MOE_BF16);
  a.K = H;
  a.N = I;
  a.A = xa;
  a.A_scales = xs;
  a.a_pitch = a_row_bytes(dt, H);
  a.a_f16 = dt == MOE_NVFP4 ? 1 : 0;
  a.a_scale_rows = dt == MOE_FP8_E4M3 ? 128 : 1;
  a.a_rows = r2f;
  a.a_row_div = k;
  a.G = d->E_loc;
  a.offsets = offsets;
  a.max_rows = slots;
  // tile shapes are chosen for the rows this GPU's slice receives under balanced routing; the
  // grid still covers every slot, so skewed routing only changes the speed
  a.expected_rows = static_cast<int>(std::min<long long>(slots, ((long long)slots * d->E_loc + d->E - 1) / d->E));
  a.B = w->w_gate;
  a.Bs = w->w_gate_scales;
  a.B2 = w->w_up;
  a.B2s = w->w_up_scales;
  a.b_stride = row_bytes(dt, H) * (long long)I;
  a.bs_stride = scale_bytes(dt, I, H);
  if (shared_fused(d)) {
    a.x_rows = T;
    a.x_row0 = slots;
    a.x_a_off = slots;
    a.xB = w->sh_gate;
    a.xBs = w->sh_gate_scales;
    a.xB2 = w->sh_up;
    a.xB2s = w->sh_up_scales;
  }
  a.C = base + L.h;
  a.C_scales = hq ? base + L.hs : nullptr;
  a.c_pitch = hq ? row_bytes(dt, I) : (long long)I * io_bytes(io);
  st = hip_status(launch_gemm(a, stream));
  if (st != MOE_OK) return st;
  const long long hsh_pitch = hq ? row_bytes(dt, d->I_s) : (long long)d->I_s * io_bytes(io);
  if (shared_apart(d)) {
    // the shared expert alone: no routed groups, one extra group of T rows in token order
    GemmArgs sa = a;
    sa.N = d->I_s;
    sa.a_rows = nullptr;
    sa.a_row_div = 1;
    sa.G = 0;
    sa.offsets = nullptr;
    sa.max_rows = 0;
    sa.expected_rows = 0;
    sa.B = sa.B2 = sa.Bs = sa.B2s = nullptr;
    sa.x_rows = T;
    sa.x_row0 = 0;
    sa.x_a_off = 0;
    sa.xB = w->sh_gate;
    sa.xBs = w->sh_gate_scales;
    sa.xB2 = w->sh_up;
    sa.xB2s = w->sh_up_scales;
    sa.C = base + L.hsh;
    sa.C_scales = hq ? base + L.hshs : nullptr;
    sa.c_pitch = hsh_pitch;
    st = hip_status(launch_gemm(sa, stream));
    if (st != MOE_OK) return st;
  }

  // 5. down GEMM: y rows = h rows
  const int ydt = y_dtype_of(d);
  GemmArgs b{};
  b.dtype = dt;
  b.epilogue = MOE_EPI_STORE;
  b.out_dtype = ydt;
  b.K = I;
  b.N = H;
  b.A = base + L.h;
  b.A_scales = hq ? base + L.hs : nullptr;
  b.a_pitch = hq ? row_bytes(dt, I) : (long long)I * io_bytes(io);
  b.a_scale_rows = 1;
  b.a_row_div = 1;
  b.G = d->E_loc;
  b.offsets = offsets;
  b.max_rows = slots;
  b.expected_rows = a.expected_rows;
  b.B = w->w_down;
  b.Bs = w->w_down_scales;
  b.b_stride = row_bytes(dt, I) * (long long)H;
  b.bs_stride = scale_bytes(dt, H, I);
  if (shared_fused(d)) {
    b.x_rows = T;
    b.x_row0 = slots;
    b.x_a_off = 0;
    b.xB = w->sh_down;
    b.xBs = w->sh_down_scales;
  }
  b.C = base + L.y;
  b.c_pitch = y_row_bytes(ydt, H);
  st = hip_status(launch_gemm(b, stream));
  if (st != MOE_OK) return st;
  if (shared_apart(d)) {
    // shared rows of y (rows slots .. slots + T) from the shared h [T, I_s]
    GemmArgs sb = b;
    sb.K = d->I_s;
    sb.A = base + L.hsh;
    sb.A_scales = hq ? base + L.hshs : nullptr;
    sb.a_pitch = hsh_pitch;
    sb.G = 0;
    sb.offsets = nullptr;
    sb.max_rows = 0;
    sb.expected_rows = 0;
    sb.B = sb.Bs = nullptr;
    sb.x_rows = T;
    sb.x_row0 = slots;
    sb.x_a_off = slots;
    sb.xB = w->sh_down;
    sb.xBs = w->sh_down_scales;
    st = hip_status(launch_gemm(sb, stream));
    if (st != MOE_OK) return st;
  }

  // 6. combine (+ shared expert rows, times their per-token gate when the layer has one)
  const void* shared = d->I_s ? base + L.y + (size_t)slots * y_row_bytes(ydt, H) : nullptr;
  float* sw = nullptr;
  if (d->I_s && w->w_shared_gate) {
    sw = reinterpret_cast<float*>(base + L.sw);
    st = hip_status(launch_shared_gate(T, H, io, x, w->w_shared_gate, sw, stream));
    if (st != MOE_OK) return st;
  }
  return hip_status(launch_combine(T, H, k, ydt, d->out_dtype, base + L.y, tw, s2r, shared, sw,
                                   out, stream));
}

moe_status moe_layer_noalloc(const moe_desc* d, const moe_weights* w, const void* x,
                             const float* bias, void* out, float* logits, int32_t* topk_ids,
                             float* topk_w, hipStream_t stream) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return moe_layer(d, w, x, bias, out, logits, topk_ids, topk_w, nullptr, 0, stream);
  if (layer_ws(d).total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != MOE_OK) return st;
  return moe_layer(d, w, x, bias, out, logits, topk_ids, topk_w, ws, MOE_NOALLOC_SCRATCH_BYTES,
                   stream);
}

}  // extern "C"
