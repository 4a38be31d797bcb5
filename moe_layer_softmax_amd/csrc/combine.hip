// combine.hip -- weighted un-permute back to token order on gfx950.
//
// "CuTeDSL at Perplexity", section "MoE dispatch and combine": the combine is a vectorised
// weighted accumulation in registers that reads the routing information and the positions the
// dispatch computed, writing the final tokens to the output buffer. Here a token's k rows (found
// through slot_to_row) are read with 16-byte (fp32) or 8-byte (bf16) loads per lane, accumulated in
// fp32 in slot order j = 0..k-1, the shared expert row added last (times its per-token gate when
// one is given), and the sum rounded once.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// Workgroup (t, c): token t, columns [c * 256 * CPL, (c + 1) * 256 * CPL), CPL per thread (8 for
// bf16 rows, 4 for fp32: one 16-byte load per row). All KMAX rows' loads are issued before the
// first is added (unconditional: a non-local slot, and a slot j >= k, reads row 0 and adds
// nothing), so one token's latency is one memory round trip. KMAX (8 or 16) bounds k: the k rows' values are held in registers, and
// with KMAX = 8 twice as many waves fit on a CU to keep loads in flight.
template <bool Y_BF16, bool OUT_BF16, int KMAX>
__global__ void __launch_bounds__(256) combine_kernel(int H, int k, const void* __restrict__ y,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ slot_to_row,
                                                      const void* __restrict__ shared,
                                                      const float* __restrict__ shared_w,
                                                      void* __restrict__ out) {
  constexpr int CPL = Y_BF16 ? 8 : 4;
  const int t = blockIdx.x;
  const int c0 = (blockIdx.y * 256 + threadIdx.x) * CPL;
  __shared__ int rows[KMAX];
  __shared__ float wts[KMAX];
  if (threadIdx.x < KMAX) {
    const bool in = threadIdx.x < k;
    rows[threadIdx.x] = in ? slot_to_row[(size_t)t * k + threadIdx.x] : -1;
    wts[threadIdx.x] = in ? w[(size_t)t * k + threadIdx.x] : 0.0f;
  }
  __syncthreads();
  if (c0 >= H) return;                      // H % 8 == 0: a thread's columns are all in or all out
  // raw 16-byte row pieces (bf16 values are widened only when added, which keeps the registers
  // per row at four)
  auto load_raw = [&](const void* base, long long r) -> i32x4 {
    if (Y_BF16) return *reinterpret_cast<const i32x4*>(static_cast<const uint16_t*>(base) + r * H + c0);
    return *reinterpret_cast<const i32x4*>(static_cast<const float*>(base) + r * H + c0);
  };
  auto widen = [&](const i32x4& b, float* v) {
    if (Y_BF16) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[2 * q] = __uint_as_float(static_cast<uint32_t>(b[q]) << 16);
        v[2 * q + 1] = __uint_as_float(static_cast<uint32_t>(b[q]) & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = __int_as_float(b[q]);
    }
  };
  i32x4 raw[KMAX];                          // y holds T * k >= 1 rows, so row 0 exists
#pragma unroll
  for (int j = 0; j < KMAX; ++j) raw[j] = load_raw(y, rows[j] < 0 ? 0 : rows[j]);
  i32x4 sh_raw = {};
  if (shared) sh_raw = load_raw(shared, t);
  // fp32 accumulation in slot order j = 0..k-1, the shared row last, one rounding
  float acc[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k && rows[j] >= 0) {
      const float wj = wts[j];
      float v[CPL];
      widen(raw[j], v);
#pragma unroll
      for (int i = 0; i < CPL; ++i) acc[i] += wj * v[i];
    }
  }
  float sh[CPL];
  widen(sh_raw, sh);
  if (shared) {
    const float gs = shared_w ? shared_w[t] : 1.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) acc[i] += gs * sh[i];
  }
  if (OUT_BF16) {
    uint32_t o[CPL / 2];
#pragma unroll
    for (int i = 0; i < CPL / 2; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
    uint16_t* dst = static_cast<uint16_t*>(out) + (size_t)t * H + c0;
    if (CPL == 8) *reinterpret_cast<i32x4*>(dst) = i32x4{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
    else *reinterpret_cast<uint2*>(dst) = make_uint2(o[0], o[1]);
  } else {
    float* dst = static_cast<float*>(out) + (size_t)t * H + c0;
#pragma unroll
    for (int q = 0; q < CPL / 4; ++q)
      *reinterpret_cast<f32x4*>(dst + 4 * q) = f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
  }
}

hipError_t launch_combine(int T, int H, int k, int y_dtype, int out_dtype, const void* y,
                          const float* w, const int32_t* slot_to_row, const void* shared,
                          const float* shared_w, void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const bool yb = y_dtype == MOE_BF16, ob = out_dtype == MOE_BF16;
  const int cols_per_wg = 256 * (yb ? 8 : 4);
  dim3 grid(T, (H + cols_per_wg - 1) / cols_per_wg), block(256);
  auto k_ = combine_kernel<false, false, 16>;
  if (k <= 8) {
    k_ = combine_kernel<false, false, 8>;
    if (yb && ob) k_ = combine_kernel<true, true, 8>;
    else if (yb) k_ = combine_kernel<true, false, 8>;
    else if (ob) k_ = combine_kernel<false, true, 8>;
  } else {
    if (yb && ob) k_ = combine_kernel<true, true, 16>;
    else if (yb) k_ = combine_kernel<true, false, 16>;
    else if (ob) k_ = combine_kernel<false, true, 16>;
  }
  k_<<<grid, block, 0, s>>>(H, k, y, w, slot_to_row, shared, shared_w, out);
  return hipGetLastError();
}

}  // namespace moe
