// combine.hip -- weighted un-permute back to token order on gfx950.
//
// "CuTeDSL at Perplexity", section "MoE dispatch and combine": the combine is a vectorised
// weighted accumulation in registers that reads the routing information and the positions the
// dispatch computed, writing the final tokens to the output buffer. Here each workgroup owns one
// token: its k rows (found through slot_to_row) are read with 16-byte loads, accumulated in fp32 in
// slot order j = 0..k-1, the shared expert row added last, and the sum rounded once.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

template <bool Y_BF16, bool OUT_BF16>
__global__ void __launch_bounds__(256) combine_kernel(int H, int k, const void* __restrict__ y,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ slot_to_row,
                                                      const void* __restrict__ shared,
                                                      void* __restrict__ out) {
  const int t = blockIdx.x;
  __shared__ int rows[16];
  __shared__ float wts[16];
  if (threadIdx.x < k) {
    rows[threadIdx.x] = slot_to_row[(size_t)t * k + threadIdx.x];
    wts[threadIdx.x] = w[(size_t)t * k + threadIdx.x];
  }
  __syncthreads();
  for (int c0 = threadIdx.x * 8; c0 < H; c0 += 256 * 8) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int r = rows[j];
      if (r < 0) continue;
      const float wj = wts[j];
      if (Y_BF16) {
        const i32x4 v = *reinterpret_cast<const i32x4*>(static_cast<const uint16_t*>(y) + (size_t)r * H + c0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += wj * __uint_as_float(static_cast<uint32_t>(v[i]) << 16);
          acc[2 * i + 1] += wj * __uint_as_float(static_cast<uint32_t>(v[i]) & 0xFFFF0000u);
        }
      } else {
        const float* yr = static_cast<const float*>(y) + (size_t)r * H + c0;
        const f32x4 a = *reinterpret_cast<const f32x4*>(yr);
        const f32x4 b = *reinterpret_cast<const f32x4*>(yr + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) { acc[i] += wj * a[i]; acc[4 + i] += wj * b[i]; }
      }
    }
    if (shared) {
      if (Y_BF16) {
        const i32x4 v = *reinterpret_cast<const i32x4*>(static_cast<const uint16_t*>(shared) + (size_t)t * H + c0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += __uint_as_float(static_cast<uint32_t>(v[i]) << 16);
          acc[2 * i + 1] += __uint_as_float(static_cast<uint32_t>(v[i]) & 0xFFFF0000u);
        }
      } else {
        const float* sr = static_cast<const float*>(shared) + (size_t)t * H + c0;
        const f32x4 a = *reinterpret_cast<const f32x4*>(sr);
        const f32x4 b = *reinterpret_cast<const f32x4*>(sr + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) { acc[i] += a[i]; acc[4 + i] += b[i]; }
      }
    }
    if (OUT_BF16) {
      i32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = static_cast<int>(pack_bf16x2(acc[2 * i], acc[2 * i + 1]));
      *reinterpret_cast<i32x4*>(static_cast<uint16_t*>(out) + (size_t)t * H + c0) = o;
    } else {
      float* orow = static_cast<float*>(out) + (size_t)t * H + c0;
      *reinterpret_cast<f32x4*>(orow) = f32x4{acc[0], acc[1], acc[2], acc[3]};
      *reinterpret_cast<f32x4*>(orow + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    }
  }
}

hipError_t launch_combine(int T, int H, int k, int y_dtype, int out_dtype, const void* y,
                          const float* w, const int32_t* slot_to_row, const void* shared,
                          void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const bool yb = y_dtype == MOE_BF16, ob = out_dtype == MOE_BF16;
  if (yb && ob) combine_kernel<true, true><<<T, 256, 0, s>>>(H, k, y, w, slot_to_row, shared, out);
  else if (yb) combine_kernel<true, false><<<T, 256, 0, s>>>(H, k, y, w, slot_to_row, shared, out);
  else if (ob) combine_kernel<false, true><<<T, 256, 0, s>>>(H, k, y, w, slot_to_row, shared, out);
  else combine_kernel<false, false><<<T, 256, 0, s>>>(H, k, y, w, slot_to_row, shared, out);
  return hipGetLastError();
}

}  // namespace moe
