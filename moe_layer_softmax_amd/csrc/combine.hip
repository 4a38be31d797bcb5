// combine.hip -- weighted un-permute back to token order on gfx950.
//
// "CuTeDSL at Perplexity", section "MoE dispatch and combine": the combine is a vectorised
// weighted accumulation in registers that reads the routing information and the positions the
// dispatch computed, writing the final tokens to the output buffer. Here a token's k rows (found
// through slot_to_row) are read with 16-byte (fp32) or 8-byte (bf16) loads per lane, accumulated in
// fp32 in slot order j = 0..k-1, the shared expert row added last, and the sum rounded once.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// Workgroup (t, c): token t, columns [c * 1024, c * 1024 + 1024), four per thread. All k rows'
// loads are issued before the first is added (unconditional: a non-local slot reads row 0 and adds
// nothing), so one token's latency is one memory round trip.
template <bool Y_BF16, bool OUT_BF16>
__global__ void __launch_bounds__(256) combine_kernel(int H, int k, const void* __restrict__ y,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ slot_to_row,
                                                      const void* __restrict__ shared,
                                                      void* __restrict__ out) {
  constexpr int KMAX = 16;
  const int t = blockIdx.x;
  const int c0 = blockIdx.y * 1024 + threadIdx.x * 4;
  __shared__ int rows[KMAX];
  __shared__ float wts[KMAX];
  if (threadIdx.x < KMAX) {
    const bool in = threadIdx.x < k;
    rows[threadIdx.x] = in ? slot_to_row[(size_t)t * k + threadIdx.x] : -1;
    wts[threadIdx.x] = in ? w[(size_t)t * k + threadIdx.x] : 0.0f;
  }
  __syncthreads();
  if (c0 >= H) return;
  f32x4 v[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
      const long long r = rows[j] < 0 ? 0 : rows[j];
      if (Y_BF16) {
        const uint2 b = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(y) + r * H + c0);
        v[j] = f32x4{__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xFFFF0000u),
                     __uint_as_float(b.y << 16), __uint_as_float(b.y & 0xFFFF0000u)};
      } else {
        v[j] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(y) + r * H + c0);
      }
    }
  }
  f32x4 sh = f32x4{};
  if (shared) {
    if (Y_BF16) {
      const uint2 b = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(shared) + (size_t)t * H + c0);
      sh = f32x4{__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xFFFF0000u),
                 __uint_as_float(b.y << 16), __uint_as_float(b.y & 0xFFFF0000u)};
    } else {
      sh = *reinterpret_cast<const f32x4*>(static_cast<const float*>(shared) + (size_t)t * H + c0);
    }
  }
  // fp32 accumulation in slot order j = 0..k-1, the shared row last, one rounding
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k && rows[j] >= 0) {
      const float wj = wts[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += wj * v[j][i];
    }
  }
  if (shared) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += sh[i];
  }
  if (OUT_BF16) {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + (size_t)t * H + c0) =
        make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + (size_t)t * H + c0) =
        f32x4{acc[0], acc[1], acc[2], acc[3]};
  }
}

hipError_t launch_combine(int T, int H, int k, int y_dtype, int out_dtype, const void* y,
                          const float* w, const int32_t* slot_to_row, const void* shared,
                          void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const bool yb = y_dtype == MOE_BF16, ob = out_dtype == MOE_BF16;
  dim3 grid(T, (H + 1023) / 1024), block(256);
  if (yb && ob) combine_kernel<true, true><<<grid, block, 0, s>>>(H, k, y, w, slot_to_row, shared, out);
  else if (yb) combine_kernel<true, false><<<grid, block, 0, s>>>(H, k, y, w, slot_to_row, shared, out);
  else if (ob) combine_kernel<false, true><<<grid, block, 0, s>>>(H, k, y, w, slot_to_row, shared, out);
  else combine_kernel<false, false><<<grid, block, 0, s>>>(H, k, y, w, slot_to_row, shared, out);
  return hipGetLastError();
}

}  // namespace moe
