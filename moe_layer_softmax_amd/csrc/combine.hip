// combine.hip -- weighted un-permute back to token order on gfx950.
//
// "CuTeDSL at Perplexity", section "MoE dispatch and combine": the combine is a vectorised
// weighted accumulation in registers that reads the routing information and the positions the
// dispatch computed, writing the final tokens to the output buffer. Here a token's k rows (found
// through slot_to_row) are read with one 16-byte load per lane and row (4 fp32 or 8 bf16 / fp16
// values), accumulated in fp32 in slot order j = 0..k-1, the shared expert row added last (times
// its per-token gate when one is given), and the sum rounded once.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// Row formats of y (and of the shared rows)
enum { kYF32 = 0, kYBf16 = 1, kYF16S = 2 };

// Workgroup (t, c): token t, columns [c * 256 * CPL, (c + 1) * 256 * CPL), CPL per thread (8 for
// bf16 and scaled fp16 rows, 4 for fp32: one 16-byte load per row). All KMAX rows' loads are issued
// before the first is added (unconditional: a non-local slot, and a slot j >= k, reads row 0 and
// adds nothing), so one token's latency is one memory round trip. KMAX (8, 12 or 16) bounds k: the
// k rows' values are held in registers, and the smallest KMAX >= k is launched, so that fewer
// registers per wave let more waves keep loads in flight and no more dead loads are issued than
// needed. Scaled fp16 rows (MOE_F16_SCALED) also load the fp32 scale of the thread's
// 64-column block, which multiplies the row's weight (a power of two: exact).
template <int YF, bool OUT_BF16, int KMAX>
__global__ void __launch_bounds__(256) combine_kernel(int H, int k, long long pitch, const void* __restrict__ y,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ slot_to_row,
                                                      const void* __restrict__ shared,
                                                      const float* __restrict__ shared_w,
                                                      void* __restrict__ out) {
  constexpr int CPL = YF == kYF32 ? 4 : 8;
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
  // raw 16-byte row pieces (bf16 and fp16 values are widened only when added, which keeps the
  // registers per row at four); rows are `pitch` bytes apart
  auto row_at = [&](const void* base, long long r) -> const char* {
    return static_cast<const char*>(base) + r * pitch;
  };
  auto load_raw = [&](const void* base, long long r) -> i32x4 {
    return *reinterpret_cast<const i32x4*>(row_at(base, r) + (long long)c0 * (YF == kYF32 ? 4 : 2));
  };
  auto load_scale = [&](const void* base, long long r) -> float {
    if constexpr (YF == kYF16S) return *reinterpret_cast<const float*>(row_at(base, r) + (long long)H * 2 + (c0 / 64) * 4);
    else return 1.0f;
  };
  auto widen = [&](const i32x4& b, float* v) {
    if constexpr (YF == kYBf16) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[2 * q] = __uint_as_float(static_cast<uint32_t>(b[q]) << 16);
        v[2 * q + 1] = __uint_as_float(static_cast<uint32_t>(b[q]) & 0xFFFF0000u);
      }
    } else if constexpr (YF == kYF16S) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // through a scalar copy: hipcc miscompiles a bit cast of a vector element in place (every
        // q read element 0)
        const int bits = b[q];
        const f16x2 h = __builtin_bit_cast(f16x2, bits);
        v[2 * q] = static_cast<float>(h[0]);
        v[2 * q + 1] = static_cast<float>(h[1]);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = __int_as_float(b[q]);
    }
  };
  i32x4 raw[KMAX];                          // y holds T * k >= 1 rows, so row 0 exists
  float scl[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const long long r = rows[j] < 0 ? 0 : rows[j];
    raw[j] = load_raw(y, r);
    scl[j] = load_scale(y, r);
  }
  i32x4 sh_raw = {};
  float sh_scl = 1.0f;
  if (shared) {
    sh_raw = load_raw(shared, t);
    sh_scl = load_scale(shared, t);
  }
  // fp32 accumulation in slot order j = 0..k-1, the shared row last, one rounding
  float acc[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k && rows[j] >= 0) {
      const float wj = wts[j] * scl[j];
      float v[CPL];
      widen(raw[j], v);
#pragma unroll
      for (int i = 0; i < CPL; ++i) acc[i] += wj * v[i];
    }
  }
  float sh[CPL];
  widen(sh_raw, sh);
  if (shared) {
    const float gs = (shared_w ? shared_w[t] : 1.0f) * sh_scl;
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

template <int YF>
hipError_t run_combine(int T, int H, int k, bool ob, long long pitch, const void* y, const float* w,
                       const int32_t* slot_to_row, const void* shared, const float* shared_w,
                       void* out, hipStream_t s) {
  const int cols_per_wg = 256 * (YF == kYF32 ? 4 : 8);
  dim3 grid(T, (H + cols_per_wg - 1) / cols_per_wg), block(256);
  auto k_ = k <= 8    ? (ob ? combine_kernel<YF, true, 8> : combine_kernel<YF, false, 8>)
            : k <= 12 ? (ob ? combine_kernel<YF, true, 12> : combine_kernel<YF, false, 12>)
                      : (ob ? combine_kernel<YF, true, 16> : combine_kernel<YF, false, 16>);
  k_<<<grid, block, 0, s>>>(H, k, pitch, y, w, slot_to_row, shared, shared_w, out);
  return hipGetLastError();
}

hipError_t launch_combine(int T, int H, int k, int y_dtype, int out_dtype, const void* y,
                          const float* w, const int32_t* slot_to_row, const void* shared,
                          const float* shared_w, void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const bool ob = out_dtype == MOE_BF16;
  switch (y_dtype) {
    case MOE_F32: return run_combine<kYF32>(T, H, k, ob, (long long)H * 4, y, w, slot_to_row, shared, shared_w, out, s);
    case MOE_BF16: return run_combine<kYBf16>(T, H, k, ob, (long long)H * 2, y, w, slot_to_row, shared, shared_w, out, s);
    case MOE_F16_SCALED:
      if (H % 64) return hipErrorInvalidValue;
      return run_combine<kYF16S>(T, H, k, ob, moe_f16_scaled_row_bytes(H), y, w, slot_to_row, shared,
                                 shared_w, out, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
