// quant.hip -- fp8 (e4m3, fp32 block scales), MXFP4 (e2m1 + E8M0 per 32) and MXFP8 (e4m3 + E8M0 per
// 32) quantisers on gfx950.
//
// Block scaling "as used for models like DeepSeek" ("Hosting Qwen on Blackwell", section
// "Quantization"); 4-bit weights packed two per byte with per-group scales and activations
// quantised to 4 bits before dispatch ("Driving vLLM WideEP ... on Blackwell (Part I)", section on
// lower-precision operations); absmax over 32 elements for the MX formats ("CuTeDSL at
// Perplexity", Blackwell section). Element formats and the MX scale rule follow the OCP 8-bit FP
// and OCP MX v1.0 specifications. Codes come from gfx950's packed conversions (v_cvt_pk_fp8_f32 on
// operands clamped to +-448, v_cvt_scalef32_pk_fp4_f32 with a unit scale), which round to nearest
// even in the default rounding mode; quant_dev.hpp also keeps the integer/compare encoders they were
// checked against bit for bit, and the GPU tests compare the codes with the oracle's on every grid
// value, tie, neighbour, subnormal, +-0 and the 440..620 saturation range.
#include "common.hpp"
#include "kernels.hpp"
#include "quant_dev.hpp"

namespace moe {

// 8 consecutive source elements starting at element i (i a multiple of 8), as fp32
template <bool SRC_BF16>
__device__ __forceinline__ void load8(const void* src, size_t i, float* v) {
  if (SRC_BF16) {
    const i32x4 w = *reinterpret_cast<const i32x4*>(static_cast<const uint16_t*>(src) + i);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(static_cast<uint32_t>(w[q]) << 16);
      v[2 * q + 1] = __uint_as_float(static_cast<uint32_t>(w[q]) & 0xFFFF0000u);
    }
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(static_cast<const float*>(src) + i);
    const f32x4 b = *reinterpret_cast<const f32x4*>(static_cast<const float*>(src) + i + 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) { v[q] = a[q]; v[4 + q] = b[q]; }
  }
}

// One workgroup per (batch, block of block_rows x 128); block_rows is 1 or 128. Each thread holds
// up to 8 chunks of 8 consecutive elements (16-byte loads) in registers, so the block is read once:
// amax over the block, then the codes (8 per 8-byte store).
template <bool SRC_BF16>
__global__ void __launch_bounds__(256) quant_fp8_kernel(int rows, int cols, int block_rows,
                                                        const void* __restrict__ src,
                                                        uint8_t* __restrict__ codes,
                                                        float* __restrict__ scales) {
  const int nbc = cols / 128;
  const int nbr = (rows + block_rows - 1) / block_rows;
  const int b = blockIdx.y;
  const int bi = blockIdx.x / nbc, bj = blockIdx.x % nbc;
  const size_t mat = (size_t)b * rows * cols;
  const int r0 = bi * block_rows;
  const int r1 = r0 + block_rows < rows ? r0 + block_rows : rows;
  const int nch = (r1 - r0) * 16;          // 8-element chunks of the block (<= 2048)
  float v[8][8];
  float amax = 0.0f;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int i = threadIdx.x + u * 256;
    if (i < nch) {
      load8<SRC_BF16>(src, mat + (size_t)(r0 + i / 16) * cols + bj * 128 + (i % 16) * 8, v[u]);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[u][e]));
    }
  }
  __shared__ float red[4];
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  if (threadIdx.x == 0) scales[((size_t)b * nbr + bi) * nbc + bj] = s;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int i = threadIdx.x + u * 256;
    if (i < nch) {
      const uint32_t lo = e4m3x4_rne_sat(v[u][0] / s, v[u][1] / s, v[u][2] / s, v[u][3] / s);
      const uint32_t hi = e4m3x4_rne_sat(v[u][4] / s, v[u][5] / s, v[u][6] / s, v[u][7] / s);
      *reinterpret_cast<uint2*>(codes + mat + (size_t)(r0 + i / 16) * cols + bj * 128 + (i % 16) * 8) =
          make_uint2(lo, hi);
    }
  }
}

// Four lanes per 32-element group, 8 elements (one 16-byte bf16 load) each: group amax over the
// four lanes, then each lane packs its 8 codes into one 32-bit word (element 2i in the low nibble
// of byte i); the first lane writes the E8M0 scale.
template <bool SRC_BF16>
__global__ void __launch_bounds__(256) quant_mx4_kernel(long long groups, const void* __restrict__ src,
                                                        uint8_t* __restrict__ packed,
                                                        uint8_t* __restrict__ scales) {
  const long long tid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long g = tid >> 2;
  const int sub = static_cast<int>(tid & 3);
  const bool live = g < groups;
  float v[8];
  if (live) load8<SRC_BF16>(src, (size_t)g * 32 + sub * 8, v);
  else
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.0f;
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  const int e8 = mx_shared_exp(amax);
  const float mul = ldexpf(1.0f, -e8);
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = v[e] * mul;
  const uint32_t word = e2m1x8_rne_sat(y);
  if (!live) return;
  *reinterpret_cast<uint32_t*>(packed + (size_t)g * 16 + sub * 4) = word;
  if (sub == 0) scales[g] = static_cast<uint8_t>(e8 + 127);
}

// MXFP8: four lanes per 32-element group as for MXFP4; each lane writes its 8 codes as one 8-byte
// store.
template <bool SRC_BF16>
__global__ void __launch_bounds__(256) quant_mx8_kernel(long long groups, const void* __restrict__ src,
                                                        uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales) {
  const long long tid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long g = tid >> 2;
  const int sub = static_cast<int>(tid & 3);
  const bool live = g < groups;
  float v[8];
  if (live) load8<SRC_BF16>(src, (size_t)g * 32 + sub * 8, v);
  else
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.0f;
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  const int e8 = mx_shared_exp<8>(amax);
  const float mul = ldexpf(1.0f, -e8);
  const uint32_t lo = e4m3x4_rne_sat(v[0] * mul, v[1] * mul, v[2] * mul, v[3] * mul);
  const uint32_t hi = e4m3x4_rne_sat(v[4] * mul, v[5] * mul, v[6] * mul, v[7] * mul);
  if (!live) return;
  *reinterpret_cast<uint2*>(codes + (size_t)g * 32 + sub * 8) = make_uint2(lo, hi);
  if (sub == 0) scales[g] = static_cast<uint8_t>(e8 + 127);
}

hipError_t launch_quant_fp8(int src_dtype, int batch, int rows, int cols, int block_rows,
                            const void* src, uint8_t* codes, float* scales, hipStream_t s) {
  if (rows == 0 || batch == 0) return hipSuccess;
  const int nbr = (rows + block_rows - 1) / block_rows;
  dim3 grid(nbr * (cols / 128), batch);
  if (src_dtype == MOE_BF16)
    quant_fp8_kernel<true><<<grid, 256, 0, s>>>(rows, cols, block_rows, src, codes, scales);
  else
    quant_fp8_kernel<false><<<grid, 256, 0, s>>>(rows, cols, block_rows, src, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quant_mx8(int src_dtype, int batch, int rows, int cols, const void* src,
                            uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const long long groups = (long long)batch * rows * (cols / 32);
  if (groups == 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>((groups * 4 + 255) / 256));
  if (src_dtype == MOE_BF16)
    quant_mx8_kernel<true><<<grid, 256, 0, s>>>(groups, src, codes, scales);
  else
    quant_mx8_kernel<false><<<grid, 256, 0, s>>>(groups, src, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quant_mx4(int src_dtype, int batch, int rows, int cols, const void* src,
                            uint8_t* packed, uint8_t* scales, hipStream_t s) {
  const long long groups = (long long)batch * rows * (cols / 32);
  if (groups == 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>((groups * 4 + 255) / 256));
  if (src_dtype == MOE_BF16)
    quant_mx4_kernel<true><<<grid, 256, 0, s>>>(groups, src, packed, scales);
  else
    quant_mx4_kernel<false><<<grid, 256, 0, s>>>(groups, src, packed, scales);
  return hipGetLastError();
}

}  // namespace moe
