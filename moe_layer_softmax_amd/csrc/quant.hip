// quant.hip -- fp8 (e4m3, fp32 block scales) and MXFP4 (e2m1 + E8M0 per 32) quantisers on gfx950.
//
// Block scaling "as used for models like DeepSeek" ("Hosting Qwen on Blackwell", section
// "Quantization"); 4-bit weights packed two per byte with per-group scales and activations
// quantised to 4 bits before dispatch ("Driving vLLM WideEP ... on Blackwell (Part I)", section on
// lower-precision operations); absmax over 32 elements for the MX formats ("CuTeDSL at
// Perplexity", Blackwell section). Element formats and the MX scale rule follow the OCP 8-bit FP
// and OCP MX v1.0 specifications. The conversions are written out in integer/compare form so the
// codes are exactly round-to-nearest-even, independent of any hardware conversion mode.
#include "common.hpp"
#include "kernels.hpp"
#include "quant_dev.hpp"

namespace moe {

template <bool SRC_BF16>
__device__ __forceinline__ float load_src(const void* src, size_t i) {
  if (SRC_BF16) return bf16_to_f32(static_cast<const uint16_t*>(src)[i]);
  return static_cast<const float*>(src)[i];
}

// one workgroup per (batch, block of block_rows x 128)
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
  const int n = (r1 - r0) * 128;
  float amax = 0.0f;
  for (int i = threadIdx.x; i < n; i += 256) {
    const int r = r0 + i / 128, c = bj * 128 + (i & 127);
    amax = fmaxf(amax, fabsf(load_src<SRC_BF16>(src, mat + (size_t)r * cols + c)));
  }
  __shared__ float red[4];
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  if (threadIdx.x == 0) scales[((size_t)b * nbr + bi) * nbc + bj] = s;
  for (int i = threadIdx.x; i < n; i += 256) {
    const int r = r0 + i / 128, c = bj * 128 + (i & 127);
    const size_t idx = mat + (size_t)r * cols + c;
    codes[idx] = e4m3_rne_sat(load_src<SRC_BF16>(src, idx) / s);
  }
}

// one thread per 32-element group
template <bool SRC_BF16>
__global__ void __launch_bounds__(256) quant_mx4_kernel(long long groups, const void* __restrict__ src,
                                                        uint8_t* __restrict__ packed,
                                                        uint8_t* __restrict__ scales) {
  const long long g = (long long)blockIdx.x * 256 + threadIdx.x;
  if (g >= groups) return;
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = load_src<SRC_BF16>(src, (size_t)g * 32 + i);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e = mx_shared_exp(amax);
  scales[g] = static_cast<uint8_t>(e + 127);
  const float mul = ldexpf(1.0f, -e);
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) word |= static_cast<uint32_t>(e2m1_rne_sat(v[q * 8 + i] * mul)) << (4 * i);
    w[q] = word;
  }
  *reinterpret_cast<i32x4*>(packed + (size_t)g * 16) =
      i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
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

hipError_t launch_quant_mx4(int src_dtype, int batch, int rows, int cols, const void* src,
                            uint8_t* packed, uint8_t* scales, hipStream_t s) {
  const long long groups = (long long)batch * rows * (cols / 32);
  if (groups == 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>((groups + 255) / 256));
  if (src_dtype == MOE_BF16)
    quant_mx4_kernel<true><<<grid, 256, 0, s>>>(groups, src, packed, scales);
  else
    quant_mx4_kernel<false><<<grid, 256, 0, s>>>(groups, src, packed, scales);
  return hipGetLastError();
}

}  // namespace moe
