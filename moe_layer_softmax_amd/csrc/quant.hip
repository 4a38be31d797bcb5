// quant.hip -- fp8 (e4m3, fp32 block scales), MXFP4 (e2m1 + E8M0 per 32), MXFP8 (e4m3 + E8M0 per
// 32) and NVFP4 (e2m1 + e4m3 per 16 + fp32 per row) quantisers on gfx950.
//
// Block scaling "as used for models like DeepSeek" ("Hosting Qwen on Blackwell", section
// "Quantization"); 4-bit weights packed two per byte with per-group scales and activations
// quantised to 4 bits before dispatch ("Driving vLLM WideEP ... on Blackwell (Part I)", section on
// lower-precision operations); absmax over 32 elements for the MX formats and over 16 for NVFP4
// ("CuTeDSL at Perplexity", Blackwell section). Element formats and the MX scale rule follow the OCP 8-bit FP
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
  // every chunk load is issued before the first is used: indices past the block's end are clamped
  // to its last chunk (in bounds, nch >= 16) and those values are left out of the maximum (a
  // guarded load became a branch with a full wait after each of the 8 loads)
  float v[8][8];
  float amax = 0.0f;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int i = min((int)threadIdx.x + u * 256, nch - 1);
    load8<SRC_BF16>(src, mat + (size_t)(r0 + i / 16) * cols + bj * 128 + (i % 16) * 8, v[u]);
  }
#pragma unroll
  for (int u = 0; u < 8; ++u)
    if ((int)threadIdx.x + u * 256 < nch)
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[u][e]));
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

// NVFP4, one wave per row (four rows per workgroup): the row's absolute maximum gives the row scale
// g = amax / 2688 (1 when that is 0); then per 16-element block (two neighbouring lanes of 8
// elements each) the e4m3 block scale code of bamax / (6 g), s its value, d = s * g, and the e2m1
// codes of v / d (signed zeros when d = 0). Every step is one IEEE fp32 operation, taken in the
// same order as the definition, so the codes are exact decisions. The row is read twice (the
// second pass finds it in L2).
//   MODE kNv4Packed: packed codes [rows, cols/2]; scale record per matrix of `rows` rows: e4m3
//                block scales [rows, cols/16], then fp32 row scales [rows].
//   MODE kNv4ValuesBf16 / kNv4ValuesF16: the block values q * s as bf16 / fp16 [rows, cols] (exact
//                in both) and the row scales g [rows] (the layer's activation operand).
template <bool SRC_BF16, int MODE>
__global__ void __launch_bounds__(256) quant_nv4_kernel(long long total_rows, int rows, int cols,
                                                        const void* __restrict__ src,
                                                        uint8_t* __restrict__ out,
                                                        uint8_t* __restrict__ scales,
                                                        float* __restrict__ row_scale) {
  constexpr bool DEQ = MODE != kNv4Packed;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= total_rows) return;                   // wave-uniform
  const int lane = threadIdx.x & 63;
  const int nch = cols / 8;                        // 8-element chunks; cols % 64 == 0
  const size_t base = (size_t)row * cols;
  float amax = 0.0f;
  for (int c = lane; c < nch; c += 64) {
    float v[8];
    load8<SRC_BF16>(src, base + (size_t)c * 8, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
  }
  amax = wave_max(amax);
  float g = amax / 2688.0f;
  if (!(g > 0.0f)) g = 1.0f;
  const float d6 = 6.0f * g;
  const long long mat = row / rows, r = row % rows;
  uint8_t* bs = nullptr;
  if (!DEQ) {
    const long long rec = (long long)rows * (cols / 16) + (long long)rows * 4;
    bs = scales + mat * rec + r * (cols / 16);
    if (lane == 0) reinterpret_cast<float*>(scales + mat * rec + (long long)rows * (cols / 16))[r] = g;
  } else if (lane == 0) {
    row_scale[row] = g;
  }
  for (int c = lane; c < nch; c += 64) {           // nch is even: block partners share c / 64
    float v[8];
    load8<SRC_BF16>(src, base + (size_t)c * 8, v);
    float bamax = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) bamax = fmaxf(bamax, fabsf(v[e]));
    bamax = fmaxf(bamax, __shfl_xor(bamax, 1, 64));
    const uint8_t sc = e4m3_rne_sat(bamax / d6);
    const float sv = e4m3_to_f32(sc);
    const float d = sv * g;
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = d == 0.0f ? v[e] * 0.0f : v[e] / d;
    const uint32_t word = e2m1x8_rne_sat(y);
    if (!DEQ) {
      *reinterpret_cast<uint32_t*>(out + (size_t)row * (cols / 2) + (size_t)c * 4) = word;
      if ((c & 1) == 0) bs[c / 2] = sc;
    } else {
      *reinterpret_cast<i32x4*>(out + base * 2 + (size_t)c * 16) =
          MODE == kNv4ValuesF16 ? e2m1x8_times_f16(word, sv) : e2m1x8_times(word, sv);
    }
  }
}

// Dispatch copy of NVFP4 activation rows: a_perm[r] = the block values q * s (bf16) of token row
// row_to_flat[r] / k of the packed input, a_perm_scales[r] = its row scale; one wave per row.
__global__ void __launch_bounds__(256) gather_nv4_kernel(long long max_rows, int k, int T, int cols,
                                                         const int32_t* __restrict__ offsets_end,
                                                         const int32_t* __restrict__ row_to_flat,
                                                         const uint8_t* __restrict__ packed,
                                                         const uint8_t* __restrict__ scales,
                                                         uint16_t* __restrict__ dst,
                                                         float* __restrict__ dst_scales) {
  const long long r = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= max_rows || r >= *offsets_end) return;  // wave-uniform
  const int lane = threadIdx.x & 63;
  const long long t = row_to_flat[r] / k;
  const uint8_t* bs = scales + t * (cols / 16);
  const float* rs = reinterpret_cast<const float*>(scales + (long long)T * (cols / 16));
  for (int c = lane; c < cols / 8; c += 64) {
    const uint32_t word = *reinterpret_cast<const uint32_t*>(packed + t * (cols / 2) + (long long)c * 4);
    *reinterpret_cast<i32x4*>(dst + r * cols + (long long)c * 8) = e2m1x8_times(word, e4m3_to_f32(bs[c / 2]));
  }
  if (lane == 0) dst_scales[r] = rs[t];
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

hipError_t launch_quant_nv4(int src_dtype, int batch, int rows, int cols, const void* src,
                            uint8_t* out, uint8_t* scales, float* row_scale, int out_mode,
                            hipStream_t s) {
  const long long total = (long long)batch * rows;
  if (total == 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>((total + 3) / 4));
  const bool bf = src_dtype == MOE_BF16;
#define MOE_RUN(BF, MODE) quant_nv4_kernel<BF, MODE><<<grid, 256, 0, s>>>(total, rows, cols, src, out, scales, row_scale)
  if (out_mode == kNv4Packed) { if (bf) MOE_RUN(true, kNv4Packed); else MOE_RUN(false, kNv4Packed); }
  else if (out_mode == kNv4ValuesBf16) { if (bf) MOE_RUN(true, kNv4ValuesBf16); else MOE_RUN(false, kNv4ValuesBf16); }
  else if (out_mode == kNv4ValuesF16) { if (bf) MOE_RUN(true, kNv4ValuesF16); else MOE_RUN(false, kNv4ValuesF16); }
  else return hipErrorInvalidValue;
#undef MOE_RUN
  return hipGetLastError();
}

hipError_t launch_gather_nv4(long long max_rows, int k, int T, int cols, const int32_t* offsets_end,
                             const int32_t* row_to_flat, const uint8_t* packed,
                             const uint8_t* scales, uint16_t* dst, float* dst_scales,
                             hipStream_t s) {
  if (max_rows == 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>((max_rows + 3) / 4));
  gather_nv4_kernel<<<grid, 256, 0, s>>>(max_rows, k, T, cols, offsets_end, row_to_flat, packed,
                                         scales, dst, dst_scales);
  return hipGetLastError();
}

}  // namespace moe
