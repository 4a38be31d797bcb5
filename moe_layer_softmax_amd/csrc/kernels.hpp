// kernels.hpp -- host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Arguments of one grouped-GEMM launch.
//   routed groups g < G: rows [offsets[g], offsets[g+1]) of C, weights B + g * b_stride
//   optional extra group ("shared expert"): rows [x_row0, x_row0 + x_rows) of C, A row = r - x_row0,
//   weights xB / xB2
struct GemmArgs {
  int dtype;            // moe_dtype of A and B
  int epilogue;         // moe_epilogue
  int out_dtype;        // moe_dtype of C
  int K, N;             // reduction length; output columns
  const void* A;        // [rows of A, K] in dtype (row pitch a_pitch bytes)
  const void* A_scales;
  long long a_pitch;    // bytes between A rows
  int a_scale_rows;     // FP8: A scales per a_scale_rows-row block
  const int32_t* a_rows;
  int a_row_div;
  int G;
  const int32_t* offsets;
  int max_rows;         // bound on offsets[G] (sizes the grid)
  int expected_rows;    // rows the routed groups are expected to hold (tile-shape choice only;
                        // 0: take max_rows); results never depend on it
  const void* B; const void* Bs; const void* B2; const void* B2s;
  long long b_stride;   // bytes between groups' B (and B2)
  long long bs_stride;  // bytes between groups' scales
  int x_rows, x_row0;   // extra group rows of C
  int x_a_off;          // extra group: A row = C row - x_a_off
  const void* xB; const void* xBs; const void* xB2; const void* xB2s;
  const float* bias;    // STORE epilogue: per-column fp32 bias, or null
  void* C;
  void* C_scales;
  long long c_pitch;    // bytes between C rows
  int a_f16;            // NVFP4 only: A holds the block values as fp16 (else bf16); the product runs
                        // on the fp16 MFMA with the weights dequantised to fp16
};

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s);
// the router as a grouped GEMM (one extra group of T rows): a tile shape for N = E and many rows
hipError_t launch_gemm_router(const GemmArgs& a, hipStream_t s);
// block-scaled fp8 / MXFP4 / MXFP8 grouped GEMM (A and B in a.dtype)
hipError_t launch_gemm_q(const GemmArgs& a, hipStream_t s);

// Top-k selection and weights. With nsplit > 1, logits[t, e] is first formed as the sum of the
// router's K-split partials partial[s][t][e] (s ascending) plus bias[e] and written to `logits`.
hipError_t launch_topk(int T, int E, int k, int scoring, int renormalize, float* logits,
                       const float* partial, int nsplit, const float* bias, int32_t* ids, float* w,
                       hipStream_t s);
// bf16 router logits (E % 16 == 0, H % 64 == 0); nsplit = router_splits(T, H, E). With nsplit > 1
// the partial sums go to `partial` ([nsplit, T, E] fp32, router_ws_bytes) and the top-k kernel
// finishes the logits; otherwise logits (+ bias) are written directly.
int router_splits(int T, int H, int E);
size_t router_ws_bytes(int T, int H, int E);
hipError_t launch_router(int T, int H, int E, const void* x, const void* w_router,
                         const float* bias, float* logits, float* partial, int nsplit,
                         hipStream_t s);

// Dispatch maps. ws must hold permute_ws_bytes(T*k, E_loc) bytes.
size_t permute_ws_bytes(long long slots, int E_loc);
hipError_t launch_permute_maps(int T, int k, int e0, int E_loc, const int32_t* ids, int32_t* counts,
                               int32_t* offsets, int32_t* slot_to_row, int32_t* row_to_flat,
                               void* ws, hipStream_t s);
// a_perm[r] = a_in[row_to_flat[r] / k] for r < offsets[E_loc]; row_bytes % 16 == 0.
// With scales: the same gather of scale rows (scale_row_bytes % 4 == 0), the source scale row of
// token t being t / scale_rows_per_block.
hipError_t launch_gather_rows(long long max_rows, int k, const int32_t* offsets_end,
                              const int32_t* row_to_flat, const void* src, long long row_bytes,
                              void* dst, const void* src_scales, long long scale_row_bytes,
                              int scale_rows_per_block, void* dst_scales, hipStream_t s);

hipError_t launch_combine(int T, int H, int k, int y_dtype, int out_dtype, const void* y, const float* w,
                          const int32_t* slot_to_row, const void* shared, const float* shared_w,
                          void* out, hipStream_t s);
// g[t] = 1 / (1 + exp(-(x_t . w_sg))), fp32 accumulation; x [T, H], w_sg [H] in io_dtype; H % 8 == 0.
hipError_t launch_shared_gate(int T, int H, int io_dtype, const void* x, const void* w_sg, float* g,
                              hipStream_t s);

hipError_t launch_quant_fp8(int src_dtype, int batch, int rows, int cols, int block_rows,
                            const void* src, uint8_t* codes, float* scales, hipStream_t s);
hipError_t launch_quant_mx4(int src_dtype, int batch, int rows, int cols, const void* src,
                            uint8_t* packed, uint8_t* scales, hipStream_t s);
hipError_t launch_quant_mx8(int src_dtype, int batch, int rows, int cols, const void* src,
                            uint8_t* codes, uint8_t* scales, hipStream_t s);
// NVFP4: out_mode 0: packed [batch*rows, cols/2] + per-matrix scale records (e4m3 [rows, cols/16]
// then fp32 [rows]) in `scales`; out_mode 1 / 2: the block values as bf16 / fp16 [batch*rows, cols]
// in `out` and fp32 row scales in `row_scale`. cols % 64 == 0.
enum { kNv4Packed = 0, kNv4ValuesBf16 = 1, kNv4ValuesF16 = 2 };
hipError_t launch_quant_nv4(int src_dtype, int batch, int rows, int cols, const void* src,
                            uint8_t* out, uint8_t* scales, float* row_scale, int out_mode,
                            hipStream_t s);
// a_perm[r] = bf16 block values of packed NVFP4 row row_to_flat[r] / k (scales: one record of T
// rows), a_perm_scales[r] = its row scale; rows r < *offsets_end. cols % 64 == 0.
hipError_t launch_gather_nv4(long long max_rows, int k, int T, int cols, const int32_t* offsets_end,
                             const int32_t* row_to_flat, const uint8_t* packed,
                             const uint8_t* scales, uint16_t* dst, float* dst_scales,
                             hipStream_t s);
// NVFP4 weights (B) with bf16 (or, a_f16, fp16) block-value activations (A) and fp32 row scales
// (A_scales, may be null); K % 256 == 0, N % 128 == 0; a_f16 needs SWIGLU with bf16 out
hipError_t launch_gemm_nv4(const GemmArgs& a, hipStream_t s);

}  // namespace moe
