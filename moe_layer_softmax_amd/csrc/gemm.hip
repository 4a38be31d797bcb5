// gemm.hip -- grouped (per-expert) GEMM on gfx950 MFMA with fused epilogues.
//
// The expert GEMMs of a MoE layer: at prefill each expert gets a dense problem (a 6000-token input
// routed top-8 over 128 experts gives ~375 rows per expert, "Hosting Qwen on Blackwell", section
// "Prefillers"), at decode the problem is bound by reading the weights from HBM (same page,
// section "Decoders"; "CuTeDSL at Perplexity", section on prefill versus decode kernels).
//
// Structure (all variants):
//   * Tile scheduler on the device: workgroup -> (group, m-tile, n-tile) from the device-resident
//     group offsets (a wave-wide prefix sum over per-group tile counts), so no host synchronisation
//     is needed to learn the number of rows per expert. The grid is sized for the worst case and
//     workgroups without a tile exit at once. Workgroups are remapped so that the n-tiles of one
//     m-tile run on one XCD (they share the A rows in that XCD's L2).
//   * A rows are optionally gathered through a row map (the dispatch's row_to_flat / k), so the
//     layer can read expert rows straight from the token-order activations.
//   * K loop: row slices of A and B go from global memory straight into a ring of LDS stages
//     (direct-to-LDS loads), several K-steps ahead of the MFMAs; 16-byte chunks are XOR-swizzled
//     by row so MFMA fragment reads (ds_read_b128) are bank-conflict free.
//   * Epilogues: STORE (optional per-column bias, fp32 or bf16 out) and SWIGLU, where each wave
//     holds matching gate and up columns so h = silu(g) * u is formed in registers.
#include "gemm_common.hpp"
#include "quant_dev.hpp"

namespace moe {

template <int BM, int BN, int WM, int WN, int MI, int BK, int S, bool SWIGLU, bool OUT_F32>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_bf16_pipe_kernel(GemmArgs p, int n_tiles, int x_tiles, int span, int total, int gm) {
  using Geo = SliceGeo<BK>;
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / MI, FN = TN / MI;
  constexpr int MK = (MI == 32) ? 16 : 32;
  constexpr int KS = BK / MK;
  constexpr int RPI = Geo::kRowsPerIns;
  constexpr int A_INS = BM / (RPI * NW), B_INS = BN / (RPI * NW);
  constexpr int INS = A_INS + B_INS;                   // DMA instructions per wave per K-step
  constexpr int STAGE = (BM + BN) * BK;                // uint16 per LDS stage
  static_assert(BM % (RPI * NW) == 0 && BN % (RPI * NW) == 0, "tile rows per wave region");
  static_assert(KS % 2 == 0, "fragment double buffer assumes an even number of substeps");
  static_assert(!SWIGLU || (FN % 2 == 0), "SWIGLU needs gate and up fragments in every wave");
  static_assert(S >= 3 && (S - 2) * INS < 64, "pipeline depth");

  // dynamic LDS (S * STAGE uint16), written only by the DMA loads
  extern __shared__ __attribute__((aligned(1024))) uint16_t lds[];

  const int logical = xcd_remap(blockIdx.x, span);
  if (logical >= total) return;
  Tile t;
  if (!resolve_tile(p, BM, n_tiles, x_tiles, logical, t, gm)) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int K = p.K;
  const int nk = K / BK;
  const int lrow = lane / Geo::kChunks;

  const char* a_src[A_INS];
#pragma unroll
  for (int j = 0; j < A_INS; ++j) {
    const int r = (j * NW + wave) * RPI + lrow;
    const int lch = (lane % Geo::kChunks) ^ Geo::swz(r);
    a_src[j] = static_cast<const char*>(p.A) + a_src_row(p, t, t.row0 + r) * p.a_pitch + lch * 16;
  }
  const char* b_src[B_INS];
#pragma unroll
  for (int j = 0; j < B_INS; ++j) {
    const int rb = (j * NW + wave) * RPI + lrow;
    const int lch = (lane % Geo::kChunks) ^ Geo::swz(rb);
    long long n;
    const char* base = t.B;
    if (SWIGLU) {
      const int within = rb % TN;
      const int half = TN / 2;
      n = (long long)t.nt * (BN / 2) + (rb / TN) * half + (within % half);
      if (within >= half) base = t.B2;
    } else {
      n = (long long)t.nt * BN + rb;
    }
    if (n >= p.N) n = p.N - 1;             // columns past N: read a valid row, never stored
    b_src[j] = base + n * (long long)K * 2 + lch * 16;
  }

  // K-step kt's slices into stage kt % S (steps past the end issue nothing)
  auto issue = [&](int kt) {
    if (kt >= nk) return;
    uint16_t* la = lds + (kt % S) * STAGE;
    uint16_t* lb = la + BM * BK;
#pragma unroll
    for (int j = 0; j < A_INS; ++j)
      dma_16b(a_src[j] + (long long)kt * Geo::kRowBytes, la + (j * NW + wave) * RPI * BK);
#pragma unroll
    for (int j = 0; j < B_INS; ++j)
      dma_16b(b_src[j] + (long long)kt * Geo::kRowBytes, lb + (j * NW + wave) * RPI * BK);
  };

  bf16x8 fa[2][FM], fb[2][FN];
  auto lfrag = [&](int stage, int s, int slot) {
    const uint16_t* la = lds + stage * STAGE;
    const uint16_t* lb = la + BM * BK;
    const int cidx = s * (MK / 8) + lane / MI;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = wm * TM + i * MI + (lane % MI);
      fa[slot][i] = *reinterpret_cast<const bf16x8*>(la + r * BK + ((cidx ^ Geo::swz(r)) * 8));
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int r = wn * TN + j * MI + (lane % MI);
      fb[slot][j] = *reinterpret_cast<const bf16x8*>(lb + r * BK + ((cidx ^ Geo::swz(r)) * 8));
    }
  };

  f32x16 acc32[MI == 32 ? FM : 1][MI == 32 ? FN : 1];
  f32x4 acc16[MI == 16 ? FM : 1][MI == 16 ? FN : 1];
  if constexpr (MI == 32) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc32[i][j] = f32x16{};
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc16[i][j] = f32x4{};
  }

  // prologue: steps 0 .. S-2 in flight, wait for step 0
#pragma unroll
  for (int q = 0; q < S - 1; ++q) issue(q);
  if (nk >= S - 1) wait_vmem_n<(S - 2) * INS>();
  else wait_vmem();
  barrier_lds();
  lfrag(0, 0, 0);

  // Step kt: substeps 0..KS-2 on fragments already in registers (each prefetching the next
  // substep's); then wait for step kt+1's slices and pass the barrier while those MFMAs drain
  // (the barrier also releases stage kt-1, read during step kt-1, for step kt+S-1's loads); the
  // last substep's MFMAs then overlap the reads of step kt+1's first fragments.
  for (int kt = 0; kt < nk; ++kt) {
    const int stage = kt % S;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int slot = s & 1;
      if (s == KS - 1) {
        if (kt + S - 2 < nk) wait_vmem_n<(S - 3) * INS>();   // step kt+1 landed
        else wait_vmem();
        barrier_lds();
        issue(kt + S - 1);
        if (kt + 1 < nk) lfrag((kt + 1) % S, 0, slot ^ 1);
      } else {
        lfrag(stage, s + 1, slot ^ 1);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if constexpr (MI == 32)
            acc32[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][i], fb[slot][j], acc32[i][j], 0, 0, 0);
          else
            acc16[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[slot][i], fb[slot][j], acc16[i][j], 0, 0, 0);
        }
#pragma unroll
      for (int q = 0; q < FM + FN; ++q) {
        MOE_SCHED_GROUP(0x100, 1);
        MOE_SCHED_GROUP(0x008, (FM * FN) / (FM + FN) > 0 ? (FM * FN) / (FM + FN) : 1);
      }
      MOE_SCHED_GROUP(0x008, FM * FN);
    }
  }

// ---- epilogue ----
  constexpr int VPF = (MI == 32) ? 16 : 4;
  auto acc_at = [&](int i, int j, int v) -> float {
    if constexpr (MI == 32) return acc32[i][j][v];
    else return acc16[i][j][v];
  };
  auto row_of = [&](int v) -> int {
    if constexpr (MI == 32) return (v / 4) * 8 + (lane / 32) * 4 + (v % 4);
    else return (lane / 16) * 4 + v;
  };
  const int colw = lane % MI;
  char* C = static_cast<char*>(p.C);
  if constexpr (SWIGLU) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN / 2; ++j)
#pragma unroll
        for (int v = 0; v < VPF; ++v) {
          const int r = t.row0 + wm * TM + i * MI + row_of(v);
          if (r >= t.row1) continue;
          const float g = acc_at(i, j, v), u = acc_at(i, j + FN / 2, v);
          const float h = silu_fast(g) * u;
          const long long col = (long long)t.nt * (BN / 2) + wn * (TN / 2) + j * MI + colw;
          if (col >= p.N) continue;
          if (OUT_F32) reinterpret_cast<float*>(C + r * p.c_pitch)[col] = h;
          else reinterpret_cast<uint16_t*>(C + r * p.c_pitch)[col] = f32_to_bf16(h);
        }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const long long col = (long long)t.nt * BN + wn * TN + j * MI + colw;
        if (col >= p.N) continue;
        const float bias = p.bias ? p.bias[col] : 0.0f;
#pragma unroll
        for (int v = 0; v < VPF; ++v) {
          const int r = t.row0 + wm * TM + i * MI + row_of(v);
          if (r >= t.row1) continue;
          const float val = acc_at(i, j, v) + bias;
          if (OUT_F32) reinterpret_cast<float*>(C + r * p.c_pitch)[col] = val;
          else reinterpret_cast<uint16_t*>(C + r * p.c_pitch)[col] = f32_to_bf16(val);
        }
      }
  }
}

// ------------------------------------------------------------------------------------------------
// fp32 kernel (VALU FMA; the fp32 vector rate equals the fp32 matrix rate on this chip)
//   64 x 64 tile, BK = 16, 256 threads with 4 x 4 outputs each: rows 4*ty.., columns
//   {2tx, 2tx+1, 32+2tx, 33+2tx} so that for SWIGLU the gate column c and up column c + 32 sit in
//   the same thread (h tile 64 x 32).
// ------------------------------------------------------------------------------------------------
template <bool SWIGLU>
__global__ void __launch_bounds__(256) gemm_f32_kernel(GemmArgs p, int n_tiles, int x_tiles,
                                                       int span, int total) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  const int logical = xcd_remap(blockIdx.x, span);
  if (logical >= total) return;
  Tile t;
  if (!resolve_tile(p, BM, n_tiles, x_tiles, logical, t)) return;
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const int K = p.K;
  // loads: 64 rows x 16 k per operand = 1024 floats = 4 per thread: row tid/4, k (tid%4)*4..+3
  const int lr = tid / 4, lk = (tid % 4) * 4;
  const float* arow = reinterpret_cast<const float*>(static_cast<const char*>(p.A) +
                                                     a_src_row(p, t, t.row0 + lr) * p.a_pitch);
  long long n;
  const char* bb = t.B;
  if (SWIGLU) {
    n = (long long)t.nt * (BN / 2) + (lr % 32);
    if (lr >= 32) bb = t.B2;
  } else {
    n = (long long)t.nt * BN + lr;
  }
  if (n >= p.N) n = p.N - 1;
  const float* brow = reinterpret_cast<const float*>(bb) + n * K;
  const int cols[4] = {2 * tx, 2 * tx + 1, 32 + 2 * tx, 33 + 2 * tx};
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += BK) {
    const f32x4 av = *reinterpret_cast<const f32x4*>(arow + k0 + lk);
    const f32x4 bv = *reinterpret_cast<const f32x4*>(brow + k0 + lk);
#pragma unroll
    for (int q = 0; q < 4; ++q) { As[lk + q][lr] = av[q]; Bs[lk + q][lr] = bv[q]; }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][4 * ty + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][cols[j]];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  char* C = static_cast<char*>(p.C);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = t.row0 + 4 * ty + i;
    if (r >= t.row1) continue;
    float* crow = reinterpret_cast<float*>(C + r * p.c_pitch);
    if (SWIGLU) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float g = acc[i][j], u = acc[i][j + 2];
        const long long col = (long long)t.nt * (BN / 2) + cols[j];
        if (col < p.N) crow[col] = g / (1.0f + expf(-g)) * u;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const long long col = (long long)t.nt * BN + cols[j];
        if (col < p.N) crow[col] = acc[i][j] + (p.bias ? p.bias[col] : 0.0f);
      }
    }
  }
}

// ------------------------------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------------------------------
namespace {

// Tile order of the 256 x 256 configurations: groups of 8 m-tiles with the m-tile index fastest,
// 64 consecutive logical tiles per XCD. The 32 tiles an XCD runs at once then cover 8 m-tiles x 4
// n-tiles, so each K-step slice of A is shared by 4 tiles and each slice of B by 8 in that XCD's L2
// (12 distinct slices per 32 tiles).
constexpr int kTileGroupM = 8;
constexpr int kTileSpan = 64;

template <int BM, int BN, int WM, int WN, int MI, int BK, int S>
hipError_t run_bf16(const GemmArgs& a, hipStream_t s, int gm = 1, int span = 0) {
  const bool sw = a.epilogue == MOE_EPI_SWIGLU;
  Grid g = make_grid(a, BM, sw ? BN / 2 : BN, gm, span);
  if (g.total == 0) return hipSuccess;
  dim3 grid(g.blocks), block(WM * WN * 64);
  const bool f32 = a.out_dtype == MOE_F32;
  const size_t lds_bytes = (size_t)S * (BM + BN) * BK * sizeof(uint16_t);
#define MOE_RUN(SWI, F32)                                                                    \
  gemm_bf16_pipe_kernel<BM, BN, WM, WN, MI, BK, S, SWI, F32><<<grid, block, lds_bytes, s>>>(  \
      a, g.n_tiles, g.x_tiles, g.span, g.total, g.gm)
  if (sw && f32) MOE_RUN(true, true);
  else if (sw) MOE_RUN(true, false);
  else if (f32) MOE_RUN(false, true);
  else MOE_RUN(false, false);
#undef MOE_RUN
  return hipGetLastError();
}

hipError_t run_f32(const GemmArgs& a, hipStream_t s) {
  const bool sw = a.epilogue == MOE_EPI_SWIGLU;
  Grid g = make_grid(a, 64, sw ? 32 : 64);
  if (g.total == 0) return hipSuccess;
  dim3 grid(g.blocks), block(256);
  if (sw) gemm_f32_kernel<true><<<grid, block, 0, s>>>(a, g.n_tiles, g.x_tiles, g.span, g.total);
  else gemm_f32_kernel<false><<<grid, block, 0, s>>>(a, g.n_tiles, g.x_tiles, g.span, g.total);
  return hipGetLastError();
}

}  // namespace

// Tile shape choice: the expected rows per group decide between a compute-shaped tile (large
// groups, MFMA-bound) and a weight-streaming tile (few rows per group, HBM-bound).
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  if (a.dtype == MOE_FP8_E4M3 || a.dtype == MOE_MXFP4) return launch_gemm_q(a, s);
  if (a.dtype == MOE_F32) return run_f32(a, s);
  if (a.dtype == MOE_BF16) {
    const long long rows = (long long)a.max_rows + a.x_rows;
    const int groups = a.G + (a.x_rows > 0 ? 1 : 0);
    const long long per_group = groups ? rows / groups : rows;
    const int n_full = a.epilogue == MOE_EPI_SWIGLU ? 2 * a.N : a.N;   // B rows per tile row
    if (per_group >= 512 && n_full >= 256) {
      // 256 x 256 tiles, K-steps of 32 through LDS stages of 32 KB. SwiGLU: 8 waves (2 per SIMD),
      // each 128 x 64, 4 stages; plain store: 16 waves, each 64 x 64, 5 stages.
      if (a.epilogue == MOE_EPI_SWIGLU)
        return run_bf16<256, 256, 2, 4, 32, 32, 4>(a, s, kTileGroupM, kTileSpan);
      return run_bf16<256, 256, 4, 4, 32, 32, 5>(a, s, kTileGroupM, kTileSpan);
    }
    if (per_group >= 96 && n_full >= 128) return run_bf16<128, 128, 2, 2, 32, 64, 3>(a, s);
    return run_bf16<32, 128, 1, 4, 16, 64, 4>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
