// gemm_fp8.hip -- grouped GEMM for fp8 e4m3 experts with fp32 block scales (128 x 128 blocks of
// the weights, 128-element row blocks of the activations) on gfx950: block scaling "as used for
// models like DeepSeek" ("Hosting Qwen on Blackwell", section "Quantization").
//
// Kept in a translation unit of its own so that its MFMAs can be compiled in their VGPR form: the
// per-step fp32 rescale reads every MFMA result with the vector ALU, which cannot address the
// MFMA-only registers (in their AGPR form each result needs four extra register moves).
#include <algorithm>

#include "gemm_common.hpp"
#include "quant_dev.hpp"

namespace moe {

enum { QEPI_STORE_F32 = 0, QEPI_STORE_BF16 = 1, QEPI_SWIGLU_BF16 = 2, QEPI_SWIGLU_Q = 3 };

// fp32 scales staged per K-step beside the operands: 128 A rows, then the two B block scales (read
// from the first two words of loader 2's 256-byte slot), then loader 3's spare slot (every loader
// issues one 4-byte scale load per step, so every loader's vmcnt waits count the same loads)
constexpr int kFp8ScaleStageBytes = 1024;
// compute waves of the fp8 tile kernel (4: 64 x 128 per wave, 8: 64 x 64)
#ifndef MOE_FP8_COMPUTE_WAVES
#define MOE_FP8_COMPUTE_WAVES 4
#endif
constexpr int kFp8ComputeWaves = MOE_FP8_COMPUTE_WAVES;

// ------------------------------------------------------------------------------------------------
// fp8 (e4m3 with fp32 scales per 128 x 128 block of the weights and per 128-element row block of
// the activations) on 128 x 256 tiles.
//
// A K-step is one 128-element scale block: each fragment's MFMA (16 x 16 x 128, unit scales) goes
// into a temporary that is added into the accumulator times the step's scale product in fp32.
// The accumulators must stay in arch VGPRs for that (the vector ALU cannot address the MFMA-only
// registers); the 16 x 16 shape keeps each temporary at 4 registers, and a ring of four lets the
// MFMAs of fragment pair p run while pair p - 3 is scaled. The weights are the MFMA's row operand
// and the activations its column operand, so a lane's entries of a fragment belong to one
// activation row and one 128-row weight block: one scale product per fragment and step.
//
// Warp-specialised: NC compute waves and 4 loader waves. Compute wave c: wt = c / (NC / 2) takes
// activation rows [64 wt, 64 wt + 64); wn = c % (NC / 2) takes TW = 512 / NC weight rows: rows
// [TW wn, +TW) (STORE), or gate rows [TW/2 wn, +TW/2) and the matching up rows (SWIGLU: h columns
// [TW/2 wn, +TW/2) of the tile). The loader waves only move data (3-stage direct-to-LDS ring,
// block scales staged with their step): they issue step kt + 2 into the stage released by the
// barrier that ended step kt - 1, wait for step kt + 1, and meet the compute waves at the barrier
// that ends step kt. A wave whose load cannot issue (the memory pipeline full) stalls in order:
// with one wave per SIMD doing both, such stalls also held back its MFMAs (measured on the
// 4096-token DeepSeek-V3 slice's gate/up: loads alone 268 us, loads and compute in the same waves
// 403 us, split between loader and compute waves 372 us). fp8 h: the row amax of the tile's 128
// h-columns is exchanged between the compute waves of a row through LDS.
// ------------------------------------------------------------------------------------------------
template <int EPI>
__global__ void __launch_bounds__((kFp8ComputeWaves + 4) * 64)
gemm_fp8_tile_kernel(GemmArgs p, int n_tiles, int x_tiles, int span, int total, int gm) {
  constexpr bool SWIGLU = EPI >= QEPI_SWIGLU_BF16;
  constexpr int BM = 128, BN = 256, S = 3;
  constexpr int NC = kFp8ComputeWaves, NW = 4;    // compute waves, loader waves
  constexpr int WNS = NC / 2;              // compute waves per activation-row half
  constexpr int TW = BN / WNS;             // weight rows per compute wave
  constexpr int RB = 128;                  // bytes per row slice (one K-step)
  constexpr int A_INS = BM / (8 * NW), B_INS = BN / (8 * NW);
  constexpr int INS = A_INS + B_INS + 1;   // + one 4-byte scale load
  constexpr int DATA = (BM + BN) * RB;
  constexpr int STAGE = DATA + kFp8ScaleStageBytes;
  constexpr int FT = 4, FW = TW / 16;      // 16-row activation and weight fragments per wave
  constexpr int NP = FT * FW;              // fragment pairs per step
  constexpr int RING = 4;                  // temporaries in flight
  using Geo = SliceGeo<64>;
  static_assert(NC == 4 || NC == 8, "compute waves");
  static_assert((S - 2) * INS < 64, "pipeline depth");

  extern __shared__ __attribute__((aligned(1024))) uint8_t ldsf[];

  const int logical = xcd_remap(blockIdx.x, span);
  if (logical >= total) return;
  Tile t;
  if (!resolve_tile(p, BM, n_tiles, x_tiles, logical, t, gm)) return;

  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);   // scalar: DMA targets
  const int K = p.K;
  const int nk = K / 128;

  if (wave >= NC) {
    // ---- loader wave lw: DMA sources as a uniform base and a 32-bit byte offset per lane (the
    // host checks that A and every weight matrix span less than 4 GiB), so a K-step moves only the
    // scalar base ----
    const int lw = wave - NC;
    const int lrow = lane >> 3;
    unsigned a_off[A_INS];
#pragma unroll
    for (int j = 0; j < A_INS; ++j) {
      const int r = (j * NW + lw) * 8 + lrow;
      a_off[j] = static_cast<unsigned>(a_src_row(p, t, t.row0 + r) * p.a_pitch) +
                 ((lane & 7) ^ Geo::swz(r)) * 16;
    }
    const char* b_base[B_INS];
    unsigned b_off[B_INS];
#pragma unroll
    for (int j = 0; j < B_INS; ++j) {
      const int rb0 = (j * NW + lw) * 8;   // wave-uniform: gate or up for the whole instruction
      const int rb = rb0 + lrow;
      long long n;
      if (SWIGLU) {
        n = (long long)t.nt * (BN / 2) + (rb % (BN / 2));
        b_base[j] = rb0 >= BN / 2 ? t.B2 : t.B;
      } else {
        n = (long long)t.nt * BN + rb;
        b_base[j] = t.B;
      }
      if (n >= p.N) n = p.N - 1;
      b_off[j] = static_cast<unsigned>(n * K) + ((lane & 7) ^ Geo::swz(rb)) * 16;
    }
    const char* const a_base = static_cast<const char*>(p.A);
    const unsigned lds0 = static_cast<unsigned>(reinterpret_cast<uintptr_t>(ldsf));
    // scales: loaders 0 and 1 move the A scales of rows [64 lw, 64 lw + 64) (one fp32 per row and
    // step), loader 2 the two B block scales (lane i: block i & 1), loader 3 the same into a spare
    // slot
    const int kb = K / 128;
    const char* s_src;
    int s_dst;
    if (lw < 2) {
      const int r = lw * 64 + lane;
      s_src = static_cast<const char*>(p.A_scales) +
              (long long)(a_src_row(p, t, t.row0 + r) / p.a_scale_rows) * kb * 4;
      s_dst = DATA + lw * 256;
    } else {
      const char* b0;
      const char* b1;
      if (SWIGLU) {                        // the tile's 128 h-columns: one gate and one up block
        b0 = t.Bs + (long long)t.nt * kb * 4;
        b1 = t.B2s + (long long)t.nt * kb * 4;
      } else {                             // two 128-column blocks
        b0 = t.Bs + (long long)(t.nt * 2) * kb * 4;
        b1 = t.Bs + (long long)min(t.nt * 2 + 1, (p.N - 1) / 128) * kb * 4;
      }
      s_src = (lane & 1) ? b1 : b0;
      s_dst = DATA + 512 + (lw - 2) * 256;
    }
    auto issue = [&](int kt) {
      const int stage = kt % S;
      const unsigned st = lds0 + stage * STAGE;
      const long long kb8 = (long long)kt * RB;
#pragma unroll
      for (int j = 0; j < A_INS; ++j) dma_16b_sbase(a_base + kb8, a_off[j], st + (j * NW + lw) * 8 * RB);
#pragma unroll
      for (int j = 0; j < B_INS; ++j)
        dma_16b_sbase(b_base[j] + kb8, b_off[j], st + BM * RB + (j * NW + lw) * 8 * RB);
      dma_4b_asm(s_src + kt * 4, ldsf + stage * STAGE + s_dst);
    };
    // prologue: steps 0 .. S-2 in flight, step 0 landed before the first barrier
#pragma unroll
    for (int qq = 0; qq < S - 1; ++qq)
      if (qq < nk) issue(qq);
    if (nk >= S - 1) wait_vmem_n<(S - 2) * INS>();
    else wait_vmem();
    barrier_lds();
    for (int kt = 0; kt < nk; ++kt) {
      // step kt + S - 1 into the stage the last barrier released; step kt + 1 landed before the
      // barrier that ends step kt
      if (kt + S - 1 < nk) {
        issue(kt + S - 1);
        wait_vmem_n<(S - 2) * INS>();
      } else {
        wait_vmem();
      }
      barrier_lds();
    }
    if constexpr (EPI == QEPI_SWIGLU_Q) __syncthreads();   // the compute waves' amax exchange
    return;
  }

  // ---- compute waves ----
  const int wt = wave / WNS, wn = wave % WNS;
  const int l16 = lane & 15, q = lane >> 4;
  // 16 rows x 32 bytes per lane (the fp8 operand of 16 x 16 x 128): chunks 2 q and 2 q + 1 of
  // rows r0 + l16 (any K order shared by both operands gives the same sum)
  auto frag = [&](const uint8_t* base, int r0) -> i32x8 {
    const int r = r0 + l16;
    const i32x4 v0 = *reinterpret_cast<const i32x4*>(base + r * RB + (((2 * q) ^ Geo::swz(r)) * 16));
    const i32x4 v1 = *reinterpret_cast<const i32x4*>(base + r * RB + (((2 * q + 1) ^ Geo::swz(r)) * 16));
    return i32x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
  };
  // first tile B-row of weight fragment i, and its 128-row block (0: b0, 1: b1)
  auto wrow = [&](int i) -> int {
    if (SWIGLU) return i < FW / 2 ? wn * (TW / 2) + i * 16 : BN / 2 + wn * (TW / 2) + (i - FW / 2) * 16;
    return wn * TW + i * 16;
  };
  auto wblk = [&](int i) -> int { return SWIGLU && i >= FW / 2 ? 1 : 0; };

  f32x4 acc[FW][FT];
#pragma unroll
  for (int i = 0; i < FW; ++i)
#pragma unroll
    for (int j = 0; j < FT; ++j) acc[i][j] = f32x4{};

  barrier_lds();                           // step 0 landed (the loaders' prologue)
  for (int kt = 0; kt < nk; ++kt) {
    const uint8_t* la = ldsf + (kt % S) * STAGE;
    const uint8_t* lb = la + BM * RB;
    const float* ls = reinterpret_cast<const float*>(la + DATA);
    i32x8 xf[FT];
#pragma unroll
    for (int j = 0; j < FT; ++j) xf[j] = frag(la, wt * 64 + j * 16);
    i32x8 wf[2];
    wf[0] = frag(lb, wrow(0));
    // scale products: SWIGLU fragments use the gate (0) or up (1) block, STORE the wave's block
    float fac[2][FT];
    const float sb0 = SWIGLU ? ls[128] : ls[128 + (wn * TW) / 128], sb1 = ls[129];
#pragma unroll
    for (int j = 0; j < FT; ++j) {
      const float sa = ls[wt * 64 + j * 16 + l16];
      fac[0][j] = sa * sb0;
      fac[1][j] = sa * sb1;
    }
    // pairs p = FT i + j: pair p's MFMA into temporary p % RING, then pair p - RING + 1 scaled
    // into its accumulator; weight fragment i + 1 read with the first pair of fragment i
    f32x4 tmp[RING];
#pragma unroll
    for (int pp = 0; pp < NP + RING - 1; ++pp) {
      if (pp < NP) {
        const int i = pp / FT, j = pp % FT;
        if (j == 0 && i + 1 < FW) wf[(i + 1) & 1] = frag(lb, wrow(i + 1));
        tmp[pp % RING] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            wf[i & 1], xf[j], f32x4{}, 0, 0, 0, 127, 0, 127);
      }
      const int pd = pp - (RING - 1);
      if (pd >= 0) {
        const int i = pd / FT, j = pd % FT;
        const float f = fac[wblk(i)][j];
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[i][j][v] = fmaf(tmp[pd % RING][v], f, acc[i][j][v]);
      }
    }
    wait_lgkm();                           // this wave's reads of stage kt are done
    barrier_lds();                         // and step kt + 1 has landed (the loaders waited)
  }

  // ---- epilogue: lane l16 of fragment j is activation row r; entries v of weight fragment i are
  // the 4 consecutive weight rows 16 i + 4 q + v ----
  char* C = static_cast<char*>(p.C);
  if constexpr (!SWIGLU) {
#pragma unroll
    for (int j = 0; j < FT; ++j) {
      const int r = t.row0 + wt * 64 + j * 16 + l16;
      if (r >= t.row1) continue;
      char* crow = C + (long long)r * p.c_pitch;
#pragma unroll
      for (int i = 0; i < FW; ++i) {
        const long long col = (long long)t.nt * BN + wn * TW + i * 16 + q * 4;
        if (col >= p.N) continue;          // N % 128 == 0: 4 columns all in or all out
        const f32x4 v = acc[i][j];
        if (EPI == QEPI_STORE_F32) *reinterpret_cast<f32x4*>(crow + col * 4) = v;
        else *reinterpret_cast<uint2*>(crow + col * 2) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
    }
  } else {
    constexpr int HF = FW / 2;             // gate fragments (TW / 2 h-columns per wave)
    f32x4 hv[FT][HF];
#pragma unroll
    for (int j = 0; j < FT; ++j)
#pragma unroll
      for (int i = 0; i < HF; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) hv[j][i][v] = silu_fast(acc[i][j][v]) * acc[i + HF][j][v];
    const long long hcol0 = (long long)t.nt * (BN / 2) + wn * (TW / 2);
    if constexpr (EPI == QEPI_SWIGLU_BF16) {
#pragma unroll
      for (int j = 0; j < FT; ++j) {
        const int r = t.row0 + wt * 64 + j * 16 + l16;
        if (r >= t.row1) continue;
        char* crow = C + (long long)r * p.c_pitch;
#pragma unroll
        for (int i = 0; i < HF; ++i) {
          const long long col = hcol0 + i * 16 + q * 4;
          if (col >= p.N) continue;
          *reinterpret_cast<uint2*>(crow + col * 2) =
              make_uint2(pack_bf16x2(hv[j][i][0], hv[j][i][1]), pack_bf16x2(hv[j][i][2], hv[j][i][3]));
        }
      }
    } else {
      // fp8 h in 1 x 128 blocks: the tile's 128 h-columns of a row are held by the four lanes
      // l16 + 16 q of the WNS compute waves of its row half; their amax goes through LDS
      float* xch = reinterpret_cast<float*>(ldsf + S * STAGE);      // [WNS wn][BM rows]
#pragma unroll
      for (int j = 0; j < FT; ++j) {
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < HF; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v) a = fmaxf(a, fabsf(hv[j][i][v]));
        a = fmaxf(a, __shfl_xor(a, 16, 64));
        a = fmaxf(a, __shfl_xor(a, 32, 64));
        if (q == 0) xch[wn * BM + wt * 64 + j * 16 + l16] = a;
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < FT; ++j) {
        const int rt = wt * 64 + j * 16 + l16;
        float amax = 0.0f;
#pragma unroll
        for (int w = 0; w < WNS; ++w) amax = fmaxf(amax, xch[w * BM + rt]);
        const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
        const int r = t.row0 + rt;
        if (r >= t.row1) continue;
        uint8_t* crow = reinterpret_cast<uint8_t*>(C + (long long)r * p.c_pitch);
#pragma unroll
        for (int i = 0; i < HF; ++i) {
          const long long col = hcol0 + i * 16 + q * 4;
          *reinterpret_cast<uint32_t*>(crow + col) =
              e4m3x4_rne_sat(hv[j][i][0] / sc, hv[j][i][1] / sc, hv[j][i][2] / sc, hv[j][i][3] / sc);
        }
        if (wn == 0 && q == 0)
          reinterpret_cast<float*>(p.C_scales)[(long long)r * (p.N / 128) + t.nt] = sc;
      }
    }
  }
}


namespace {
// the fp8 tile kernel addresses A and each weight matrix with 32-bit byte offsets
inline bool fp8_tile_fits(const GemmArgs& a) {
  const long long a_rows = std::max<long long>(a.max_rows, (long long)a.x_row0 + a.x_rows) + 1;
  return a_rows * a.a_pitch < (1ll << 32) && (long long)a.N * a.K < (1ll << 32);
}

template <int EPI>
hipError_t run_fp8_tile(const GemmArgs& a, hipStream_t s) {
  constexpr int BM = 128, BN = 256, S = 3;
  constexpr bool SWIGLU = EPI >= QEPI_SWIGLU_BF16;
  // groups of 4 m-tiles, 32 tiles per XCD (one per CU): an XCD runs 8 n-tiles of 4 m-tiles at
  // once. 4096-token DeepSeek-V3 fp8 slice, two reps: 0.764-0.768 ms against 0.832-0.840 with 8 /
  // 64 (2 / 32 0.772-0.773, 4 / 64 0.844-0.848, 16 / 64 0.831-0.833)
  Grid g = make_grid(a, BM, SWIGLU ? BN / 2 : BN, 4, 32);
  if (g.total == 0) return hipSuccess;
  const size_t lds = (size_t)S * ((BM + BN) * 128 + kFp8ScaleStageBytes) + (kFp8ComputeWaves / 2) * BM * 4;
  gemm_fp8_tile_kernel<EPI><<<dim3(g.blocks), dim3((kFp8ComputeWaves + 4) * 64), lds, s>>>(a, g.n_tiles, g.x_tiles, g.span,
                                                                  g.total, g.gm);
  return hipGetLastError();
}

}  // namespace

bool launch_fp8_tile(const GemmArgs& a, int epi, hipStream_t s, hipError_t* err) {
  if (!fp8_tile_fits(a)) return false;
  switch (epi) {
    case QEPI_STORE_F32: *err = run_fp8_tile<QEPI_STORE_F32>(a, s); break;
    case QEPI_STORE_BF16: *err = run_fp8_tile<QEPI_STORE_BF16>(a, s); break;
    case QEPI_SWIGLU_BF16: *err = run_fp8_tile<QEPI_SWIGLU_BF16>(a, s); break;
    default: *err = run_fp8_tile<QEPI_SWIGLU_Q>(a, s); break;
  }
  return true;
}

}  // namespace moe
