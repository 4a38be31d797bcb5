// gemm_q.hip -- grouped (per-expert) GEMM for block-scaled 8-bit and 4-bit expert formats on the
// gfx950 scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4).
//
// Formats (weights and the activations fed to the expert GEMMs):
//   * fp8: OCP e4m3 codes with one fp32 scale per 128 x 128 block of each weight matrix and, for
//     activations, per 128-token x 128-channel block of x or per 1 x 128 block of h (block scaling
//     "as used for models like DeepSeek", "Hosting Qwen on Blackwell", section "Quantization").
//     A K-step is 128 elements = one scale block: the MFMA runs with unit scales into a temporary
//     and the product of the two fp32 block scales is applied in fp32 before accumulation.
//   * MXFP4: OCP e2m1 codes, two per byte, with one E8M0 scale per 32 elements along K (4-bit
//     weights packed two per byte with per-group scales, "Driving vLLM WideEP ... on Blackwell
//     (Part I)", section on lower-precision operations; absmax over 32 elements for MX formats,
//     "CuTeDSL at Perplexity", Blackwell section). The E8M0 scales go straight into the MFMA's
//     per-lane scale operands, so the dequantisation happens inside the matrix core.
//   * MXFP8: OCP e4m3 codes with one E8M0 scale per 32 elements along K (the MXFP8 MoE GEMMs of
//     "Hosting Qwen on Blackwell", section "Quantization"). The 32-byte fp8 operand of lane group q
//     (lanes 16q .. 16q + 15) holds K-elements [16q, 16q + 16) in its first 16 bytes and
//     [64 + 16q, 64 + 16q + 16) in its last 16, and the scale byte of lane group q applies to
//     K-elements [32q, 32q + 32); so the operand is built from 16-byte chunks q and q + 4 of the
//     128-element row slice, and lane group q passes the E8M0 scale of group q.
//
// Tile: 128 rows x 256 B-rows, 4 waves each owning 32 rows x all 256 B-rows (so a wave holds the
// full 128 h-columns of the SwiGLU tile: the epilogue can form fp8 1x128 or MX 1x32 blocks of h
// in registers, with the row amax reduced across 16 lanes by shuffles). K-steps are 128-byte row
// slices (128 fp8 or 256 fp4 elements) staged through a 3-stage direct-to-LDS ring, with the same
// bank swizzle, tile scheduler and row gathering as the bf16 kernel. The block scales of a K-step
// travel in the same stage as its operands (4-byte direct-to-LDS loads), so the loop has no other
// global loads: every wait in it is an explicit count of this wave's own loads.
#include <algorithm>

#include "gemm_common.hpp"
#include "quant_dev.hpp"

namespace moe {

enum { QEPI_STORE_F32 = 0, QEPI_STORE_BF16 = 1, QEPI_SWIGLU_BF16 = 2, QEPI_SWIGLU_Q = 3 };

// m-tiles per tile-order group (and per XCD span) of the weight-streaming kernel, per format.
// Measured (layer ms, two reps; groups of 4 / 8 / 16): 256-token DeepSeek-V3 fp8 slice 0.319 /
// 0.319 / 0.314; 64-token Qwen3-235B MXFP8 slice 0.1795 / 0.185 / 0.192; 64-token DeepSeek-V3
// MXFP4 slice 0.178 / 0.177 / 0.177.
template <int FMT>
constexpr int q_stream_group() {
  return FMT == MOE_FP8_E4M3 ? 16 : FMT == MOE_MXFP8 ? 4 : 8;
}


// Block scales of a K-step follow its operands in the LDS stage: MXFP4 E8M0 [128 A rows][8 B] then
// [256 B rows][8 B]; MXFP8 E8M0 [128][4 B] then [256][4 B] and 512 spare bytes (the target of the
// padding loads that keep every wave's load count equal); fp8 fp32 [128 A rows] then the two B
// block scales (1 KB).
template <int FMT>
constexpr int q_scale_stage_bytes() {
  return FMT == MOE_MXFP4 ? (128 + 256) * 8 : (FMT == MOE_MXFP8 ? (128 + 256) * 4 + 512 : 1024);
}

template <int FMT, int EPI>
__global__ void __launch_bounds__(256)
gemm_q_kernel(GemmArgs p, int n_tiles, int x_tiles, int span, int total, int gm) {
  constexpr bool MX4 = FMT == MOE_MXFP4;   // e2m1 elements, E8M0 per 32
  constexpr bool MX8 = FMT == MOE_MXFP8;   // e4m3 elements, E8M0 per 32
  constexpr bool MX = MX4 || MX8;          // E8M0 scales go straight into the MFMA
  constexpr bool SWIGLU = EPI >= QEPI_SWIGLU_BF16;
  constexpr int BM = 128, BN = 256, NW = 4, TM = 32, FM = 2, FN = 16, S = 3;
  constexpr int RB = 128;                  // bytes per row slice (one K-step)
  constexpr int KE = MX4 ? 256 : 128;      // elements per K-step
  constexpr int SUB = MX4 ? 2 : 1;         // 128-element MFMA substeps per K-step
  constexpr int A_INS = BM / (8 * NW), B_INS = BN / (8 * NW);
  constexpr int SINS = MX4 ? 3 : (MX8 ? 2 : 1);   // 4-byte scale loads per wave per K-step
  constexpr int INS = A_INS + B_INS + SINS;
  constexpr int DATA = (BM + BN) * RB;     // operand bytes per LDS stage
  constexpr int SCALE_BYTES = q_scale_stage_bytes<FMT>();
  constexpr int STAGE = DATA + SCALE_BYTES; // bytes per LDS stage
  constexpr int NB = 4;                    // B fragments per MFMA batch
  constexpr int FMT_CODE = MX4 ? 4 : 0;    // f8f6f4 operand format: 0 = fp8 e4m3, 4 = fp4 e2m1
  using Geo = SliceGeo<64>;                // 128-byte rows
  static_assert((S - 2) * INS < 64, "pipeline depth");

  extern __shared__ __attribute__((aligned(1024))) uint8_t ldsq[];

  const int logical = xcd_remap(blockIdx.x, span);
  if (logical >= total) return;
  Tile t;
  if (!resolve_tile(p, BM, n_tiles, x_tiles, logical, t, gm)) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K = p.K;
  const int nk = K / KE;
  const long long b_row_bytes = MX4 ? K / 2 : K;
  const int lrow = lane >> 3;

  // ---- DMA sources of this lane's rows ----
  const char* a_src[A_INS];
#pragma unroll
  for (int j = 0; j < A_INS; ++j) {
    const int r = (j * NW + wave) * 8 + lrow;
    a_src[j] = static_cast<const char*>(p.A) + a_src_row(p, t, t.row0 + r) * p.a_pitch +
               ((lane & 7) ^ Geo::swz(r)) * 16;
  }
  // B row (and matrix) behind tile row rb
  auto b_row = [&](int rb, const char*& base, const char*& sbase) -> long long {
    long long n;
    base = t.B;
    sbase = t.Bs;
    if (SWIGLU) {
      n = (long long)t.nt * (BN / 2) + (rb % (BN / 2));
      if (rb >= BN / 2) { base = t.B2; sbase = t.B2s; }
    } else {
      n = (long long)t.nt * BN + rb;
    }
    return n < p.N ? n : p.N - 1;
  };
  const char* b_src[B_INS];
#pragma unroll
  for (int j = 0; j < B_INS; ++j) {
    const int rb = (j * NW + wave) * 8 + lrow;
    const char *base, *sb;
    const long long n = b_row(rb, base, sb);
    b_src[j] = base + n * b_row_bytes + ((lane & 7) ^ Geo::swz(rb)) * 16;
  }
  // ---- scale sources (one 4-byte direct-to-LDS load per lane and instruction) ----
  // MXFP4: wave w moves A scale rows [32w, 32w + 32) and B scale rows [64w, 64w + 64), 8 bytes
  //        (one K-step) per row, two lanes per row.
  // MXFP8: 4 bytes per row and K-step, one lane per row: wave w's loads c = 0, 1 take 64-row slot
  //        u = 2w + c: A rows for u < 2, B rows for 2 <= u < 6, and for u >= 6 the A rows again
  //        into the spare bytes.
  // fp8:   waves 0 and 1 move A scale rows [64w, 64w + 64) (one fp32 per row and K-step); wave 2
  //        the two B block scales (lane i: scale i & 1); wave 3 the same into a spare slot (every
  //        wave issues the same number of loads, so the wait counts are uniform).
  const char* s_src[SINS];
  int s_dst[SINS];
  long long s_step[SINS];                  // bytes between consecutive K-steps of a source
  if constexpr (MX8) {
    const int gpr = K / 32;                // scale bytes per row
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int u = wave * 2 + c;
      if (u < 2 || u >= 6) {
        const int r = (u & 1) * 64 + lane;
        s_src[c] = static_cast<const char*>(p.A_scales) + a_src_row(p, t, t.row0 + r) * gpr;
        s_dst[c] = u < 2 ? DATA + u * 256 : DATA + (BM + BN) * 4 + (u - 6) * 256;
      } else {
        const int rb = (u - 2) * 64 + lane;
        long long n;
        const char* sbase = t.Bs;
        if (SWIGLU) {
          n = (long long)t.nt * (BN / 2) + (rb % (BN / 2));
          if (rb >= BN / 2) sbase = t.B2s;
        } else {
          n = (long long)t.nt * BN + rb;
        }
        if (n >= p.N) n = p.N - 1;
        s_src[c] = sbase + n * gpr;
        s_dst[c] = DATA + BM * 4 + (u - 2) * 256;
      }
      s_step[c] = 4;
    }
  } else if constexpr (MX4) {
    const int gpr = K / 32;                // scale bytes per row
    {
      const int r = wave * 32 + (lane >> 1);
      s_src[0] = static_cast<const char*>(p.A_scales) + a_src_row(p, t, t.row0 + r) * gpr + (lane & 1) * 4;
      s_dst[0] = DATA + wave * 256;
      s_step[0] = 8;
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int rb = (wave * 2 + c) * 32 + (lane >> 1);
      long long n;
      const char* sbase = t.Bs;
      if (SWIGLU) {
        n = (long long)t.nt * (BN / 2) + (rb % (BN / 2));
        if (rb >= BN / 2) sbase = t.B2s;
      } else {
        n = (long long)t.nt * BN + rb;
      }
      if (n >= p.N) n = p.N - 1;
      s_src[1 + c] = sbase + n * gpr + (lane & 1) * 4;
      s_dst[1 + c] = DATA + BM * 8 + (wave * 2 + c) * 256;
      s_step[1 + c] = 8;
    }
  } else {
    const int kb = K / 128;                // fp32 scales per row
    if (wave < 2) {
      const int r = wave * 64 + lane;
      s_src[0] = static_cast<const char*>(p.A_scales) +
                 (long long)(a_src_row(p, t, t.row0 + r) / p.a_scale_rows) * kb * 4;
      s_dst[0] = DATA + wave * 256;
    } else {
      const char* b0;
      const char* b1;
      if (SWIGLU) {                        // 128 h-columns = one block of gate and one of up
        b0 = t.Bs + (long long)t.nt * kb * 4;
        b1 = t.B2s + (long long)t.nt * kb * 4;
      } else {                             // two 128-column blocks
        b0 = t.Bs + (long long)(t.nt * 2) * kb * 4;
        b1 = t.Bs + (long long)min(t.nt * 2 + 1, (p.N - 1) / 128) * kb * 4;
      }
      s_src[0] = (lane & 1) ? b1 : b0;
      s_dst[0] = DATA + 512 + (wave - 2) * 256;
    }
    s_step[0] = 4;
  }

  // load q of this wave's share of K-step kt (q < A_INS: A rows, then B rows, then scales)
  auto issue_one = [&](int kt, int q, int stage) {
    uint8_t* la = ldsq + stage * STAGE;
    if (q < A_INS) {
      dma_16b_asm(a_src[q] + (long long)kt * RB, la + (q * NW + wave) * 8 * RB);
    } else if (q < A_INS + B_INS) {
      const int j = q - A_INS;
      dma_16b_asm(b_src[j] + (long long)kt * RB, la + BM * RB + (j * NW + wave) * 8 * RB);
    } else {
      const int j = q - A_INS - B_INS;
      dma_4b_asm(s_src[j] + kt * s_step[j], la + s_dst[j]);
    }
  };
  auto issue = [&](int kt) {
    if (kt >= nk) return;
#pragma unroll
    for (int q = 0; q < INS; ++q) issue_one(kt, q, kt % S);
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{};

  // fragment readers (operand of the 16x16x128 f8f6f4 MFMA: lane l holds row/column l % 16; for
  // MXFP4 the 32 K-elements [32 (l / 16), +32) of the 128; for MXFP8 chunks l / 16 and l / 16 + 4,
  // the hardware's K order; for fp8 with whole-step block scales any K order shared by both
  // operands gives the same dot product: chunks 2 (l / 16) and 2 (l / 16) + 1)
  const int q = lane >> 4;
  auto read_frag = [&](const uint8_t* base, int r, int s) -> i32x8 {
    i32x8 out;
    if constexpr (MX4) {
      const int c = s * 4 + q;                       // 16 bytes = 32 fp4
      const i32x4 v = *reinterpret_cast<const i32x4*>(base + r * RB + ((c ^ Geo::swz(r)) * 16));
      out = i32x8{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
    } else {
      const int c0 = MX8 ? q : 2 * q, c1 = MX8 ? q + 4 : 2 * q + 1;   // 32 bytes = 32 fp8
      const i32x4 v0 = *reinterpret_cast<const i32x4*>(base + r * RB + ((c0 ^ Geo::swz(r)) * 16));
      const i32x4 v1 = *reinterpret_cast<const i32x4*>(base + r * RB + ((c1 ^ Geo::swz(r)) * 16));
      out = i32x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    }
    return out;
  };

  // prologue: steps 0 .. S-2 in flight, wait for step 0
#pragma unroll
  for (int qq = 0; qq < S - 1; ++qq) issue(qq);
  if (nk >= S - 1) wait_vmem_n<(S - 2) * INS>();
  else wait_vmem();
  barrier_lds();

  // The loads of step kt + S - 1 (its stage was released by the last barrier) are spread through
  // the MFMAs of step kt, a few after each batch: issuing them in one block stalls the wave for
  // as long as the address unit takes to accept them, with the matrix unit idle.
  constexpr int BATCHES = SUB * (FN / NB);
  constexpr int PER_BATCH = (INS + BATCHES - 1) / BATCHES;
  for (int kt = 0; kt < nk; ++kt) {
    // step kt + S - 1 goes into the stage the last barrier released; past the end the last step
    // loads itself again there, unread: no branch in the loop, so nothing can move the MFMAs out
    // of their place between the loads
    const int kn = kt + S - 1 < nk ? kt + S - 1 : nk - 1;
    const uint8_t* la = ldsq + (kt % S) * STAGE;
    const uint8_t* lb = la + BM * RB;

    // scales of this K-step, staged with its operands
    const uint8_t* ls = la + DATA;
    float fs[MX ? 1 : FM * 4][2];
    u32x2 sam[MX4 ? FM : 1], sbm[MX4 ? FN : 1];
    uint32_t sa8[MX8 ? FM : 1], sb8[MX8 ? FN : 1];
    if constexpr (MX8) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
        sa8[i] = *reinterpret_cast<const uint32_t*>(ls + (wave * TM + i * 16 + (lane & 15)) * 4);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        sb8[j] = *reinterpret_cast<const uint32_t*>(ls + BM * 4 + (j * 16 + (lane & 15)) * 4);
    } else if constexpr (!MX) {
      const float g0 = reinterpret_cast<const float*>(ls + 512)[0];
      const float g1 = reinterpret_cast<const float*>(ls + 512)[1];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const f32x4 a4 = *reinterpret_cast<const f32x4*>(ls + (wave * TM + i * 16 + q * 4) * 4);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          fs[i * 4 + v][0] = a4[v] * g0;
          fs[i * 4 + v][1] = a4[v] * g1;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i)
        sam[i] = *reinterpret_cast<const u32x2*>(ls + (wave * TM + i * 16 + (lane & 15)) * 8);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        sbm[j] = *reinterpret_cast<const u32x2*>(ls + BM * 8 + (j * 16 + (lane & 15)) * 8);
    }

#pragma unroll
    for (int s = 0; s < SUB; ++s) {
      i32x8 fa[FM];
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[i] = read_frag(la, wave * TM + i * 16 + (lane & 15), s);
#pragma unroll
      for (int b0 = 0; b0 < FN; b0 += NB) {
        i32x8 fb[NB];
#pragma unroll
        for (int jj = 0; jj < NB; ++jj) fb[jj] = read_frag(lb, (b0 + jj) * 16 + (lane & 15), s);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int jj = 0; jj < NB; ++jj) {
            const int j = b0 + jj;
            if constexpr (MX) {
              // lane group q passes the scale of K group q of the (sub)step
              const int sa = static_cast<int>(((MX4 ? sam[i][s] : sa8[i]) >> (8 * q)) & 0xFFu);
              const int sb = static_cast<int>(((MX4 ? sbm[j][s] : sb8[j]) >> (8 * q)) & 0xFFu);
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  fa[i], fb[jj], acc[i][j], FMT_CODE, FMT_CODE, 0, sa, 0, sb);
            } else {
              const f32x4 tmp = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  fa[i], fb[jj], f32x4{}, FMT_CODE, FMT_CODE, 0, 127, 0, 127);
              const int half = j >= FN / 2 ? 1 : 0;
#pragma unroll
              for (int v = 0; v < 4; ++v) acc[i][j][v] = fmaf(tmp[v], fs[i * 4 + v][half], acc[i][j][v]);
            }
          }
        MOE_SCHED_FENCE();
        {
          const int batch = s * (FN / NB) + b0 / NB;
#pragma unroll
          for (int u = 0; u < PER_BATCH; ++u) {
            const int q = batch * PER_BATCH + u;
            if (q < INS) issue_one(kn, q, (kt + S - 1) % S);
          }
        }
        MOE_SCHED_FENCE();
      }
    }
    wait_vmem_n<(S - 2) * INS>();          // step kt+1 landed (only step kt+2's loads remain)
    barrier_lds();
  }
  wait_vmem();                             // the unread tail loads, before the stores

  // ---- epilogue ----
  char* C = static_cast<char*>(p.C);
  const int colw = lane & 15;
  if constexpr (!SWIGLU) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const long long col = (long long)t.nt * BN + j * 16 + colw;
        if (col >= p.N) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = t.row0 + wave * TM + i * 16 + q * 4 + v;
          if (r >= t.row1) continue;
          if (EPI == QEPI_STORE_F32) reinterpret_cast<float*>(C + r * p.c_pitch)[col] = acc[i][j][v];
          else reinterpret_cast<uint16_t*>(C + r * p.c_pitch)[col] = f32_to_bf16(acc[i][j][v]);
        }
      }
  } else {
    constexpr int HF = FN / 2;             // h fragments: 8 x 16 = 128 columns
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = t.row0 + wave * TM + i * 16 + q * 4 + v;
        const bool live = r < t.row1;       // uniform per 16-lane group
        float h[HF];
#pragma unroll
        for (int j = 0; j < HF; ++j) h[j] = silu_fast(acc[i][j][v]) * acc[i][j + HF][v];
        if constexpr (EPI == QEPI_SWIGLU_BF16) {
          if (!live) continue;
#pragma unroll
          for (int j = 0; j < HF; ++j) {
            const long long col = (long long)t.nt * (BN / 2) + j * 16 + colw;
            if (col < p.N) reinterpret_cast<uint16_t*>(C + r * p.c_pitch)[col] = f32_to_bf16(h[j]);
          }
        } else if constexpr (MX8) {
          // MXFP8 h: four 1 x 32 groups per row (fragments 2g, 2g+1), one code byte per lane
          uint8_t* crow = reinterpret_cast<uint8_t*>(C + r * p.c_pitch);
#pragma unroll
          for (int g = 0; g < HF / 2; ++g) {
            float amax = fmaxf(fabsf(h[2 * g]), fabsf(h[2 * g + 1]));
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
            const int e = mx_shared_exp<8>(amax);
            const float mul = ldexpf(1.0f, -e);
            if (!live) continue;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const long long col = (long long)t.nt * (BN / 2) + (2 * g + hh) * 16 + colw;
              crow[col] = e4m3_rne_sat(h[2 * g + hh] * mul);
            }
            if (colw == 0)
              reinterpret_cast<uint8_t*>(p.C_scales)[(long long)r * (p.N / 32) + (t.nt * (BN / 2)) / 32 + g] =
                  static_cast<uint8_t>(e + 127);
          }
        } else if constexpr (!MX) {
          // fp8 h: one 1 x 128 block per row per tile (the 128 h-columns of this tile)
          float amax = 0.0f;
#pragma unroll
          for (int j = 0; j < HF; ++j) amax = fmaxf(amax, fabsf(h[j]));
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
          const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
          if (!live) continue;
          uint8_t* crow = reinterpret_cast<uint8_t*>(C + r * p.c_pitch);
#pragma unroll
          for (int j = 0; j < HF; ++j) {
            const long long col = (long long)t.nt * (BN / 2) + j * 16 + colw;
            crow[col] = e4m3_rne_sat(h[j] / sc);
          }
          if (colw == 0)
            reinterpret_cast<float*>(p.C_scales)[(long long)r * (p.N / 128) + t.nt] = sc;
        } else {
          // MXFP4 h: four 1 x 32 groups per row (fragments 2g, 2g+1)
          uint8_t* crow = reinterpret_cast<uint8_t*>(C + r * p.c_pitch);
#pragma unroll
          for (int g = 0; g < HF / 2; ++g) {
            float amax = fmaxf(fabsf(h[2 * g]), fabsf(h[2 * g + 1]));
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
            const int e = mx_shared_exp(amax);
            const float mul = ldexpf(1.0f, -e);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const uint32_t code = e2m1_rne_sat(h[2 * g + hh] * mul);
              const uint32_t other = __shfl_xor(code, 1, 64);     // neighbouring column
              const long long col = (long long)t.nt * (BN / 2) + (2 * g + hh) * 16 + colw;
              if (live && (colw & 1) == 0) crow[col / 2] = static_cast<uint8_t>(code | (other << 4));
            }
            if (live && colw == 0)
              reinterpret_cast<uint8_t*>(p.C_scales)[(long long)r * (p.N / 32) + (t.nt * (BN / 2)) / 32 + g] =
                  static_cast<uint8_t>(e + 127);
          }
        }
      }
  }
}

// ------------------------------------------------------------------------------------------------
// Weight-streaming variant for decode-sized groups (fp8 and MXFP4 weights), after the bf16 one in
// gemm.hip: the weights are the scaled MFMA's first operand and go straight to registers, 128
// bytes of every row per K-pair (one 128-element step for fp8, two for MXFP4), each load
// instruction covering 8 rows x 128 contiguous bytes, redistributed to the operand lanes with
// ds_bpermute; activations and block scales are loaded in the operand layout directly; pairs are
// double-buffered. For fp8 a lane's 32-byte operand is chunks kq and kq + 4 of the pair (the same
// chunks of the activation row, so the dot product is unchanged); for MXFP4 step s uses chunk
// 4 s + kq and scale byte 4 s + kq of the row's 8 scale bytes per pair; MXFP8 uses the fp8
// operand (chunks kq and kq + 4, the hardware's K order) and scale byte kq of the pair.
// Workgroup: 4 waves on 16 * FM rows x 4 adjacent column blocks of one group (SWIGLU: 128 h-columns,
// wave w on 32 of them = 32 gate + 32 up weight rows; STORE: 256 columns, 64 per wave), so the
// fp8 1 x 128 blocks of h are complete inside the workgroup (row amax exchanged through LDS) and
// the MXFP4 1 x 32 groups inside one wave.
// ------------------------------------------------------------------------------------------------
// The body of gemm_q_stream_kernel for a tile whose rows fill L of its 16-row fragments (only
// those fragments' activation rows and scales are loaded and multiplied). amax_x: [4][ASTR] fp8 h
// row amax exchange; part: the K-split's LDS partial sums, [KS - 1][4][L][64].
template <int L, int FMT, int EPI, int KS, int ASTR>
__device__ __forceinline__ void stream_q_tile(const GemmArgs& p, const Tile& t, float* amax_x, f32x4* part) {
  constexpr bool MX4 = FMT == MOE_MXFP4, MX8 = FMT == MOE_MXFP8, MX = MX4 || MX8;
  constexpr bool SWIGLU = EPI >= QEPI_SWIGLU_BF16;
  constexpr int FMT_CODE = MX4 ? 4 : 0;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  constexpr int NCB = 4 / KS;              // column blocks of 64 weight rows per tile
  const int cw = wave % NCB;               // column block of the wave inside the tile
  const int kh = wave / NCB;               // the wave's K range
  const int lr = lane & 15, kq = lane >> 4;
  const int K = p.K;
  const long long wrow = MX4 ? K / 2 : K;  // weight row bytes
  const int np_all = MX4 ? K / 256 : K / 128;   // K-pairs (128 bytes of every row)
  const int c0 = np_all * kh / KS;         // this wave's K-pairs [c0, c0 + np)
  const int np = np_all * (kh + 1) / KS - c0;
  // weight rows of fragment j (SWIGLU: j < 2 gate, else up; 16 rows each) of this wave
  auto wrow_of = [&](int j, int r, const char*& base, const char*& sbase) -> long long {
    long long n;
    base = t.B;
    sbase = t.Bs;
    if (SWIGLU) {
      n = (long long)t.nt * (128 / KS) + cw * 32 + (j & 1) * 16 + r;
      if (j >= 2) { base = t.B2; sbase = t.B2s; }
    } else {
      n = (long long)t.nt * (256 / KS) + cw * 64 + j * 16 + r;
    }
    return n < p.N ? n : p.N - 1;          // columns past N: valid row, never stored
  };
  const char* wp[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const char *base, *sb;
      const long long n = wrow_of(j, h * 8 + (lane >> 3), base, sb);
      wp[j][h] = base + n * wrow + (lane & 7) * 16;
    }
  const char* A = static_cast<const char*>(p.A);
  const char* ap[L];
  long long arow[L];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    arow[i] = a_src_row(p, t, t.row0 + i * 16 + lr);
    ap[i] = A + arow[i] * p.a_pitch + kq * 16;
  }
  // block scales: MX E8M0 bytes of the operand rows (8 per pair for MXFP4, 4 for MXFP8); fp8 fp32
  // block scales
  const uint8_t* wsc[MX ? 4 : 1];
  const uint8_t* asc[MX ? L : 1];
  const float* wsf[MX ? 1 : 2];
  const float* asf[MX ? 1 : L];
  if constexpr (MX) {
    const int gpr = K / 32;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const char *base, *sb;
      const long long n = wrow_of(j, lr, base, sb);
      wsc[j] = reinterpret_cast<const uint8_t*>(sb) + n * gpr;
    }
#pragma unroll
    for (int i = 0; i < L; ++i) asc[i] = static_cast<const uint8_t*>(p.A_scales) + arow[i] * gpr;
  } else {
    const int kb = K / 128;
    const char *b0, *s0, *b1, *s1;
    const long long n0 = wrow_of(0, 0, b0, s0), n1 = wrow_of(SWIGLU ? 2 : 0, 0, b1, s1);
    wsf[0] = reinterpret_cast<const float*>(s0) + (n0 / 128) * kb;
    wsf[1] = reinterpret_cast<const float*>(s1) + (n1 / 128) * kb;   // SWIGLU: the up block
#pragma unroll
    for (int i = 0; i < L; ++i)
      asf[i] = static_cast<const float*>(p.A_scales) + (arow[i] / p.a_scale_rows) * kb;
  }
  const int src0 = ((lr & 7) * 8 + kq) * 4, src1 = src0 + 16;
  const bool upper = lr >= 8;

  i32x4 wraw[2][4][2];
  i32x4 av[2][L][2];
  u32x2 wsm[2][MX ? 4 : 1], asm_[2][MX ? L : 1];
  float wss[2][2], ass[2][MX ? 1 : L];
  auto load = [&](int c, int set) {
    c = c0 + (c < np ? c : np - 1);
    const long long off = (long long)c * 128;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        wraw[set][j][h] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(wp[j][h] + off));
#pragma unroll
    for (int i = 0; i < L; ++i)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        av[set][i][s2] = *reinterpret_cast<const i32x4*>(ap[i] + off + s2 * 64);
    if constexpr (MX4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) wsm[set][j] = *reinterpret_cast<const u32x2*>(wsc[j] + c * 8);
#pragma unroll
      for (int i = 0; i < L; ++i) asm_[set][i] = *reinterpret_cast<const u32x2*>(asc[i] + c * 8);
    } else if constexpr (MX8) {
#pragma unroll
      for (int j = 0; j < 4; ++j) wsm[set][j][0] = *reinterpret_cast<const uint32_t*>(wsc[j] + c * 4);
#pragma unroll
      for (int i = 0; i < L; ++i) asm_[set][i][0] = *reinterpret_cast<const uint32_t*>(asc[i] + c * 4);
    } else {
      wss[set][0] = wsf[0][c];
      wss[set][1] = wsf[1][c];
#pragma unroll
      for (int i = 0; i < L; ++i) ass[set][i] = asf[i][c];
    }
  };
  f32x4 acc[4][L];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < L; ++i) acc[j][i] = f32x4{};
  auto piece = [&](int set, int j, int src) -> i32x4 {
    i32x4 w;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int lo = __builtin_amdgcn_ds_bpermute(src, wraw[set][j][0][q]);
      const int hi = __builtin_amdgcn_ds_bpermute(src, wraw[set][j][1][q]);
      w[q] = upper ? hi : lo;
    }
    return w;
  };
  auto compute = [&](int set) {
    if constexpr (MX8) {
      i32x8 wf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const i32x4 w0 = piece(set, j, src0), w1 = piece(set, j, src1);
        wf[j] = i32x8{w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
      }
#pragma unroll
      for (int i = 0; i < L; ++i) {
        const i32x4 a0 = av[set][i][0], a1 = av[set][i][1];
        const i32x8 a = i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        const int sa = static_cast<int>((asm_[set][i][0] >> (8 * kq)) & 0xFFu);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int sw = static_cast<int>((wsm[set][j][0] >> (8 * kq)) & 0xFFu);
          acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[j], a, acc[j][i], FMT_CODE,
                                                                      FMT_CODE, 0, sw, 0, sa);
        }
      }
    } else if constexpr (MX4) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        i32x8 wf[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const i32x4 w = piece(set, j, s2 ? src1 : src0);
          wf[j] = i32x8{w[0], w[1], w[2], w[3], 0, 0, 0, 0};
        }
        const int sh = 8 * (s2 * 4 + kq);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int sw = static_cast<int>(((s2 ? wsm[set][j][1] : wsm[set][j][0]) >> (sh - 32 * s2)) & 0xFFu);
#pragma unroll
          for (int i = 0; i < L; ++i) {
            const int sa = static_cast<int>(((s2 ? asm_[set][i][1] : asm_[set][i][0]) >> (sh - 32 * s2)) & 0xFFu);
            const i32x4 a = av[set][i][s2];
            acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                wf[j], i32x8{a[0], a[1], a[2], a[3], 0, 0, 0, 0}, acc[j][i], FMT_CODE, FMT_CODE, 0, sw, 0, sa);
          }
        }
      }
    } else {
      i32x8 wf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const i32x4 w0 = piece(set, j, src0), w1 = piece(set, j, src1);
        wf[j] = i32x8{w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
      }
#pragma unroll
      for (int i = 0; i < L; ++i) {
        const i32x4 a0 = av[set][i][0], a1 = av[set][i][1];
        const i32x8 a = i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 tmp = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              wf[j], a, f32x4{}, FMT_CODE, FMT_CODE, 0, 127, 0, 127);
          const float sc = ass[set][i] * wss[set][(SWIGLU && j >= 2) ? 1 : 0];
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[j][i][v] = fmaf(tmp[v], sc, acc[j][i][v]);
        }
      }
    }
  };
  if (np > 0) {                            // wave-uniform; np = 0 only if K-pairs < KS
    load(0, 0);
    int c = 0;
    for (; c + 1 < np; c += 2) {
      MOE_SCHED_FENCE();
      load(c + 1, 1);
      MOE_SCHED_FENCE();
      compute(0);
      MOE_SCHED_FENCE();
      load(c + 2, 0);
      MOE_SCHED_FENCE();
      compute(1);
    }
    MOE_SCHED_FENCE();
    if (c < np) compute(0);                  // odd number of pairs: the last is in set 0
  }
  if constexpr (KS > 1) {
    // K-split: the waves of K ranges 1.. hand their partial sums to the wave of range 0 of the
    // same column block through LDS, which adds them in range order and finishes the block
    // part: [KS - 1][NCB][4][L][64]
    if (kh > 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < L; ++i)
          part[((((kh - 1) * NCB + cw) * 4 + j) * L + i) * 64 + lane] = acc[j][i];
    }
    __syncthreads();
    if (kh > 0) return;
#pragma unroll
    for (int w = 0; w < KS - 1; ++w)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < L; ++i) acc[j][i] += part[(((w * NCB + cw) * 4 + j) * L + i) * 64 + lane];
  }

  // ---- epilogue: acc[j][i][v] = weight row j * 16 + kq * 4 + v of the wave, C row row0 + i*16 + lr
  char* C = static_cast<char*>(p.C);
  if constexpr (!SWIGLU) {
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int r = t.row0 + i * 16 + lr;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const long long col = (long long)t.nt * (256 / KS) + cw * 64 + j * 16 + kq * 4;
        if (r >= t.row1 || col >= p.N) continue;
        char* crow = C + (long long)r * p.c_pitch;
        if (EPI == QEPI_STORE_F32) {
          *reinterpret_cast<f32x4*>(crow + col * 4) = acc[j][i];
        } else {
          *reinterpret_cast<uint2*>(crow + col * 2) =
              make_uint2(pack_bf16x2(acc[j][i][0], acc[j][i][1]), pack_bf16x2(acc[j][i][2], acc[j][i][3]));
        }
      }
    }
  } else {
    // h[i][jj][v]: h column (jj * 16 + kq * 4 + v) of the wave's 32, C row row0 + i*16 + lr
    float h[L][2][4];
#pragma unroll
    for (int i = 0; i < L; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int v = 0; v < 4; ++v) h[i][jj][v] = silu_fast(acc[jj][i][v]) * acc[jj + 2][i][v];
    const long long col0 = (long long)t.nt * (128 / KS) + cw * 32;   // first h column of the wave
    if constexpr (EPI == QEPI_SWIGLU_BF16) {
#pragma unroll
      for (int i = 0; i < L; ++i) {
        const int r = t.row0 + i * 16 + lr;
        if (r >= t.row1) continue;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
          *reinterpret_cast<uint2*>(C + (long long)r * p.c_pitch + (col0 + jj * 16 + kq * 4) * 2) =
              make_uint2(pack_bf16x2(h[i][jj][0], h[i][jj][1]), pack_bf16x2(h[i][jj][2], h[i][jj][3]));
      }
    } else if constexpr (MX8) {
      // one 1 x 32 group per row: the wave's 32 columns; row amax over the 4 lanes of the row
#pragma unroll
      for (int i = 0; i < L; ++i) {
        float amax = 0.0f;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int v = 0; v < 4; ++v) amax = fmaxf(amax, fabsf(h[i][jj][v]));
        amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        const int e = mx_shared_exp<8>(amax);
        const float mul = ldexpf(1.0f, -e);
        const int r = t.row0 + i * 16 + lr;
        if (r >= t.row1) continue;
        uint8_t* crow = reinterpret_cast<uint8_t*>(C + (long long)r * p.c_pitch);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const uint32_t word = e4m3x4_rne_sat(h[i][jj][0] * mul, h[i][jj][1] * mul, h[i][jj][2] * mul,
                                               h[i][jj][3] * mul);
          *reinterpret_cast<uint32_t*>(crow + col0 + jj * 16 + kq * 4) = word;
        }
        if (kq == 0)
          static_cast<uint8_t*>(p.C_scales)[(long long)r * (p.N / 32) + col0 / 32] = static_cast<uint8_t>(e + 127);
      }
    } else if constexpr (MX4) {
      // one 1 x 32 group per row: the wave's 32 columns; row amax over the 4 lanes of the row
#pragma unroll
      for (int i = 0; i < L; ++i) {
        float amax = 0.0f;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int v = 0; v < 4; ++v) amax = fmaxf(amax, fabsf(h[i][jj][v]));
        amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        const int e = mx_shared_exp(amax);
        const float mul = ldexpf(1.0f, -e);
        const int r = t.row0 + i * 16 + lr;
        if (r >= t.row1) continue;
        uint8_t* crow = reinterpret_cast<uint8_t*>(C + (long long)r * p.c_pitch);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          uint32_t b[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) b[v] = e2m1_rne_sat(h[i][jj][v] * mul);
          const uint16_t two = static_cast<uint16_t>((b[0] | (b[1] << 4)) | ((b[2] | (b[3] << 4)) << 8));
          *reinterpret_cast<uint16_t*>(crow + (col0 + jj * 16 + kq * 4) / 2) = two;
        }
        if (kq == 0)
          static_cast<uint8_t*>(p.C_scales)[(long long)r * (p.N / 32) + col0 / 32] = static_cast<uint8_t>(e + 127);
      }
    } else {
      // fp8: one 1 x 128 block per row over the workgroup's 128 columns (4 waves)
#pragma unroll
      for (int i = 0; i < L; ++i) {
        float amax = 0.0f;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int v = 0; v < 4; ++v) amax = fmaxf(amax, fabsf(h[i][jj][v]));
        amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        if (kq == 0) amax_x[wave * ASTR + i * 16 + lr] = amax;
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < L; ++i) {
        const int rl = i * 16 + lr;
        const float amax = fmaxf(fmaxf(amax_x[rl], amax_x[ASTR + rl]), fmaxf(amax_x[2 * ASTR + rl], amax_x[3 * ASTR + rl]));
        const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
        const int r = t.row0 + rl;
        if (r >= t.row1) continue;
        uint8_t* crow = reinterpret_cast<uint8_t*>(C + (long long)r * p.c_pitch);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const uint32_t word = e4m3x4_rne_sat(h[i][jj][0] / sc, h[i][jj][1] / sc, h[i][jj][2] / sc,
                                               h[i][jj][3] / sc);
          *reinterpret_cast<uint32_t*>(crow + col0 + jj * 16 + kq * 4) = word;
        }
        if (wave == 0 && kq == 0)
          reinterpret_cast<float*>(p.C_scales)[(long long)r * (p.N / 128) + t.nt] = sc;
      }
    }
  }
}

template <int FMT, int EPI, int FM, int KS>
__global__ void __launch_bounds__(256)
gemm_q_stream_kernel(GemmArgs p, int n_tiles, int x_tiles, int total) {
  // KS = 1: the 4 waves take 4 adjacent column blocks (fp8's 1 x 128 h blocks need all four);
  // KS = 4: they share one column block and split it over four K ranges, whose partial sums meet
  // through LDS at the end
  static_assert(KS == 1 || KS == 4, "K split");
  static_assert(KS == 1 || !(EPI == QEPI_SWIGLU_Q && FMT == MOE_FP8_E4M3), "fp8 h blocks span 4 waves");
  static_assert(FM == 1 || FM == 2, "tile rows");
  constexpr int BM = 16 * FM;
  __shared__ float amax_x[4 * BM];         // fp8 h: per-wave row amax
  __shared__ f32x4 part[KS > 1 ? (KS - 1) * (4 / KS) * 4 * FM * 64 : 1];

  constexpr int GM = q_stream_group<FMT>();
  const int logical = xcd_remap(blockIdx.x, GM);
  if (logical >= total) return;            // uniform per workgroup
  Tile t;
  if (!resolve_tile(p, BM, n_tiles, x_tiles, logical, t, GM)) return;
  // 16-row fragments holding rows of the tile (uniform over the workgroup): each count runs its
  // own instantiation, so every load and MFMA stays unconditional. Not for MXFP8: with both
  // bodies in one kernel its K-split form needs more than 256 registers (one wave per SIMD
  // instead of two; measured 14% slower on the 64-token Qwen3-235B slice)
  if constexpr (FM == 2) {
    if (FMT == MOE_MXFP8 || t.row1 - t.row0 > 16) {
      stream_q_tile<2, FMT, EPI, KS, BM>(p, t, amax_x, part);
      return;
    }
  }
  if constexpr (FMT != MOE_MXFP8 || FM == 1) stream_q_tile<1, FMT, EPI, KS, BM>(p, t, amax_x, part);
}

// ------------------------------------------------------------------------------------------------
// Wide-tile variant for prefill-sized groups in the MX formats: 256 x 256 tiles, 4 waves in a 2 x 2
// arrangement, each owning 128 rows x 128 B-rows as 4 x 4 fragments of 32 x 32 (256 accumulator
// registers), on v_mfma_scale_f32_32x32x64_f8f6f4: measured on the MI355X with one wave per SIMD
// it issues at the full fp8 and fp4 rates, while the 16 x 16 x 128 form loses ~20% there and runs
// fp4 only at the fp8 rate. A wave reads (128 + 128) x 128 bytes of fragments per 128-byte K-step
// (half the LDS bytes per flop of the 32-row wave tile above). The E8M0 scales go to the MFMA
// directly, so the accumulators never leave the matrix core's registers (fp8's fp32 block scales
// would need a vector FMA per MFMA on them; fp8 keeps the 32-row kernel).
// Operand layout of the 32 x 32 x 64 MFMA (measured): lane l holds row l % 32; lane half
// h = l / 32 holds, for fp8, K-elements [16h, 16h + 16) in bytes 0-15 and [32 + 16h, +16) in bytes
// 16-31, for fp4 K-elements [32h, 32h + 32) in bytes 0-15, and passes the E8M0 scale of K-elements
// [32h, 32h + 32). A 128-byte K-step is SUB = 2 (fp8) or 4 (fp4) substeps of 64 elements.
// Schedule: two LDS stages of 64 KB of operands plus the step's scales. Fragments of the next
// substep are read while the current one's MFMAs run. At the start of a step's last substep a
// wave waits for the next step's loads and the workgroup meets at a barrier; the wave then reads
// the next step's first fragments and issues the loads of the step after it into the stage just
// released, both while the last substep's MFMAs run, so the loads have a whole step to land.
// SwiGLU: wave column wn holds gate rows [64 wn, 64 wn + 64) and the up rows of the same h-columns,
// so gate and up of one h-column meet in one lane and a 1 x 32 MX group of h is one fragment row.
// ------------------------------------------------------------------------------------------------
constexpr int kQWideBM = 256, kQWideBN = 256, kQWideStages = 2;
// E8M0 scales travel in chunks of 16 bytes per row (4 K-steps of MXFP8, 2 of MXFP4), each lane
// loading one row's 16 bytes: per K-step that is a quarter (half) of the 4-byte loads' requests,
// which otherwise are as many as the operand loads'. Two chunk slots of [256 A + 256 B rows][16 B].
constexpr int kQWideScaleSlot = (kQWideBM + kQWideBN) * 16;
constexpr size_t kQWideLds = (size_t)kQWideStages * (kQWideBM + kQWideBN) * 128 + 2 * kQWideScaleSlot;

template <int FMT, int EPI>
__global__ void __launch_bounds__(256)
gemm_q_wide_kernel(GemmArgs p, int n_tiles, int x_tiles, int span, int total, int gm) {
  constexpr bool MX4 = FMT == MOE_MXFP4, MX8 = FMT == MOE_MXFP8;
  static_assert(MX4 || MX8, "E8M0-scaled formats only");
  constexpr bool SWIGLU = EPI >= QEPI_SWIGLU_BF16;
  constexpr int BM = kQWideBM, BN = kQWideBN, NW = 4, FM = 4, FN = 4, S = kQWideStages;
  constexpr int RB = 128;                  // bytes per row slice (one K-step)
  constexpr int KE = MX4 ? 256 : 128;      // elements per K-step
  constexpr int SUB = MX4 ? 4 : 2;         // 64-element MFMA substeps per K-step
  constexpr int A_INS = BM / (8 * NW), B_INS = BN / (8 * NW);
  constexpr int INS = A_INS + B_INS;       // operand loads per wave per K-step
  constexpr int SCH = 2;                   // scale chunk loads per wave (512 rows / 4 waves / 64)
  constexpr int DATA = (BM + BN) * RB;
  constexpr int STAGE = DATA;
  constexpr int SC_BASE = S * DATA;        // the two scale chunk slots
  constexpr int SRB = MX4 ? 8 : 4;         // E8M0 bytes per row and K-step
  constexpr int CH = 16 / SRB;             // K-steps per scale chunk
  constexpr int FMT_CODE = MX4 ? 4 : 0;
  using Geo = SliceGeo<64>;
  using SW = typename std::conditional<MX4, u32x2, uint32_t>::type;   // a row's scales of a step
  static_assert(INS + SCH < 64, "vmcnt range");
  static_assert(SUB % 2 == 0, "fragment sets alternate by substep parity");

  extern __shared__ __attribute__((aligned(1024))) uint8_t ldsw[];

  const int logical = xcd_remap(blockIdx.x, span);
  if (logical >= total) return;
  Tile t;
  if (!resolve_tile(p, BM, n_tiles, x_tiles, logical, t, gm)) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int K = p.K;
  const int nk = K / KE;
  const long long b_row_bytes = MX4 ? K / 2 : K;
  const int lrow = lane >> 3;
  const int l32 = lane & 31, h = lane >> 5;

  // B row (and matrices) behind tile B-row rb: SWIGLU rows [0, 128) gate, [128, 256) up
  auto b_row = [&](int rb, const char*& base, const char*& sbase) -> long long {
    long long n;
    base = t.B;
    sbase = t.Bs;
    if (SWIGLU) {
      n = (long long)t.nt * (BN / 2) + (rb % (BN / 2));
      if (rb >= BN / 2) { base = t.B2; sbase = t.B2s; }
    } else {
      n = (long long)t.nt * BN + rb;
    }
    return n < p.N ? n : p.N - 1;
  };
  // first tile B-row of this wave's fragment j
  auto frag_brow = [&](int j) -> int {
    if (SWIGLU) return j < FN / 2 ? wn * 64 + j * 32 : BN / 2 + wn * 64 + (j - FN / 2) * 32;
    return wn * 128 + j * 32;
  };

  // ---- DMA sources: 8 A and 8 B instructions of 8 rows x 128 bytes per wave ----
  const char* a_src[A_INS];
#pragma unroll
  for (int j = 0; j < A_INS; ++j) {
    const int r = (j * NW + wave) * 8 + lrow;
    a_src[j] = static_cast<const char*>(p.A) + a_src_row(p, t, t.row0 + r) * p.a_pitch +
               ((lane & 7) ^ Geo::swz(r)) * 16;
  }
  const char* b_src[B_INS];
#pragma unroll
  for (int j = 0; j < B_INS; ++j) {
    const int rb = (j * NW + wave) * 8 + lrow;
    const char *base, *sb;
    const long long n = b_row(rb, base, sb);
    b_src[j] = base + n * b_row_bytes + ((lane & 7) ^ Geo::swz(rb)) * 16;
  }
  // ---- scale chunk sources: load c of wave w moves rows of slot u = 2w + c, A rows
  //      [64u, 64u + 64) for u < 4, B rows [64 (u - 4), +64) for u >= 4, 16 bytes per lane ----
  const char* s_src[SCH];
  {
    const int gpr = K / 32;                // scale bytes per row
#pragma unroll
    for (int c = 0; c < SCH; ++c) {
      const int u = wave * SCH + c;
      if (u < 4) {
        s_src[c] = static_cast<const char*>(p.A_scales) + a_src_row(p, t, t.row0 + u * 64 + lane) * gpr;
      } else {
        const char *base, *sbase;
        const long long n = b_row((u - 4) * 64 + lane, base, sbase);
        s_src[c] = sbase + n * gpr;
      }
    }
  }
  const int nch = nk / CH;                 // scale chunks (K % 512 == 0)
  auto issue_scales = [&](int ch, int slot) {
#pragma unroll
    for (int c = 0; c < SCH; ++c)
      dma_16b_asm(s_src[c] + (long long)ch * 16, ldsw + SC_BASE + slot * kQWideScaleSlot + (wave * SCH + c) * 64 * 16);
  };

  // load qi of this wave's share of K-step kt into LDS stage `stage`
  auto issue_one = [&](int kt, int qi, int stage) {
    uint8_t* la = ldsw + stage * STAGE;
    if (qi < A_INS) {
      dma_16b_asm(a_src[qi] + (long long)kt * RB, la + (qi * NW + wave) * 8 * RB);
    } else {
      const int j = qi - A_INS;
      dma_16b_asm(b_src[j] + (long long)kt * RB, la + BM * RB + (j * NW + wave) * 8 * RB);
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

  // fragment (32 rows from tile row r0) of substep sub of the step in stage base
  auto read_frag = [&](const uint8_t* base, int r0, int sub) -> i32x8 {
    const int r = r0 + l32;
    if constexpr (MX4) {
      const int c = sub * 2 + h;                     // 16 bytes = 32 fp4
      const i32x4 v = *reinterpret_cast<const i32x4*>(base + r * RB + ((c ^ Geo::swz(r)) * 16));
      return i32x8{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
    } else {
      const int c0 = sub * 4 + h, c1 = sub * 4 + 2 + h;
      const i32x4 v0 = *reinterpret_cast<const i32x4*>(base + r * RB + ((c0 ^ Geo::swz(r)) * 16));
      const i32x4 v1 = *reinterpret_cast<const i32x4*>(base + r * RB + ((c1 ^ Geo::swz(r)) * 16));
      return i32x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    }
  };
  // fragment sets alternate by substep parity; scale words (a row's E8M0 bytes of a step) are
  // [current step, next step]
  i32x8 fa[2][FM], fb[2][FN];
  SW sa[2][FM], sb[2][FN];
  auto stage_ptr = [&](int kt) -> const uint8_t* { return ldsw + (kt % S) * STAGE; };
  // scale words of K-step kt (a row's E8M0 bytes of the step) into set sset. Substep sub of lane
  // half h needs byte 2 sub + h; the words are shifted right by 8 h once here, so that the MFMA's
  // op_sel picks byte 2 sub (MXFP8) or 2 (sub & 1) of word sub / 2 (MXFP4) for every lane with no
  // per-MFMA extraction
  auto read_scales = [&](int kt, int sset) {
    const uint8_t* ls = ldsw + SC_BASE + ((kt / CH) & 1) * kQWideScaleSlot + (kt % CH) * SRB;
#pragma unroll
    for (int jj = 0; jj < FN; ++jj)
      sb[sset][jj] = *reinterpret_cast<const SW*>(ls + (BM + frag_brow(jj) + l32) * 16) >> (8 * h);
#pragma unroll
    for (int ii = 0; ii < FM; ++ii)
      sa[sset][ii] = *reinterpret_cast<const SW*>(ls + (wm * 128 + ii * 32 + l32) * 16) >> (8 * h);
  };
  auto scale_word = [&](const SW& w, int sub) -> int {
    if constexpr (MX4) return static_cast<int>(w[sub >> 1]);
    else return static_cast<int>(w);
  };

  // prologue: scale chunk 0, steps 0 and 1, scale chunk 1 in flight; wait for the first two
  issue_scales(0, 0);
#pragma unroll
  for (int qi = 0; qi < INS; ++qi) issue_one(0, qi, 0);
#pragma unroll
  for (int qi = 0; qi < INS; ++qi) issue_one(nk > 1 ? 1 : 0, qi, 1);
  issue_scales(nch > 1 ? 1 : 0, 1);
  wait_vmem_n<INS + SCH>();
  barrier_lds();
  read_scales(0, 0);
#pragma unroll
  for (int ii = 0; ii < FM; ++ii) fa[0][ii] = read_frag(stage_ptr(0), wm * 128 + ii * 32, 0);
#pragma unroll
  for (int jj = 0; jj < FN; ++jj) fb[0][jj] = read_frag(stage_ptr(0) + BM * RB, frag_brow(jj), 0);

  // Each substep runs its 16 MFMAs in four rows (A fragment i against the four B fragments). The
  // fragments of the next substep are read one row at a time, each read placed between two
  // MFMAs: a burst of reads would hold up the in-order issue of the MFMAs behind it while the
  // LDS queue drains. In the last substep the loads of step kt + 2 go out after each row.
  constexpr int DS_PER_ROW = MX4 ? 2 : 4;  // ds_read_b128 of one A and one B fragment
  constexpr int PER_BATCH = (INS + FM - 1) / FM;
  for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
    for (int sub = 0; sub < SUB; ++sub) {
      const int cur = sub & 1;
      const bool last = sub == SUB - 1;
      if (last) {
        // step kt + 1 landed and every wave is done with stage kt % S: the next step's first
        // fragments come from stage (kt + 1) % S, and step kt + 2 goes into stage kt % S (past the
        // end: the last step again, unread, which keeps the loop free of branches)
        wait_vmem();
        wait_lgkm();
        barrier_lds();
        // the scale chunk after the next one goes into the slot of the chunk just finished
        const int nc = (kt + 1) / CH + 1;
        if ((kt + 1) % CH == 0) issue_scales(nc < nch ? nc : nch - 1, nc & 1);
      }
      const int rk = last ? (kt + 1 < nk ? kt + 1 : kt) : kt;   // step and substep read next
      const int rs = last ? 0 : sub + 1;
      const uint8_t* la = stage_ptr(rk);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if (last && i == 0) read_scales(rk, 1);
        fa[cur ^ 1][i] = read_frag(la, wm * 128 + i * 32, rs);
        fb[cur ^ 1][i] = read_frag(la + BM * RB, frag_brow(i), rs);
#pragma unroll
        for (int jj = 0; jj < FN; ++jj) {
          const int wa = scale_word(sa[0][i], sub), wb = scale_word(sb[0][jj], sub);
          if ((MX4 ? (sub & 1) : sub) == 0)   // op_sel byte 0 or 2 (resolved at compile time)
            acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                fa[cur][i], fb[cur][jj], acc[i][jj], FMT_CODE, FMT_CODE, 0, wa, 0, wb);
          else
            acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                fa[cur][i], fb[cur][jj], acc[i][jj], FMT_CODE, FMT_CODE, 2, wa, 2, wb);
        }
        if (last && i == 0) MOE_SCHED_GROUP(0x100, 2 * FN);   // the scale reads first
#pragma unroll
        for (int m = 0; m < FN; ++m) {
          MOE_SCHED_GROUP(0x008, 1);                          // one MFMA
          if (m < DS_PER_ROW) MOE_SCHED_GROUP(0x100, 1);      // one fragment read
        }
        MOE_SCHED_FENCE();
        if (last) {
          const int kn = kt + 2 < nk ? kt + 2 : nk - 1;
#pragma unroll
          for (int u = 0; u < PER_BATCH; ++u) {
            const int qi = i * PER_BATCH + u;
            if (qi < INS) issue_one(kn, qi, kt % S);
          }
          MOE_SCHED_FENCE();
        }
      }
    }
    // the next step's scale words become the current ones
#pragma unroll
    for (int i = 0; i < FM; ++i) sa[0][i] = sa[1][i];
#pragma unroll
    for (int j = 0; j < FN; ++j) sb[0][j] = sb[1][j];
  }
  wait_vmem();                             // the unread tail loads, before the stores
  wait_lgkm();

  // ---- epilogue ----
  // A lane holds column l32 of rows 8 g + 4 h + v (g, v = 0..3) of fragment (i, j), entry 4 g + v.
  // A 4 x 4 transpose inside each quad of lanes (two DPP exchanges) gives quad lane qq row
  // 8 g + 4 h + rt and 4 adjacent columns, so every store writes 4 values (16 bytes fp32, 8 bf16,
  // 4 MXFP8 codes, 2 MXFP4 bytes).
  char* C = static_cast<char*>(p.C);
  const int rbase = t.row0 + wm * 128;
  const int qq = lane & 3;
  const bool odd = qq & 1, hi = qq & 2;
  const int rt = (qq & 1) * 2 + (qq >> 1);
  auto dpp = [](float x, auto ctrl) -> float {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value,
                                                      0xF, 0xF, false));
  };
  using swap1 = std::integral_constant<int, 0xB1>;     // quad_perm [1, 0, 3, 2]: lane ^ 1
  using swap2 = std::integral_constant<int, 0x4E>;     // quad_perm [2, 3, 0, 1]: lane ^ 2
  auto quad_t = [&](const float (&a)[4]) -> f32x4 {
    const float r0 = dpp(odd ? a[0] : a[2], swap1{}), r1 = dpp(odd ? a[1] : a[3], swap1{});
    const float x0 = odd ? r0 : a[0], x1 = odd ? a[2] : r0;
    const float x2 = odd ? r1 : a[1], x3 = odd ? a[3] : r1;
    const float s0 = dpp(hi ? x0 : x2, swap2{}), s1 = dpp(hi ? x1 : x3, swap2{});
    return hi ? f32x4{s0, s1, x2, x3} : f32x4{x0, x1, s0, s1};
  };
  if constexpr (!SWIGLU || EPI == QEPI_SWIGLU_BF16) {
    constexpr int JN = SWIGLU ? FN / 2 : FN;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < JN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float a[4];
#pragma unroll
          for (int v = 0; v < 4; ++v)
            a[v] = SWIGLU ? silu_fast(acc[i][j][4 * g + v]) * acc[i][j + FN / 2][4 * g + v]
                          : acc[i][j][4 * g + v];
          const f32x4 v4 = quad_t(a);
          const int r = rbase + i * 32 + g * 8 + h * 4 + rt;
          const long long col = SWIGLU ? (long long)t.nt * (BN / 2) + wn * 64 + j * 32 + (l32 & ~3)
                                       : (long long)t.nt * BN + wn * 128 + j * 32 + (l32 & ~3);
          if (r >= t.row1 || col >= p.N) continue;         // N % 128 == 0: 4 columns all in or out
          char* dst = C + (long long)r * p.c_pitch;
          if (EPI == QEPI_STORE_F32) {
            *reinterpret_cast<f32x4*>(dst + col * 4) = v4;
          } else {
            *reinterpret_cast<uint2*>(dst + col * 2) =
                make_uint2(pack_bf16x2(v4[0], v4[1]), pack_bf16x2(v4[2], v4[3]));
          }
        }
  } else {
    // h re-quantised to 1 x 32 MX groups, one fragment row each: the group amax is reduced over
    // the lanes holding the row after the transpose (DPP inside 16-lane rows, then one exchange
    // between the two), the codes are formed by the hardware conversions (fp8: operands clamped to +-448 first, which
    // makes its round-to-nearest-even saturating; fp4: saturating itself) on the values times
    // 2^-e, as the element rule prescribes
    constexpr int HF = FN / 2;             // h fragments: 2 x 32 = 64 columns per wave
    using ror4 = std::integral_constant<int, 0x124>;    // row_ror:4 inside a 16-lane row
    using ror8 = std::integral_constant<int, 0x128>;    // row_ror:8
    const long long col0 = (long long)t.nt * (BN / 2) + wn * 64;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // after the transpose a lane holds 4 columns of its row; the row's other 28 columns are in
        // the lanes 4, 8, ... apart (same quad position), 16 of them across the two 16-lane rows
        f32x4 hv[HF];
        int ex[HF];
#pragma unroll
        for (int j = 0; j < HF; ++j) {
          float a[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) a[v] = silu_fast(acc[i][j][4 * g + v]) * acc[i][j + HF][4 * g + v];
          hv[j] = quad_t(a);
          float am = fmaxf(fmaxf(fabsf(hv[j][0]), fabsf(hv[j][1])), fmaxf(fabsf(hv[j][2]), fabsf(hv[j][3])));
          am = fmaxf(am, dpp(am, ror4{}));
          am = fmaxf(am, dpp(am, ror8{}));
          am = fmaxf(am, __shfl_xor(am, 16, 64));
          ex[j] = mx_shared_exp<MX8 ? 8 : 2>(am);
        }
        const int r = rbase + i * 32 + g * 8 + h * 4 + rt;
        const bool live = r < t.row1;
        uint8_t* crow = reinterpret_cast<uint8_t*>(C + (long long)r * p.c_pitch);
#pragma unroll
        for (int j = 0; j < HF; ++j) {
          const f32x4 v4 = hv[j];
          const float mul = ldexpf(1.0f, -ex[j]);
          const long long col = col0 + j * 32 + (l32 & ~3);
          if constexpr (MX8) {
            auto cl = [&](float x) { return fminf(fmaxf(x * mul, -448.0f), 448.0f); };
            int w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(v4[0]), cl(v4[1]), 0, false);
            w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(v4[2]), cl(v4[3]), w, true);
            if (live) *reinterpret_cast<uint32_t*>(crow + col) = static_cast<uint32_t>(w);
          } else {
            uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v4[0] * mul, v4[1] * mul, 1.0f, 0);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v4[2] * mul, v4[3] * mul, 1.0f, 1);
            if (live) *reinterpret_cast<uint16_t*>(crow + col / 2) = static_cast<uint16_t>(w);
          }
        }
        if (live && l32 < 4)
          *reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(p.C_scales) + (long long)r * (p.N / 32) + col0 / 32) =
              static_cast<uint16_t>((ex[0] + 127) | ((ex[1] + 127) << 8));
      }
  }

}
// fp8 tile kernel (gemm_fp8.hip): false if the operands do not fit its 32-bit offsets
bool launch_fp8_tile(const GemmArgs& a, int epi, hipStream_t s, hipError_t* err);

namespace {

template <int FMT, int EPI>
hipError_t run_q(const GemmArgs& a, hipStream_t s) {
  constexpr int BM = 128, BN = 256, S = 3;
  constexpr bool SWIGLU = EPI >= QEPI_SWIGLU_BF16;
  Grid g = make_grid(a, BM, SWIGLU ? BN / 2 : BN, 8, 64);
  if (g.total == 0) return hipSuccess;
  const size_t lds = (size_t)S * ((BM + BN) * 128 + q_scale_stage_bytes<FMT>());
  gemm_q_kernel<FMT, EPI><<<dim3(g.blocks), dim3(256), lds, s>>>(a, g.n_tiles, g.x_tiles, g.span,
                                                                  g.total, g.gm);
  return hipGetLastError();
}

template <int FMT, int EPI>
hipError_t run_q_stream(const GemmArgs& a, hipStream_t s) {
  constexpr int FM = 2;
  constexpr bool SWIGLU = EPI >= QEPI_SWIGLU_BF16;
  // MXFP8 splits K over the workgroup's waves (4x the workgroups: more weight loads in flight per
  // CU; measured on the 64-token Qwen3-235B slice: layer 0.205 -> 0.187 ms; 2 column blocks x 2
  // K ranges 0.200 ms, no split 0.200 ms). fp8 does not: its h blocks of 128 columns need the four
  // column blocks in one workgroup, and its down projection streams faster whole (256-token
  // DeepSeek-V3 slice: 0.336 ms with the 4-way split, 0.323 with 2 x 2, 0.318-0.322 without).
  // Nor does MXFP4, whose K-split form needs more registers than two waves per SIMD allow
  // (0.193 -> 0.251 ms).
  constexpr int KS = FMT == MOE_MXFP8 ? 4 : 1;
  Grid g = make_grid(a, 16 * FM, (SWIGLU ? 128 : 256) / KS, q_stream_group<FMT>(), q_stream_group<FMT>());
  if (g.total == 0) return hipSuccess;
  gemm_q_stream_kernel<FMT, EPI, FM, KS><<<dim3(g.blocks), dim3(256), 0, s>>>(a, g.n_tiles, g.x_tiles,
                                                                            g.total);
  return hipGetLastError();
}

template <int FMT, int EPI>
hipError_t run_q_wide(const GemmArgs& a, hipStream_t s) {
  constexpr bool SWIGLU = EPI >= QEPI_SWIGLU_BF16;
  Grid g = make_grid(a, kQWideBM, SWIGLU ? kQWideBN / 2 : kQWideBN, 8, 64);
  if (g.total == 0) return hipSuccess;
  gemm_q_wide_kernel<FMT, EPI><<<dim3(g.blocks), dim3(256), kQWideLds, s>>>(
      a, g.n_tiles, g.x_tiles, g.span, g.total, g.gm);
  return hipGetLastError();
}

// decode-sized groups (few rows per group on average) stream the weights; prefill-sized groups
// (a full 256-row tile or more per group) of the MX formats with K % 512 == 0 (whole scale
// chunks) use the wide tiles; others the 128-row tiles
template <int FMT, int EPI>
hipError_t run_q_choice(const GemmArgs& a, hipStream_t s) {
  const long long rows = (long long)(a.expected_rows > 0 ? a.expected_rows : a.max_rows) + a.x_rows;
  const int groups = a.G + (a.x_rows > 0 ? 1 : 0);
  const long long per_group = groups ? rows / groups : rows;
  if (per_group <= 32 && a.N % 128 == 0) return run_q_stream<FMT, EPI>(a, s);
  if constexpr (FMT == MOE_MXFP4 || FMT == MOE_MXFP8)
    if (per_group >= kQWideBM && a.K % 512 == 0) return run_q_wide<FMT, EPI>(a, s);
  if constexpr (FMT == MOE_FP8_E4M3) {
    hipError_t e;
    if (launch_fp8_tile(a, EPI, s, &e)) return e;
  }
  return run_q<FMT, EPI>(a, s);
}

template <int FMT>
hipError_t run_q_fmt(const GemmArgs& a, hipStream_t s) {
  if (a.epilogue == MOE_EPI_SWIGLU) {
    if (a.out_dtype == FMT) return run_q_choice<FMT, QEPI_SWIGLU_Q>(a, s);
    if (a.out_dtype == MOE_BF16) return run_q_choice<FMT, QEPI_SWIGLU_BF16>(a, s);
    return hipErrorInvalidValue;
  }
  if (a.out_dtype == MOE_F32) return run_q_choice<FMT, QEPI_STORE_F32>(a, s);
  if (a.out_dtype == MOE_BF16) return run_q_choice<FMT, QEPI_STORE_BF16>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm_q(const GemmArgs& a, hipStream_t s) {
  if (a.dtype == MOE_FP8_E4M3) return run_q_fmt<MOE_FP8_E4M3>(a, s);
  if (a.dtype == MOE_MXFP4) return run_q_fmt<MOE_MXFP4>(a, s);
  if (a.dtype == MOE_MXFP8) return run_q_fmt<MOE_MXFP8>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
