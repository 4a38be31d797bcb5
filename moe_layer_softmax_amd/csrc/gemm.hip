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
#include <atomic>
#include <cstdlib>
#include <mutex>
#include <type_traits>

#include "gemm_common.hpp"
#include "quant_dev.hpp"

namespace moe {

// m-tiles per tile-order group (and per XCD span) of the weight-streaming kernel
constexpr int kStreamGroupM = 8;

// STORE epilogue of 32 x 32 fragments with one store of 4 columns per lane and 4 rows (16 bytes
// fp32, 8 bytes bf16 or fp16): in a quad of lanes (4 consecutive columns) each lane holds 4
// consecutive rows of its column for entries 4g .. 4g + 3; two cross-lane exchanges (lane ^ 1,
// then lane ^ 2, as DPP quad permutations) transpose the 4 x 4 block so lane q holds row
// (q & 1) * 2 + (q >> 1) of the block, 4 columns. Stores are non-temporal (C is read by the next
// kernel from HBM anyway).
// F16S: MOE_F16_SCALED rows (TN = 64: one scale block per wave and row). The lanes holding one row
// after the transposition differ in lane bits 2-4 (8 quads x 4 columns x FN fragments), so the
// block maximum is a reduction over those lanes; lanes 0-3 and 32-35 store the scales.
// Returns true when every row and column of the wave's block is inside the tile: the wave then
// issued exactly FM * FN * 4 store instructions, plus FM * 4 scale stores for F16S (callers count
// them in their vmcnt waits).
template <int FM, int FN, int TM, int TN, int BN, bool OUT_F32, bool F16S, class AccAt>
__device__ __forceinline__ bool store_tile_x4(const GemmArgs& p, const Tile& t, int wm, int wn,
                                                 AccAt acc_at) {
  static_assert(!F16S || (!OUT_F32 && TN == 64), "scaled fp16 rows: 64-column waves");
  const int lane = lane_id();
  const int q = lane & 3;
  const bool odd = q & 1, hi = q & 2;
  auto dpp = [](float x, auto ctrl) -> float {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value, 0xF, 0xF, false));
  };
  using swap1 = std::integral_constant<int, 0xB1>;     // quad_perm [1, 0, 3, 2]: lane ^ 1
  using swap2 = std::integral_constant<int, 0x4E>;     // quad_perm [2, 3, 0, 1]: lane ^ 2
  // the 4 columns of lane q's row of the 4 x 4 block of entries 4g .. 4g + 3 of fragment (i, j)
  auto transpose = [&](int i, int j, int g) -> f32x4 {
    const float a0 = acc_at(i, j, 4 * g), a1 = acc_at(i, j, 4 * g + 1);
    const float a2 = acc_at(i, j, 4 * g + 2), a3 = acc_at(i, j, 4 * g + 3);
    // step 1: even lanes keep rows 0, 1 and take the partner column's rows 0, 1; odd lanes keep
    // rows 2, 3 and take the partner's rows 2, 3
    const float r0 = dpp(odd ? a0 : a2, swap1{}), r1 = dpp(odd ? a1 : a3, swap1{});
    const float x0 = odd ? r0 : a0, x1 = odd ? a2 : r0;
    const float x2 = odd ? r1 : a1, x3 = odd ? a3 : r1;
    // step 2: lanes 0, 1 keep their first row (x0, x1) and take the other column pair's; lanes
    // 2, 3 keep their second row (x2, x3)
    const float s0 = dpp(hi ? x0 : x2, swap2{}), s1 = dpp(hi ? x1 : x3, swap2{});
    return hi ? f32x4{s0, s1, x2, x3} : f32x4{x0, x1, s0, s1};
  };
  const int row_in = (lane / 32) * 4 + (q & 1) * 2 + (q >> 1);
  const long long c_blk = (long long)t.nt * BN + wn * TN;
  const long long col0 = c_blk + ((lane % 32) & ~3);
  const int rbase = t.row0 + wm * TM;
  const bool full = rbase + TM <= t.row1 && c_blk + TN <= p.N;
  char* C = static_cast<char*>(p.C);
  if constexpr (F16S) {
    const bool in_n = c_blk < p.N;                     // N % 64 == 0: the block is all in or out
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v[FN];
        float m = 0.0f;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          v[j] = transpose(i, j, g);
          m = fmaxf(m, fmaxf(fmaxf(fabsf(v[j][0]), fabsf(v[j][1])), fmaxf(fabsf(v[j][2]), fabsf(v[j][3]))));
        }
        const int e = f16s_exp(lanes_max<28>(m));
        const int r = rbase + i * 32 + g * 8 + row_in;
        if (full || (r < t.row1 && in_n)) {
          char* crow = C + (long long)r * p.c_pitch;
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const u32x2 w = u32x2{pack_f16x2_scaled(v[j][0], v[j][1], e), pack_f16x2_scaled(v[j][2], v[j][3], e)};
            __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(crow + (col0 + j * 32) * 2));
          }
          // the scale is an ordinary store: the row's other scales (the same 128-byte line) come
          // from the tiles of the other n-tiles, most of which run at the same time on this XCD,
          // and merge with it in L2 (as non-temporal stores each went to HBM on its own, ~64 bytes
          // written per 4-byte scale)
          if ((lane & 28) == 0)
            *reinterpret_cast<float*>(crow + (long long)p.N * 2 + c_blk / 16) = f16s_scale(e);
        }
      }
    return full;
  }
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 v = transpose(i, j, g);
        const int r = rbase + i * 32 + g * 8 + row_in;
        const long long col = col0 + j * 32;
        if (full || (r < t.row1 && col < p.N)) {
          if constexpr (OUT_F32) {
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(C + (long long)r * p.c_pitch + col * 4));
          } else {
            const u32x2 w = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(C + (long long)r * p.c_pitch + col * 2));
          }
        }
      }
  return full;
}

// Per-wave direct-to-LDS load plan of one BM x BN tile. Slot j of A moves tile rows
// (j * NW + wave) * RPI ... + RPI - 1 of a K-slice (RPI rows per wave-wide instruction, lanes on
// 16-byte chunks, swizzled), likewise slot j of B (SWIGLU: the B rows of each wave column are TN/2
// gate rows then TN/2 up rows; a slot never straddles the two). Each slot has a wave-uniform base
// pointer and a fixed per-lane byte offset, so a K-step only moves the base (scalar arithmetic).
// If some lane's offset needs more than 32 bits the wave uses the 64-bit per-lane address form.
// When BM is not a multiple of RPI * NW the last A slot covers the remaining rows only: waves
// whose slot would start at or past BM skip it (a wave-uniform branch), so they issue one
// instruction less per K-step (a_slots).
template <class Geo, int BM, int BN, int TN, int NW, bool SWIGLU>
struct LoadPlan {
  static constexpr int RPI = Geo::kRowsPerIns;
  static constexpr int A_INS = (BM + RPI * NW - 1) / (RPI * NW), B_INS = BN / (RPI * NW);
  static_assert(BM % RPI == 0 && BN % (RPI * NW) == 0, "whole instructions");
  static constexpr bool A_FULL = BM % (RPI * NW) == 0;
  // slot j of A is used by wave w (always when every slot is full: no check is compiled then)
  __host__ __device__ static constexpr bool a_active(int j, int w) {
    return A_FULL || (j * NW + w) * RPI < BM;
  }
  // A instructions wave w issues per K-step
  __host__ __device__ static constexpr int a_slots(int w) {
    int c = 0;
    for (int j = 0; j < A_INS; ++j) c += a_active(j, w) ? 1 : 0;
    return c;
  }
  static constexpr int BK = Geo::kRowBytes / 2;
  const char* a_base;
  const char* b_base[B_INS];
  unsigned long long a_off[A_INS], b_off[B_INS];
  bool wide;

  __device__ __forceinline__ void init(const GemmArgs& p, const Tile& t, int wave, int lane) {
    const int lrow = lane / Geo::kChunks;
    a_base = static_cast<const char*>(p.A);
#pragma unroll
    for (int j = 0; j < A_INS; ++j) {
      const int r = (j * NW + wave) * RPI + lrow;
      const int lch = (lane % Geo::kChunks) ^ Geo::swz(r);
      a_off[j] = a_active(j, wave) ? (unsigned long long)a_src_row(p, t, t.row0 + r) * p.a_pitch + lch * 16 : 0;
    }
#pragma unroll
    for (int j = 0; j < B_INS; ++j) {
      const int rb0 = (j * NW + wave) * RPI;           // wave-uniform
      const int rb = rb0 + lrow;
      const int lch = (lane % Geo::kChunks) ^ Geo::swz(rb);
      long long n;
      if (SWIGLU) {
        const int half = TN / 2;
        b_base[j] = (rb0 % TN) >= half ? t.B2 : t.B;
        n = (long long)t.nt * (BN / 2) + (rb / TN) * half + (rb % TN) % half;
      } else {
        b_base[j] = t.B;
        n = (long long)t.nt * BN + rb;
      }
      if (n >= p.N) n = p.N - 1;           // columns past N: read a valid row, never stored
      b_off[j] = (unsigned long long)n * p.K * 2 + lch * 16;
    }
    bool w = false;
#pragma unroll
    for (int j = 0; j < A_INS; ++j) w |= (a_off[j] >> 32) != 0;
#pragma unroll
    for (int j = 0; j < B_INS; ++j) w |= (b_off[j] >> 32) != 0;
    wide = __ballot(w) != 0;
  }

  // K-slice starting at byte kb of every row into the stage at `stage` (ring pointer) whose LDS
  // byte address is st
  template <bool WIDE>
  __device__ __forceinline__ void issue(long long kb, uint16_t* stage, unsigned st, int wave) const {
#pragma unroll
    for (int j = 0; j < A_INS; ++j) {
      const int row = (j * NW + wave) * RPI;
      if (!a_active(j, wave)) continue;                // wave-uniform
      if constexpr (WIDE) dma_16b_asm(a_base + a_off[j] + kb, stage + row * BK);
      else dma_16b_sbase(a_base + kb, static_cast<unsigned>(a_off[j]), st + row * BK * 2);
    }
#pragma unroll
    for (int j = 0; j < B_INS; ++j) {
      const int row = BM + (j * NW + wave) * RPI;
      if constexpr (WIDE) dma_16b_asm(b_base[j] + b_off[j] + kb, stage + row * BK);
      else dma_16b_sbase(b_base[j] + kb, static_cast<unsigned>(b_off[j]), st + row * BK * 2);
    }
  }
};

template <int BM, int BN, int WM, int WN, int MI, int BK, int S, bool SWIGLU, bool OUT_F32,
          bool PERSIST, bool F16S = false>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_bf16_pipe_kernel(GemmArgs p, int n_tiles, int x_tiles, int span, int total, int gm, int nphys) {
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

  // PERSIST: the grid holds one workgroup per CU slot and workgroup b takes the tiles of workgroup
  // positions b, b + gridDim.x, ... (gridDim.x is a multiple of the XCD count, so they all map to
  // b's XCD). After a tile's K loop the next tile is resolved, the finished tile's stores are issued
  // and the next tile's first S - 1 K-steps are loaded, so the store drain, the load latency and
  // the next tile's set-up overlap instead of running back to back in separate workgroups.
  int phys = blockIdx.x;
  auto next_tile = [&](Tile& tt) -> bool {
    for (; phys < nphys; phys += gridDim.x) {
      const int logical = xcd_remap(phys, span);
      if (logical < total && resolve_tile(p, BM, n_tiles, x_tiles, logical, tt, gm)) return true;
      if (!PERSIST) break;
    }
    return false;
  };
  Tile t;
  if (!next_tile(t)) return;

  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int nk = p.K / BK;

  LoadPlan<Geo, BM, BN, TN, NW, SWIGLU> lp;
  lp.init(p, t, wave, lane);
  const unsigned lds0 = static_cast<unsigned>(reinterpret_cast<uintptr_t>(lds));
  // K-step kt's slices into stage kt % S (steps past the end issue nothing)
  auto issue = [&](int kt, auto wide_tag) {
    if (kt >= nk) return;
    lp.template issue<decltype(wide_tag)::value>((long long)kt * Geo::kRowBytes, lds + (kt % S) * STAGE,
                                                 lds0 + (kt % S) * (STAGE * 2), wave);
  };

  bf16x8 fa[2][FM], fb[2][FN];
  unsigned lane_off[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) lane_off[s] = frag_lane_off<Geo, MI, MK>(s, lane);
  const char* const lds_bytes = reinterpret_cast<const char*>(lds);
  auto lfrag = [&](int stage, int s, int slot) {
    const char* lb = lds_bytes + stage * (STAGE * 2) + lane_off[s];
#pragma unroll
    for (int i = 0; i < FM; ++i)
      fa[slot][i] = *reinterpret_cast<const bf16x8*>(lb + (wm * TM + i * MI) * BK * 2);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      fb[slot][j] = *reinterpret_cast<const bf16x8*>(lb + (BM + wn * TN + j * MI) * BK * 2);
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

  auto prime = [&](auto wide_tag) {
  #pragma unroll
    for (int q = 0; q < S - 1; ++q) issue(q, wide_tag);
  };
  auto k_loop = [&](auto wide_tag, bool primed) {
    // prologue: steps 0 .. S-2 in flight (issued here unless already primed), wait for step 0 (and,
    // as vmcnt retires in issue order, for anything issued before those loads)
    if (!primed) prime(wide_tag);
    if (nk >= S - 1) wait_vmem_n<(S - 2) * INS>();
    else wait_vmem();
    barrier_lds();
    lfrag(0, 0, 0);
    wait_lgkm();   // nothing but these reads pending on entry, so the loop can count them in order

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
          issue(kt + S - 1, wide_tag);
          // unconditional (past the last step it reads a stale stage, never used): a branch here
          // would make the compiler wait for these reads before the MFMAs below
          lfrag((kt + 1) % S, 0, slot ^ 1);
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
        // the next substep's fragment reads go out first, so they have this substep's MFMAs to land
        MOE_SCHED_GROUP(0x100, FM + FN);
        MOE_SCHED_GROUP(0x008, FM * FN);
      }
    }
  };
  bool primed = false;
  for (;;) {
    if (lp.wide) k_loop(std::true_type{}, primed);
    else k_loop(std::false_type{}, primed);
    // next tile and its load plan first: their loads (group offsets, gathered row ids) find nothing
    // else in flight here, whereas after the stores below they would wait for those to retire
    Tile tn;
    bool more = false;
    if constexpr (PERSIST) {
      phys += gridDim.x;
      more = next_tile(tn);
      if (more) lp.init(p, tn, wave, lane);
    }
    // ---- epilogue ---- (fp32 C of 256-row tiles, i.e. a large C, streamed past L2)
    store_tile<MI, FM, FN, TM, TN, BN, SWIGLU, OUT_F32, (BM >= 256), F16S>(p, t, wm, wn, [&](int i, int j, int v) -> float {
      if constexpr (MI == 32) return acc32[i][j][v];
      else return acc16[i][j][v];
    });
    if (!more) break;
    t = tn;
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
    barrier_lds();                                     // every wave is past its last LDS read
    if (lp.wide) prime(std::true_type{});
    else prime(std::false_type{});
    primed = true;
  }
}

// ------------------------------------------------------------------------------------------------
// Ping-pong variant of the 256 x 256 tile (8 waves, each 128 x 64, K-steps of 32).
//
// The waves form two groups of four, one wave of each group per SIMD (waves 0-3: tile rows 0-127,
// waves 4-7: rows 128-255). Between two workgroup barriers one group is in its memory phase
// (reads all of one K-step's fragments from LDS into registers and issues its share of the DMA for
// a later step) while the other is in its compute phase (the 16 MFMAs of the K-step it read in its
// previous phase). Each barrier swaps the roles, so a SIMD's MFMA unit is fed by one wave while
// its sibling's LDS traffic and waits are hidden, instead of both waves reading, computing and
// stalling in lockstep.
//
// Barrier schedule (b0 after the prologue; group 1 passes one extra barrier b1 first):
//   group 0: M(0) b1 C(0) b2 M(1) b3 C(1) b4 ... M(kt) = (b2kt, b2kt+1), C(kt) = (b2kt+1, b2kt+2)
//   group 1: b1 M(0) b2 C(0) b3 M(1) ...           M(kt) = (b2kt+1, b2kt+2), C(kt) = (b2kt+2, ...)
// so both groups pass 2 nk + 1 barriers (group 1 skips the one after its last compute phase).
//   * stage of step j is read in M(j) by group 0 before b2j+1 and by group 1 before b2j+2 (each
//     wave drains its LDS reads before the barrier that ends its memory phase);
//   * the DMA for step j + S - 1 is issued in M(j), after b2j (group 0) or b2j+1 (group 1) --
//     after the previous user of that stage, step j - 1, was drained at b2j;
//   * step j + 1 must have landed, from every wave, before b2j+2: group 0 waits for its own share at
//     the end of C(j), group 1 at the end of M(j); the barrier then publishes it.
// ------------------------------------------------------------------------------------------------

template <bool SWIGLU, bool OUT_F32, int S, bool PERSIST, bool F16S = false, int BM = 256>
__global__ void __launch_bounds__(512)
gemm_bf16_pp_kernel(GemmArgs p, int n_tiles, int x_tiles, int span, int total, int gm, int nphys) {
  constexpr int BN = 256, WN = 4, MI = 32, BK = 32;
  constexpr int NW = 8, TM = BM / 2, TN = 64, FM = TM / MI, FN = TN / MI, MK = 16, KS = BK / MK;
  static_assert(BM == 256 || BM == 192, "tile rows");
  using Geo = SliceGeo<BK>;
  using Plan = LoadPlan<Geo, BM, BN, TN, NW, SWIGLU>;
  constexpr int B_INS = Plan::B_INS;
  // DMA instructions per wave per K-step, per wave group (192-row tiles: the second group's waves
  // have no row of the last A slot)
  constexpr int INS0 = Plan::a_slots(0) + B_INS, INS1 = Plan::a_slots(NW / 2) + B_INS;
  static_assert(Plan::a_slots(NW / 2 - 1) + B_INS == INS0 && Plan::a_slots(NW - 1) + B_INS == INS1,
                "one count per wave group");
  constexpr int INS = INS0 > INS1 ? INS0 : INS1;
  constexpr int STAGE = (BM + BN) * BK;                // uint16 per LDS stage
  static_assert(S >= 3 && (S - 2) * INS < 64, "pipeline depth");
  static_assert(!SWIGLU || (FN % 2 == 0), "SWIGLU needs gate and up fragments in every wave");

  extern __shared__ __attribute__((aligned(1024))) uint16_t lds[];

  // PERSIST: one workgroup per CU slot takes the tiles of workgroup positions b, b + gridDim.x, ...
  // (as in gemm_bf16_pipe_kernel): the next tile's first S - 1 K-steps are loaded while the
  // finished tile's stores drain.
  int phys = blockIdx.x;
  auto next_tile = [&](Tile& tt) -> bool {
    for (; phys < nphys; phys += gridDim.x) {
      const int logical = xcd_remap(phys, span);
      if (logical < total && resolve_tile(p, BM, n_tiles, x_tiles, logical, tt, gm)) return true;
      if (!PERSIST) break;
    }
    return false;
  };
  Tile t;
  if (!next_tile(t)) return;

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int grp = wave >> 2;                           // wave-uniform (scalar branches below)
  const int wm = grp, wn = wave & (WN - 1);
  const int nk = p.K / BK;

  Plan lp;
  lp.init(p, t, wave, lane);
  const unsigned lds0 = static_cast<unsigned>(reinterpret_cast<uintptr_t>(lds));
  auto issue = [&](int kt, auto wide_tag) {
    if (kt >= nk) return;
    lp.template issue<decltype(wide_tag)::value>((long long)kt * Geo::kRowBytes, lds + (kt % S) * STAGE,
                                                 lds0 + (kt % S) * (STAGE * 2), wave);
  };
  // Store instructions of the epilogue of a wave whose block lies inside the tile: 16-byte stores
  // for STORE (4 per 32 x 32 fragment, fp32 or bf16), otherwise 2-column stores (8 per fragment
  // pair row group, see store_tile).
  constexpr bool X4 = !SWIGLU;
  constexpr int NST = X4 ? FM * FN * 4 + (F16S ? FM * 4 : 0) : FM * (SWIGLU ? FN / 2 : FN) * 8;
  // stores left in flight must fit the vmcnt counter (6 bits) with the loads
  constexpr bool OVERLAP = PERSIST && (S - 2) * INS + NST < 64;
  constexpr int NPEND = OVERLAP ? NST : 0;
  // this wave's share of step kt + 1 has landed (steps up to kt + S - 1 may have been issued).
  // pend: the wave issued NST stores after the first S - 1 steps of this tile (the previous
  // tile's epilogue, see tile_loop); vmcnt retires in issue order, so while those stores are
  // younger than step kt + 1 (kt + 1 <= S - 2) they are left in flight by counting them too.
  // vmcnt((S - 2) * (this wave group's instructions per step) + extra)
  auto wait_steps = [&](auto extra) {
    constexpr int X = decltype(extra)::value;
    if constexpr (INS0 == INS1) {
      wait_vmem_n<(S - 2) * INS0 + X>();
    } else {
      if (grp == 0) wait_vmem_n<(S - 2) * INS0 + X>();
      else wait_vmem_n<(S - 2) * INS1 + X>();
    }
  };
  using NoPend = std::integral_constant<int, 0>;
  using Pend = std::integral_constant<int, NPEND>;
  auto wait_next = [&](int kt, bool pend) {
    if (kt + S - 1 < nk) {
      if (OVERLAP && pend && kt <= S - 3) wait_steps(Pend{});
      else wait_steps(NoPend{});
    } else {
      wait_vmem();
    }
  };

  // Fragment reads: every fragment row is (32-row block) + lane % 32, and the swizzle only depends
  // on row % 32, so a lane's byte offset is a per-substep constant plus an immediate per fragment.
  bf16x8 fa[KS][FM], fb[KS][FN];
  unsigned lane_off[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) lane_off[s] = frag_lane_off<Geo, MI, MK>(s, lane);
  const char* const lds_bytes = reinterpret_cast<const char*>(lds);
  auto read_step = [&](int stage) {
    const char* sb = lds_bytes + stage * (STAGE * 2);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const char* lb = sb + lane_off[s];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        fa[s][i] = *reinterpret_cast<const bf16x8*>(lb + (wm * TM + i * MI) * BK * 2);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        fb[s][j] = *reinterpret_cast<const bf16x8*>(lb + (BM + wn * TN + j * MI) * BK * 2);
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

  auto prime = [&](auto wide_tag) {
#pragma unroll
    for (int q = 0; q < S - 1; ++q) issue(q, wide_tag);
  };
  // The K loop, instantiated for the 32-bit-offset and the 64-bit-address load forms.
  // On return every wave has finished its LDS reads of the tile: group 0 leaves through its last
  // barrier, which group 1 passes right after its last memory phase.
  auto k_loop = [&](auto wide_tag, bool primed, bool pend) {
    // prologue: steps 0 .. S-2 in flight (issued here unless already primed); step 0 published by
    // b0. Stores issued after the primed steps are left in flight (pend), others are waited for.
    if (!primed) prime(wide_tag);
    if (nk >= S - 1) {
      if (OVERLAP && pend) wait_steps(Pend{});
      else wait_steps(NoPend{});
    } else {
      wait_vmem();
    }
    phase_barrier();                                   // b0
    if (grp == 1) phase_barrier();                     // b1 (group 1 starts one phase later)

    for (int kt = 0; kt < nk; ++kt) {
      // memory phase
      read_step(kt % S);
      issue(kt + S - 1, wide_tag);
      if (grp == 1) wait_next(kt, pend);
      wait_lgkm();
      phase_barrier();
      // compute phase
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s][i], fb[s][j], acc[i][j], 0, 0, 0);
      if (grp == 0) wait_next(kt, pend);
      if (grp == 0 || kt + 1 < nk) phase_barrier();
    }
  };
  // The workgroup's tiles, in one address form. Returns false (with the next tile in t, not yet
  // loaded) when that tile needs the 64-bit form and this loop runs the 32-bit one. The two forms
  // run as consecutive loops rather than one loop choosing per tile: a loop body holding both K
  // loops needs more registers than a wave has at this occupancy.
  //
  // Between tiles the next tile's first S - 1 K-steps are issued before the finished tile's
  // stores, and a wave whose stores all went out (its block lies inside the tile) does not wait
  // for them before the next tile's MFMAs: the stores drain behind the first K-steps.
  auto tile_loop = [&](auto wide_tag, bool primed) -> bool {
    bool pend = false;
    for (;;) {
      k_loop(wide_tag, primed, pend);
      // next tile and its load plan (their loads find nothing else in flight), then its first
      // K-steps if it uses this loop's address form
      Tile tn;
      bool more = false, next_primed = false;
      if constexpr (PERSIST) {
        phys += gridDim.x;
        more = next_tile(tn);
        if (more) {
          lp.init(p, tn, wave, lane);
          if (decltype(wide_tag)::value || !lp.wide) {   // lp.wide is wave-uniform (a ballot)
            prime(wide_tag);
            next_primed = true;
          }
        }
      }
      bool full;
      if constexpr (X4) {
        full = store_tile_x4<FM, FN, TM, TN, BN, OUT_F32, F16S>(p, t, wm, wn,
                                                          [&](int i, int j, int v) { return acc[i][j][v]; });
      } else {
        full = t.row0 + wm * TM + TM <= t.row1 &&
               (long long)t.nt * (SWIGLU ? BN / 2 : BN) + wn * (SWIGLU ? TN / 2 : TN) +
                       (SWIGLU ? TN / 2 : TN) <= p.N;
        store_tile<MI, FM, FN, TM, TN, BN, SWIGLU, OUT_F32, OUT_F32>(
            p, t, wm, wn, [&](int i, int j, int v) { return acc[i][j][v]; });
      }
      if (!more) return true;
      t = tn;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};
      if (!next_primed) return false;                  // the next tile needs the 64-bit form
      primed = true;
      pend = OVERLAP && full;
    }
  };
  if (!lp.wide && tile_loop(std::false_type{}, false)) return;
  tile_loop(std::true_type{}, false);                  // the 64-bit form serves every later tile
}

// ------------------------------------------------------------------------------------------------
// Weight-streaming kernel for decode-sized groups ("Hosting Qwen on Blackwell", section
// "Decoders": decode is limited by reading the weights from HBM).
//
// One wave per workgroup and per tile of 16 * FM C rows x 64 weight rows (SWIGLU: 32 gate rows and
// the 32 matching up rows). The weights are the MFMA's first operand, so the 16 x 16 accumulator
// fragment gives each lane four consecutive output columns of one C row. Both operands go from
// global memory straight into registers -- every weight byte is used by this wave only, so no LDS
// staging is needed. K advances in pairs of 32-wide steps (128 bytes of every row):
//   * weights: non-temporal loads (each weight byte is read once per layer; on MI355X a plain-load
//     stream of a row-major weight matrix reaches ~5.9 TB/s, the same stream with non-temporal
//     loads ~6.1 TB/s); one load instruction covers 8 rows x 128 contiguous bytes (measured: a
//     weight stream read as 16 rows x 64 bytes per instruction, the MFMA operand's own shape,
//     reaches ~4.8 TB/s; 8 rows x 128 bytes reaches ~5.8 TB/s). Cross-lane permutes (ds_bpermute,
//     no LDS storage) then move each 16-byte piece to the lane that holds it in the MFMA operand;
//   * activations (a few rows, resident in L2): loaded in the operand's layout directly.
// Pairs are double-buffered: the loads of pair c + 1 are issued before the MFMAs of pair c (the
// loop is unrolled by two so the register sets alternate statically; scheduling barriers keep the
// loads where they are written -- left alone, the scheduler sinks each load next to its use).
// Loads past the end re-read the last pair and rows past the group's end re-read its last row, so
// every load is unconditional and in bounds. Rows of C beyond 16 * FM per group take further tiles.
//
// KS > 1: the workgroup's KS waves split the tile's K pairs into KS contiguous ranges (more loads in
// flight per CU for the same registers per wave); their fp32 partial sums meet in LDS and wave 0
// adds them in wave order (deterministic) before the epilogue.
// ------------------------------------------------------------------------------------------------
// The body of gemm_bf16_stream_kernel for a tile whose rows fill L of its 16-row fragments: only
// those fragments' activation rows are loaded and multiplied (a 64-row tile of a group with a few
// rows would otherwise issue as many activation loads as weight loads, all but one re-reading a
// clamped row). part: the K-split's LDS partial sums, [KS - 1][4][L][64].
template <int L, int KS, bool SWIGLU, bool OUT_F32, bool F16S>
__device__ __forceinline__ void stream_tile(const GemmArgs& p, const Tile& t, f32x4* part) {
  const int lane = lane_id();
  const int lr = lane & 15, kq = lane >> 4;            // operand row; 16-byte quarter of a step
  const uint32_t kbytes = static_cast<uint32_t>(p.K) * 2u;
  // weight loads: fragment j, row half h: lane -> row h * 8 + lane / 8, 16-byte chunk lane % 8.
  // Addresses are a wave-uniform matrix base plus a 32-bit lane offset inside that matrix (the
  // launcher keeps N * K * 2 below 2^32), so each load takes a scalar base and a vector offset.
  const char* const wb0 = t.B;
  const char* const wb1 = SWIGLU ? t.B2 : t.B;
  uint32_t wo[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = h * 8 + (lane >> 3);
      int n = SWIGLU ? t.nt * 32 + (j & 1) * 16 + r : t.nt * 64 + j * 16 + r;
      if (n >= p.N) n = p.N - 1;                        // columns past N: valid row, never stored
      wo[j][h] = static_cast<uint32_t>(n) * kbytes + (lane & 7) * 16;
    }
  const char* A = static_cast<const char*>(p.A);
  const char* ap[L];
#pragma unroll
  for (int i = 0; i < L; ++i) ap[i] = A + a_src_row(p, t, t.row0 + i * 16 + lr) * p.a_pitch + kq * 16;
  // operand lane (row lr, quarter kq) of step s holds chunk s * 4 + kq of row lr: loaded by row
  // half lr / 8, lane (lr % 8) * 8 + s * 4 + kq (byte index for ds_bpermute)
  const int src0 = ((lr & 7) * 8 + kq) * 4, src1 = src0 + 16;
  const bool upper = lr >= 8;

  // this wave's pairs of K-steps: [c0, c0 + np)
  const int wave = KS > 1 ? (int)(threadIdx.x >> 6) : 0;
  const int np_all = p.K / 64;
  const int c0 = np_all * wave / KS, np = np_all * (wave + 1) / KS - c0;
  i32x4 wraw[2][4][2];
  bf16x8 av[2][L][2];
  auto load = [&](int c, int set) {
    const uint32_t woff = static_cast<uint32_t>(c0 + min(c, np - 1)) * 128u;
    const long long off = woff;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        wraw[set][j][h] = __builtin_nontemporal_load(
            reinterpret_cast<const i32x4*>((SWIGLU && j >= 2 ? wb1 : wb0) + (wo[j][h] + woff)));
#pragma unroll
    for (int i = 0; i < L; ++i)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) av[set][i][s2] = *reinterpret_cast<const bf16x8*>(ap[i] + off + s2 * 64);
  };
  f32x4 acc[4][L];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < L; ++i) acc[j][i] = f32x4{};
  auto compute = [&](int set) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int src = s2 ? src1 : src0;
      bf16x8 wf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        i32x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int lo = __builtin_amdgcn_ds_bpermute(src, wraw[set][j][0][q]);
          const int hi = __builtin_amdgcn_ds_bpermute(src, wraw[set][j][1][q]);
          w[q] = upper ? hi : lo;
        }
        wf[j] = __builtin_bit_cast(bf16x8, w);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < L; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j], av[set][i][s2], acc[j][i], 0, 0, 0);
    }
  };
  if (np > 0) {                                        // wave-uniform; np = 0 only if K < 64 * KS
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
    if (c < np) compute(0);                            // odd number of pairs: the last is in set 0
  }
  if constexpr (KS > 1) {
    // part: [KS - 1][4][L][64] partial sums of waves 1 .. KS - 1
    if (wave > 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < L; ++i) part[(((wave - 1) * 4 + j) * L + i) * 64 + lane] = acc[j][i];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < KS - 1; ++w)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < L; ++i) acc[j][i] += part[((w * 4 + j) * L + i) * 64 + lane];
  }

  // acc[j][i][v]: weight row j * 16 + kq * 4 + v of the tile, C row row0 + i * 16 + lr
  char* C = static_cast<char*>(p.C);
  if constexpr (F16S) {
    // MOE_F16_SCALED rows: the tile's 64 columns are one scale block (N % 64 == 0, so every tile
    // lies inside N); the lanes of one row (lr) differ in lane bits 4 and 5
    static_assert(!SWIGLU && !OUT_F32, "scaled fp16 rows: STORE");
    const long long c_blk = (long long)t.nt * 64;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      float v4[4][4], m = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          v4[j][v] = acc[j][i][v] + (p.bias ? p.bias[c_blk + j * 16 + kq * 4 + v] : 0.0f);
          m = fmaxf(m, fabsf(v4[j][v]));
        }
      const int e = f16s_exp(lanes_max<48>(m));
      const int r = t.row0 + i * 16 + lr;
      if (r >= t.row1) continue;
      char* crow = C + (long long)r * p.c_pitch;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<uint2*>(crow + (c_blk + j * 16 + kq * 4) * 2) =
            make_uint2(pack_f16x2_scaled(v4[j][0], v4[j][1], e), pack_f16x2_scaled(v4[j][2], v4[j][3], e));
      if (kq == 0) *reinterpret_cast<float*>(crow + (long long)p.N * 2 + c_blk / 16) = f16s_scale(e);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int r = t.row0 + i * 16 + lr;
    if (r >= t.row1) continue;
    char* crow = C + (long long)r * p.c_pitch;
#pragma unroll
    for (int j = 0; j < (SWIGLU ? 2 : 4); ++j) {
      float v4[4];
      long long col;
      if (SWIGLU) {
        col = (long long)t.nt * 32 + j * 16 + kq * 4;
#pragma unroll
        for (int v = 0; v < 4; ++v) v4[v] = silu_fast(acc[j][i][v]) * acc[j + 2][i][v];
      } else {
        col = (long long)t.nt * 64 + j * 16 + kq * 4;
#pragma unroll
        for (int v = 0; v < 4; ++v) v4[v] = acc[j][i][v] + (p.bias ? p.bias[min(col + v, (long long)p.N - 1)] : 0.0f);
      }
      if (col >= p.N) continue;                       // N is a multiple of 16: all four or none
      if (OUT_F32) {
        *reinterpret_cast<f32x4*>(crow + col * 4) = f32x4{v4[0], v4[1], v4[2], v4[3]};
      } else {
        const uint32_t lo = pack_bf16x2(v4[0], v4[1]), hi = pack_bf16x2(v4[2], v4[3]);
        *reinterpret_cast<uint2*>(crow + col * 2) = make_uint2(lo, hi);
      }
    }
  }
}

// Single-wave tiles (KS = 1) and the SwiGLU tiles are compiled for two waves per SIMD: the 64-row
// tiles otherwise took 268 (store) and 312 (SwiGLU) registers single-wave, 324 split over 4 waves,
// one wave per SIMD; held to 256 they keep every value in registers and twice the waves -- twice
// the weight loads -- are in flight (single-wave tiles: 64-token Qwen3-235B slice 0.2353 -> 0.2323
// ms, 1024-token Qwen3.5-397B slice 0.4157 -> 0.4098 ms, two reps). The K-split store tiles would
// spill 16-24 registers at that bound and stay at one wave per SIMD.
template <int FM, int KS, bool SWIGLU, bool OUT_F32, bool F16S = false>
__global__ void __launch_bounds__(64 * KS)
__attribute__((amdgpu_waves_per_eu((KS == 1 || SWIGLU) ? 2 : 1)))
gemm_bf16_stream_kernel(GemmArgs p, int n_tiles, int x_tiles, int total) {
  constexpr int BM = 16 * FM;                          // C rows per tile (FM fragments of 16)
  // tile order: groups of 8 m-tiles with the m-tile fastest, 8 consecutive tiles per XCD, so the
  // m-tiles of one group that needs several (the same weights) read them through one L2
  const int logical = xcd_remap(blockIdx.x, kStreamGroupM);
  if (logical >= total) return;
  Tile t;
  if (!resolve_tile(p, BM, n_tiles, x_tiles, logical, t, kStreamGroupM)) return;
  __shared__ f32x4 part[KS > 1 ? (KS - 1) * 4 * FM * 64 : 1];
  // 16-row fragments holding rows of the tile (uniform over the workgroup): each count runs its
  // own instantiation, so every load and MFMA stays unconditional
  const int live = (t.row1 - t.row0 + 15) / 16;
  if constexpr (FM >= 4) {
    if (live >= 4) { stream_tile<4, KS, SWIGLU, OUT_F32, F16S>(p, t, part); return; }
  }
  if constexpr (FM >= 3) {
    if (live == 3) { stream_tile<3, KS, SWIGLU, OUT_F32, F16S>(p, t, part); return; }
  }
  if constexpr (FM >= 2) {
    if (live == 2) { stream_tile<2, KS, SWIGLU, OUT_F32, F16S>(p, t, part); return; }
  }
  stream_tile<1, KS, SWIGLU, OUT_F32, F16S>(p, t, part);
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
// 192-row tiles (groups that fill about one m-tile each, their own weights per tile): groups of 4
// m-tiles, 32 tiles per XCD, so an XCD's CUs run every n-tile of 4 experts at once and share
// their activation rows in L2 (8192-token Qwen3.5-397B slice, two reps: 4 / 32 0.828-0.832 ms,
// 8 / 64 0.858-0.864, 4 / 64 0.864, 16 / 64 0.880-0.885)
constexpr int kTileGroupM192 = 4;
constexpr int kTileSpan192 = 32;
// LDS stages of the persistent ping-pong kernel. Measured on the 16384-token Qwen3-235B slice
// (same box, gate/up / down): 3 stages 2.52 / 1.61 ms, 4 stages 2.54 / 1.63 ms, 5 stages 2.60-2.63 /
// 1.65-1.67 ms -- fewer loads in flight per CU run faster here.
constexpr int kPPStages = 3;
// 192-row tiles: 4 stages of 28 KB (their groups' weights, each read by one m-tile, stream from HBM;
// measured on the 8192-token Qwen3.5-397B slice: 3 stages 0.905 ms, 4 stages 0.890, 5 stages 0.905)
constexpr int kPPStages192 = 4;
// weight-streaming tiles of 32 rows from 9 up to this many routed rows per group on average
constexpr int kStreamRows32 = 24;
// single-wave tiles below which a long-K weight stream splits K over 4 waves. 64-token Qwen3-235B
// slice (1536 tiles), layer ms, two reps per box: whole-K waves (two per SIMD) 0.2312-0.2315 on one
// box and 0.2587-0.2597 on another, the K split 0.2322-0.2324 and 0.2327-0.2349 -- with every
// whole-K wave resident at once, all start at the same K offset of rows 8 KB apart, and how
// those spread over the HBM channels depends on where the weights were placed
constexpr long long kStreamSplitTiles = 2048;
// weight streaming: K pairs (128 bytes of every weight row) per wave at or above which a tile is
// split over 4 waves (the long-K gate/up projection; a short K loop is dominated by its start-up)
constexpr int kStreamSplitPairs = 64;

// Workgroups of a persistent launch with one workgroup per CU: the current device's CU count rounded
// down to a multiple of the XCD count (0 if it cannot be queried; the caller then launches one
// workgroup per tile). Cached per device.
unsigned persistent_slots() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    v = (cus / kNumXcd) * kNumXcd;
    if (v <= 0) return 0;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return static_cast<unsigned>(v);
}

template <int BM, int BN, int WM, int WN, int MI, int BK, int S, bool PERSIST = false>
hipError_t run_bf16(const GemmArgs& a, hipStream_t s, int gm = 1, int span = 0) {
  const bool sw = a.epilogue == MOE_EPI_SWIGLU;
  Grid g = make_grid(a, BM, sw ? BN / 2 : BN, gm, span);
  if (g.total == 0) return hipSuccess;
  const bool f32 = a.out_dtype == MOE_F32;
  const size_t lds_bytes = (size_t)S * (BM + BN) * BK * sizeof(uint16_t);
  unsigned blocks = g.blocks;
  if (PERSIST) {
    const unsigned slots = persistent_slots();          // a multiple of the XCD count
    if (slots > 0 && slots < blocks) blocks = slots;
  }
  dim3 grid(blocks), block(WM * WN * 64);
#define MOE_RUN(SWI, F32, F16S)                                                              \
  gemm_bf16_pipe_kernel<BM, BN, WM, WN, MI, BK, S, SWI, F32, PERSIST, F16S><<<grid, block, lds_bytes, s>>>( \
      a, g.n_tiles, g.x_tiles, g.span, g.total, g.gm, (int)g.blocks)
  if (a.out_dtype == MOE_F16_SCALED) {
    // scaled fp16 rows need waves of 64 columns of 32 x 32 fragments
    if constexpr (MI == 32 && BN / WN == 64) {
      if (sw) return hipErrorInvalidValue;
      MOE_RUN(false, false, true);
    } else {
      return hipErrorInvalidValue;
    }
  }
  else if (sw && f32) MOE_RUN(true, true, false);
  else if (sw) MOE_RUN(true, false, false);
  else if (f32) MOE_RUN(false, true, false);
  else MOE_RUN(false, false, false);
#undef MOE_RUN
  return hipGetLastError();
}

template <int S, bool PERSIST = false, int BM = 256>
hipError_t run_bf16_pp(const GemmArgs& a, hipStream_t s, int gm, int span) {
  const bool sw = a.epilogue == MOE_EPI_SWIGLU;
  Grid g = make_grid(a, BM, sw ? 128 : 256, gm, span);
  if (g.total == 0) return hipSuccess;
  unsigned blocks = g.blocks;
  if (PERSIST) {
    const unsigned slots = persistent_slots();          // a multiple of the XCD count
    if (slots > 0 && slots < blocks) blocks = slots;
  }
  dim3 grid(blocks), block(512);
  const bool f32 = a.out_dtype == MOE_F32;
  const size_t lds_bytes = (size_t)S * (BM + 256) * 32 * sizeof(uint16_t);
#define MOE_RUN(SWI, F32, F16S)                                                                  \
  gemm_bf16_pp_kernel<SWI, F32, S, PERSIST, F16S, BM><<<grid, block, lds_bytes, s>>>(           \
      a, g.n_tiles, g.x_tiles, g.span, g.total, g.gm, (int)g.blocks)
  if (a.out_dtype == MOE_F16_SCALED) {
    if (sw) return hipErrorInvalidValue;
    MOE_RUN(false, false, true);
  }
  else if (sw && f32) MOE_RUN(true, true, false);
  else if (sw) MOE_RUN(true, false, false);
  else if (f32) MOE_RUN(false, true, false);
  else MOE_RUN(false, false, false);
#undef MOE_RUN
  return hipGetLastError();
}

template <int FM, int KS>
hipError_t run_bf16_stream(const GemmArgs& a, hipStream_t s) {
  const bool sw = a.epilogue == MOE_EPI_SWIGLU;
  Grid g = make_grid(a, 16 * FM, sw ? 32 : 64, kStreamGroupM, kStreamGroupM);
  if (g.total == 0) return hipSuccess;
  dim3 grid(g.blocks), block(64 * KS);
  const bool f32 = a.out_dtype == MOE_F32;
#define MOE_RUN(SWI, F32, F16S) \
  gemm_bf16_stream_kernel<FM, KS, SWI, F32, F16S><<<grid, block, 0, s>>>(a, g.n_tiles, g.x_tiles, g.total)
  if (a.out_dtype == MOE_F16_SCALED) {
    if (sw) return hipErrorInvalidValue;
    MOE_RUN(false, false, true);
  }
  else if (sw && f32) MOE_RUN(true, true, false);
  else if (sw) MOE_RUN(true, false, false);
  else if (f32) MOE_RUN(false, true, false);
  else MOE_RUN(false, false, false);
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

// Router logits of many tokens (an extra group of T rows, no routed groups, N = E experts): the
// largest of three tile shapes that still gives at least one workgroup per CU — 128 tokens x 128
// experts (4 waves of 64 x 64, 4 LDS stages), 64 x 128 (4 waves of 32 x 64, 6 stages), else 32 x 128
// (4 waves of 32 x 32 on 16 x 16 MFMAs, 7 stages). Measured with the top-k kernel (median of 10
// calls): 16384 tokens x 4096 x 128 experts 66 -> 58.5 us (64 x 128), 8192 x 4096 x 512 92 -> 69 us
// and 16384 x 7168 x 256 132 -> 99 us (128 x 128); 4096 x 7168 x 256 stays on 32 x 128 (49 us;
// the larger tiles leave CUs idle there).
hipError_t launch_gemm_router(const GemmArgs& a, hipStream_t s) {
  if (a.dtype != MOE_BF16) return launch_gemm(a, s);
  const long long e_tiles = (a.N + 127) / 128;
  if ((long long)((a.x_rows + 127) / 128) * e_tiles >= 256) return run_bf16<128, 128, 2, 2, 32, 64, 4>(a, s);
  if ((long long)((a.x_rows + 63) / 64) * e_tiles >= 256) return run_bf16<64, 128, 2, 2, 32, 64, 6>(a, s);
  return run_bf16<32, 128, 1, 4, 16, 64, 7>(a, s);
}

// Tile shape choice: the expected rows per group decide between a compute-shaped tile (large
// groups, MFMA-bound) and a weight-streaming tile (few rows per group, HBM-bound).
// MOE_FORCE_VARIANT="<swiglu>,<store>" (each one of 2x1, 2x4, 4x1, 4x4, or "-" for the default)
// forces the bf16 weight-streaming kernel's tile rows (16 x FM) and K split (KS) wherever the
// streaming kernel is chosen: a tuning and testing switch; every variant computes the same result.
// Read once per process.
static int forced_stream_variant(bool swiglu) {
  static int v[2] = {-1, -1};
  static std::once_flag once;
  std::call_once(once, [] {
    const char* e = std::getenv("MOE_FORCE_VARIANT");
    if (!e) return;
    for (int which = 0; which < 2 && *e; ++which) {
      if (e[0] >= '1' && e[0] <= '9' && e[1] == 'x' && e[2] >= '1' && e[2] <= '9')
        v[which] = (e[0] - '0') * 10 + (e[2] - '0');
      while (*e && *e != ',') ++e;
      if (*e == ',') ++e;
    }
  });
  return v[swiglu ? 0 : 1];
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  if (a.dtype == MOE_FP8_E4M3 || a.dtype == MOE_MXFP4 || a.dtype == MOE_MXFP8) return launch_gemm_q(a, s);
  if (a.dtype == MOE_NVFP4) return launch_gemm_nv4(a, s);
  if (a.dtype == MOE_F32) return run_f32(a, s);
  if (a.dtype == MOE_BF16) {
    const long long rows = (long long)(a.expected_rows > 0 ? a.expected_rows : a.max_rows) + a.x_rows;
    const int groups = a.G + (a.x_rows > 0 ? 1 : 0);
    const long long per_group = groups ? rows / groups : rows;
    const int n_full = a.epilogue == MOE_EPI_SWIGLU ? 2 * a.N : a.N;   // B rows per tile row
    // routed rows per group (the extra group's rows apart) and the rows its tiles would cover
    const long long r_bar = a.G > 0 ? (long long)(a.expected_rows > 0 ? a.expected_rows : a.max_rows) / a.G
                                    : a.x_rows;
    auto padded = [&](long long bm) { return (r_bar + bm - 1) / bm * bm; };
    // groups of ~144-192 rows (e.g. 160 on the 8192-token Qwen3.5-397B slice: top-10 of 512
    // experts, 64 local) fill one 192-row tile where a 256-row tile would be 62% padding
    const bool tile192 = r_bar >= 144 && padded(192) < padded(256);
    if (n_full >= 256 && (per_group >= 256 || tile192)) {
      // 256 (or 192) x 256 tiles, K-steps of 32 through 3 LDS stages of 32 KB, ping-pong schedule
      // of 8 waves of 128 (96) x 64, one persistent workgroup per CU: each tile's first loads are
      // issued before the previous tile's stores, which drain behind its first K-steps (measured
      // with the down projection's fp32 stores removed: the stores, waited for at every tile
      // start, took a quarter of its time).
      if (tile192) return run_bf16_pp<kPPStages192, true, 192>(a, s, kTileGroupM192, kTileSpan192);
      return run_bf16_pp<kPPStages, true>(a, s, kTileGroupM, kTileSpan);
    }
    if (per_group >= 96 && n_full >= 128) return run_bf16<128, 128, 2, 2, 32, 64, 3>(a, s);
    // decode-sized groups: stream the weights once per 32 (or 64) rows of each group
    // (each weight matrix below 4 GiB: the streaming kernel addresses inside one with 32 bits)
    if (a.N % 16 == 0 && !(a.epilogue == MOE_EPI_SWIGLU && a.N % 32) &&
        (long long)a.N * a.K * 2 < (1ll << 32)) {
      const bool split = a.K / 64 >= kStreamSplitPairs;
      switch (forced_stream_variant(a.epilogue == MOE_EPI_SWIGLU)) {
        case 21: return run_bf16_stream<2, 1>(a, s);
        case 24: return run_bf16_stream<2, 4>(a, s);
        case 41: return run_bf16_stream<4, 1>(a, s);
        case 44: return run_bf16_stream<4, 4>(a, s);
        default: break;
      }
      // the down projection streams its (short-K) weights once per 64 rows: measured ~5% faster
      // than 32-row tiles on the 64-token Qwen3-235B-shaped slice, where a few experts get more
      // than 32 rows and 32-row tiles would read their weights twice
      if (a.epilogue != MOE_EPI_SWIGLU && !split && per_group <= 64) return run_bf16_stream<4, 1>(a, s);
      // Tile rows from the routed rows each group expects under balanced routing (the extra
      // group's rows apart): 32 for ~9-24 rows, where the groups fit and the 32-row kernel holds
      // fewer registers per wave; 64 when the expectation is only a few rows, since skewed
      // routing then puts several times the average on the hottest experts and 32-row tiles
      // would read their weights twice; 64 above 24. The K split multiplies the waves by 4; it
      // pays below kStreamSplitTiles single-wave tiles. Measured with the single-wave tiles at
      // two waves per SIMD (gate/up variants, down 4x1, layer ms, two reps): 64-token Qwen3-235B
      // slice (Zipf-biased routing, ~14 rows per local expert, up to ~54) 4x4 0.2322-0.2324, 4x1
      // 0.2312-0.2315 (0.2587-0.2597 on another box), 2x1 0.2509-0.2519; 1024-token Qwen3.5-397B
      // slice + shared expert (20 rows, at most ~32) 2x1 0.4085-0.4103, 4x1 0.4178-0.4181; the
      // same with the gated shared expert 2x1 0.4143-0.4159, 4x1 0.4235-0.4245. (At one wave
      // per SIMD the 64-token slice took 4x4 0.235-0.236, 2x4 0.242-0.244, 2x1 0.250-0.251 ms.)
      const bool rows64 = r_bar <= 8 || r_bar > kStreamRows32;
      const int bm = rows64 ? 64 : 32;
      const long long m_tiles = (a.G > 0 ? (long long)a.G * ((r_bar + bm - 1) / bm) : 0) +
                                (a.x_rows + bm - 1) / bm;
      const long long n_tiles = (a.N + 31) / 32;
      const bool split_waves = split && m_tiles * n_tiles < kStreamSplitTiles;
      if (rows64) return split_waves ? run_bf16_stream<4, 4>(a, s) : run_bf16_stream<4, 1>(a, s);
      return split_waves ? run_bf16_stream<2, 4>(a, s) : run_bf16_stream<2, 1>(a, s);
    }
    return run_bf16<32, 128, 1, 4, 16, 64, 4>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
