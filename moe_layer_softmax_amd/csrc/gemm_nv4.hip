// gemm_nv4.hip -- grouped GEMM with NVFP4 weights on gfx950: the weights are dequantised in
// registers and fed to the bf16 MFMA.
//
// NVFP4 keeps 4-bit e2m1 values, two per byte, with one e4m3 scale per 16 consecutive elements
// along K (16-element absmax groups: "CuTeDSL at Perplexity", section "Blackwell"; 4-bit MoE
// weights with FP8 per-group scales, dequantised on the fly inside the matrix unit: "Driving vLLM
// WideEP and Large-Scale Serving Toward Maturity on Blackwell (Part I)", section on lower-precision
// operations), and one fp32 scale per row. gfx950's scaled MFMA takes power-of-two scales per 32
// elements, which cannot carry an e4m3 scale per 16; but an e2m1 value (2 significant bits) times
// an e4m3 scale (4 significant bits) has at most 6 significant bits and lies in [2^-10, 2688], so
// every q * s is exact in bf16. The kernels therefore form q * s in registers and run the bf16
// MFMA on those exact values, with fp32 accumulation; the two row scales (the weight row's and the
// activation row's) multiply the finished dot product in the epilogue.
//
// Layouts. B (weights of group g): packed codes [N, K/2] (element 2i in bits 0-3 of byte i); scale
// record of group g at Bs + g * bs_stride: e4m3 block scales [N, K/16], then fp32 row scales [N].
// A: bf16 [rows, K] holding the activation's block values q * s (exact; moe_permute and the
// layer's activation quantiser write them), A_scales: fp32 row scale of each A row, or null (1).
//
// The layer's gate/up projection takes its activation block values as fp16 instead (exact as
// well) and dequantises the weights to fp16 (F16), half the instructions per element of the bf16
// form; the down projection's input h is bf16, so it keeps the bf16 form.
//
// Two kernels:
//   * tile kernel (prefill-sized groups): 256 x 256 tiles of 8 waves (128 x 128 tiles of 4 waves
//     for groups under 256 rows), K-steps of 64 (four scale blocks).
//     Both operands go global -> registers -> LDS (bf16, 16-byte chunks XOR-swizzled by row as in
//     the bf16 kernels); B is dequantised on its way into LDS, once per workgroup and element, and
//     the MFMAs (32 x 32 x 16 bf16) read both operands from LDS. Two LDS stages; each step's global
//     loads are issued two steps ahead into a second register set.
//   * streaming kernel (decode-sized groups): one wave per 16 rows x 64 weight rows, weights
//     straight from HBM to registers (8 rows x 128 contiguous bytes per load instruction, moved to
//     the MFMA operand lanes with ds_bpermute), dequantised per MFMA step in registers; activations
//     loaded in the operand layout from L2; K-split over the workgroup's waves as in the bf16
//     streaming kernel.
#include <type_traits>

#include "gemm_common.hpp"
#include "quant_dev.hpp"

namespace moe {

hipError_t launch_gemm_nv4(const GemmArgs& a, hipStream_t s);

namespace {

// m-tiles per tile-order group of the streaming kernel, and the 256-element chunks of K from which
// it splits K over 4 waves (no workload shape reaches it: measured on the 64-token DeepSeek-V3
// NVFP4 slice, three reps, the gate/up split over 4 waves with groups of 8 took 0.2444-0.2453 ms,
// groups of 4 0.2392-0.2437, no split with groups of 4 0.2365-0.2393; the down projection split
// too, 0.318)
constexpr int kNvStreamGroupM = 4;
constexpr int kNvSplitChunks = 64;

// e4m3 scale byte SEL of a 32-bit word, as fp32 (exact; gfx950's fp8 conversion is OCP e4m3)
template <int SEL>
__device__ __forceinline__ float nv4_scale(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(w), SEL);
}

// F16: the activation block values arrive as fp16 and the weights are dequantised to fp16 (one
// packed multiply per two elements instead of two fp32 multiplies and a pack); the fp16 MFMA has the
// bf16 rate. Operand fragments and the MFMAs of either form:
template <bool F16>
using Frag = std::conditional_t<F16, f16x8, bf16x8>;
template <bool F16>
__device__ __forceinline__ i32x4 dequant8(uint32_t w, float s) {
  if constexpr (F16) return e2m1x8_times_f16(w, s);
  else return e2m1x8_times(w, s);
}
template <bool F16>
__device__ __forceinline__ f32x16 mfma32(Frag<F16> a, Frag<F16> b, f32x16 c) {
  if constexpr (F16) return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  else return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
template <bool F16>
__device__ __forceinline__ f32x4 mfma16(Frag<F16> a, Frag<F16> b, f32x4 c) {
  if constexpr (F16) return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  else return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fp32 row scales of the weight rows of a scale record (after its N * K/16 block-scale bytes)
__device__ __forceinline__ const float* nv4_row_scales(const char* rec, const GemmArgs& p) {
  return reinterpret_cast<const float*>(rec + (long long)p.N * (p.K / 16));
}

// ------------------------------------------------------------------------------------------------
// Tile kernel
// ------------------------------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, bool SWIGLU, bool OUT_F32, bool F16>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_nv4_tile_kernel(GemmArgs p, int n_tiles, int x_tiles, int span, int total, int gm) {
  constexpr int NT = WM * WN * 64;
  constexpr int BK = 64;
  using Geo = SliceGeo<BK>;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int STAGE = (BM + BN) * BK;              // bf16 elements per LDS stage
  constexpr int A_CH = BM * 8 / NT;                  // 16-byte A chunks per thread and step
  constexpr int B_HR = BN * 2 / NT;                  // B half rows (16 packed bytes) per thread
  static_assert(A_CH * NT == BM * 8 && B_HR * NT == BN * 2, "tile / thread split");
  static_assert(!SWIGLU || FN % 2 == 0, "SWIGLU needs gate and up fragments in every wave");
  extern __shared__ __attribute__((aligned(1024))) uint16_t lds[];

  const int logical = xcd_remap(blockIdx.x, span);
  if (logical >= total) return;
  Tile t;
  if (!resolve_tile(p, BM, n_tiles, x_tiles, logical, t, gm)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = uniform(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int nk = p.K / BK;
  const long long wrow = p.K / 2, srow = p.K / 16;

  // A: chunk c = tid + NT * u -> tile row c / 8, 16-byte chunk c % 8 of the step's 128 bytes
  const char* a_ptr[A_CH];
  unsigned a_lds[A_CH];
#pragma unroll
  for (int u = 0; u < A_CH; ++u) {
    const int c = tid + NT * u, r = c / 8, ch = c % 8;
    a_ptr[u] = static_cast<const char*>(p.A) + a_src_row(p, t, t.row0 + r) * p.a_pitch + ch * 16;
    a_lds[u] = r * BK + ((ch ^ Geo::swz(r)) * 8);
  }
  // B: half row hr = tid + NT * u -> LDS row rb = hr / 2, elements [32 h, 32 h + 32) of the step
  const char* b_ptr[B_HR];
  const char* s_ptr[B_HR];
  unsigned b_lds[B_HR][4];
#pragma unroll
  for (int u = 0; u < B_HR; ++u) {
    const int hr = tid + NT * u, rb = hr / 2, h = hr % 2;
    const char* base = t.B;
    const char* sbase = t.Bs;
    long long n;
    if (SWIGLU) {
      const int half = TN / 2;
      if ((rb % TN) >= half) { base = t.B2; sbase = t.B2s; }
      n = (long long)t.nt * (BN / 2) + (rb / TN) * half + (rb % TN) % half;
    } else {
      n = (long long)t.nt * BN + rb;
    }
    if (n >= p.N) n = p.N - 1;                       // columns past N: a valid row, never stored
    b_ptr[u] = base + n * wrow + h * 16;
    s_ptr[u] = sbase + n * srow;                     // the step's 4 scale bytes; h picks 2 of them
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int row = BM + rb, ch = 4 * h + d;
      b_lds[u][d] = row * BK + ((ch ^ Geo::swz(row)) * 8);
    }
  }

  // Barrier of the K loop: this wave's LDS writes (and reads) complete, then the workgroup barrier.
  // Not __syncthreads(): its memory fence would also wait for the global loads of the steps ahead,
  // which are in flight in registers across the barrier.
  auto lds_barrier = [] {
    wait_lgkm();
    barrier_lds();
  };
  i32x4 ra[2][A_CH], rbw[2][B_HR];
  uint32_t rs[2][B_HR];
  const int bsh = (tid % 2) * 16;                    // this thread's two scale bytes in the word
  auto load = [&](int kt, int set) {
    kt = kt < nk ? kt : nk - 1;                      // past the end: re-read the last step
#pragma unroll
    for (int u = 0; u < A_CH; ++u) ra[set][u] = *reinterpret_cast<const i32x4*>(a_ptr[u] + (long long)kt * 128);
#pragma unroll
    for (int u = 0; u < B_HR; ++u) {
      rbw[set][u] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(b_ptr[u] + (long long)kt * 32));
      rs[set][u] = *reinterpret_cast<const uint32_t*>(s_ptr[u] + (long long)kt * 4);
    }
  };
  auto write = [&](int set, int stage) {
    uint16_t* st = lds + stage * STAGE;
#pragma unroll
    for (int u = 0; u < A_CH; ++u) *reinterpret_cast<i32x4*>(st + a_lds[u]) = ra[set][u];
#pragma unroll
    for (int u = 0; u < B_HR; ++u) {
      const uint32_t w = rs[set][u] >> bsh;
      const float s0 = nv4_scale<0>(w), s1 = nv4_scale<1>(w);
#pragma unroll
      for (int d = 0; d < 4; ++d)
        *reinterpret_cast<i32x4*>(st + b_lds[u][d]) =
            dequant8<F16>(static_cast<uint32_t>(rbw[set][u][d]), d < 2 ? s0 : s1);
    }
  };

  unsigned lane_off[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) lane_off[s] = frag_lane_off<Geo, 32, 16>(s, lane);
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

  // step kt reads LDS stage kt % 2 and register set kt % 2 holds its loads until they are written;
  // the loop is unrolled by two so that the register sets are indexed statically
  auto step = [&](int kt, auto set_tag) {
    constexpr int cur = decltype(set_tag)::value;
    load(kt + 2, cur);                               // this set was written to LDS last step
    MOE_SCHED_FENCE();                               // the loads go out before this step's MFMAs
    const char* lb = reinterpret_cast<const char*>(lds + cur * STAGE);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      Frag<F16> fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        fa[i] = *reinterpret_cast<const Frag<F16>*>(lb + lane_off[s] + (wm * TM + i * 32) * BK * 2);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        fb[j] = *reinterpret_cast<const Frag<F16>*>(lb + lane_off[s] + (BM + wn * TN + j * 32) * BK * 2);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<F16>(fa[i], fb[j], acc[i][j]);
    }
    // step kt + 1 into the other stage (last read during step kt - 1, before the previous barrier);
    // fenced so that no part of it (whose operands wait for that step's loads) moves up into the
    // MFMAs
    MOE_SCHED_FENCE();
    if (kt + 1 < nk) write(cur ^ 1, cur ^ 1);
    lds_barrier();
  };
  load(0, 0);
  load(1, 1);
  write(0, 0);
  lds_barrier();
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    step(kt, std::integral_constant<int, 0>{});
    step(kt + 1, std::integral_constant<int, 1>{});
  }
  if (kt < nk) step(kt, std::integral_constant<int, 0>{});

  // epilogue: acc * (activation row scale * weight row scale), then the common store
  const float* grs = nv4_row_scales(t.Bs, p);
  const float* grs2 = SWIGLU ? nv4_row_scales(t.B2s, p) : nullptr;
  const float* ars = static_cast<const float*>(p.A_scales);
  float gb[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    long long n;
    if (SWIGLU) n = (long long)t.nt * (BN / 2) + wn * (TN / 2) + (j % (FN / 2)) * 32 + (lane & 31);
    else n = (long long)t.nt * BN + wn * TN + j * 32 + (lane & 31);
    if (n >= p.N) n = p.N - 1;
    gb[j] = (SWIGLU && j >= FN / 2) ? grs2[n] : grs[n];
  }
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = t.row0 + wm * TM + i * 32 + (v / 4) * 8 + (lane / 32) * 4 + (v % 4);
      const float ga = ars ? ars[a_src_row(p, t, r)] : 1.0f;
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j][v] *= ga * gb[j];
    }
  store_tile<32, FM, FN, TM, TN, BN, SWIGLU, OUT_F32>(p, t, wm, wn,
                                                      [&](int i, int j, int v) -> float { return acc[i][j][v]; });
}

// ------------------------------------------------------------------------------------------------
// Streaming kernel
//
// Per 256-element chunk of K (128 packed bytes of every weight row): weight loads cover 8 rows x
// 128 bytes per instruction (lane -> row h * 8 + lane / 8, 16-byte piece lane % 8 = elements
// [32 (lane % 8), +32) of the chunk). MFMA step s (0..7) of the chunk: operand lane (row lr,
// quarter kq) takes dword s % 4 of piece 4 (s / 4) + kq of row lr, i.e. elements
// 32 (4 (s / 4) + kq) + 8 (s % 4) .. + 7 -- a fixed permutation of K that the activation operand
// follows (its lane loads those same 8 elements), so the dot product is unchanged. The piece's two
// scale blocks are bytes 8 (s / 4) + 2 kq and + 1 of the row's 16 scale bytes of the chunk.
// ------------------------------------------------------------------------------------------------
template <int KS, bool SWIGLU, bool OUT_F32, bool F16>
__global__ void __launch_bounds__(64 * KS)
gemm_nv4_stream_kernel(GemmArgs p, int n_tiles, int x_tiles, int total) {
  constexpr int BM = 16;
  const int logical = xcd_remap(blockIdx.x, kNvStreamGroupM);
  if (logical >= total) return;
  Tile t;
  if (!resolve_tile(p, BM, n_tiles, x_tiles, logical, t, kNvStreamGroupM)) return;

  const int lane = lane_id();
  const int lr = lane & 15, kq = lane >> 4;
  const long long wrow = p.K / 2, srow = p.K / 16;
  // weight row of fragment j (SWIGLU: j < 2 gate, j >= 2 the matching up rows), row r in 0..15
  auto wrow_of = [&](int j, int r, const char*& base, const char*& sbase) -> long long {
    long long n;
    base = t.B;
    sbase = t.Bs;
    if (SWIGLU) {
      n = (long long)t.nt * 32 + (j & 1) * 16 + r;
      if (j >= 2) { base = t.B2; sbase = t.B2s; }
    } else {
      n = (long long)t.nt * 64 + j * 16 + r;
    }
    return n < p.N ? n : p.N - 1;                  // columns past N: a valid row, never stored
  };
  const char* wp[4][2];
  const char* sp[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const char *base, *sb;
      const long long n = wrow_of(j, h * 8 + (lane >> 3), base, sb);
      wp[j][h] = base + n * wrow + (lane & 7) * 16;
    }
    const char *base, *sb;
    const long long n = wrow_of(j, lr, base, sb);
    sp[j] = sb + n * srow + 2 * kq;
  }
  const char* ap = static_cast<const char*>(p.A) + a_src_row(p, t, t.row0 + lr) * p.a_pitch + kq * 64;
  const int src0 = ((lr & 7) * 8 + kq) * 4, src1 = src0 + 16;
  const bool upper = lr >= 8;

  const int wave = KS > 1 ? (int)(threadIdx.x >> 6) : 0;
  const int nc_all = p.K / 256;
  const int c0 = nc_all * wave / KS, nc = nc_all * (wave + 1) / KS - c0;
  i32x4 wraw[2][4][2];
  i32x4 av[2][2][4];
  uint32_t wsc[2][4][2];
  auto load = [&](int c, int set) {
    const long long cc = c0 + (c < nc ? c : nc - 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        wraw[set][j][h] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(wp[j][h] + cc * 128));
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        wsc[set][j][hh] = *reinterpret_cast<const uint16_t*>(sp[j] + cc * 16 + hh * 8);
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        av[set][hh][q] = *reinterpret_cast<const i32x4*>(ap + cc * 512 + hh * 256 + q * 16);
  };
  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{};
  auto compute = [&](int set) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int src = hh ? src1 : src0;
      float sc[4][2];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sc[j][0] = nv4_scale<0>(wsc[set][j][hh]);
        sc[j][1] = nv4_scale<1>(wsc[set][j][hh]);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        Frag<F16> wf[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int lo = __builtin_amdgcn_ds_bpermute(src, wraw[set][j][0][q]);
          const int hi = __builtin_amdgcn_ds_bpermute(src, wraw[set][j][1][q]);
          wf[j] = __builtin_bit_cast(Frag<F16>, dequant8<F16>(static_cast<uint32_t>(upper ? hi : lo), sc[j][q >> 1]));
        }
        const Frag<F16> a = __builtin_bit_cast(Frag<F16>, av[set][hh][q]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = mfma16<F16>(wf[j], a, acc[j]);
      }
    }
  };
  if (nc > 0) {                                      // wave-uniform; nc = 0 only if chunks < KS
    load(0, 0);
    int c = 0;
    for (; c + 1 < nc; c += 2) {
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
    if (c < nc) compute(0);                          // odd number of chunks: the last is in set 0
  }
  if constexpr (KS > 1) {
    __shared__ f32x4 part[KS - 1][4][64];
    if (wave > 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) part[wave - 1][j][lane] = acc[j];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < KS - 1; ++w)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] += part[w][j][lane];
  }

  // acc[j][v]: weight row j * 16 + kq * 4 + v of the tile, C row row0 + lr
  const int r = t.row0 + lr;
  if (r >= t.row1) return;
  const float ga = p.A_scales ? static_cast<const float*>(p.A_scales)[a_src_row(p, t, r)] : 1.0f;
  f32x4 gsc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const char *base, *sb;
    const long long n = wrow_of(j, kq * 4, base, sb);   // 4 consecutive rows (N % 16 == 0)
    gsc[j] = *reinterpret_cast<const f32x4*>(nv4_row_scales(sb, p) + n);
  }
  char* crow = static_cast<char*>(p.C) + (long long)r * p.c_pitch;
#pragma unroll
  for (int j = 0; j < (SWIGLU ? 2 : 4); ++j) {
    float v4[4];
    long long col;
    if (SWIGLU) {
      col = (long long)t.nt * 32 + j * 16 + kq * 4;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        v4[v] = silu_fast(acc[j][v] * (ga * gsc[j][v])) * (acc[j + 2][v] * (ga * gsc[j + 2][v]));
    } else {
      col = (long long)t.nt * 64 + j * 16 + kq * 4;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        v4[v] = acc[j][v] * (ga * gsc[j][v]) + (p.bias ? p.bias[min(col + v, (long long)p.N - 1)] : 0.0f);
    }
    if (col >= p.N) continue;                        // N is a multiple of 16: all four or none
    if (OUT_F32) {
      *reinterpret_cast<f32x4*>(crow + col * 4) = f32x4{v4[0], v4[1], v4[2], v4[3]};
    } else {
      const uint32_t lo = pack_bf16x2(v4[0], v4[1]), hi = pack_bf16x2(v4[2], v4[3]);
      *reinterpret_cast<uint2*>(crow + col * 2) = make_uint2(lo, hi);
    }
  }
}

template <int BM, int BN, int WM, int WN, bool SWIGLU, bool OUT_F32, bool F16>
hipError_t run_tile(const GemmArgs& a, hipStream_t s) {
  Grid g = make_grid(a, BM, SWIGLU ? BN / 2 : BN, 8, 64);
  if (g.total == 0) return hipSuccess;
  const size_t lds = 2 * (size_t)(BM + BN) * 64 * 2;
  gemm_nv4_tile_kernel<BM, BN, WM, WN, SWIGLU, OUT_F32, F16><<<dim3(g.blocks), dim3(WM * WN * 64), lds, s>>>(
      a, g.n_tiles, g.x_tiles, g.span, g.total, g.gm);
  return hipGetLastError();
}

template <int KS, bool SWIGLU, bool OUT_F32, bool F16>
hipError_t run_stream(const GemmArgs& a, hipStream_t s) {
  Grid g = make_grid(a, 16, SWIGLU ? 32 : 64, kNvStreamGroupM, kNvStreamGroupM);
  if (g.total == 0) return hipSuccess;
  gemm_nv4_stream_kernel<KS, SWIGLU, OUT_F32, F16><<<dim3(g.blocks), dim3(64 * KS), 0, s>>>(
      a, g.n_tiles, g.x_tiles, g.total);
  return hipGetLastError();
}

template <bool SWIGLU, bool OUT_F32, bool F16 = false>
hipError_t run_choice(const GemmArgs& a, hipStream_t s) {
  const long long rows = (long long)(a.expected_rows > 0 ? a.expected_rows : a.max_rows) + a.x_rows;
  const int groups = a.G + (a.x_rows > 0 ? 1 : 0);
  const long long per_group = groups ? rows / groups : rows;
  if (per_group <= 32) {
    if (a.K / 256 >= kNvSplitChunks) return run_stream<4, SWIGLU, OUT_F32, F16>(a, s);
    return run_stream<1, SWIGLU, OUT_F32, F16>(a, s);
  }
  // groups of a full 256-row tile: 256 x 256 tiles of 8 waves (128 x 64 each, one workgroup per
  // CU in 128 KB of LDS), twice the MFMAs per dequantised weight and per fragment read of the
  // 128 x 128 tiles (4 waves of 64 x 64, two workgroups per CU), which serve smaller groups
  if (per_group >= 256) return run_tile<256, 256, 2, 4, SWIGLU, OUT_F32, F16>(a, s);
  return run_tile<128, 128, 2, 2, SWIGLU, OUT_F32, F16>(a, s);
}

}  // namespace

// NVFP4 grouped GEMM: K % 256 == 0, N % 128 == 0; out fp32 or bf16 (SWIGLU: h, STORE: C)
hipError_t launch_gemm_nv4(const GemmArgs& a, hipStream_t s) {
  if (a.K % 256 || a.N % 128) return hipErrorInvalidValue;
  const bool swiglu = a.epilogue == MOE_EPI_SWIGLU;
  if (a.a_f16) {                                     // the layer's gate/up projection only
    if (!swiglu || a.out_dtype != MOE_BF16) return hipErrorInvalidValue;
    return run_choice<true, false, true>(a, s);
  }
  if (a.out_dtype == MOE_F32) return swiglu ? run_choice<true, true>(a, s) : run_choice<false, true>(a, s);
  if (a.out_dtype == MOE_BF16) return swiglu ? run_choice<true, false>(a, s) : run_choice<false, false>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
