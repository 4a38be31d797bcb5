// gemm_common.hpp -- tile scheduling, row gathering, LDS slice geometry and the MFMA-fragment
// epilogue shared by the grouped GEMM kernels (bf16, block-scaled fp8 / MX formats, NVFP4).
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

struct Tile {
  int row0, row1;       // rows of C covered by this tile
  int nt;               // n-tile
  bool extra;           // the extra (shared-expert) group
  const char* B;
  const char* B2;
  const char* Bs;
  const char* B2s;
};

// Find the group and row range of routed m-tile `mt` (every lane of the wave calls this; the
// result is wave-uniform). Returns false if `mt` is past the last tile.
__device__ __forceinline__ bool find_group(const int32_t* __restrict__ off, int G, int BM, int mt,
                                           int& g_out, int& row0, int& row1) {
  const int lane = lane_id();
  int base = 0;
  for (int g0 = 0; g0 < G; g0 += 64) {
    const int g = g0 + lane;
    int beg = 0, end = 0, tiles = 0;
    if (g < G) {
      beg = off[g];
      end = off[g + 1];
      tiles = (end - beg + BM - 1) / BM;
    }
    int inc = tiles;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(inc, o, 64);
      if (lane >= o) inc += v;
    }
    const unsigned long long hit = __ballot(base + inc > mt);
    if (hit) {
      const int first = __builtin_ctzll(hit);
      const int before = __shfl(inc - tiles, first, 64) + base;
      const int b = __shfl(beg, first, 64), e = __shfl(end, first, 64);
      g_out = uniform(g0 + first);
      row0 = uniform(b + (mt - before) * BM);
      row1 = uniform(min(row0 + BM, e));
      return true;
    }
    base += __shfl(inc, 63, 64);
  }
  return false;
}

// logical tile -> (m-tile, n-tile): m-tiles are taken in groups of gm; inside a group the m-tile
// index runs fastest, so consecutive logical tiles share B (same expert, same n-tile) and a short
// run of them shares A rows.
__device__ __forceinline__ bool resolve_tile(const GemmArgs& p, int BM, int n_tiles, int x_tiles,
                                             int logical, Tile& t, int gm = 1) {
  const int per_group = gm * n_tiles;
  const int grp = logical / per_group;
  const int within = logical - grp * per_group;
  const int mt = grp * gm + within % gm;
  t.nt = within / gm;
  if (mt < x_tiles) {
    t.extra = true;
    t.row0 = p.x_row0 + mt * BM;
    t.row1 = min(t.row0 + BM, p.x_row0 + p.x_rows);
    t.B = static_cast<const char*>(p.xB);
    t.B2 = static_cast<const char*>(p.xB2);
    t.Bs = static_cast<const char*>(p.xBs);
    t.B2s = static_cast<const char*>(p.xB2s);
    return true;
  }
  int g;
  if (!find_group(p.offsets, p.G, BM, mt - x_tiles, g, t.row0, t.row1)) return false;
  t.extra = false;
  t.B = static_cast<const char*>(p.B) + g * p.b_stride;
  t.B2 = p.B2 ? static_cast<const char*>(p.B2) + g * p.b_stride : nullptr;
  t.Bs = p.Bs ? static_cast<const char*>(p.Bs) + g * p.bs_stride : nullptr;
  t.B2s = p.B2s ? static_cast<const char*>(p.B2s) + g * p.bs_stride : nullptr;
  return true;
}

// source row of A for row r of C (r clamped into the tile so padding rows read valid memory)
__device__ __forceinline__ long long a_src_row(const GemmArgs& p, const Tile& t, int r) {
  r = r < t.row1 ? r : t.row1 - 1;
  if (t.extra) return r - p.x_a_off;
  if (p.a_rows) return p.a_rows[r] / p.a_row_div;
  return r;
}

// silu(g) = g * sigmoid(g) with the hardware exp2 and reciprocal (about 1 ulp each); the result is
// rounded to the expert format (bf16 or coarser) right after, far above their error.
__device__ __forceinline__ float silu_fast(float g) {
  return __fdividef(g, 1.0f + __expf(-g));
}

template <int BK>
struct SliceGeo {
  static constexpr int kRowBytes = BK * 2;             // bytes of one row slice
  static constexpr int kChunks = kRowBytes / 16;       // 16-byte chunks per row slice
  static constexpr int kRowsPerIns = 64 / kChunks;     // rows one wave-wide DMA instruction covers
  static constexpr int kRowsPerLine = 256 / kRowBytes; // rows sharing one 256-byte LDS bank line
  // gfx950's LDS serves a ds_read_b128 16 lanes at a time from 64 four-byte banks; an MFMA fragment
  // read has 16 lanes on 16 consecutive rows at one logical chunk. XOR-ing the chunk with
  // (row / rows-per-line) mod chunks gives those lanes 16 distinct bank groups.
  __device__ static __forceinline__ int swz(int r) { return (r / kRowsPerLine) & (kChunks - 1); }
};

// A lane's byte offset of its MFMA fragment row inside a stage region for substep s: fragments
// cover MI-row blocks starting at multiples of 16 rows, where the chunk swizzle repeats, so the
// offset depends on the lane only (the block adds an immediate).
template <class Geo, int MI, int MK>
__device__ __forceinline__ unsigned frag_lane_off(int s, int lane) {
  constexpr int BK = Geo::kRowBytes / 2;
  const int r = lane % MI;
  const int cidx = s * (MK / 8) + lane / MI;
  return (r * BK + ((cidx ^ Geo::swz(r)) * 8)) * 2;
}

// s_waitcnt vmcnt(n) with every other counter left alone (n is a compile-time count)
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt((N & 15) | (((N >> 4) & 3) << 14) | 0x70 | 0xF00);
#endif
}

// ---- MOE_F16_SCALED rows: fp16 values, then one fp32 power-of-two scale per 64 columns -----------
// Maximum over the lanes that differ from this one only in the lane-index bits of MASK (bits 2 and
// 3 only together: two rotations within a 16-lane row). Every lane must execute it.
template <int MASK>
__device__ __forceinline__ float lanes_max(float v) {
  static_assert((MASK & 12) == 0 || (MASK & 12) == 12, "bits 2 and 3 go together");
  auto dpp = [](float x, auto ctrl) -> float {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value, 0xF, 0xF, false));
  };
  if constexpr (MASK & 1) v = fmaxf(v, dpp(v, std::integral_constant<int, 0xB1>{}));    // lane ^ 1
  if constexpr (MASK & 2) v = fmaxf(v, dpp(v, std::integral_constant<int, 0x4E>{}));    // lane ^ 2
  if constexpr (MASK & 12) {
    v = fmaxf(v, dpp(v, std::integral_constant<int, 0x124>{}));                         // row_ror 4
    v = fmaxf(v, dpp(v, std::integral_constant<int, 0x128>{}));                         // row_ror 8
  }
  if constexpr (MASK & 16) v = fmaxf(v, __shfl_xor(v, 16, kWave));
  if constexpr (MASK & 32) v = fmaxf(v, __shfl_xor(v, 32, kWave));
  return v;
}
// Scale exponent of a 64-column block whose largest magnitude is m: with m in [2^(e-1), 2^e) the
// block is stored as its values times 2^-(e - 15), all below 2^15 in magnitude (fp16's largest
// finite value is 65504), the block maximum keeping fp16's 11 significant bits; the exponent is
// kept at or above -126 so that the stored scale is a normal fp32 number.
__device__ __forceinline__ int f16s_exp(float m) { return max(__builtin_amdgcn_frexp_expf(m) - 15, -126); }
// two values times 2^-e, rounded to fp16 (nearest even), packed low-first
__device__ __forceinline__ uint32_t pack_f16x2_scaled(float lo, float hi, int e) {
  const f16x2 h = f16x2{static_cast<_Float16>(__builtin_amdgcn_ldexpf(lo, -e)),
                        static_cast<_Float16>(__builtin_amdgcn_ldexpf(hi, -e))};
  return __builtin_bit_cast(uint32_t, h);
}
// the stored scale 2^e
__device__ __forceinline__ float f16s_scale(int e) { return __builtin_amdgcn_ldexpf(1.0f, e); }
// barrier_lds with no instruction scheduled across it (the phase boundaries of the ping-pong
// kernels, where the memory phase's reads and loads must stay on their side)
__device__ __forceinline__ void phase_barrier() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_sched_barrier(0);
  barrier_lds();
  __builtin_amdgcn_sched_barrier(0);
#endif
}

// Launch geometry of a grouped GEMM.
struct Grid {
  int n_tiles, x_tiles, span, total, gm;
  unsigned blocks;
};

// gm: m-tiles per tile-order group; span: consecutive logical tiles given to one XCD
inline Grid make_grid(const GemmArgs& a, int BM, int n_cols_per_tile, int gm = 1, int span = 0) {
  Grid g;
  g.n_tiles = (a.N + n_cols_per_tile - 1) / n_cols_per_tile;
  g.x_tiles = a.x_rows > 0 ? (a.x_rows + BM - 1) / BM : 0;
  // routed tiles: sum_g ceil(m_g / BM) <= floor(max_rows / BM) + G
  const long long routed = a.G > 0 ? (long long)a.max_rows / BM + a.G : 0;
  const long long m_tiles = g.x_tiles + routed;
  g.gm = gm;
  g.total = static_cast<int>(((m_tiles + gm - 1) / gm) * gm * g.n_tiles);
  g.span = span > 0 ? span : g.n_tiles;
  const long long blk = (long long)kNumXcd * g.span;
  g.blocks = static_cast<unsigned>(((g.total + blk - 1) / blk) * blk);
  return g;
}


// Write one wave's accumulators (FM x FN fragments of MI x MI, the wave's TM x TN block of the
// BM x BN tile at wave position (wm, wn)). SWIGLU: fragment j < FN/2 holds gate columns and
// j + FN/2 the matching up columns; h = silu(g) * u is stored. STORE: optional per-column bias.
// Rows past the tile's end and columns past N are skipped.
//
// In both MFMA layouts a lane holds one column and, for accumulator entries 2u and 2u + 1, two
// consecutive rows; the neighbouring lane (lane ^ 1) holds the next column for the same rows. One
// cross-lane swap (DPP) per pair gives the even lane both columns of the first row and the odd lane
// both columns of the second, so every store writes two adjacent values (4 bytes bf16, 8 fp32).
// STREAM: fp32 stores are non-temporal (a large C that the next kernel reads from HBM anyway, e.g.
// the down projection's y, is not left occupying L2; measured ~3% faster down projection).
// F16S (STORE, 32 x 32 fragments, 64-column waves): MOE_F16_SCALED rows. After the pair swap the
// lanes holding one row differ in lane bits 1-4 (16 lanes x 2 columns x FN fragments = the wave's
// 64 columns), so the block maximum is a reduction over those lanes; lanes 0, 1, 32 and 33 store
// the scale of their row.
template <int MI, int FM, int FN, int TM, int TN, int BN, bool SWIGLU, bool OUT_F32,
          bool STREAM = false, bool F16S = false, class AccAt>
__device__ __forceinline__ void store_tile(const GemmArgs& p, const Tile& t, int wm, int wn,
                                           AccAt acc_at) {
  constexpr int VPF = (MI == 32) ? 16 : 4;
  const int lane = lane_id();
  const bool odd = lane & 1;
  auto row_of = [&](int v) -> int {
    if constexpr (MI == 32) return (v / 4) * 8 + (lane / 32) * 4 + (v % 4);
    else return (lane / 16) * 4 + v;
  };
  auto swap_pair = [](float x) -> float {   // value of lane ^ 1 (quad_perm [1, 0, 3, 2])
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  };
  const int colw = (lane % MI) & ~1;                   // even column of this lane's pair
  char* C = static_cast<char*>(p.C);
  if constexpr (F16S) {
    static_assert(!SWIGLU && !OUT_F32 && MI == 32 && TN == 64, "scaled fp16 rows: 64-column waves");
    const long long c_blk = (long long)t.nt * BN + wn * TN;   // first column of the wave's block
    if (c_blk >= p.N) return;                                  // N % 64 == 0: all in or all out
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int u = 0; u < VPF / 2; ++u) {
        float lo[FN], hi[FN], m = 0.0f;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const long long col = c_blk + j * MI + colw;
          const float b0 = p.bias ? p.bias[col] : 0.0f, b1 = p.bias ? p.bias[col + 1] : 0.0f;
          const float a = acc_at(i, j, 2 * u), b = acc_at(i, j, 2 * u + 1);
          const float recv = swap_pair(odd ? a : b);
          lo[j] = (odd ? recv : a) + b0;
          hi[j] = (odd ? b : recv) + b1;
          m = fmaxf(m, fmaxf(fabsf(lo[j]), fabsf(hi[j])));
        }
        const int e = f16s_exp(lanes_max<30>(m));
        const int r = t.row0 + wm * TM + i * MI + row_of(odd ? 2 * u + 1 : 2 * u);
        if (r < t.row1) {
          char* crow = C + (long long)r * p.c_pitch;
#pragma unroll
          for (int j = 0; j < FN; ++j)
            *reinterpret_cast<uint32_t*>(crow + (c_blk + j * MI + colw) * 2) = pack_f16x2_scaled(lo[j], hi[j], e);
          if ((lane & 30) == 0)
            *reinterpret_cast<float*>(crow + (long long)p.N * 2 + c_blk / 16) = f16s_scale(e);
        }
      }
    return;
  }
  auto put = [&](int r, long long col, float lo, float hi) {
    if (r >= t.row1 || col >= p.N) return;
    char* crow = C + (long long)r * p.c_pitch;
    if (col + 1 < p.N) {
      if (OUT_F32 && STREAM) __builtin_nontemporal_store(f32x2{lo, hi}, reinterpret_cast<f32x2*>(crow + col * 4));
      else if (OUT_F32) *reinterpret_cast<float2*>(crow + col * 4) = make_float2(lo, hi);
      else *reinterpret_cast<uint32_t*>(crow + col * 2) = pack_bf16x2(lo, hi);
    } else {
      if (OUT_F32) reinterpret_cast<float*>(crow)[col] = lo;
      else reinterpret_cast<uint16_t*>(crow)[col] = f32_to_bf16(lo);
    }
  };
  constexpr int JN = SWIGLU ? FN / 2 : FN;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < JN; ++j) {
      const long long col = SWIGLU ? (long long)t.nt * (BN / 2) + wn * (TN / 2) + j * MI + colw
                                   : (long long)t.nt * BN + wn * TN + j * MI + colw;
      float b0 = 0.0f, b1 = 0.0f;
      if (!SWIGLU && p.bias) {
        b0 = p.bias[min(col, (long long)p.N - 1)];
        b1 = p.bias[min(col + 1, (long long)p.N - 1)];
      }
#pragma unroll
      for (int u = 0; u < VPF / 2; ++u) {
        float a, b;                                    // rows row_of(2u), row_of(2u + 1)
        if (SWIGLU) {
          a = silu_fast(acc_at(i, j, 2 * u)) * acc_at(i, j + FN / 2, 2 * u);
          b = silu_fast(acc_at(i, j, 2 * u + 1)) * acc_at(i, j + FN / 2, 2 * u + 1);
        } else {
          a = acc_at(i, j, 2 * u);
          b = acc_at(i, j, 2 * u + 1);
        }
        const float recv = swap_pair(odd ? a : b);
        const float lo = odd ? recv : a, hi = odd ? b : recv;
        const int r = t.row0 + wm * TM + i * MI + row_of(odd ? 2 * u + 1 : 2 * u);
        put(r, col, lo + b0, hi + b1);
      }
    }
}


}  // namespace moe
