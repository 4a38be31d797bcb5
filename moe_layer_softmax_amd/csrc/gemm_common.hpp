// gemm_common.hpp -- tile scheduling, row gathering and LDS slice geometry shared by the grouped
// GEMM kernels (bf16 and block-scaled fp8 / MXFP4).
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

// s_waitcnt vmcnt(n) with every other counter left alone (n is a compile-time count)
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt((N & 15) | (((N >> 4) & 3) << 14) | 0x70 | 0xF00);
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


}  // namespace moe
