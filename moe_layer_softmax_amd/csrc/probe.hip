// probe.hip -- HBM read-ceiling probe (measurement only; built into libmoe_probe.so, not into the
// layer library, and called by bench.py --stream-ceiling).
//
// Reads a row-major matrix of 8 KB rows (4096 bf16 elements: the gate/up weight row of the
// Qwen3-235B-shaped slice) with the decode kernels' access pattern: every wave of a 256-thread
// workgroup owns RPW consecutive rows and walks them along K; one load instruction covers ROWS rows
// x (1024 / ROWS) contiguous bytes (ROWS = 8: the weight-streaming kernels' 8 rows x 128 bytes;
// ROWS = 1: 1 KB of one row, the most contiguous form), U instructions in flight per wave,
// non-temporal loads as in those kernels. The values are folded into one word per thread so the
// loads cannot be removed.
#include <hip/hip_runtime.h>

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
constexpr long long kRowBytes = 8192;

template <int ROWS, int RPW, int U>
__global__ void __launch_bounds__(256) read_rows_kernel(const char* __restrict__ src, int* __restrict__ out) {
  constexpr int SEG = 1024 / ROWS;                   // contiguous bytes per row per instruction
  constexpr int PER_STEP = RPW / ROWS;               // instructions covering the wave's RPW rows
  constexpr int TOTAL = (kRowBytes / SEG) * PER_STEP;
  static_assert(RPW % ROWS == 0 && TOTAL % U == 0, "whole groups of loads");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const char* base = src + ((long long)blockIdx.x * 4 * RPW + wave * RPW) * kRowBytes;
  const int r_in = lane / (64 / ROWS), c_in = (lane % (64 / ROWS)) * 16;
  int acc = 0;
  for (int i = 0; i < TOTAL; i += U) {
    i32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = i + u, step = q / PER_STEP, rg = q % PER_STEP;
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(
          base + (long long)(rg * ROWS + r_in) * kRowBytes + (long long)step * SEG + c_in));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc;
}

template <int ROWS, int RPW, int U>
int launch(const char* s, long long bytes, int* out, hipStream_t stream) {
  if (bytes % (4 * RPW * kRowBytes)) return static_cast<int>(hipErrorInvalidValue);
  const unsigned wgs = static_cast<unsigned>(bytes / (4 * RPW * kRowBytes));
  read_rows_kernel<ROWS, RPW, U><<<wgs, 256, 0, stream>>>(s, out);
  return static_cast<int>(hipGetLastError());
}

}  // namespace

// Read `bytes` from src in one of three patterns:
//   0: 8 rows x 128 bytes per load, 16 rows per wave, 8 loads in flight (the streaming kernels' shape)
//   1: 1 row x 1024 bytes per load, 16 rows per wave, 8 loads in flight
//   2: 8 rows x 128 bytes per load, 64 rows per wave, 16 loads in flight (fewer, longer streams)
// bytes must be a multiple of 4 waves x the pattern's rows per wave x 8 KB; out holds one int per
// thread of the launch (at most bytes / 64 KB * 256 / 4 ints for pattern 0 and 1, a quarter of that
// for pattern 2). Returns the launch's hipError_t.
extern "C" int moe_probe_read_rows(const void* src, long long bytes, int pattern, int* out,
                                   hipStream_t stream) {
  if (!src || !out || bytes <= 0) return static_cast<int>(hipErrorInvalidValue);
  const char* s = static_cast<const char*>(src);
  switch (pattern) {
    case 0: return launch<8, 16, 8>(s, bytes, out, stream);
    case 1: return launch<1, 16, 8>(s, bytes, out, stream);
    case 2: return launch<8, 64, 16>(s, bytes, out, stream);
    default: return static_cast<int>(hipErrorInvalidValue);
  }
}
