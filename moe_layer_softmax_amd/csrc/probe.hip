// probe.hip -- HBM read-ceiling probe (measurement only; built into libmoe_probe.so, not into the
// layer library, and called by bench.py --stream-ceiling).
//
// Reads a row-major matrix of 8 KB rows (4096 bf16 elements: the gate/up weight row of the
// Qwen3-235B-shaped slice) with the decode kernels' access pattern: every wave of a 256-thread
// workgroup owns 16 consecutive rows and walks them along K; one load instruction covers ROWS rows
// x (1024 / ROWS) contiguous bytes (ROWS = 8: the weight-streaming kernels' 8 rows x 128 bytes;
// ROWS = 1: 1 KB of one row, the most contiguous form), eight instructions in flight per wave,
// non-temporal loads as in those kernels. The values are folded into one word per thread so the
// loads cannot be removed.
#include <hip/hip_runtime.h>

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
constexpr long long kRowBytes = 8192;

template <int ROWS>
__global__ void __launch_bounds__(256) read_rows_kernel(const char* __restrict__ src, int* __restrict__ out) {
  constexpr int U = 8;                               // loads in flight per wave
  constexpr int SEG = 1024 / ROWS;                   // contiguous bytes per row per instruction
  constexpr int PER_STEP = 16 / ROWS;                // instructions covering the wave's 16 rows
  constexpr int TOTAL = (kRowBytes / SEG) * PER_STEP;
  static_assert(TOTAL % U == 0, "whole groups of loads");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const char* base = src + ((long long)blockIdx.x * 64 + wave * 16) * kRowBytes;
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

}  // namespace

// Read `bytes` (a multiple of 64 rows of 8 KB) from src with ROWS = rows_per_load (1 or 8); out
// holds bytes / 512 KB * 256 ints. Returns the launch's hipError_t.
extern "C" int moe_probe_read_rows(const void* src, long long bytes, int rows_per_load, int* out,
                                   hipStream_t stream) {
  if (!src || !out || bytes <= 0 || bytes % (64 * kRowBytes)) return static_cast<int>(hipErrorInvalidValue);
  const unsigned wgs = static_cast<unsigned>(bytes / (64 * kRowBytes));
  const char* s = static_cast<const char*>(src);
  if (rows_per_load == 8) read_rows_kernel<8><<<wgs, 256, 0, stream>>>(s, out);
  else if (rows_per_load == 1) read_rows_kernel<1><<<wgs, 256, 0, stream>>>(s, out);
  else return static_cast<int>(hipErrorInvalidValue);
  return static_cast<int>(hipGetLastError());
}
