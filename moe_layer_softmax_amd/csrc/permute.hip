// permute.hip -- dispatch on gfx950: per-expert counts, expert offsets, a unique row for every
// local slot, and the row copy into expert-contiguous order.
//
// "CuTeDSL at Perplexity", section "MoE dispatch and combine": the local kernel counts the tokens
// of each expert from the routing table and gives each token a unique index inside its expert's
// list; the prefill variant counts in shared memory per block and accumulates the counts of all
// blocks in global memory, the decode variant handles the small routing table in one block.
// Unlike the atomics-ordered slots of that design, the rows here are placed in a unique order:
// the rows of one expert follow ascending flat slot index t*k+j. Counts use LDS atomics (their
// order does not matter); ranks come from wave ballots ("multisplit"), so the result does not
// depend on scheduling.
//
// Work split: the flat slot range [0, T*k) is cut into chunks of kChunk slots, one wave per chunk.
//   hist:    counts of every local expert inside each chunk  -> partial[chunk][E_loc]
//   scan:    counts, offsets (exclusive prefix over experts), and the base row of each
//            (chunk, expert) = offsets[e] + counts of e in earlier chunks
//   scatter: each wave walks its chunk in order, 64 slots at a time, ranking equal experts with
//            ballots and advancing a running row per expert kept in LDS.
// Count tables of up to 8192 entries fold the scan into the scatter kernel (every workgroup reads
// the whole table), so the dispatch is two launches; larger ones run the scan as a kernel of its
// own. For small tables (decode) one 1024-thread workgroup does all three phases in LDS.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kChunk = 1024;          // slots per wave-chunk (16 steps of 64)
constexpr int kMaxLocal = 1024;       // E_loc <= E <= 1024

size_t permute_ws_bytes(long long slots, int E_loc) {
  long long chunks = (slots + kChunk - 1) / kChunk;
  if (chunks < 1) chunks = 1;
  return static_cast<size_t>(chunks) * E_loc * sizeof(int32_t) + 256;
}

// lanes of the wave holding the same key as this lane
__device__ __forceinline__ unsigned long long match_key(int key, int nbits) {
  unsigned long long m = __ballot(1);
  for (int b = 0; b < nbits; ++b) {
    const int bit = (key >> b) & 1;
    const unsigned long long bal = __ballot(bit);
    m &= bit ? bal : ~bal;
  }
  return m;
}

__device__ __forceinline__ int key_bits(int E_loc) {
  int n = 1;
  while ((1 << n) <= E_loc + 1) ++n;
  return n;
}

// The keys of one wave's slots [c0, c1) (c1 - c0 <= 64 * N), lane-strided: key[i] belongs to
// slot c0 + 64 i + lane. Every load is issued before the first is used (clamped to the last slot of
// the range, so none is predicated), so a chunk costs one memory round trip. Keys: the local expert,
// E_loc for a slot routed off this GPU, E_loc + 1 past the range.
template <int N>
__device__ __forceinline__ void load_keys(const int32_t* ids, long long c0, long long c1, int e0,
                                          int E_loc, int (&key)[N]) {
  const int lane = lane_id();
  if (c0 >= c1) {                           // wave-uniform: an empty range reads nothing
#pragma unroll
    for (int i = 0; i < N; ++i) key[i] = E_loc + 1;
    return;
  }
  int raw[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const long long f = c0 + i * 64 + lane;
    raw[i] = ids[f < c1 ? f : c1 - 1];
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int el = raw[i] - e0;
    key[i] = c0 + i * 64 + lane >= c1 ? E_loc + 1 : ((el >= 0 && el < E_loc) ? el : E_loc);
  }
}

// count the local experts among the keys into cnt[E_loc] (LDS, zeroed by the caller)
template <int N>
__device__ __forceinline__ void hist_keys(const int (&key)[N], int E_loc, int* cnt) {
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (key[i] < E_loc) atomicAdd(&cnt[key[i]], 1);
}

// place the slots of one wave's range in order, 64 at a time; run[E_loc] (LDS) holds the next row
// of each expert
template <int N>
__device__ __forceinline__ void scatter_keys(const int (&key)[N], long long c0, long long c1,
                                             int E_loc, int* run, int32_t* slot_to_row,
                                             int32_t* row_to_flat) {
  const int lane = lane_id();
  const int nbits = key_bits(E_loc);
  const unsigned long long lt = (1ull << lane) - 1ull;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (c0 + i * 64 >= c1) break;           // wave-uniform
    const long long f = c0 + i * 64 + lane;
    const unsigned long long peers = match_key(key[i], nbits);
    const int rank = __popcll(peers & lt);
    int row = -1;
    if (key[i] < E_loc) row = run[key[i]] + rank;
    __builtin_amdgcn_wave_barrier();
    if (key[i] < E_loc && rank == 0) run[key[i]] += __popcll(peers);
    __builtin_amdgcn_wave_barrier();
    if (f < c1) {
      slot_to_row[f] = row;
      if (row >= 0) row_to_flat[row] = static_cast<int32_t>(f);
    }
  }
}

__global__ void __launch_bounds__(256) perm_hist_kernel(const int32_t* __restrict__ ids,
                                                        long long slots, int e0, int E_loc,
                                                        int n_chunks, int32_t* __restrict__ partial) {
  __shared__ int cnt[4][kMaxLocal];
  const int w = threadIdx.x >> 6;
  const int c = blockIdx.x * 4 + w;
  for (int i = threadIdx.x & 63; i < E_loc; i += 64) cnt[w][i] = 0;
  __syncthreads();
  if (c < n_chunks) {
    long long c0 = (long long)c * kChunk, c1 = c0 + kChunk < slots ? c0 + kChunk : slots;
    int key[kChunk / 64];
    load_keys(ids, c0, c1, e0, E_loc, key);
    hist_keys(key, E_loc, cnt[w]);
  }
  __syncthreads();
  if (c < n_chunks)
    for (int i = threadIdx.x & 63; i < E_loc; i += 64) partial[(size_t)c * E_loc + i] = cnt[w][i];
}

// exclusive scan of v over the NW * 64 threads of the block (returns the exclusive prefix, total)
template <int NW>
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int& total) {
  static_assert(NW <= 16, "wave totals in one 16-lane scan");
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int u = __shfl_up(inc, o, 64);
    if (lane >= o) inc += u;
  }
  if (lane == 63) tmp[w] = inc;
  __syncthreads();
  if (w == 0) {
    int x = lane < NW ? tmp[lane] : 0;
    int xi = x;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      int u = __shfl_up(xi, o, 64);
      if (lane >= o) xi += u;
    }
    if (lane < 16) tmp[16 + lane] = xi - x;   // exclusive prefix of wave totals
    if (lane == 15) tmp[32] = xi;
  }
  __syncthreads();
  int res = tmp[16 + w] + inc - v;
  total = tmp[32];
  __syncthreads();
  return res;
}

// counts, offsets and the base row of every (chunk, expert). One wave per expert (16 waves,
// experts w, w + 16, ...): lane l sums chunks l, l + 64, ...; then the chunk bases are an in-order
// scan over chunks, 64 chunks per wave-wide prefix sum.
__global__ void __launch_bounds__(1024) perm_scan_kernel(int32_t* __restrict__ partial, int n_chunks,
                                                         int E_loc, int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets) {
  __shared__ int tmp[64];
  __shared__ int tot_of[kMaxLocal];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int e = w; e < E_loc; e += 16) {
    int sum = 0;
    for (int c = lane; c < n_chunks; c += 64) sum += partial[(size_t)c * E_loc + e];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
    if (lane == 0) tot_of[e] = sum;
  }
  __syncthreads();
  const int el = threadIdx.x;
  const int tot = el < E_loc ? tot_of[el] : 0;
  int total;
  const int off = block_exclusive_scan<16>(tot, tmp, total);   // ends with a barrier
  if (el < E_loc) {
    counts[el] = tot;
    offsets[el] = off;
    tot_of[el] = off;                                             // each thread rewrites its own
  }
  if (threadIdx.x == 0) offsets[E_loc] = total;
  __syncthreads();
  for (int e = w; e < E_loc; e += 16) {
    int run = tot_of[e];
    for (int c0 = 0; c0 < n_chunks; c0 += 64) {
      const int c = c0 + lane;
      const int v = c < n_chunks ? partial[(size_t)c * E_loc + e] : 0;
      int inc = v;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(inc, o, 64);
        if (lane >= o) inc += u;
      }
      if (c < n_chunks) partial[(size_t)c * E_loc + e] = run + inc - v;
      run += __shfl(inc, 63, 64);
    }
  }
}

__global__ void __launch_bounds__(256) perm_scatter_kernel(const int32_t* __restrict__ ids,
                                                           long long slots, int e0, int E_loc,
                                                           int n_chunks,
                                                           const int32_t* __restrict__ base,
                                                           int32_t* __restrict__ slot_to_row,
                                                           int32_t* __restrict__ row_to_flat) {
  __shared__ int run[4][kMaxLocal];
  const int w = threadIdx.x >> 6;
  const int c = blockIdx.x * 4 + w;
  if (c >= n_chunks) return;                 // per-wave exit; no block barrier below
  long long c0 = (long long)c * kChunk, c1 = c0 + kChunk < slots ? c0 + kChunk : slots;
  int key[kChunk / 64];
  load_keys(ids, c0, c1, e0, E_loc, key);    // in flight together with the bases below
  for (int i = threadIdx.x & 63; i < E_loc; i += 64) run[w][i] = base[(size_t)c * E_loc + i];
  __builtin_amdgcn_wave_barrier();
  scatter_keys(key, c0, c1, E_loc, run[w], slot_to_row, row_to_flat);
}

// Scan folded into the scatter (count tables of up to kFusedTable entries): each workgroup loads
// the whole table with every load in flight and folds it, as it arrives, into per-expert LDS sums:
// the total over all chunks and the sum over the chunks before the workgroup's first; it keeps the
// rows of its own first three chunks. A wave's chunk base is then offsets[e] + that sum + the rows
// of the workgroup's chunks before it. Workgroup 0 also writes the counts and offsets. This
// replaces the one-workgroup scan kernel between the count and scatter kernels.
constexpr int kFusedTable = 8192;

__global__ void __launch_bounds__(256) perm_scan_scatter_kernel(const int32_t* __restrict__ ids,
                                                                long long slots, int e0, int E_loc,
                                                                int n_chunks,
                                                                const int32_t* __restrict__ partial,
                                                                int32_t* __restrict__ counts,
                                                                int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ slot_to_row,
                                                                int32_t* __restrict__ row_to_flat) {
  constexpr int PER = kFusedTable / 256;
  __shared__ int tot[kMaxLocal], pre[kMaxLocal], own[3][kMaxLocal], run[4][kMaxLocal];
  __shared__ int tmp[64];
  const int tid = threadIdx.x, w = tid >> 6;
  const int cw = blockIdx.x * 4, c = cw + w;
  // this wave's keys (empty past the last chunk) and the table, all loads in flight together
  const long long c0 = (long long)c * kChunk, c1 = c0 + kChunk < slots ? c0 + kChunk : slots;
  int key[kChunk / 64];
  load_keys(ids, c0, c1, e0, E_loc, key);
  const int n = n_chunks * E_loc;
  int v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) v[j] = partial[min(j * 256 + tid, n - 1)];
  for (int e = tid; e < E_loc; e += 256) tot[e] = pre[e] = 0;
  __syncthreads();
  // entry j * 256 + tid is (chunk cc, expert e); 256 = dq * E_loc + dr steps both
  const int dq = 256 / E_loc, dr = 256 - dq * E_loc;
  int cc = tid / E_loc, e = tid - cc * E_loc;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (j * 256 + tid < n) {
      atomicAdd(&tot[e], v[j]);
      if (cc < cw) atomicAdd(&pre[e], v[j]);
      else if (cc < cw + 3) own[cc - cw][e] = v[j];
    }
    cc += dq;
    e += dr;
    if (e >= E_loc) { e -= E_loc; ++cc; }
  }
  __syncthreads();
  // offsets: exclusive scan over the experts, 4 consecutive experts per thread (E_loc <= 1024)
  int t4[4], s4 = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    t4[i] = 4 * tid + i < E_loc ? tot[4 * tid + i] : 0;
    s4 += t4[i];
  }
  int total;
  int off = block_exclusive_scan<4>(s4, tmp, total);             // ends with a barrier
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int el = 4 * tid + i;
    if (el < E_loc) {
      if (blockIdx.x == 0) {
        counts[el] = t4[i];
        offsets[el] = off;
      }
      tot[el] = off;                                             // each thread rewrites its own
    }
    off += t4[i];
  }
  if (blockIdx.x == 0 && tid == 0) offsets[E_loc] = total;
  __syncthreads();
  if (c >= n_chunks) return;                 // per-wave exit; no block barrier below
  for (int el = tid & 63; el < E_loc; el += 64) {
    int b = tot[el] + pre[el];
    for (int r = 0; r < w; ++r) b += own[r][el];
    run[w][el] = b;
  }
  __builtin_amdgcn_wave_barrier();
  scatter_keys(key, c0, c1, E_loc, run[w], slot_to_row, row_to_flat);
}

// All three phases in one workgroup of 16 waves (small routing tables).
__global__ void __launch_bounds__(1024) perm_small_kernel(const int32_t* __restrict__ ids,
                                                          long long slots, int e0, int E_loc,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ slot_to_row,
                                                          int32_t* __restrict__ row_to_flat) {
  __shared__ int cnt[16][kMaxLocal];
  __shared__ int tmp[64];
  const int w = threadIdx.x >> 6;
  long long per = ((slots + 16 * 64 - 1) / (16 * 64)) * 64;   // slots per wave, multiple of 64
  long long c0 = w * per, c1 = c0 + per < slots ? c0 + per : slots;
  if (c0 > slots) c0 = slots;
  int key[16];                                                // per <= 16 * 64
  load_keys(ids, c0, c1, e0, E_loc, key);
  for (int i = threadIdx.x & 63; i < E_loc; i += 64) cnt[w][i] = 0;
  __syncthreads();
  hist_keys(key, E_loc, cnt[w]);
  __syncthreads();
  const int el = threadIdx.x;
  int tot = 0;
  if (el < E_loc)
    for (int v = 0; v < 16; ++v) tot += cnt[v][el];
  int total;
  const int off = block_exclusive_scan<16>(el < E_loc ? tot : 0, tmp, total);
  if (el < E_loc) {
    counts[el] = tot;
    offsets[el] = off;
    int run = off;
    for (int v = 0; v < 16; ++v) {
      int c = cnt[v][el];
      cnt[v][el] = run;
      run += c;
    }
  }
  if (threadIdx.x == 0) offsets[E_loc] = total;
  __syncthreads();
  scatter_keys(key, c0, c1, E_loc, cnt[w], slot_to_row, row_to_flat);
}

hipError_t launch_permute_maps(int T, int k, int e0, int E_loc, const int32_t* ids, int32_t* counts,
                               int32_t* offsets, int32_t* slot_to_row, int32_t* row_to_flat,
                               void* ws, hipStream_t s) {
  const long long slots = (long long)T * k;
  if (slots <= 16 * kChunk) {
    perm_small_kernel<<<1, 1024, 0, s>>>(ids, slots, e0, E_loc, counts, offsets, slot_to_row,
                                         row_to_flat);
    return hipGetLastError();
  }
  const int n_chunks = static_cast<int>((slots + kChunk - 1) / kChunk);
  int32_t* partial = static_cast<int32_t*>(ws);
  const int blocks = (n_chunks + 3) / 4;
  perm_hist_kernel<<<blocks, 256, 0, s>>>(ids, slots, e0, E_loc, n_chunks, partial);
  if ((long long)n_chunks * E_loc <= kFusedTable) {
    perm_scan_scatter_kernel<<<blocks, 256, 0, s>>>(ids, slots, e0, E_loc, n_chunks, partial, counts,
                                                    offsets, slot_to_row, row_to_flat);
    return hipGetLastError();
  }
  perm_scan_kernel<<<1, 1024, 0, s>>>(partial, n_chunks, E_loc, counts, offsets);
  perm_scatter_kernel<<<blocks, 256, 0, s>>>(ids, slots, e0, E_loc, n_chunks, partial, slot_to_row,
                                             row_to_flat);
  return hipGetLastError();
}

// ---- row copy: a_perm[r] = a_in[row_to_flat[r] / k] ------------------------------------------------
__global__ void __launch_bounds__(256) gather_rows_kernel(long long max_rows, int k,
                                                          const int32_t* __restrict__ offsets_end,
                                                          const int32_t* __restrict__ row_to_flat,
                                                          const uint8_t* __restrict__ src,
                                                          long long row_bytes, uint8_t* __restrict__ dst,
                                                          const uint8_t* __restrict__ src_scales,
                                                          long long scale_row_bytes, int scale_block,
                                                          uint8_t* __restrict__ dst_scales) {
  const long long r = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int R = *offsets_end;
  if (r >= R || r >= max_rows) return;
  const int lane = threadIdx.x & 63;
  const long long t = row_to_flat[r] / k;
  const i32x4* s4 = reinterpret_cast<const i32x4*>(src + t * row_bytes);
  i32x4* d4 = reinterpret_cast<i32x4*>(dst + r * row_bytes);
  for (long long c = lane; c < row_bytes / 16; c += 64) d4[c] = s4[c];
  if (src_scales) {
    const int32_t* ss = reinterpret_cast<const int32_t*>(src_scales + (t / scale_block) * scale_row_bytes);
    int32_t* ds = reinterpret_cast<int32_t*>(dst_scales + r * scale_row_bytes);
    for (long long c = lane; c < scale_row_bytes / 4; c += 64) ds[c] = ss[c];
  }
}

hipError_t launch_gather_rows(long long max_rows, int k, const int32_t* offsets_end,
                              const int32_t* row_to_flat, const void* src, long long row_bytes,
                              void* dst, const void* src_scales, long long scale_row_bytes,
                              int scale_rows_per_block, void* dst_scales, hipStream_t s) {
  if (max_rows == 0) return hipSuccess;
  const long long blocks = (max_rows + 3) / 4;
  gather_rows_kernel<<<dim3(static_cast<unsigned>(blocks)), 256, 0, s>>>(
      max_rows, k, offsets_end, row_to_flat, static_cast<const uint8_t*>(src), row_bytes,
      static_cast<uint8_t*>(dst), static_cast<const uint8_t*>(src_scales), scale_row_bytes,
      scale_rows_per_block, static_cast<uint8_t*>(dst_scales));
  return hipGetLastError();
}

}  // namespace moe
