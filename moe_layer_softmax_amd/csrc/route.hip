// route.hip -- scores, top-k and routing weights on gfx950.
//
// One wave64 per token. Each lane holds ceil(E/64) logits as 64-bit keys
//   key = (order-preserving u32 of the fp32 logit) << 32 | (~expert id)
// so that the wave-wide maximum key is the largest logit and, among equal logits, the lowest
// expert id (the tie rule of the tiny workload; -0.0 is canonicalised to +0.0 first so the two
// compare equal). k rounds of a wave max pick the experts in rank order.
// Routing as int ids + float weights of shape [T, k]: "How we served a 397B MoE model ... on
// TPU v7", section "Three collectives become two".
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

__device__ __forceinline__ uint32_t ordered_bits(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);   // -0 -> +0 (round-to-nearest: -0 + +0 = +0)
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}

template <int VPL>
__global__ void __launch_bounds__(256) topk_kernel(int T, int E, int k, int scoring, int renorm,
                                                   const float* __restrict__ logits,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;                       // uniform per wave
  const int lane = threadIdx.x & 63;
  const float* L = logits + (size_t)t * E;

  unsigned long long key[VPL];
  float val[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    int e = v * 64 + lane;
    if (e < E) {
      val[v] = L[e];
      key[v] = (static_cast<unsigned long long>(ordered_bits(val[v])) << 32) |
               static_cast<uint32_t>(~e);
    } else {
      val[v] = 0.0f;
      key[v] = 0ull;                        // below every real key
    }
  }

  float my_l = 0.0f, top_l = 0.0f;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    unsigned long long best = key[0];
#pragma unroll
    for (int v = 1; v < VPL; ++v) best = key[v] > best ? key[v] : best;
    best = wave_max_u64(best);
    const int e = static_cast<int>(~static_cast<uint32_t>(best));
    const float l = from_ordered(static_cast<uint32_t>(best >> 32));
    if (j == 0) top_l = l;
    if (lane == j) { my_l = l; my_e = e; }
    if ((e & 63) == lane) {
#pragma unroll
      for (int v = 0; v < VPL; ++v)
        if (v == (e >> 6)) key[v] = 0ull;
    }
  }

  float wt;
  if (scoring == MOE_SOFTMAX) {
    // softmax over all experts at the chosen ones; renormalised: softmax over the chosen logits
    float z;
    const float num = (lane < k) ? expf(my_l - top_l) : 0.0f;
    if (renorm) {
      z = wave_sum(num);
    } else {
      float part = 0.0f;
#pragma unroll
      for (int v = 0; v < VPL; ++v)
        if (v * 64 + lane < E) part += expf(val[v] - top_l);
      z = wave_sum(part);
    }
    wt = num / z;
  } else {
    const float p = (lane < k) ? 1.0f / (1.0f + expf(-my_l)) : 0.0f;
    wt = renorm ? p / wave_sum(p) : p;
  }
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_e;
    w[(size_t)t * k + lane] = wt;
  }
}

hipError_t launch_topk(int T, int E, int k, int scoring, int renormalize, const float* logits,
                       int32_t* ids, float* w, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((T + 3) / 4), block(256);
  int vpl = (E + 63) / 64;
  if (vpl <= 1)
    topk_kernel<1><<<grid, block, 0, s>>>(T, E, k, scoring, renormalize, logits, ids, w);
  else if (vpl <= 2)
    topk_kernel<2><<<grid, block, 0, s>>>(T, E, k, scoring, renormalize, logits, ids, w);
  else if (vpl <= 4)
    topk_kernel<4><<<grid, block, 0, s>>>(T, E, k, scoring, renormalize, logits, ids, w);
  else if (vpl <= 8)
    topk_kernel<8><<<grid, block, 0, s>>>(T, E, k, scoring, renormalize, logits, ids, w);
  else
    topk_kernel<16><<<grid, block, 0, s>>>(T, E, k, scoring, renormalize, logits, ids, w);
  return hipGetLastError();
}

}  // namespace moe
