// route.hip -- scores, top-k and routing weights on gfx950.
//
// One wave64 per token. Each lane holds ceil(E/64) logits as order-preserving u32 codes of the
// fp32 values (-0.0 canonicalised to +0.0 first so the two compare equal; 0 marks a padding or an
// already chosen entry). Each of k rounds takes the wave-wide maximum code and, among the entries
// holding it, the lowest expert id (the tie rule of the tiny workload): one ballot per register
// of codes, the first nonzero one giving the expert. The rounds pick the experts in rank order.
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
// code of a real entry: never 0 (only the negative NaN with every bit set maps to 0; it becomes
// the next NaN code)
__device__ __forceinline__ uint32_t entry_code(float f) {
  const uint32_t o = ordered_bits(f);
  return o > 1u ? o : 1u;
}
// wave-wide maximum: within each row of 16 lanes by DPP (quad swaps, then row rotations by 4 and
// 8), then the four rows' maxima through scalar registers
__device__ __forceinline__ uint32_t wave_max_code(uint32_t v) {
  auto dmax = [](uint32_t x, auto ctrl) {
    const uint32_t y = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(x), decltype(ctrl)::value, 0xF, 0xF, false));
    return x > y ? x : y;
  };
  v = dmax(v, std::integral_constant<int, 0xB1>{});
  v = dmax(v, std::integral_constant<int, 0x4E>{});
  v = dmax(v, std::integral_constant<int, 0x124>{});
  v = dmax(v, std::integral_constant<int, 0x128>{});
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  const uint32_t a = r0 > r1 ? r0 : r1, b = r2 > r3 ? r2 : r3;
  return a > b ? a : b;
}

// With nsplit > 1 the logits are first formed from the router's K-split partial sums
// (partial[s][t][e], s ascending, then the bias) and written to `logits`; the selection then uses
// exactly the values written.
template <int VPL>
__global__ void __launch_bounds__(256) topk_kernel(int T, int E, int k, int scoring, int renorm,
                                                   float* __restrict__ logits,
                                                   const float* __restrict__ partial, int nsplit,
                                                   const float* __restrict__ bias,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;                       // uniform per wave
  const int lane = threadIdx.x & 63;
  float* L = logits + (size_t)t * E;

  uint32_t code[VPL];
  float val[VPL];
  // every logit load is issued before the first is used (clamped to the last expert, never
  // guarded: a guarded load became a branch with a full wait after each one)
  if (nsplit <= 1) {
#pragma unroll
    for (int v = 0; v < VPL; ++v) val[v] = L[min(v * 64 + lane, E - 1)];
  }
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    if (v * 64 + lane < E) {
      if (nsplit > 1) val[v] = 0.0f;
      code[v] = entry_code(val[v]);
    } else {
      val[v] = 0.0f;
      code[v] = 0u;                         // below every real entry
    }
  }

  if (nsplit > 1) {
    // logits from the router's K-split partials, added in slice order (then the bias); a batch of
    // partials of every value is loaded before any is added so that their latencies overlap
    constexpr int BATCH = VPL <= 2 ? 16 : (VPL <= 4 ? 8 : 4);
    const size_t stride = (size_t)T * E;
    const float* pp = partial + (size_t)t * E;
    for (int sp0 = 0; sp0 < nsplit; sp0 += BATCH) {
      float pv[VPL][BATCH];
      // unconditional loads (clamped indices): a predicated load becomes a branch that the
      // wait-count pass must drain at
#pragma unroll
      for (int v = 0; v < VPL; ++v)
#pragma unroll
        for (int q = 0; q < BATCH; ++q)
          pv[v][q] = pp[min(sp0 + q, nsplit - 1) * stride + min(v * 64 + lane, E - 1)];
#pragma unroll
      for (int v = 0; v < VPL; ++v)
#pragma unroll
        for (int q = 0; q < BATCH; ++q)
          if (sp0 + q < nsplit) val[v] = (sp0 + q == 0) ? pv[v][q] : val[v] + pv[v][q];
    }
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = v * 64 + lane;
      if (e < E) {
        if (bias) val[v] += bias[e];
        L[e] = val[v];
        code[v] = entry_code(val[v]);
      }
    }
  }

  float my_l = 0.0f, top_l = 0.0f;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t m = code[0];
#pragma unroll
    for (int v = 1; v < VPL; ++v) m = code[v] > m ? code[v] : m;
    const uint32_t best = wave_max_code(m);            // wave-uniform, >= 1 while j < k <= E
    // lowest expert holding the best code: the registers from last to first, the last nonzero
    // ballot (lowest register) deciding, its lowest lane within it
    int e = 0;
#pragma unroll
    for (int v = VPL - 1; v >= 0; --v) {
      const unsigned long long b = __ballot(code[v] == best);
      e = b != 0ull ? v * 64 + static_cast<int>(__builtin_ctzll(b)) : e;
    }
    e = __builtin_amdgcn_readfirstlane(e);
    const float l = from_ordered(best);
    if (j == 0) top_l = l;
    if (lane == j) { my_l = l; my_e = e; }
    // clear the chosen entry: a compare per register, or (16 registers) one indexed register
    // access through the uniform register index
    if constexpr (VPL >= 16) {
      const int vw = e >> 6;
      code[vw] = lane == (e & 63) ? 0u : code[vw];
    } else {
      const int el = e - lane;                                    // v * 64 in the owning lane
#pragma unroll
      for (int v = 0; v < VPL; ++v) code[v] = el == v * 64 ? 0u : code[v];
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

hipError_t launch_topk(int T, int E, int k, int scoring, int renormalize, float* logits,
                       const float* partial, int nsplit, const float* bias, int32_t* ids, float* w,
                       hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((T + 3) / 4), block(256);
  int vpl = (E + 63) / 64;
#define MOE_TOPK(V) \
  topk_kernel<V><<<grid, block, 0, s>>>(T, E, k, scoring, renormalize, logits, partial, nsplit, bias, ids, w)
  if (vpl <= 1) MOE_TOPK(1);
  else if (vpl <= 2) MOE_TOPK(2);
  else if (vpl <= 4) MOE_TOPK(4);
  else if (vpl <= 8) MOE_TOPK(8);
  else MOE_TOPK(16);
#undef MOE_TOPK
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// Router logits, bf16: L[t, e] = sum_h x[t, h] * W_r[e, h] (+ bias[e]) with fp32 accumulation.
//
// The router is a skinny GEMM (E = 128..512 output columns) whose shape swings from 64 tokens
// (decode: a 1-8 MB weight read) to 16K tokens. One wave owns 16 * FT tokens x 64 experts over one
// slice of K; the slices (K-split) multiply the number of waves when there are few tokens, and
// their fp32 partial sums are added in slice order by the top-k kernel, so the result does not
// depend on timing. The router weight is the MFMA's first operand, so each lane's accumulator
// fragment holds four consecutive experts of one token (16-byte stores). Operands go from global
// memory straight into registers in double-buffered chunks of D K-steps; loads are unconditional
// (clamped to the slice and to the last token / expert), only the MFMAs past the slice's end are
// skipped.
// ------------------------------------------------------------------------------------------------
template <int FT, int D>
__global__ void __launch_bounds__(256)
router_kernel(int T, int H, int E, const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
              const float* __restrict__ bias, float* __restrict__ out, int n_tb, int n_eb,
              int nsplit, int kps) {
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= n_tb * n_eb * nsplit) return;             // uniform per wave
  const int eb = wid % n_eb;
  const int rest = wid / n_eb;
  const int tb = rest % n_tb, sp = rest / n_tb;
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, kq = lane >> 4;
  const int k0 = sp * kps;                              // first K-step (32 elements) of the slice

  const uint16_t* wp[4];
  const uint16_t* xp[FT];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = min(eb * 64 + j * 16 + lr, E - 1);
    wp[j] = wr + (size_t)e * H + k0 * 32 + kq * 8;
  }
#pragma unroll
  for (int i = 0; i < FT; ++i) {
    const int t = min(tb * 16 * FT + i * 16 + lr, T - 1);
    xp[i] = x + (size_t)t * H + k0 * 32 + kq * 8;
  }
  // chunks of D K-steps, double-buffered (loads of chunk c + 1 before the MFMAs of chunk c; the
  // chunk loop is unrolled by two so the register sets alternate statically, and scheduling
  // barriers keep the loads where they are written)
  bf16x8 wv[2][D][4], xv[2][D][FT];
  auto load = [&](int c, int set) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int off = min(c * D + d, kps - 1) * 32;
#pragma unroll
      for (int j = 0; j < 4; ++j) wv[set][d][j] = *reinterpret_cast<const bf16x8*>(wp[j] + off);
#pragma unroll
      for (int i = 0; i < FT; ++i) xv[set][d][i] = *reinterpret_cast<const bf16x8*>(xp[i] + off);
    }
  };
  f32x4 acc[4][FT];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < FT; ++i) acc[j][i] = f32x4{};
  auto compute = [&](int c, int set) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (c * D + d < kps) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < FT; ++i)
            acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv[set][d][j], xv[set][d][i], acc[j][i], 0, 0, 0);
      }
    }
  };
  const int nc = (kps + D - 1) / D;
  load(0, 0);
  for (int c = 0; c < nc; c += 2) {
    MOE_SCHED_FENCE();
    load(c + 1, 1);
    MOE_SCHED_FENCE();
    compute(c, 0);
    MOE_SCHED_FENCE();
    load(c + 2, 0);
    MOE_SCHED_FENCE();
    compute(c + 1, 1);
  }
  MOE_SCHED_FENCE();
  // acc[j][i][v]: expert eb * 64 + j * 16 + kq * 4 + v, token tb * 16 FT + i * 16 + lr
  float* dst = nsplit > 1 ? out + (size_t)sp * T * E : out;
#pragma unroll
  for (int i = 0; i < FT; ++i) {
    const int t = tb * 16 * FT + i * 16 + lr;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = eb * 64 + j * 16 + kq * 4;
      if (e >= E) continue;                             // E % 16 == 0: all four or none
      f32x4 v = acc[j][i];
      if (nsplit == 1 && bias) {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] += bias[e + q];
      }
      *reinterpret_cast<f32x4*>(dst + (size_t)t * E + e) = v;
    }
  }
}

namespace {
// K-split until the router has about one wave per CU: more slices give more waves but more fp32
// partials for the top-k kernel to add (decode slices, two reps, 1024 / 2048 / 4096 waves:
// 64-token Qwen3-235B 0.2346-0.2351 / 0.2355-0.2362 / 0.2354-0.2361 ms, 256-token DeepSeek-V3
// fp8 0.3118-0.3130 / 0.3153-0.3173 / 0.3137-0.3155 ms)
constexpr int kRouterMinWaves = 1024;
constexpr int kRouterMaxSplit = 32;
int router_ft(int T) { return T >= 1024 ? 4 : 1; }
}  // namespace

int router_splits(int T, int H, int E) {
  if (T <= 0) return 1;
  const int ft = router_ft(T);
  const long long base = (long long)((T + 16 * ft - 1) / (16 * ft)) * ((E + 63) / 64);
  const int nk = H / 32;
  int ns = 1;
  while (ns < kRouterMaxSplit && base * ns < kRouterMinWaves && nk % (ns * 2) == 0) ns *= 2;
  return ns;
}

size_t router_ws_bytes(int T, int H, int E) {
  const int ns = router_splits(T, H, E);
  return ns > 1 ? (size_t)ns * T * E * sizeof(float) : 0;
}

hipError_t launch_router(int T, int H, int E, const void* x, const void* w_router,
                         const float* bias, float* logits, float* partial, int nsplit,
                         hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int ft = router_ft(T);
  const int n_tb = (T + 16 * ft - 1) / (16 * ft), n_eb = (E + 63) / 64;
  const int kps = H / 32 / nsplit;
  const long long waves = (long long)n_tb * n_eb * nsplit;
  dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  float* out = nsplit > 1 ? partial : logits;
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* wb = static_cast<const uint16_t*>(w_router);
  if (ft == 4)
    router_kernel<4, 2><<<grid, block, 0, s>>>(T, H, E, xb, wb, bias, out, n_tb, n_eb, nsplit, kps);
  else
    router_kernel<1, 2><<<grid, block, 0, s>>>(T, H, E, xb, wb, bias, out, n_tb, n_eb, nsplit, kps);
  return hipGetLastError();
}

// Gate of the shared expert ("Hosting Qwen on Blackwell", introduction: the layer adapts to the
// newer models' additional gate terms; read as g_t = 1 / (1 + exp(-(x_t . w_sg))) on the
// unquantised token). One wave per token, four tokens per workgroup: each lane loads 16 bytes of
// x_t and of w_sg per step (8 bf16 or 4 fp32 columns), accumulates in fp32, and the wave sums
// the lanes. x and w_sg are read once; H % 8 == 0.
template <bool BF16>
__global__ void __launch_bounds__(256) shared_gate_kernel(int T, int H, const void* __restrict__ x,
                                                          const void* __restrict__ wsg,
                                                          float* __restrict__ g) {
  constexpr int CPL = BF16 ? 8 : 4;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;                                   // whole waves leave together
  float acc = 0.0f;
  for (int c = lane * CPL; c < H; c += 64 * CPL) {
    if (BF16) {
      const i32x4 a = *reinterpret_cast<const i32x4*>(static_cast<const uint16_t*>(x) + (size_t)t * H + c);
      const i32x4 b = *reinterpret_cast<const i32x4*>(static_cast<const uint16_t*>(wsg) + c);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t ua = static_cast<uint32_t>(a[q]), ub = static_cast<uint32_t>(b[q]);
        acc = fmaf(__uint_as_float(ua << 16), __uint_as_float(ub << 16), acc);
        acc = fmaf(__uint_as_float(ua & 0xFFFF0000u), __uint_as_float(ub & 0xFFFF0000u), acc);
      }
    } else {
      const f32x4 a = *reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + (size_t)t * H + c);
      const f32x4 b = *reinterpret_cast<const f32x4*>(static_cast<const float*>(wsg) + c);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc = fmaf(a[q], b[q], acc);
    }
  }
  acc = wave_sum(acc);
  if (lane == 0) g[t] = 1.0f / (1.0f + expf(-acc));
}

hipError_t launch_shared_gate(int T, int H, int io_dtype, const void* x, const void* w_sg, float* g,
                              hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((T + 3) / 4), block(256);
  if (io_dtype == MOE_BF16) shared_gate_kernel<true><<<grid, block, 0, s>>>(T, H, x, w_sg, g);
  else shared_gate_kernel<false><<<grid, block, 0, s>>>(T, H, x, w_sg, g);
  return hipGetLastError();
}

}  // namespace moe
