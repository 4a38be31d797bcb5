// common.hpp -- device types and helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;   // MI355X: 8 XCDs, workgroups dispatched round-robin over them

// ---- bf16 <-> fp32 (bit level; bf16 kept as uint16_t in memory) -----------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// ---- wave-level reductions (wave64) -------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    unsigned long long w = __shfl_xor(v, o, kWave);
    v = w > v ? w : v;
  }
  return v;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Device-only builtins, wrapped so that the host compilation pass (which only emits kernel launch
// stubs) never sees them in a kernel body.
// 16 bytes per lane from global memory straight into LDS: lane i writes lds_region + 16 * i.
__device__ __forceinline__ void dma_16b(const void* g, void* lds_region) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, lds_region, 16, 0, 0);
#endif
}
// The two inline-assembly forms below write M0, which the compiler reserves. That is sound here
// because nothing in these kernels relies on a compiler-set M0 across them: the only M0 user is the
// direct-to-LDS load, and the compiler sets M0 immediately before each one it emits itself.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// The same load written as inline assembly. The compiler's wait-count pass does not see it, so it
// neither treats it as an LDS access (which makes every LDS-read wait in a loop a full drain) nor
// counts it: the caller owns every vmcnt wait for these loads. M0 holds the wave's LDS base; the
// s_nop covers the M0-write-to-use hazard.
__device__ __forceinline__ void dma_16b_asm(const void* g, const void* lds_region) {
#if defined(__HIP_DEVICE_COMPILE__)
  const unsigned base = __builtin_amdgcn_readfirstlane(
      static_cast<unsigned>(reinterpret_cast<uintptr_t>(lds_region)));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(base), "v"(g) : "memory", "m0");
#endif
}
// 4 bytes per lane from global memory straight into LDS (lane i writes lds_region + 4 * i); like
// dma_16b_asm, invisible to the compiler's wait-count pass.
__device__ __forceinline__ void dma_4b_asm(const void* g, const void* lds_region) {
#if defined(__HIP_DEVICE_COMPILE__)
  const unsigned base = __builtin_amdgcn_readfirstlane(
      static_cast<unsigned>(reinterpret_cast<uintptr_t>(lds_region)));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :: "s"(base), "v"(g) : "memory", "m0");
#endif
}
// The same load with a scalar base address and a 32-bit per-lane byte offset, and the LDS target
// given as a wave-uniform byte address for M0. A K loop then advances the scalar base only, so the
// loads cost no per-lane address arithmetic (vector ALU instructions in the loop take issue cycles
// from the MFMAs of the same SIMD).
__device__ __forceinline__ void dma_16b_sbase(const void* sbase, unsigned voff, unsigned lds_addr) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds_addr), "v"(voff), "s"(sbase) : "memory", "m0");
#endif
}
#pragma clang diagnostic pop
// s_waitcnt vmcnt(0): all of this wave's vector memory loads (including LDS DMA) have completed
__device__ __forceinline__ void wait_vmem() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt(0x0F70);
#endif
}
// s_waitcnt lgkmcnt(0): all of this wave's LDS (and scalar memory) reads have completed
__device__ __forceinline__ void wait_lgkm() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt(0xC07F);
#endif
}
// Workgroup barrier for LDS filled by dma_16b. __syncthreads() carries a workgroup memory fence,
// which makes every wave drain ALL of its outstanding LDS DMA first; a pipelined K loop only needs
// the stage it is about to read. Callers therefore wait for that stage's DMA explicitly
// (wait_vmem_n) and then use this plain hardware barrier; the empty asm statements with memory
// clobbers keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// scheduling hint: `count` instructions of class `mask` (0x008 MFMA, 0x100 DS read, ...) next
#define MOE_SCHED_GROUP(mask, count) __builtin_amdgcn_sched_group_barrier((mask), (count), 0)
// no instruction is scheduled across this point
#define MOE_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Workgroup order -> logical tile order: consecutive groups of `span` logical tiles run on one XCD
// (so tiles sharing an operand share that XCD's L2), while consecutive spans rotate over the XCDs.
// `total` must be a multiple of kNumXcd * span.
__device__ __forceinline__ int xcd_remap(int bid, int span) {
  int blk = kNumXcd * span;
  int base = (bid / blk) * blk;
  int r = bid - base;
  return base + (r % kNumXcd) * span + (r / kNumXcd);
}

}  // namespace moe
