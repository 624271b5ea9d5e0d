// Device helpers shared by the bf16 kernels (the prefill in fwd_bf16.hip and
// fwd_gda3_bf16.hip, the backward in bwd_ring_bf16.hip): the global->LDS tile
// DMA, load-counter waits, opaque lane offsets, the transposed-score row
// reductions and the block weights of the lazy-reference online softmax.
// Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace da {
namespace fwdc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) int lds_i32;

// LDS accesses through address-space-3 byte pointers (32-bit arithmetic; a
// pointer plus a constant folds into the instruction's offset field)
__device__ __forceinline__ bf16x8 lds_ld16(const lds_u8* a) { return *(const lds_bf16x8*)a; }
__device__ __forceinline__ void lds_st16(lds_u8* a, const bf16x8& v) { *(lds_bf16x8*)a = v; }
__device__ __forceinline__ bf16x4 lds_ld_tr8(const lds_u8* a) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)a);
}
__device__ __forceinline__ float lds_ldf(const lds_u8* a) { return *(const lds_f32*)a; }
__device__ __forceinline__ void lds_stf(lds_u8* a, float v) { *(lds_f32*)a = v; }
__device__ __forceinline__ int lds_ldi(const lds_u8* a) { return *(const lds_i32*)a; }
__device__ __forceinline__ void lds_sti(lds_u8* a, int v) { *(lds_i32*)a = v; }

// 16 bytes per lane from gbase + goff straight into LDS: lane l writes LDS bytes
// [lds + 16 l, lds + 16 l + 16).  Issued as inline assembly so the compiler does
// not order the ring's LDS reads behind these loads; completion is awaited
// explicitly (s_waitcnt vmcnt + barrier) before a slot is read.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t goff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(goff), "s"(gbase), "s"(lds)
               : "memory");
}
// A per-step lane address made opaque to the compiler, so that the constant
// parts of the reads that use it (row steps, tensors of a stage) stay in the
// instructions' offset fields instead of being hoisted into one register each.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lds_and_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Entry i (wavefront-uniform) of a 4-byte-aligned int16 table in the kernel
// arguments, through a 4-byte scalar load: a 2-byte element would be fetched
// by a vector load, which the ring's load-counter waits would then include.
__device__ __forceinline__ int arg16(const int16_t* table, int i) {
  const int w = ((const int*)table)[i >> 1];
  return (int)(int16_t)((i & 1) ? (w >> 16) : w);
}

// maxima are NaN-propagating (v_maximum3_f32): no operand canonicalisation
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float max16(const f32x16& s) {
  const float a = vmax(vmax(s[0], s[1]), s[2]), b = vmax(vmax(s[3], s[4]), s[5]);
  const float c = vmax(vmax(s[6], s[7]), s[8]), d = vmax(vmax(s[9], s[10]), s[11]);
  const float e = vmax(vmax(s[12], s[13]), s[14]);
  return vmax(vmax(vmax(a, b), c), vmax(vmax(d, e), s[15]));
}

// bf16 weights 2^(s sc - m) of a block as the P^T operands of its two 16-key
// P.V steps; returns the sum of this lane's 16 bf16-rounded weights
// (v_dot2_f32_bf16 against (1, 1)), i.e. exactly what the P.V product uses.
__device__ __forceinline__ float block_weights(const f32x16& s, float sc, float m, bf16x8& p0, bf16x8& p1) {
  float pr[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sc, -m));
  const f32x8 lo = {pr[0], pr[1], pr[2], pr[3], pr[4], pr[5], pr[6], pr[7]};
  const f32x8 hi = {pr[8], pr[9], pr[10], pr[11], pr[12], pr[13], pr[14], pr[15]};
  p0 = __builtin_convertvector(lo, bf16x8);
  p1 = __builtin_convertvector(hi, bf16x8);
  const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
  float t0 = 0.f, t1 = 0.f;
  t0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p0, p0, 0, 1), one2, t0, false);
  t1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p1, p1, 0, 1), one2, t1, false);
  t0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p0, p0, 2, 3), one2, t0, false);
  t1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p1, p1, 2, 3), one2, t1, false);
  t0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p0, p0, 4, 5), one2, t0, false);
  t1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p1, p1, 4, 5), one2, t1, false);
  t0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p0, p0, 6, 7), one2, t0, false);
  t1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p1, p1, 6, 7), one2, t1, false);
  return t0 + t1;
}

// S^T[r] of lane (q, half) is key k0 + 4 half + 8 (r/4) + r%4; keys past lim
// (the last key this lane's query sees, relative to k0 + 4 half) are hidden
__device__ __forceinline__ void mask_scores(f32x16& s, int lim) {
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = (8 * (r / 4) + (r & 3) > lim) ? -INFINITY : s[r];
}

// XCD-contiguous work order: workgroup ids congruent mod 8 run on one XCD; the
// ids of XCD x map to the contiguous logical range [x q8 + min(x, r8), ...)
__device__ __forceinline__ int xcd_logical(int bid, int total) {
  const int xcd = bid & 7, q8 = total >> 3, r8 = total & 7;
  return xcd * q8 + min(xcd, r8) + (bid >> 3);
}

}  // namespace fwdc
}  // namespace da
