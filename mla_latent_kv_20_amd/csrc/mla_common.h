// Shared device helpers for the gfx950 kernels of the MLA decode library.
#pragma once

#include <hip/hip_runtime.h>

#include "rope_spec.h"
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t bf16_bits;

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 <-> fp32.  The narrowing rounds to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ float bf16_to_f32(bf16_bits b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// RoPE of one rotate-half pair (x, y) = (v_k, v_{k+d/2}) at `pos`: rotation by the angle
// pos * f_k, f_k the pair's frequency (rope_spec.h).  The frequency and the angle are fp64
// (angles reach 1e5 rad at long context); the angle is reduced to [-pi, pi] in fp64 (error
// ~1e-11 rad), its sine and cosine taken in fp32 and the rotation done in fp64: ~1e-7
// relative, far below the bf16 and fp32 outputs' rounding.
__device__ __forceinline__ double rope_inv_freq(int k, int d, const RopeSpec& r) {
  const double f = exp(-(2.0 * k / d) * r.log_theta);
  if (!(r.yarn_s > 1.0)) return f;
  const double turns = r.yarn_len * f * 0.15915494309189535;   // turns over the training length
  double g = (turns - r.yarn_alpha) / (r.yarn_beta - r.yarn_alpha);
  g = g < 0.0 ? 0.0 : (g > 1.0 ? 1.0 : g);
  return (1.0 - g) * f / r.yarn_s + g * f;
}
__device__ __forceinline__ void rope_rotate(double& x, double& y, int64_t pos, double inv_freq) {
  const double ang = (double)pos * inv_freq;
  const double red = ang - 6.283185307179586 * rint(ang * 0.15915494309189535);
  float sn, cs;
  sincosf((float)red, &sn, &cs);
  const double nx = x * cs - y * sn;
  const double ny = y * cs + x * sn;
  x = nx;
  y = ny;
}
__device__ __forceinline__ void rope_pair(double& x, double& y, int64_t pos, int k, int d,
                                          const RopeSpec& r) {
  rope_rotate(x, y, pos, rope_inv_freq(k, d, r));
}
__device__ __forceinline__ bf16_bits f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_bits, (__bf16)f);
}
// Two floats -> packed bf16 pair (low half = a), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// D = A x B + C for 32x32x16 bf16 MFMA (gfx950). Lane l holds A[l%32][8(l/32)+j],
// B[8(l/32)+j][l%32] (j = 0..7) and D[8(r/4)+4(l/32)+r%4][l%32] (r = 0..15).
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read: within each 16-lane group, lane i receives element i%4 of
// the 4-element vectors addressed by group lanes i/4, 4+i/4, 8+i/4, 12+i/4.
__device__ __forceinline__ i16x4 lds_read_tr16(const void* lds_ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)lds_ptr);
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)p);
}

// Asynchronous 16-byte global -> LDS copy; lane l's 16 bytes land at LDS address
// lds_base + 16*l (lds_base wave-uniform).  Issued from asm so that the compiler
// does not treat every later LDS read as dependent on it (it would otherwise wait
// for all outstanding loads, including prefetches of later tiles); callers order
// it with wait_vmcnt and lds_barrier.  The instruction writes no VGPR.
__device__ __forceinline__ void global_to_lds16(const void* gptr, uint32_t lds_base) {
  uint32_t saved_m0;
  // M0 is reserved by the compiler, so the block restores it; the load reads M0 at issue.
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved_m0)
      : "v"(gptr), "s"(lds_base)
      : "memory");
}

// As global_to_lds16, addressed as a wave-uniform 64-bit base plus a per-lane 32-bit
// byte offset (the saddr form), so no per-lane 64-bit address arithmetic is needed.
__device__ __forceinline__ void global_to_lds16_sv(const void* sbase, uint32_t voff, uint32_t lds_base) {
  uint32_t saved_m0;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved_m0)
      : "v"(voff), "s"(sbase), "s"(lds_base)
      : "memory");
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Workgroup barrier that also orders LDS traffic: every wave's LDS reads are
// complete before any wave passes.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// max(x[l], x[l ^ 32]) over the two halves of the wave, through v_permlane32_swap:
// swapping a register with itself leaves x[l] in one result and x[l ^ 32] in the other.
__device__ __forceinline__ float pair_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// acc += A . B (v_mfma_f32_32x32x16_bf16) with the accumulator in VGPRs, issued from inline
// assembly so that it stays in VGPRs while the compiler's own MFMAs keep their
// accumulators in the AGPR file.  The compiler does not see this MFMA's latency:
//  - back-to-back calls on the same accumulator need no wait (the MFMA forwards srcC);
//  - a VALU write of the accumulator or operands needs 2 wait states before the call
//    (keep such writes a few instructions away);
//  - before any other instruction reads the accumulator, call mfma_vgpr_drain().
__device__ __forceinline__ void mfma_acc_vgpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

// 12 wait states (what the compiler places between this MFMA and a VALU read of its
// result on gfx950), with the accumulator as an operand so later reads stay behind it.
__device__ __forceinline__ void mfma_vgpr_drain(f32x16& acc) {
  asm volatile("s_nop 11" : "+v"(acc));
}
__device__ __forceinline__ void mfma_vgpr_drain2(f32x16& acc0, f32x16& acc1) {
  asm volatile("s_nop 11" : "+v"(acc0), "+v"(acc1));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// a *= alpha for an MFMA accumulator that lives in AGPRs.  VALU arithmetic cannot
// read AGPRs, so each element goes AGPR -> VGPR -> AGPR inside one asm block; this
// keeps the accumulator's only uses AGPR-compatible, so the register allocator
// never copies the whole accumulator to VGPRs around a loop.
__device__ __forceinline__ void scale_acc_agpr(f32x16& a, float alpha) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float v = a[i];
    float tmp;
    asm volatile(
        "v_accvgpr_read_b32 %1, %0\n\t"
        "v_mul_f32 %1, %1, %2\n\t"
        "v_accvgpr_write_b32 %0, %1"
        : "+a"(v), "=&v"(tmp)
        : "v"(alpha));
    a[i] = v;
  }
}

}  // namespace mla
