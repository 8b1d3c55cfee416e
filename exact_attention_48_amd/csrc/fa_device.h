// fa_device.h -- gfx950 device primitives shared by the attention kernels.
//
// MFMA operand/result layouts (checked on gfx950 with an in-bounds probe):
//   v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] * B[16x32]
//     A: lane l holds A[l % 32][8 * (l / 32) + e], e = 0..7
//     B: lane l holds B[8 * (l / 32) + e][l % 32]
//     D: lane l, register r holds D[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32]
//   ds_read_b64_tr_b16 (per group of 16 lanes, each lane addressing 4 bf16):
//     lane i receives element (i % 4) of the vectors addressed by lanes
//     i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4 of its group.
//   v_permlane32_swap(x, x) returns {x[l], x[l ^ 32]} in some order on every lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// v_mfma_f32_32x32x16_bf16 with the register file of each operand fixed by inline asm
// (the compiler would otherwise put every accumulator in AGPRs and copy the
// ones the VALU reads back every tile). The compiler does not see these as
// MFMAs, so their users keep the hazard rules themselves: a VALU write of an
// operand is followed by at least 2 other instructions before the MFMA that
// reads it, and an MFMA result is not read or overwritten by the VALU within
// 19 wait states of the MFMA (mfma_result_wait() pads where nothing else does).
//   acc (VGPR) = A * B (accumulator start 0), B held in AGPRs
__device__ __forceinline__ void mfma_v_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "a"(b));
}
//   acc (VGPR) += A * B, B held in AGPRs
__device__ __forceinline__ void mfma_v(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
}
//   acc (VGPR) = A * B + C, B held in AGPRs, C a VGPR tuple (left unchanged)
__device__ __forceinline__ void mfma_v_init(f32x16& acc, const bf16x8& a, const bf16x8& b, const f32x16& c) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(acc) : "v"(a), "a"(b), "v"(c));
}
//   acc (AGPR) += A * B, A and B in VGPRs
__device__ __forceinline__ void mfma_a(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Every operand in VGPRs (kernels at two waves per SIMD, whose 256 registers
// per wave go to the VGPRs alone; the MFMA rate is the same as with AGPR
// accumulators):
//   acc = A * B (accumulator start 0)
__device__ __forceinline__ void mfma_vv_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
//   acc += A * B
__device__ __forceinline__ void mfma_vv(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// 8-bit MFMA: S^T (VGPR accumulator) from K (A, VGPRs) and Q^T (B, AGPRs), both
// OCP E4M3 (format fields 0), 32 bytes of the contraction per lane and operand.
__device__ __forceinline__ void mfma8_v_first(f32x16& acc, const i32x8& a, const i32x8& b) {
  asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma8_v(f32x16& acc, const i32x8& a, const i32x8& b) {
  asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_result_wait() { asm volatile("s_nop 7\n s_nop 7\n s_nop 7" ::: "memory"); }
// Keeps an asm MFMA result allocated up to this point (a result that is never
// read would otherwise free its registers while the MFMA still writes them).
__device__ __forceinline__ void keep_live(const f32x16& x) { asm volatile("" ::"v"(x)); }

// f(integral_constant<int, i>) for i = B .. E-1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// -inf where the element offset E (a compile-time constant in [0, 64]) is at
// least thr, else x: one compare into VCC and one select, so that masking a tile
// does not build up one SGPR pair per element.
template <int E>
__device__ __forceinline__ float mask_ge(float x, int thr, float ninf) {
  asm("v_cmp_le_i32 vcc, %1, %2\n\tv_cndmask_b32 %0, %0, %3, vcc" : "+v"(x) : "v"(thr), "n"(E), "v"(ninf) : "vcc");
  return x;
}

// Both lanes of the pair (l, l ^ 32) receive max(x[l], x[l ^ 32]).
// Maxima as plain v_max / v_max3. fmaxf on values produced by inline asm
// costs an extra canonicalising v_max per operand; scores are never
// signalling NaNs, so the plain instructions give the same result.
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Both lanes of the pair (l, l ^ 32) receive x[l] + x[l ^ 32].
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bool wave_any(bool p) {
  return __builtin_amdgcn_ballot_w64(p) != 0;
}

// Two floats to packed bf16 (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x2 pack_bf16(float a, float b) {
  bf16x2 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return r;
}

__device__ __forceinline__ bf16x8 cat(const bf16x4& lo, const bf16x4& hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Transposing LDS read (ds_read_b64_tr_b16); `p` is this lane's 8-byte address.
__device__ __forceinline__ bf16x4 lds_read_tr(const void FA_LDS* p) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 FA_LDS*)p);
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 lds_read16(const void FA_LDS* p) {
  return *(const bf16x8 FA_LDS*)p;
}

// HBM -> LDS loads without register staging use the buffer form
// (buffer_load_dword{,x4} ... lds): the global (FLAT-encoded) form makes the
// compiler treat every later LDS read as ordered behind it on the LDS counter,
// so each wait for an operand would drain all reads in flight.
// A buffer descriptor over `base` with no range limit in practice (callers
// keep every offset inside the tensor themselves).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}
// The same for a `base` that is equal in every lane but that the compiler may
// have computed on the vector unit: the address goes through readfirstlane so
// the descriptor is built in scalar registers (otherwise every load that uses
// it is wrapped in a loop over the lanes' distinct values).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc_uniform(const void* base) {
  const unsigned long long a = (unsigned long long)base;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  return buffer_rsrc((const void*)(((unsigned long long)hi << 32) | lo));
}
// A pointer that is equal in every lane, passed through readfirstlane so the
// compiler keeps it (and what is computed from it) in scalar registers.
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const unsigned long long a = (unsigned long long)p;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  return (T*)(((unsigned long long)hi << 32) | lo);
}
// `bytes` (4 or 16) per lane from rsrc + voffset into LDS: the 64 lanes fill
// 64 * bytes of LDS starting at `lds` (wave-uniform), lane i at lds + bytes * i.
__device__ __forceinline__ void buf2lds16(__amdgpu_buffer_rsrc_t rsrc, unsigned voffset, void FA_LDS* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, lds, 16, (int)voffset, 0, 0, 0);
}
__device__ __forceinline__ void buf2lds4(__amdgpu_buffer_rsrc_t rsrc, unsigned voffset, void FA_LDS* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, lds, 4, (int)voffset, 0, 0, 0);
}

// s_waitcnt immediate: at most `vm` vector-memory operations (which include the
// HBM->LDS copies) and no LDS operation of this wave outstanding.
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 15) | (7 << 4) | (0 << 8) | (((vm >> 4) & 3) << 14); }
// Workgroup barrier WITHOUT the memory fence of __syncthreads(): that fence
// waits for every outstanding vector-memory operation, i.e. it would drain the
// HBM->LDS copies still in flight for later tiles. Callers wait explicitly for
// the copies they need (s_waitcnt) before calling this; the memory clobber
// keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

// exp2 on the FMA pipe: exact split x = n + f with n = floor(x), f in [0, 1),
// 2^f from a minimax polynomial (coefficients fitted by gen_exp2_poly.py),
// 2^n applied by v_ldexp_f32. Range handling:
//   x < -125   -> 0 (a masked -inf gives exactly 0, and no result is denormal:
//                 p(f) may be slightly below 1, which would push 2^-126 p(f)
//                 out of the normal range);
//   x >= 128   -> +inf (2^128 is past the float32 range; selected at the end,
//                 since p(0) is slightly below 1);
//   NaN        -> NaN (the clamp is a select, which keeps a NaN where fmaxf
//                 would replace it by the bound, and (int)NaN is 0 on
//                 v_cvt_i32_f32, so v_ldexp_f32 returns the NaN).
#include "exp2_poly_coeffs.h"
__device__ __forceinline__ float exp2_poly(float x) {
  const bool under = x < -125.0f;
  const float xc = under ? -125.0f : x;
  const float n = __builtin_floorf(xc);
  const float f = xc - n;
  float p = kExp2Poly[kExp2PolyDegree];
#pragma unroll
  for (int i = kExp2PolyDegree - 1; i >= 0; --i) p = __builtin_fmaf(p, f, kExp2Poly[i]);
  float r = __builtin_amdgcn_ldexpf(p, (int)n);
  r = x >= 128.0f ? __builtin_inff() : r;
  return under ? 0.0f : r;
}

// XOR swizzle of the 16-byte chunks of row `row` of a bf16 [rows][D] tile in
// LDS (physical chunk = logical chunk ^ lds_swz<D>(row)). Conflict-free for
// both access patterns the kernels use:
//   * 16 consecutive rows, one 16-byte chunk each (ds_read_b128 MFMA operands);
//   * 4 consecutive rows x 4 consecutive chunks (ds_read_b64_tr_b16 groups).
template <int D>
__device__ __forceinline__ int lds_swz(int row) {
  if constexpr (D == 128) {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  } else {
    const int x = row >> 1;   // two 128-byte rows share one 256-byte bank line
    return ((x & 1) << 2) | ((x >> 1) & 3);
  }
}

template <int EXPMODE>
__device__ __forceinline__ float exp2_sel(float x) {
  if constexpr (EXPMODE == 1) return exp2_poly(x);
  else return __builtin_amdgcn_exp2f(x);
}

}  // namespace fa
