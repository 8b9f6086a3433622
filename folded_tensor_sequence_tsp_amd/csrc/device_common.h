// Device helpers shared by the gfx950 kernels of libtsp: vector types for the
// MFMA operands, bf16 rounding and the tanh-form GELU in fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float F16_MAX = 65504.0f;

// fp32 -> bf16 bits with the hardware conversion (v_cvt_pk_bf16_f32, round to
// nearest even).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two fp32 -> packed bf16x2 (low half = a) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Two fp32 -> packed fp16x2 (low half = a), round to nearest even, saturated
// to the finite fp16 range (one v_cvt_pk_f16_f32 after the clamps).
__device__ __forceinline__ uint32_t pack_f16x2_sat(float a, float b) {
  f16x2 v;
  v[0] = (_Float16)fminf(fmaxf(a, -F16_MAX), F16_MAX);
  v[1] = (_Float16)fminf(fmaxf(b, -F16_MAX), F16_MAX);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// GELU, tanh form: 0.5 u (1 + tanh(z)) with z = sqrt(2/pi) (u + 0.044715 u^3).
// With r = 1 / (1 + exp(2z)), 1 + tanh(z) = 2 (1 - r), so GELU(u) = u - u r,
// one fma; exp(2z) = 2^(u (k1 + k2 u^2)) on the hardware exp2, with
// k1 = 2 log2(e) sqrt(2/pi) and k2 = 0.044715 k1.  Saturates for finite u:
// exp2 -> inf gives r = 0 (GELU = u), exp2 -> 0 gives r = 1 (GELU = 0).
__device__ __forceinline__ float gelu_tanh(float u) {
  const float k1 = 2.30220819814432488913f, k2 = 0.10294323958002348742f;
  const float e = __builtin_amdgcn_exp2f(u * __builtin_fmaf(k2, u * u, k1));
  const float r = __builtin_amdgcn_rcpf(e + 1.0f);
  return __builtin_fmaf(-u, r, u);
}

// Derivative of gelu_tanh: 0.5 (1 + t) + 0.5 u (1 - t^2) c (1 + 3 a u^2) with
// t = tanh(c (u + a u^3)), c = sqrt(2/pi), a = 0.044715; t from the same exp2
// form as gelu_tanh.
__device__ __forceinline__ float gelu_tanh_grad(float u) {
  const float c = 0.79788456080286535588f, a = 0.044715f;
  const float two_log2e = 2.88539008177792681472f;
  const float z = c * (u + a * u * u * u);
  const float e = __builtin_amdgcn_exp2f(two_log2e * z);
  const float t = 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
  return 0.5f * (1.0f + t) + 0.5f * u * (1.0f - t * t) * c * (1.0f + 3.0f * a * u * u);
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32_f16(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ f16x8 as_f16x8(const u32x4& v) { return __builtin_bit_cast(f16x8, v); }

// 32x32x16 MFMA on 16-bit operands given as raw bits: fp16 when F16, else bf16.
template <bool F16>
__device__ __forceinline__ f32x16 mfma32_bits(const u32x4& a, const u32x4& b, const f32x16& c) {
  if constexpr (F16)
    return mfma32_f16(as_f16x8(a), as_f16x8(b), c);
  else
    return mfma32(as_bf16x8(a), as_bf16x8(b), c);
}

// max of x over the lane pair (l, l xor 32), one v_permlane32_swap (gfx950):
// with both operands x, the swap leaves (x_lo | x_lo) and (x_hi | x_hi).
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// ---- direct global->LDS loads and their synchronisation (shared by the kernels).
// s_waitcnt vmcnt(N) alone (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Direct global->LDS load of 16 bytes per lane (global_load_lds_dwordx4): lane L
// of the wave writes its 16 bytes at lds_block + 16 * L; lds_block is wave-uniform.
__device__ __forceinline__ void dma16(const void* src, void* lds_block) {
  __builtin_amdgcn_global_load_lds(const_cast<void*>(src), (__attribute__((address_space(3))) void*)lds_block, 16,
                                   0, 0);
}

// Buffer resource (V#) over `bytes` bytes from `base` (raw buffer: stride 0;
// offsets at or past `bytes` read as zero).  Built from SGPRs when the
// arguments are wave-uniform, so rebasing it per tile is scalar work.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Direct buffer->LDS load of 16 bytes per lane (buffer_load_dwordx4 ... lds):
// lane L reads rsrc + voffset + soffset (soffset wave-uniform, in an SGPR) and
// writes its 16 bytes at lds_block + 16 * L; lds_block is wave-uniform.
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t rsrc, uint32_t voffset, void* lds_block,
                                          uint32_t soffset = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds_block, 16, voffset,
                                           soffset, 0, 0);
}

// Transposing LDS read of four 16-bit values per lane (ds_read_b64_tr_b16,
// gfx950).  Within each group of 16 lanes, lane 4m + q names 8 bytes (four
// consecutive 16-bit columns of one row, row m of the group's four rows), and
// lane j receives column j of the group's 16 columns from rows m = 0..3, in
// order: a 4 x 16 block of rows comes back as 16 columns of 4.
__device__ __forceinline__ u32x2 lds_read_tr16x4(const void* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p));
}

// Workgroup barrier that the compiler may not move memory operations across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace tsp
