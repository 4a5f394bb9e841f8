// Device-side vector types and small helpers for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ca {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 f32x16_zero() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ f32x4 f32x4_zero() {
  f32x4 z;
#pragma unroll
  for (int i = 0; i < 4; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ bf16x8 bf16x8_zero() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.f;
  return z;
}

__device__ __forceinline__ int64_t clamp64(int64_t x, int64_t lo, int64_t hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

// Marks a rarely taken, wave-uniform branch body as having a side effect so
// the compiler keeps it as a branch instead of executing it unconditionally
// under a select.
__device__ __forceinline__ void keep_branch() { asm volatile("" ::: "memory"); }

// 2^x on the hardware transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives element i % 4 of the 8-byte rows addressed by lanes
// i / 4, i / 4 + 4, i / 4 + 8 and i / 4 + 12 (in that order).
__device__ __forceinline__ bf16x4 ds_read_tr16(const __bf16* lds_ptr) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(lds_ptr));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource over [base, base + bytes): loads past the end return 0
// (hardware range check), which zero-fills ragged tiles without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buffer_load_16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}

// 16 bytes per lane from a raw buffer straight into LDS (no registers): lane i
// of the wave writes lds_block + 16 i; lds_block must be wave-uniform.
__device__ __forceinline__ void buffer_load_lds_16(__amdgpu_buffer_rsrc_t r, void* lds_block, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_block, 16, voff, soff, 0, 0);
}

// Wait for this wave's outstanding vector-memory operations (including loads
// into LDS); other counters untouched.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Value of lane l and of lane l ^ 32 combined (v_permlane32_swap, no LDS).
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// sum of the 8 bf16 values of v, accumulated into acc in fp32 (v_dot2 with 1s)
__device__ __forceinline__ float sum_bf16x8(bf16x8 v, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[0], v[1]}, one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[2], v[3]}, one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[4], v[5]}, one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[6], v[7]}, one, acc, false);
  return acc;
}

__device__ __forceinline__ bf16x8 concat_bf16x4(bf16x4 lo, bf16x4 hi) {
  bf16x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

}  // namespace ca
