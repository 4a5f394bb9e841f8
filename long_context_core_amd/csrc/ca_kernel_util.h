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

// A struct of 32-bit words that every lane loaded from the same address,
// moved to scalar registers.  Needed where the load cannot be a scalar load
// (the kernel has already stored to global memory, so the compiler cannot
// prove the data unchanged): without it every value derived from the struct
// lives in vector registers and each scalar use (buffer descriptors, loop
// bounds) pays a readfirstlane.
template <class T>
__device__ __forceinline__ T wave_uniform(const T& v) {
  static_assert(sizeof(T) % 4 == 0, "whole 32-bit words");
  T r;
  const int32_t* src = reinterpret_cast<const int32_t*>(&v);
  int32_t* dst = reinterpret_cast<int32_t*>(&r);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 4); ++i) dst[i] = __builtin_amdgcn_readfirstlane(src[i]);
  return r;
}

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
// Only the per-lane offset is relied on for that check: a tile is addressed
// by moving the base, and the scalar offset of the loads stays 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Resource over n rows (n <= 0: none) that start at row0_ptr and lie
// row_bytes apart; loads of rows >= n return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* row0_ptr, int n, uint32_t row_bytes) {
  return make_rsrc(row0_ptr, n > 0 ? (uint32_t)n * row_bytes : 0u);
}

__device__ __forceinline__ uint4 buffer_load_16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}

// The same load with the nontemporal hint, for data read exactly once
// (streamed K/V caches): measured on a 2 GiB streaming read, 7.2 TB/s with
// the hint against 6.3 TB/s without.
__device__ __forceinline__ uint4 buffer_load_16_stream(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2 /* nt */);
  return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}

__device__ __forceinline__ float buffer_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// Value of lane l and of lane l ^ 32 combined (v_permlane32_swap, no LDS).
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x8 concat_bf16x4(bf16x4 lo, bf16x4 hi) {
  bf16x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

typedef float f32x4v __attribute__((ext_vector_type(4)));

// One chunk of partials into the running Equation-4 state (M: running max,
// den: sum of weights relative to M, out: weighted sum of O's); partials
// with LSE = -inf carry weight 0.
template <int VEC, int CHUNK>
__device__ __forceinline__ void merge_chunk(const float (&l)[CHUNK], const f32x4v (&x)[CHUNK][VEC], float& M,
                                            float& den, float4 (&out)[VEC]) {
  float mc = M;
#pragma unroll
  for (int k = 0; k < CHUNK; ++k) mc = fmaxf(mc, l[k]);
  if (mc == -INFINITY) return;
  if (mc != M) {
    const float a = (M == -INFINITY) ? 0.f : __expf(M - mc);
    den *= a;
#pragma unroll
    for (int v = 0; v < VEC; ++v) { out[v].x *= a; out[v].y *= a; out[v].z *= a; out[v].w *= a; }
    M = mc;
  }
#pragma unroll
  for (int k = 0; k < CHUNK; ++k) {
    const float w = (l[k] == -INFINITY) ? 0.f : __expf(l[k] - M);
    den += w;
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      out[v].x = fmaf(w, x[k][v][0], out[v].x);
      out[v].y = fmaf(w, x[k][v][1], out[v].y);
      out[v].z = fmaf(w, x[k][v][2], out[v].z);
      out[v].w = fmaf(w, x[k][v][3], out[v].w);
    }
  }
}

// Final O = out / den and LSE = M + ln den (0 and -inf if every LSE was -inf).
template <int VEC>
__device__ __forceinline__ float merge_finish(float M, float den, float4 (&out)[VEC]) {
  const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
  for (int v = 0; v < VEC; ++v) { out[v].x *= inv; out[v].y *= inv; out[v].z *= inv; out[v].w *= inv; }
  return den > 0.f ? M + __logf(den) : -INFINITY;
}

// Log-sum-exp merge of n partial results of one (row, head) ("Context
// Parallelism for Scalable Million-Token Inference", Section 3.4, Equation 4):
//   M = max_s LSE_s,  O = sum_s e^(LSE_s - M) O_s / sum_s e^(LSE_s - M),
//   LSE = M + ln sum_s e^(LSE_s - M).
// The calling lane owns VEC float4s of the row, at o + v * (D / VEC) of each
// partial; partial s sits at lse[s * lse_stride] and o + s * o_stride.  A
// partial with LSE = -inf is skipped without reading its O.  Eight partials'
// LSEs and O's are loaded together; earlier chunks are rescaled when the
// running maximum grows.  out receives the merged O (0 if every LSE is -inf);
// the merged LSE is returned (-inf then).
template <int D, int VEC>
__device__ __forceinline__ float merge_lse_parts(const float* lse, int64_t lse_stride, const float* o,
                                                 int64_t o_stride, int n, float4 (&out)[VEC]) {
  constexpr int CHUNK = 8;
  float M = -INFINITY, den = 0.f;
#pragma unroll
  for (int v = 0; v < VEC; ++v) out[v] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < n; s0 += CHUNK) {
    float l[CHUNK];
    f32x4v x[CHUNK][VEC];
#pragma unroll
    for (int k = 0; k < CHUNK; ++k) l[k] = s0 + k < n ? lse[(s0 + k) * lse_stride] : -INFINITY;
    // partials are read once: nontemporal loads
#pragma unroll
    for (int k = 0; k < CHUNK; ++k)
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        x[k][v] = f32x4v{0.f, 0.f, 0.f, 0.f};
        if (l[k] != -INFINITY) x[k][v] = __builtin_nontemporal_load((const f32x4v*)(o + (s0 + k) * o_stride + v * (D / VEC)));
      }
    merge_chunk<VEC, CHUNK>(l, x, M, den, out);
  }
  return merge_finish<VEC>(M, den, out);
}

// Store VEC float4s (at dst + v * (D / VEC)) as fp32 or rounded to bf16.  The
// merged rows are written once and not read back by the kernel: nontemporal
// stores (on the 5.4 GB ring merge, 6.0 TB/s against 5.5 TB/s with plain
// stores; without the LSE round trip, plain stores reach only 5.7).
template <int D, int VEC>
__device__ __forceinline__ void store_row_part(void* O, int64_t base, bool f32, const float4 (&r)[VEC]) {
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    const int64_t at = base + v * (D / VEC);
    if (f32) {
      __builtin_nontemporal_store(f32x4v{r[v].x, r[v].y, r[v].z, r[v].w}, (f32x4v*)((float*)O + at));
    } else {
      bf16x4 b;
      b[0] = (__bf16)r[v].x; b[1] = (__bf16)r[v].y; b[2] = (__bf16)r[v].z; b[3] = (__bf16)r[v].w;
      __builtin_nontemporal_store(b, (bf16x4*)((__bf16*)O + at));
    }
  }
}

}  // namespace ca
