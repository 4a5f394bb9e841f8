// K2 — merge of partial attention results by their log-sum-exp
// ("Context Parallelism for Scalable Million-Token Inference", Section 3.4
// Merge Attention, Equation 4, Appendix B):
//   M = max_s LSE_s,  O = sum_s O_s e^(LSE_s - M) / sum_s e^(LSE_s - M),
//   LSE = M + ln sum_s e^(LSE_s - M).
// HBM-bound: each (row, head) is D / 4 lanes holding one float4 of every
// partial; a partial with LSE = -inf is skipped without reading its O.

#include "ca_internal.h"
#include "ca_kernel_util.h"

namespace ca {

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  constexpr int LPP = D / 4;                    // lanes per (row, head)
  constexpr int CHUNK = 8;                      // partials loaded together
  const int64_t n_pairs = p.n_rows * p.hq;
  const int64_t pair = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPP;
  const int sub = threadIdx.x % LPP;
  if (pair >= n_pairs) return;
  const int64_t part_stride_o = n_pairs * D;    // floats per partial
  const float* lse = p.LSE_parts + pair;
  const float* op = p.O_parts + pair * D + sub * 4;
  float M = -INFINITY;
  for (int s = 0; s < p.n_parts; ++s) M = fmaxf(M, lse[s * n_pairs]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.f;
  if (M != -INFINITY) {
    for (int s0 = 0; s0 < p.n_parts; s0 += CHUNK) {
      float w[CHUNK];
      float4 o[CHUNK];
#pragma unroll
      for (int k = 0; k < CHUNK; ++k) {       // all loads of the chunk first
        const int s = s0 + k;
        const float l = s < p.n_parts ? lse[s * n_pairs] : -INFINITY;
        w[k] = (l == -INFINITY) ? 0.f : __expf(l - M);
        o[k] = (l == -INFINITY) ? make_float4(0.f, 0.f, 0.f, 0.f)
                                : *(const float4*)(op + s * part_stride_o);
      }
#pragma unroll
      for (int k = 0; k < CHUNK; ++k) {
        acc.x = fmaf(w[k], o[k].x, acc.x);
        acc.y = fmaf(w[k], o[k].y, acc.y);
        acc.z = fmaf(w[k], o[k].z, acc.z);
        acc.w = fmaf(w[k], o[k].w, acc.w);
        den += w[k];
      }
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  acc.x *= inv; acc.y *= inv; acc.z *= inv; acc.w *= inv;
  if (p.out_f32) {
    *(float4*)((float*)p.O + pair * D + sub * 4) = acc;
  } else {
    bf16x4 o4;
    o4[0] = (__bf16)acc.x; o4[1] = (__bf16)acc.y; o4[2] = (__bf16)acc.z; o4[3] = (__bf16)acc.w;
    *(bf16x4*)((__bf16*)p.O + pair * D + sub * 4) = o4;
  }
  if (sub == 0) p.LSE[pair] = den > 0.f ? M + __logf(den) : -INFINITY;
}

hipError_t launch_merge(const MergeParams& p, int d, hipStream_t s) {
  const int64_t threads = p.n_rows * p.hq * (d / 4);
  if (threads <= 0) return hipSuccess;
  const int64_t blocks = (threads + 255) / 256;
  if (d == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(merge_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

__global__ void zero_f32_kernel(float* p, int64_t n) {
  const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i4 + 3 < n) {
    *(float4*)(p + i4) = make_float4(0.f, 0.f, 0.f, 0.f);
  } else {
    for (int64_t i = i4; i < n; ++i) p[i] = 0.f;
  }
}

__global__ void zero_bf16_kernel(__bf16* p, int64_t n) {
  const int64_t i8 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i8 + 7 < n) {
    *(uint4*)(p + i8) = make_uint4(0, 0, 0, 0);
  } else {
    for (int64_t i = i8; i < n; ++i) p[i] = (__bf16)0.f;
  }
}

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n / 4 + 256) / 256;
  hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_zero_bf16(__bf16* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n / 8 + 256) / 256;
  hipLaunchKernelGGL(zero_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace ca
