// K2 — merge of partial attention results by their log-sum-exp
// ("Context Parallelism for Scalable Million-Token Inference", Section 3.4
// Merge Attention, Equation 4, Appendix B):
//   M = max_s LSE_s,  O = sum_s O_s e^(LSE_s - M) / sum_s e^(LSE_s - M),
//   LSE = M + ln sum_s e^(LSE_s - M).
// HBM-bound: each (row, head) is D / 8 lanes holding two float4s of every
// partial; a partial with LSE = -inf is skipped without reading its O.

#include "ca_internal.h"
#include "ca_kernel_util.h"

namespace ca {

// Two float4s of a row per lane: D / 8 lanes per (row, head).
constexpr int kMergeVec = 2;

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  constexpr int LPP = D / (4 * kMergeVec);
  const int64_t n_pairs = p.n_rows * p.hq;
  const int64_t pair = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPP;
  const int sub = threadIdx.x % LPP;
  if (pair >= n_pairs) return;
  float4 r[kMergeVec];
  const float lse = merge_lse_parts<D, kMergeVec>(p.LSE_parts + pair, n_pairs, p.O_parts + pair * D + sub * 4,
                                                  n_pairs * D, p.n_parts, r);
  store_row_part<D, kMergeVec>(p.O, pair * D + sub * 4, p.out_f32 != 0, r);
  if (sub == 0) p.LSE[pair] = lse;
}

hipError_t launch_merge(const MergeParams& p, int d, hipStream_t s) {
  const int64_t threads = p.n_rows * p.hq * (d / (4 * kMergeVec));
  if (threads <= 0) return hipSuccess;
  const int64_t blocks = (threads + 255) / 256;
  if (d == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(merge_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

// Split query shards: the key chunks' partials of every (row, head) merged
// by Equation 4 into the shard's output rows.  blockIdx.y = shard; D / 8
// lanes per (row, head) as in merge_kernel.
template <int D>
__global__ __launch_bounds__(256) void shard_merge_kernel(const ShardMerge* recs, const float* stage_O,
                                                          const float* stage_LSE, void* O, float* LSE, int out_f32,
                                                          int hq) {
  constexpr int LPP = D / (4 * kMergeVec);
  const ShardMerge r = recs[blockIdx.y];
  const int64_t pair = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPP;   // (row, head) of the shard
  const int sub = threadIdx.x % LPP;
  if (pair >= (int64_t)r.q_len * hq) return;
  const int64_t sp = r.stage_row0 * hq + pair;                            // chunk 0's (row, head)
  const int64_t stride = (int64_t)r.q_len * hq;                           // chunk to chunk
  float4 o[kMergeVec];
  const float lse = merge_lse_parts<D, kMergeVec>(stage_LSE + sp, stride, stage_O + sp * D + sub * 4, stride * D,
                                                  r.n_chunks, o);
  const int64_t op = r.o_off * hq + pair;
  store_row_part<D, kMergeVec>(O, op * D + sub * 4, out_f32 != 0, o);
  if (sub == 0) LSE[op] = lse;
}

hipError_t launch_shard_merge(const ShardMerge* recs, int32_t n_recs, int32_t max_q_len, const float* stage_O,
                              const float* stage_LSE, void* O, float* LSE, int out_f32, int hq, int d, hipStream_t s) {
  if (n_recs <= 0) return hipSuccess;
  const int64_t threads = (int64_t)max_q_len * hq * (d / (4 * kMergeVec));
  const dim3 grid((unsigned)((threads + 255) / 256), (unsigned)n_recs);
  if (d == 128)
    hipLaunchKernelGGL(shard_merge_kernel<128>, grid, dim3(256), 0, s, recs, stage_O, stage_LSE, O, LSE, out_f32, hq);
  else
    hipLaunchKernelGGL(shard_merge_kernel<64>, grid, dim3(256), 0, s, recs, stage_O, stage_LSE, O, LSE, out_f32, hq);
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
