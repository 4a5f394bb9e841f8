// K1 — fused core-attention forward over a CA-task table (gfx950).
//
// One workgroup (4 waves) per work item: 128 (query row, head) pairs that all
// read the same KV head — hpw heads x (4 / hpw) blocks of 32 rows — so each
// K/V tile staged in LDS feeds four MFMA streams.  Per 64-key tile a wave:
//
//   S^T[64 keys][32 queries] = K_tile . Q^T       (MFMA 32x32x16 bf16, fp32 acc)
//   online softmax in the exp2 domain              (rows are lane-local)
//   O^T[d][32 queries]     += V_tile^T . P^T       (MFMA 32x32x16 bf16)
//
// Computing the transposed products keeps one query per lane (lane % 32) in
// both the score and the output accumulators, so the row max / row sum need
// one exchange between the two half-waves and the rescale of O is lane-local.
// The MFMA's reduction index is permuted consistently on both operands of
// P.V, so the probabilities feed the next MFMA straight from the score
// registers; V^T comes from LDS through ds_read_b64_tr_b16.
//
// Masking follows the CA-task definition: key j of a task is visible to its
// query i iff kv_pos0 + j <= q_pos0 + i ("Efficient Long-context Language
// Model Training by Core Attention Disaggregation", Section 3.4, CA-Task
// Abstraction; diagonal included).  Tiles past the last visible key of the
// workgroup are never visited; only tiles that straddle the diagonal or the
// end of the context apply the per-element mask.
//
// Outputs: O (bf16, or fp32 partials) and LSE = ln sum exp(scale q.k), the
// statistic that makes partials mergeable by Equation 4 ("Context Parallelism
// for Scalable Million-Token Inference", Section 3.4 Merge Attention).

#include "ca_internal.h"
#include "ca_kernel_util.h"

namespace ca {

template <int D>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdParams p) {
  constexpr int BN = 64;          // keys per tile
  constexpr int KS = D + 8;       // K row stride in LDS (elements): 16 B pad
  constexpr int VS = D + 16;      // V row stride in LDS (elements): 32 B pad
  constexpr int NCB = D / 32;     // 32-channel output blocks
  constexpr int NKS = D / 16;     // 16-channel reduction steps of Q.K
  constexpr int CH = D / 8;       // 16-byte chunks per row
  constexpr int RPP = 256 / CH;   // rows per load pass
  constexpr int PASSES = BN / RPP;

  __shared__ __attribute__((aligned(16))) __bf16 lds_k[2][BN * KS];
  __shared__ __attribute__((aligned(16))) __bf16 lds_v[2][BN * VS];

  const FwdItem it = p.items[blockIdx.x];
  const ca_task t = p.tasks[it.task];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;       // half-wave

  const int hpw = p.hpw;
  const int head = it.kv_head * p.group + it.head_sub * hpw + (wave % hpw);
  const int wrow0 = it.row0 + (wave / hpw) * 32;
  const int64_t delta = t.q_pos0 - t.kv_pos0;
  const int kv_len = t.kv_len;

  // Key range of the workgroup and of this wave.
  const int rt = 32 * (4 / hpw);
  const int wg_last = min(it.row0 + rt, t.q_len) - 1;
  const int kv_hi = (int)clamp64((int64_t)wg_last + delta + 1, 0, kv_len);
  const int w_last = min(wrow0 + 32, t.q_len) - 1;
  const int w_kv_hi = (w_last < wrow0) ? 0 : (int)clamp64((int64_t)w_last + delta + 1, 0, kv_len);

  // Q^T operand: this lane's query row, channels 16 s + 8 hh .. + 7.
  const int qrow = wrow0 + l32;
  const bool qvalid = qrow < t.q_len;
  bf16x8 qf[NKS];
  {
    const __bf16* qp = p.Q + (t.q_off + qrow) * (int64_t)(p.hq * D) + head * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < NKS; ++s) qf[s] = qvalid ? *(const bf16x8*)(qp + 16 * s) : bf16x8_zero();
  }

  f32x16 o_acc[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) o_acc[c] = f32x16_zero();
  float m2 = -INFINITY;   // running max of scale*log2(e)*s
  float lsum = 0.f;       // running sum of exp2(...)

  const int n_tiles = (kv_hi + BN - 1) / BN;
  const int64_t kv_stride = (int64_t)p.hkv * D;
  const __bf16* kbase = p.K + t.kv_off * kv_stride + it.kv_head * D;
  const __bf16* vbase = p.V + t.kv_off * kv_stride + it.kv_head * D;
  const int ld_row = tid / CH;
  const int ld_chunk = tid % CH;

  uint4 kreg[PASSES], vreg[PASSES];
  auto gload = [&](int tile) {
#pragma unroll
    for (int r = 0; r < PASSES; ++r) {
      const int row = tile * BN + r * RPP + ld_row;
      if (row < kv_hi) {
        kreg[r] = *(const uint4*)(kbase + row * kv_stride + ld_chunk * 8);
        vreg[r] = *(const uint4*)(vbase + row * kv_stride + ld_chunk * 8);
      } else {
        kreg[r] = make_uint4(0, 0, 0, 0);
        vreg[r] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int r = 0; r < PASSES; ++r) {
      const int row = r * RPP + ld_row;
      *(uint4*)(&lds_k[buf][row * KS + ld_chunk * 8]) = kreg[r];
      *(uint4*)(&lds_v[buf][row * VS + ld_chunk * 8]) = vreg[r];
    }
  };

  // Per-lane LDS offsets of the two operands.
  //  K (A of S^T): key mb*32 + l32, channels 16 s + 8 hh.
  //  V^T (A of O^T) via transpose reads: the 16-lane group g16 serves channels
  //  c0 + (lane % 16), c0 = cb*32 + 16 (g16 % 2); source lane j of the group
  //  points at key k0 + j / 4, channels c0 + 4 (j % 4).
  const int k_lane_off = l32 * KS + 8 * hh;
  const int g16 = lane >> 4;
  const int j16 = lane & 15;
  const int v_lane_off = (j16 >> 2) * VS + 16 * (g16 & 1) + 4 * (j16 & 3);
  const int v_h = (g16 >> 1);     // == hh

  if (n_tiles > 0) gload(0);
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int buf = tile & 1;
    swrite(buf);
    __syncthreads();
    if (tile + 1 < n_tiles) gload(tile + 1);
    const int k0 = tile * BN;
    if (k0 < w_kv_hi) {
      f32x16 s_acc[2];
      s_acc[0] = f32x16_zero();
      s_acc[1] = f32x16_zero();
      const __bf16* kl = &lds_k[buf][k_lane_off];
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const bf16x8 kf = *(const bf16x8*)(kl + mb * 32 * KS + 16 * s);
          s_acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], s_acc[mb], 0, 0, 0);
        }
      }
      // Mask only where the tile straddles the diagonal or the context end.
      const bool need_mask = ((int64_t)k0 + BN - 1 > (int64_t)wrow0 + delta) || (k0 + BN > kv_len);
      if (need_mask) {
        const int64_t lim = (int64_t)qrow + delta;   // last visible key of this row
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = k0 + mb * 32 + 8 * (j >> 2) + 4 * hh + (j & 3);
            if (key >= kv_len || (int64_t)key > lim) s_acc[mb][j] = -INFINITY;
          }
        }
      }
      // Online softmax, exp2 domain.
      float mx = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s_acc[mb][j]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m2, mx * p.scale_log2);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2_fast(m2 - m_use);
      float rs = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float e = exp2_fast(fmaf(s_acc[mb][j], p.scale_log2, -m_use));
          s_acc[mb][j] = e;
          rs += e;
        }
      rs += __shfl_xor(rs, 32);
      lsum = lsum * alpha + rs;
      m2 = m_new;
#pragma unroll
      for (int c = 0; c < NCB; ++c)
#pragma unroll
        for (int j = 0; j < 16; ++j) o_acc[c][j] *= alpha;

      // P^T fragments: registers 8*half .. 8*half+7 of score block mb.
      bf16x8 pf[2][2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int i = 0; i < 8; ++i) pf[mb][half][i] = (__bf16)s_acc[mb][8 * half + i];

      const __bf16* vl = &lds_v[buf][v_lane_off];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int kb = mb * 32 + 16 * half + 4 * v_h;
#pragma unroll
          for (int c = 0; c < NCB; ++c) {
            const __bf16* a0 = vl + kb * VS + c * 32;
            const bf16x4 lo = ds_read_tr16(a0);
            const bf16x4 hi = ds_read_tr16(a0 + 8 * VS);
            const bf16x8 vf = concat_bf16x4(lo, hi);
            o_acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[mb][half], o_acc[c], 0, 0, 0);
          }
        }
      }
    }
  }

  // Epilogue: O = acc / l, LSE = ln 2 * (m2 + log2 l); empty rows: 0, -inf.
  if (!qvalid) return;
  const float inv_l = lsum > 0.f ? 1.f / lsum : 0.f;
  const int64_t orow = t.o_off + qrow;
  if (hh == 0) {
    p.LSE[orow * p.hq + head] = lsum > 0.f ? (m2 + __log2f(lsum)) * 0.69314718055994530942f : -INFINITY;
  }
  const int64_t obase = orow * (int64_t)(p.hq * D) + head * D;
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int ch = c * 32 + 8 * q4 + 4 * hh;
      const float v0 = o_acc[c][4 * q4 + 0] * inv_l;
      const float v1 = o_acc[c][4 * q4 + 1] * inv_l;
      const float v2 = o_acc[c][4 * q4 + 2] * inv_l;
      const float v3 = o_acc[c][4 * q4 + 3] * inv_l;
      if (p.out_f32) {
        *(float4*)((float*)p.O + obase + ch) = make_float4(v0, v1, v2, v3);
      } else {
        bf16x4 o4;
        o4[0] = (__bf16)v0;
        o4[1] = (__bf16)v1;
        o4[2] = (__bf16)v2;
        o4[3] = (__bf16)v3;
        *(bf16x4*)((__bf16*)p.O + obase + ch) = o4;
      }
    }
  }
}

hipError_t launch_forward(const FwdParams& p, int d, hipStream_t s) {
  if (p.n_items <= 0) return hipSuccess;
  if (d == 128)
    hipLaunchKernelGGL(fwd_kernel<128>, dim3(p.n_items), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(fwd_kernel<64>, dim3(p.n_items), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace ca
