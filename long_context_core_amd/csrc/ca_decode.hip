// K3 — split-KV decode: single-token queries over long KV caches (gfx950).
//
// The pass-Q ring keeps each rank's KV block stationary and runs the visiting
// queries against it, returning (O, LSE) partials that are merged by
// Equation 4 ("Context Parallelism for Scalable Million-Token Inference",
// Section 3.4 Ring Pass-Q and Batched Ring Pass-Q Decode; Merge Attention).
// On one GPU this is memory-bound: every cached key and value is read once,
// at 16 FLOPs per byte for 16 query heads, far below the MFMA ridge.
//
// Work item = (task, KV head, key chunk).  The query heads of the KV head's
// group (G <= 16) form the N = 16 columns of v_mfma_f32_16x16x32_bf16, so
// one load of K/V serves all of them.  Per 128-key tile each wave takes 32
// keys:
//   S^T[32 keys][16 heads] = K . Q^T   K straight from HBM in operand layout
//   online softmax per head (exp2 domain, lazy rescale)
//   O^T[d][16 heads]     += V^T . P^T  V^T through per-wave LDS + ds_read_b64_tr_b16
// The four waves' running states are merged by log-sum-exp at the end of the
// item; chunks of a split task are merged by dec_merge_kernel.

#include <type_traits>

#include "ca_internal.h"
#include "ca_kernel_util.h"

namespace ca {

namespace {
constexpr float kDecRescaleLog2 = 8.0f;

__device__ __forceinline__ float xor_max(float x, int m) { return fmaxf(x, __shfl_xor(x, m)); }
__device__ __forceinline__ float xor_sum(float x, int m) { return x + __shfl_xor(x, m); }
}  // namespace

template <int D, bool PAGED>
__global__ __launch_bounds__(256, PAGED ? 1 : 2) void dec_kernel(DecParams p) {
  constexpr int TK = 128;            // keys per tile, 32 per wave
  // Tiles whose K/V loads are in flight while one tile computes.  Paged
  // caches take two (two register sets, one wave per SIMD): each tile may
  // lie in another physical page, and the second set hides that page's
  // address translation (256-row shuffled pages: 0.366 -> 0.338 ms on the
  // 32 x 128K step).  Contiguous caches stream best with one set at two
  // waves per SIMD (two sets measured 2 % slower there).
  constexpr int DEPTH = PAGED ? 2 : 1;
  constexpr int NT = D / 32;         // 32-channel reduction steps of Q.K
  constexpr int NCB = D / 16;        // 16-channel blocks of O^T
  constexpr int VS = D + 16;         // V row stride in LDS (elements)
  constexpr int VCH = D / 8;         // 16-byte chunks per V row
  constexpr int VROWS = 64 / VCH;    // V rows written per wave pass
  constexpr int VPASS = 32 / VROWS;  // passes for the wave's 32 rows

  __shared__ __attribute__((aligned(16))) __bf16 lds_v[4][32 * VS];

  const DecItem it = p.items[blockIdx.x];
  const ca_task t = p.tasks[it.task];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;
  const int G = p.group;
  const int head0 = it.kv_head * G;

  // Q^T operand: head l16 of the group, channels 32 s + 8 g4 .. + 7.
  bf16x8 qf[NT];
  {
    const bool hv = l16 < G;
    const __bf16* qp = p.Q + t.q_off * (int64_t)(p.hq * D) + (head0 + (hv ? l16 : 0)) * D + 8 * g4;
#pragma unroll
    for (int s = 0; s < NT; ++s) qf[s] = hv ? *(const bf16x8*)(qp + 32 * s) : bf16x8_zero();
  }

  const int nkeys = it.k_end - it.k_begin;
  const int64_t kv_stride = (int64_t)p.hkv * D;
  const uint32_t row_bytes = (uint32_t)(kv_stride * 2);
  const int64_t row0 = t.kv_off + it.k_begin;   // virtual row of the chunk's first key
  const __bf16* kbase = p.K + it.kv_head * D;
  const __bf16* vbase = p.V + it.kv_head * D;

  // K operand loads: key 32 w + 16 b + l16, channels 32 s + 8 g4.
  uint32_t k_voff[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) k_voff[b] = (uint32_t)(32 * wave + 16 * b + l16) * row_bytes + 16 * g4;
  // V loads: wave rows 32 w + VROWS r + lane / VCH, chunk lane % VCH.
  const uint32_t v_voff = (uint32_t)(32 * wave + lane / VCH) * row_bytes + 16 * (lane % VCH);
  __bf16* vw = &lds_v[wave][0];
  const int v_st = (lane / VCH) * VS + 8 * (lane % VCH);
  // Transpose-read offsets: group g4 reads keys 4 g4 (+16), channels cb*16 + 4 (j % 4).
  const int v_rd = (4 * g4 + (l16 >> 2)) * VS + 4 * (l16 & 3);

  uint4 kr[DEPTH][2][NT], vr[DEPTH][VPASS];   // register set t % DEPTH holds tile t
  // Tile loads over the tile's own rows: keys >= nkeys read as zeros and
  // nothing past the chunk is read.  Paged K/V: chunks start at multiples of
  // 128 keys, tasks at multiples of 128 virtual rows, and pages hold a
  // multiple of 128 rows, so each tile lies inside one page.
  // Paged K/V: a tile's physical page is read DEPTH tiles before its loads
  // are issued (vector load, in order with the tile loads) and moved to a
  // scalar register where used.
  const __amdgpu_buffer_rsrc_t prs = make_rsrc(p.pages, p.page_bytes);
  auto tile_page = [&](int tile) -> int {
    if constexpr (PAGED) {
      const int64_t v = row0 + (int64_t)tile * TK;
      return __builtin_amdgcn_raw_buffer_load_b32(prs, (uint32_t)(v >> p.page_shift) * 4u, 0, 0);
    } else {
      return 0;
    }
  };
  auto gload = [&](auto set_tag, int tile, int page) {
    constexpr int SET = decltype(set_tag)::value;
    const int64_t v = row0 + (int64_t)tile * TK;
    int64_t r0 = v;
    if constexpr (PAGED) {
      const int64_t pg = __builtin_amdgcn_readfirstlane(page);
      r0 = (pg << p.page_shift) | (v & ((int64_t(1) << p.page_shift) - 1));
    }
    const int n = min(TK, nkeys - tile * TK);
    const __amdgpu_buffer_rsrc_t krs = rows_rsrc(kbase + r0 * kv_stride, n, row_bytes);
    const __amdgpu_buffer_rsrc_t vrs = rows_rsrc(vbase + r0 * kv_stride, n, row_bytes);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int s = 0; s < NT; ++s) kr[SET][b][s] = buffer_load_16_stream(krs, k_voff[b] + 64 * s, 0);
#pragma unroll
    for (int r = 0; r < VPASS; ++r) vr[SET][r] = buffer_load_16_stream(vrs, v_voff + (uint32_t)(r * VROWS) * row_bytes, 0);
  };

  f32x4 o_acc[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) o_acc[c] = f32x4_zero();
  float m2 = -INFINITY, lsum = 0.f;

  const int n_tiles = (nkeys + TK - 1) / TK;
  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, DEPTH - 1>;
  int pgs[DEPTH];                                // page of the next tile each set loads
  if (n_tiles > 0) gload(Set0{}, 0, tile_page(0));
  if (DEPTH > 1 && n_tiles > 1) gload(Set1{}, 1, tile_page(1));
#pragma unroll
  for (int i = 0; i < DEPTH; ++i) pgs[i] = DEPTH + i < n_tiles ? tile_page(DEPTH + i) : 0;

  auto process = [&](auto set_tag, int tile) __attribute__((always_inline)) {
    constexpr int SET = decltype(set_tag)::value;
    uint4 kc[2][NT];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int s = 0; s < NT; ++s) kc[b][s] = kr[SET][b][s];
    // stage this wave's 32 V rows (wave-private LDS region)
#pragma unroll
    for (int r = 0; r < VPASS; ++r) *(uint4*)(vw + v_st + r * VROWS * VS) = vr[SET][r];
    if (tile + DEPTH < n_tiles) {
      gload(set_tag, tile + DEPTH, pgs[SET]);
      if (tile + 2 * DEPTH < n_tiles) pgs[SET] = tile_page(tile + 2 * DEPTH);
    }

    f32x4 s_acc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      s_acc[b] = f32x4_zero();
#pragma unroll
      for (int s = 0; s < NT; ++s)
        s_acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kc[b][s]), qf[s], s_acc[b], 0, 0, 0);
    }
    const int kt0 = tile * TK + 32 * wave;        // first key of this wave in the chunk
    if (kt0 + 32 > nkeys) {
      keep_branch();
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (kt0 + 16 * b + 4 * g4 + j >= nkeys) s_acc[b][j] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(s_acc[0][0], s_acc[0][1]), fmaxf(s_acc[0][2], s_acc[0][3])),
                     fmaxf(fmaxf(s_acc[1][0], s_acc[1][1]), fmaxf(s_acc[1][2], s_acc[1][3])));
    mx = xor_max(xor_max(mx, 16), 32);
    const float m_tile = mx * p.scale_log2;
    if (__any(m_tile > m2 + kDecRescaleLog2)) {
      keep_branch();
      const float m_new = fmaxf(m2, m_tile);
      const float alpha = (m2 == -INFINITY) ? 0.f : exp2_fast(m2 - m_new);   // rows still empty: acc is 0
      lsum *= alpha;
#pragma unroll
      for (int c = 0; c < NCB; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) o_acc[c][j] *= alpha;
      m2 = m_new;
    }
    const float m_use = (m2 == -INFINITY) ? 0.f : m2;
    bf16x8 pf;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float e = exp2_fast(fmaf(s_acc[b][j], p.scale_log2, -m_use));
        lsum += e;
        pf[4 * b + j] = (__bf16)e;
      }
    // V^T . P^T over the wave's 32 keys
    __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0): this wave's LDS writes landed
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      const __bf16* a0 = vw + v_rd + 16 * c;
      const bf16x8 vf = concat_bf16x4(ds_read_tr16(a0), ds_read_tr16(a0 + 16 * VS));
      o_acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, o_acc[c], 0, 0, 0);
    }
  };
  for (int tile = 0; tile < n_tiles; tile += DEPTH) {
    process(Set0{}, tile);
    if (DEPTH > 1 && tile + 1 < n_tiles) process(Set1{}, tile + 1);
  }

  // Row sums: lanes of the same head (l16) across the four lane groups.
  lsum = xor_sum(xor_sum(lsum, 16), 32);

  // Merge the four waves' states through LDS.
  __syncthreads();
  float* red = (float*)&lds_v[0][0];              // [4][16][D] O, then [4][16] m, [4][16] l
  float* red_m = red + 4 * 16 * D;
  float* red_l = red_m + 64;
#pragma unroll
  for (int c = 0; c < NCB; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) red[(wave * 16 + l16) * D + 16 * c + 4 * g4 + j] = o_acc[c][j];
  if (g4 == 0) {
    red_m[wave * 16 + l16] = m2;
    red_l[wave * 16 + l16] = lsum;
  }
  __syncthreads();
  constexpr int CPT = D / 16;                     // channels per thread
  const int h = tid >> 4;                         // head 0..15
  const int c0 = (tid & 15) * CPT;
  if (h >= G) return;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, red_m[w * 16 + h]);
  float wgt[4], L = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float mw = red_m[w * 16 + h];
    wgt[w] = (mw == -INFINITY) ? 0.f : exp2_fast(mw - M);
    L += wgt[w] * red_l[w * 16 + h];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const float lse = L > 0.f ? (M + __log2f(L)) * 0.69314718055994530942f : -INFINITY;
  float o[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) a = fmaf(wgt[w], red[(w * 16 + h) * D + c0 + i], a);
    o[i] = a * inv;
  }
  if (it.part < 0) {
    const int64_t orow = t.o_off;
    const int64_t ob = orow * (int64_t)(p.hq * D) + (int64_t)(head0 + h) * D + c0;
    if (p.out_f32) {
#pragma unroll
      for (int i = 0; i < CPT; i += 4) *(float4*)((float*)p.O + ob + i) = make_float4(o[i], o[i + 1], o[i + 2], o[i + 3]);
    } else {
#pragma unroll
      for (int i = 0; i < CPT; i += 4) {
        bf16x4 v;
        v[0] = (__bf16)o[i]; v[1] = (__bf16)o[i + 1]; v[2] = (__bf16)o[i + 2]; v[3] = (__bf16)o[i + 3];
        *(bf16x4*)((__bf16*)p.O + ob + i) = v;
      }
    }
    if ((tid & 15) == 0) p.LSE[orow * p.hq + head0 + h] = lse;
  } else {
    float* po = p.part_O + ((int64_t)it.part * G + h) * D + c0;
#pragma unroll
    for (int i = 0; i < CPT; i += 4) *(float4*)(po + i) = make_float4(o[i], o[i + 1], o[i + 2], o[i + 3]);
    if ((tid & 15) == 0) p.part_LSE[(int64_t)it.part * G + h] = lse;
  }
}

// Merge of the key chunks of each split decode task (Equation 4).  D / 8
// lanes per (split task, head), two float4s each.
constexpr int kDecMergeVec = 2;

template <int D>
__global__ __launch_bounds__(256) void dec_merge_kernel(DecMergeParams p) {
  constexpr int LPP = D / (4 * kDecMergeVec);
  const int64_t pair = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPP;
  const int sub = threadIdx.x % LPP;
  if (pair >= (int64_t)p.n_split * p.group) return;
  const int rec = (int)(pair / p.group);
  const int h = (int)(pair % p.group);
  const int64_t first = p.first_part[rec];
  const ca_task t = p.tasks[p.task_of[rec]];
  const int head = p.head_of[rec] * p.group + h;
  float4 r[kDecMergeVec];
  const float lse = merge_lse_parts<D, kDecMergeVec>(p.part_LSE + first * p.group + h, p.group,
                                                     p.part_O + (first * p.group + h) * D + sub * 4,
                                                     (int64_t)p.group * D, p.n_parts[rec], r);
  store_row_part<D, kDecMergeVec>(p.O, t.o_off * (int64_t)(p.hq * D) + (int64_t)head * D + sub * 4,
                                  p.out_f32 != 0, r);
  if (sub == 0) p.LSE[t.o_off * p.hq + head] = lse;
}

template <int D>
hipError_t launch_decode_d(const DecParams& p, hipStream_t s) {
  if (p.pages)
    hipLaunchKernelGGL((dec_kernel<D, true>), dim3(p.n_items), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((dec_kernel<D, false>), dim3(p.n_items), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_decode(const DecParams& p, int d, hipStream_t s) {
  if (p.n_items <= 0) return hipSuccess;
  return d == 128 ? launch_decode_d<128>(p, s) : launch_decode_d<64>(p, s);
}

hipError_t launch_decode_merge(const DecMergeParams& p, int d, hipStream_t s) {
  const int64_t threads = (int64_t)p.n_split * p.group * (d / (4 * kDecMergeVec));
  if (threads <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  if (d == 128)
    hipLaunchKernelGGL(dec_merge_kernel<128>, dim3(blocks), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(dec_merge_kernel<64>, dim3(blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace ca
