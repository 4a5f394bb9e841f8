// Backward of core attention over a CA-task table (gfx950), without atomics.
//
// The pages fix only that the backward recomputes the attention
// probabilities from the per-row statistics saved by the forward instead of
// storing them ("Efficient Long-context Language Model Training by Core
// Attention Disaggregation", Sections 3.2 and 3.4, Property 1).  With
// P = exp(scale S - LSE) and D_i = <dO_i, O_i>:
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  dK = scale dS^T Q,
//   dQ = scale dS K.
//
//   bwd_prep_kernel  D_i = rowsum(dO_i o O_i)                      (HBM-bound)
//   bwd_kv_kernel    K/V-stationary: a workgroup owns 128 context rows of one
//                    KV head (32 per wave, K and V held as MFMA operands in
//                    registers) and sweeps every query tile and every query
//                    head of the group that sees them; dK and dV accumulate in
//                    registers across heads and tiles.  Per 32x32 block:
//                      S = Q K^T, dP = dO V^T          (lane = key)
//                      dV^T += dO^T P,  dK^T += Q^T dS (dO^T, Q^T by LDS transpose reads)
//   bwd_q_kernel     Q-stationary, shaped like the forward (eight waves, two
//                    per SIMD): S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T
//                    (K^T by transpose reads).
// Query shards over several contexts (consecutive tasks sharing their query
// rows) and context groups (tasks sharing their context rows; contexts that
// overlap are first cut into shared pieces) are swept one task after another
// inside one work item (the MULTI instantiations), so every gradient row is
// still written once per pass.  Items whose rows are too many for one item
// write fp32 partials (dK/dV slots, dQ key chunks) that a reduction sums in a
// fixed order.
// Rows are written once per pass (read-modify-write in fp32 when several
// tasks share rows), so results are deterministic.

#include <type_traits>

#include "ca_internal.h"
#include "ca_kernel_util.h"

namespace ca {

namespace {
constexpr float kLog2e = 1.4426950408889634f;

// LSE (natural log) -> log2 units; an empty row (-inf) becomes +inf so that
// exp2(s - lse) = 0 for every key.
__device__ __forceinline__ float lse_log2(float lse) {
  return lse == -INFINITY ? INFINITY : lse * kLog2e;
}
}  // namespace

// ---------------------------------------------------------------------------
// D_i = sum_c dO[i][h][c] * O[i][h][c], for every output row and head.
// 16 lanes per (row, head), 8 channels each (D = 128) or 4 (D = 64).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const __bf16* O, const __bf16* dO, float* Dv, int64_t n_pairs) {
  constexpr int EPL = D / 16;
  const int64_t pair = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
  const int sub = threadIdx.x & 15;
  float acc = 0.f;
  if (pair < n_pairs) {
    const __bf16* o = O + pair * D + sub * EPL;
    const __bf16* g = dO + pair * D + sub * EPL;
#pragma unroll
    for (int i = 0; i < EPL; ++i) acc = fmaf((float)o[i], (float)g[i], acc);
  }
  acc += __shfl_xor(acc, 8);
  acc += __shfl_xor(acc, 4);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 1);
  if (pair < n_pairs && sub == 0) Dv[pair] = acc;
}

// ---------------------------------------------------------------------------
// LDS tile of 32 query rows x D bf16 (Q or dO) in the dK/dV kernel.  It is read
// row-wise (MFMA A operand: 16 rows, one 16-byte chunk each) and by transpose
// reads (4 consecutive rows, 4 consecutive chunks).  D = 128: unpadded 256-byte
// rows with chunk c of row r stored at chunk c ^ swz(r), a layout in which
// both patterns hit every bank once.  D = 64: rows padded to 80 elements.
// ---------------------------------------------------------------------------
template <int D>
struct QTile {
  static constexpr int kRow = D + 16;
  static constexpr int kElems = 32 * kRow;
  __device__ static int off(int r, int chunk) { return r * kRow + chunk * 8; }
};
template <>
struct QTile<128> {
  static constexpr int kRow = 128;
  static constexpr int kElems = 32 * kRow;
  __device__ static int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
  __device__ static int off(int r, int chunk) { return r * kRow + ((chunk ^ swz(r)) << 3); }
};

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (task, KV head, 128 context rows).
// ---------------------------------------------------------------------------
template <int D, bool PAGED, bool WIN, bool MULTI>
__global__ __launch_bounds__(256, 1) void bwd_kv_kernel(BwdParams p) {
  using Tile = QTile<D>;
  constexpr int BQ = 32;            // query rows per step
  constexpr int NKS = D / 16;       // 16-channel reduction steps
  constexpr int NCB = D / 32;       // 32-channel output blocks
  constexpr int CH = D / 8;         // 16-byte chunks per row
  constexpr int RPP = 256 / CH;     // rows per load pass
  constexpr int PASSES = BQ / RPP;
  __shared__ __attribute__((aligned(16))) __bf16 lds_q[2][Tile::kElems];
  __shared__ __attribute__((aligned(16))) __bf16 lds_do[2][Tile::kElems];
  __shared__ __attribute__((aligned(16))) float lds_lse[2][BQ];
  __shared__ __attribute__((aligned(16))) float lds_d[2][BQ];

  const BwdItem it = p.items[blockIdx.x];
  // The item's context group: tasks p.members[it.member0 ..] share the
  // context rows; t is the task whose query rows are being swept (the only
  // one unless MULTI).
  int task_idx = p.members[it.member0];
  ca_task t = p.tasks[task_idx];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  int64_t delta = t.q_pos0 - t.kv_pos0;
  const int G = p.group;
  const int kw0 = it.key0 + 32 * wave;           // first (task-relative) key of this wave
  const int my_key = kw0 + l32;
  const bool key_ok = my_key < t.kv_len;

  // Physical row of the item's first key: the 128 keys of an item lie in
  // one page of paged K/V (pages hold a multiple of 128 rows and contexts
  // start on a 128-row boundary).
  // kv_row0 + key is the physical row of task-relative key `key` of the item.
  int64_t kv_row0 = t.kv_off;
  if constexpr (PAGED) {
    const int64_t v = t.kv_off + it.key0;
    const int64_t page = p.pages[v >> p.page_shift];
    kv_row0 = ((page << p.page_shift) | (v & ((int64_t(1) << p.page_shift) - 1))) - it.key0;
  }
  // Stationary operands: K and V rows of this lane's key (B of S = Q K^T and of dP = dO V^T).
  const int64_t kv_stride = (int64_t)p.hkv * D;
  bf16x8 kf[NKS], vf[NKS];
  {
    const int64_t roff = (kv_row0 + (key_ok ? my_key : 0)) * kv_stride + it.kv_head * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      kf[s] = key_ok ? *(const bf16x8*)(p.K + roff + 16 * s) : bf16x8_zero();
      vf[s] = key_ok ? *(const bf16x8*)(p.V + roff + 16 * s) : bf16x8_zero();
    }
  }
  f32x16 dk_acc[NCB], dv_acc[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
    dk_acc[c] = f32x16_zero();
    dv_acc[c] = f32x16_zero();
  }

  // Query rows that see at least one key of the workgroup: i + delta >= key0.
  const int wg_keys = min(128, t.kv_len - it.key0);
  // Sink + sliding-window mask (win > 0): key j is also required to lie in
  // the row's win latest positions (j > i + delta - win) or among the sink
  // keys [0, sj).  Rows past the window of the workgroup's last key see none
  // of its keys, unless it holds sink keys.
  int win, sj, r_lo, r_end, r_first, n_rt, n_steps;
  auto member = [&]() __attribute__((always_inline)) {
    win = 0;
    sj = 0;
    if (p.masks) {
      win = p.masks[task_idx].window;
      if (win > 0) sj = (int)clamp64((int64_t)p.masks[task_idx].sink - t.kv_pos0, 0, t.kv_len);
    }
    r_lo = (int)clamp64((int64_t)it.key0 - delta, 0, t.q_len);
    r_end = (win > 0 && it.key0 >= sj) ? (int)clamp64((int64_t)it.key0 + wg_keys - 1 - delta + win, r_lo, t.q_len)
                                       : t.q_len;
    if constexpr (MULTI) {
      // a split item sweeps only its rows [row_lo, row_hi) (32-aligned)
      r_lo = max(r_lo, it.row_lo);
      r_end = min(r_end, it.row_hi);
    }
    r_first = (r_lo / BQ) * BQ;
    n_rt = (r_end - r_first + BQ - 1) / BQ;
    n_steps = (wg_keys > 0 && r_end > r_lo) ? n_rt * G : 0;
  };
  member();

  // Tile loads through range-checked buffers based at the tile's first row:
  // rows past the task read as 0 (Q = dO = 0 there, so such rows add nothing
  // to dK or dV whatever their P).  The wave-uniform bases advance by fixed
  // strides from tile to tile; the lane offsets are constants.
  const int64_t q_stride = (int64_t)p.hq * D;
  const uint32_t row_bytes = (uint32_t)(q_stride * 2);
  const int ld_row = tid / CH;
  const int ld_chunk = tid % CH;
  const uint32_t ld_voff = (uint32_t)ld_row * row_bytes + (uint32_t)ld_chunk * 16;
  const uint32_t lse_voff = (uint32_t)tid * (uint32_t)p.hq * 4;
  const int head0 = it.kv_head * G;
  // next tile to load: head nx_g of the group, rows from the one nq points at
  const __bf16* nq;
  const __bf16* no;
  const float* nl;
  const float* nd;
  int nx_g, nx_left;                             // nx_left: task rows from the next tile's first row
  auto member_rows = [&]() __attribute__((always_inline)) {
    nq = p.Q + (t.q_off + r_first) * q_stride + head0 * D;
    no = p.dO + (t.o_off + r_first) * q_stride + head0 * D;
    nl = p.LSE + (t.o_off + r_first) * p.hq + head0;
    nd = p.Dvec + (t.o_off + r_first) * p.hq + head0;
    nx_g = 0;
    nx_left = t.q_len - r_first;
  };
  member_rows();
  uint4 qreg[PASSES], oreg[PASSES];
  float lse_reg = 0.f, d_reg = 0.f;
  auto gload = [&]() {
    // nx_left >= 1 here: the last row tile starts below r_end <= q_len
    const uint32_t nvalid = (uint32_t)min(BQ, nx_left);
    const uint32_t qbytes = nvalid * row_bytes;
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(nq + nx_g * D, qbytes);
    const __amdgpu_buffer_rsrc_t orr = make_rsrc(no + nx_g * D, qbytes);
#pragma unroll
    for (int r = 0; r < PASSES; ++r) {
      qreg[r] = buffer_load_16(qr, ld_voff + (uint32_t)(r * RPP) * row_bytes, 0);
      oreg[r] = buffer_load_16(orr, ld_voff + (uint32_t)(r * RPP) * row_bytes, 0);
    }
    const uint32_t lbytes = nvalid * (uint32_t)p.hq * 4;
    const __amdgpu_buffer_rsrc_t lr = make_rsrc(nl + nx_g, lbytes);
    const __amdgpu_buffer_rsrc_t dr = make_rsrc(nd + nx_g, lbytes);
    if (tid < BQ) {
      lse_reg = buffer_load_f32(lr, lse_voff, 0);
      d_reg = buffer_load_f32(dr, lse_voff, 0);
    }
    if (++nx_g == G) {
      nx_g = 0;
      nq += BQ * q_stride;
      no += BQ * q_stride;
      nl += BQ * p.hq;
      nd += BQ * p.hq;
      nx_left -= BQ;
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int r = 0; r < PASSES; ++r) {
      const int o = Tile::off(r * RPP + ld_row, ld_chunk);
      *(uint4*)(&lds_q[buf][o]) = qreg[r];
      *(uint4*)(&lds_do[buf][o]) = oreg[r];
    }
    if (tid < BQ) {
      lds_lse[buf][tid] = lse_log2(lse_reg);
      lds_d[buf][tid] = d_reg;
    }
  };

  // Row-wise operand offsets (A of S and dP: m = query l32, k = 16 s + 8 hh) and
  // transpose-read offsets (Q^T, dO^T: rows 4 hh + j16 / 4 (+8, +16 half),
  // columns 32 c + 16 (g16 & 1) + 4 (j16 & 3)).
  int a_off[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) a_off[s] = Tile::off(l32, 2 * s + hh);
  const int g16 = lane >> 4;
  const int j16 = lane & 15;
  int tr_off[NCB][2];
#pragma unroll
  for (int c = 0; c < NCB; ++c)
#pragma unroll
    for (int u = 0; u < 2; ++u)
      tr_off[c][u] = Tile::off(8 * u + 4 * hh + (j16 >> 2), 4 * c + 2 * (g16 & 1) + ((j16 & 3) >> 1)) + 4 * (j16 & 1);

  // One step: 32 query rows of one head against the wave's 32 keys, in the
  // diagonal band, where a wave may see none or only some of the (row, key)
  // pairs.
  auto diag_body = [&](int buf, int r0) {
    const __bf16* lq = &lds_q[buf][0];
    const __bf16* lo = &lds_do[buf][0];
    bf16x8 qa[NKS], oa[NKS];
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      qa[s] = *(const bf16x8*)(lq + a_off[s]);
      oa[s] = *(const bf16x8*)(lo + a_off[s]);
    }
    // S = Q K^T (lane = key l32; rows m = 8 (j/4) + 4 hh + j%4), dP = dO V^T
    f32x16 s_acc = f32x16_zero(), dp_acc = f32x16_zero();
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      s_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[s], kf[s], s_acc, 0, 0, 0);
      dp_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[s], vf[s], dp_acc, 0, 0, 0);
    }
    bf16x8 dot[2][NCB];
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int c = 0; c < NCB; ++c)
        dot[half][c] = concat_bf16x4(ds_read_tr16(lo + tr_off[c][0] + 16 * half * Tile::kRow),
                                     ds_read_tr16(lo + tr_off[c][1] + 16 * half * Tile::kRow));
    // P = exp2(scale log2e S - LSE2); masked pairs: 0.  Row m (= 8 q4 + 4 hh + j)
    // sees key l32 of the wave iff l32 - 4 hh - (r0 + delta - kw0) <= 8 q4 + j.
    float pv[16];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 l4 = *(const float4*)(&lds_lse[buf][8 * q4 + 4 * hh]);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) pv[4 * q4 + j] = exp2_fast(fmaf(s_acc[4 * q4 + j], p.scale_log2, -lv[j]));
    }
    // With a window, row m also needs m < (l32 - 4 hh) - (r0 + delta - kw0) + win
    // unless key l32 is a sink key.
    const int64_t dd = (int64_t)r0 + delta - kw0;
    const bool win_edge = win > 0 && !(kw0 + 31 < sj || dd + 31 - win < 0);
    if (dd < 31 || win_edge) {
      keep_branch();
      const int x = l32 - 4 * hh - (int)clamp64(dd, -64, 64);
      const int wthr = win > 0 ? (int)clamp64((int64_t)(l32 - 4 * hh) - dd + win, -1, 64) : 64;
      const bool sink_key = kw0 + l32 < sj;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          pv[4 * q4 + j] = (x <= 8 * q4 + j && (8 * q4 + j < wthr || sink_key)) ? pv[4 * q4 + j] : 0.f;
    }
    bf16x8 pf[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) pf[r >> 3][r & 7] = (__bf16)pv[r];
    // dV^T += dO^T P (reduction over the 32 rows)
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int c = 0; c < NCB; ++c)
        dv_acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dot[half][c], pf[half], dv_acc[c], 0, 0, 0);
    // Q^T operands, then dS = P (dP - D) and dK^T += Q^T dS
    bf16x8 qt[2][NCB];
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int c = 0; c < NCB; ++c)
        qt[half][c] = concat_bf16x4(ds_read_tr16(lq + tr_off[c][0] + 16 * half * Tile::kRow),
                                    ds_read_tr16(lq + tr_off[c][1] + 16 * half * Tile::kRow));
    bf16x8 dsf[2];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 d4 = *(const float4*)(&lds_d[buf][8 * q4 + 4 * hh]);
      const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int reg = 4 * q4 + j;
        dsf[reg >> 3][reg & 7] = (__bf16)(pv[reg] * (dp_acc[reg] - dv[j]));
      }
    }
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int c = 0; c < NCB; ++c)
        dk_acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qt[half][c], dsf[half], dk_acc[c], 0, 0, 0);
  };

  // The same step where every (row, key) pair is visible: one basic block in
  // a fixed issue order (sched_barrier fences) for a single wave per SIMD, so
  // that each MFMA runs in the shadow of independent work: the S chain with
  // the dO^T reads, the dP chain with exp(S) and the Q^T reads, the dV chain
  // with dS.
  static_assert(NKS == 2 * NCB && 16 % NKS == 0, "step layout assumes D in {64, 128}");
  auto full_body = [&](int buf) {
    const __bf16* lq = &lds_q[buf][0];
    const __bf16* lo = &lds_do[buf][0];
    bf16x8 qa[NKS], oa[NKS];
#pragma unroll
    for (int s = 0; s < NKS; ++s) qa[s] = *(const bf16x8*)(lq + a_off[s]);
#pragma unroll
    for (int s = 0; s < NKS; ++s) oa[s] = *(const bf16x8*)(lo + a_off[s]);
    float lv[16];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 l4 = *(const float4*)(&lds_lse[buf][8 * q4 + 4 * hh]);
      lv[4 * q4 + 0] = l4.x; lv[4 * q4 + 1] = l4.y; lv[4 * q4 + 2] = l4.z; lv[4 * q4 + 3] = l4.w;
    }
    __builtin_amdgcn_sched_barrier(0);
    // S chain + dO^T reads
    f32x16 s_acc = f32x16_zero(), dp_acc = f32x16_zero();
    bf16x4 dtr[2][NCB][2];
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      s_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[s], kf[s], s_acc, 0, 0, 0);
      const int half = s / NCB, c = s % NCB;
      dtr[half][c][0] = ds_read_tr16(lo + tr_off[c][0] + 16 * half * Tile::kRow);
      dtr[half][c][1] = ds_read_tr16(lo + tr_off[c][1] + 16 * half * Tile::kRow);
      __builtin_amdgcn_sched_barrier(0);
    }
    // dP chain + exp(S) + Q^T reads
    float pv[16];
    bf16x4 qtr[2][NCB][2];
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      dp_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[s], vf[s], dp_acc, 0, 0, 0);
      asm volatile("" : "+v"(dp_acc));   // keep the chain step here (IR passes sink pure calls)
#pragma unroll
      for (int k = 0; k < 16 / NKS; ++k) {
        const int r = s * (16 / NKS) + k;
        pv[r] = exp2_fast(fmaf(s_acc[r], p.scale_log2, -lv[r]));
      }
      const int half = s / NCB, c = s % NCB;
      qtr[half][c][0] = ds_read_tr16(lq + tr_off[c][0] + 16 * half * Tile::kRow);
      qtr[half][c][1] = ds_read_tr16(lq + tr_off[c][1] + 16 * half * Tile::kRow);
      __builtin_amdgcn_sched_barrier(0);
    }
    bf16x8 pf[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) pf[r >> 3][r & 7] = (__bf16)pv[r];
    float dvv[16];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 d4 = *(const float4*)(&lds_d[buf][8 * q4 + 4 * hh]);
      dvv[4 * q4 + 0] = d4.x; dvv[4 * q4 + 1] = d4.y; dvv[4 * q4 + 2] = d4.z; dvv[4 * q4 + 3] = d4.w;
    }
    __builtin_amdgcn_sched_barrier(0);
    // dV chain + dS = P (dP - D)
    bf16x8 dsf[2];
#pragma unroll
    for (int i = 0; i < 2 * NCB; ++i) {
      const int half = i / NCB, c = i % NCB;
      dv_acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(concat_bf16x4(dtr[half][c][0], dtr[half][c][1]), pf[half],
                                                          dv_acc[c], 0, 0, 0);
#pragma unroll
      for (int k = 0; k < 16 / (2 * NCB); ++k) {
        const int r = i * (16 / (2 * NCB)) + k;
        dsf[r >> 3][r & 7] = (__bf16)(pv[r] * (dp_acc[r] - dvv[r]));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // dK chain
#pragma unroll
    for (int i = 0; i < 2 * NCB; ++i) {
      const int half = i / NCB, c = i % NCB;
      dk_acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(concat_bf16x4(qtr[half][c][0], qtr[half][c][1]), dsf[half],
                                                          dk_acc[c], 0, 0, 0);
    }
  };

  // step = (query tile, head of the group), head fastest.  Row tiles before
  // n_diag_rt may hold rows that do not see every key of the workgroup.  With
  // a window, row tiles from n_win_rt on hold rows whose window ends inside the
  // workgroup's keys (and a workgroup holding sink keys is masked
  // throughout).  Steps [n_diag, n_fend) see every key and run the fixed-order
  // body; the rest run the general one.  Steps alternate between the two LDS
  // buffers and run in pairs, so that every LDS address is a lane constant
  // plus an immediate: n_diag is rounded up and n_fend down to even steps
  // (the general body is correct for any step).
  auto sweep = [&]() __attribute__((always_inline)) {
  const int n_diag_rt = (int)clamp64(((int64_t)it.key0 + 127 - delta - r_first + BQ - 1) / BQ, 0, n_rt);
  int n_diag = min(n_steps, (n_diag_rt * G + 1) & ~1);
  int n_fend = n_steps;
  if (!WIN && win > 0) n_diag = n_steps;   // masks without the windowed loop split
  if (WIN && win > 0) {
    if (it.key0 < sj) {
      n_diag = n_steps;
    } else {
      const int64_t x = (int64_t)it.key0 - delta + win - BQ - r_first;   // last full row tile start - r_first
      const int n_win_rt = x < 0 ? 0 : (int)min<int64_t>(x / BQ + 1, n_rt);
      n_fend = max(n_diag, min(n_steps, (n_win_rt * G) & ~1));
    }
  }
  int cur_g = 0, cur_r0 = r_first;
  auto do_step = [&](auto buf_tag, auto diag_tag, int step) {
    constexpr int BUF = decltype(buf_tag)::value;
    constexpr bool DIAG = decltype(diag_tag)::value;
    const int r0 = cur_r0;
    swrite(BUF);
    __syncthreads();
    if (++cur_g == G) {
      cur_g = 0;
      cur_r0 += BQ;
    }
    if (step + 1 < n_steps) gload();
    if constexpr (DIAG) {
      // Skip blocks where no row of the step sees any key of this wave: all
      // keys after the last row, or (window) all before the first row's
      // window and none of them a sink key.
      if ((int64_t)r0 + BQ - 1 + delta < kw0) return;
      if (win > 0 && kw0 >= sj && (int64_t)r0 + delta - win + 1 > (int64_t)kw0 + 31) return;
      diag_body(BUF, r0);
    } else {
      full_body(BUF);
    }
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  int step = 0;
  if (n_steps > 0) gload();
  for (; step + 1 < n_diag; step += 2) {
    do_step(B0{}, std::true_type{}, step);
    do_step(B1{}, std::true_type{}, step + 1);
  }
  if (step < n_diag) {                          // odd step count, all in the band
    do_step(B0{}, std::true_type{}, step);
    ++step;
  }
  if constexpr (WIN) {
    for (; step + 1 < n_fend; step += 2) {
      do_step(B0{}, std::false_type{}, step);
      do_step(B1{}, std::false_type{}, step + 1);
    }
    if (step < n_fend) {                        // odd count: the last step of all
      do_step(B0{}, std::false_type{}, step);
      ++step;
    }
    for (; step + 1 < n_steps; step += 2) {     // window edge
      do_step(B0{}, std::true_type{}, step);
      do_step(B1{}, std::true_type{}, step + 1);
    }
    if (step < n_steps) do_step(B0{}, std::true_type{}, step);
  } else {
    for (; step + 1 < n_steps; step += 2) {
      do_step(B0{}, std::false_type{}, step);
      do_step(B1{}, std::false_type{}, step + 1);
    }
    if (step < n_steps) do_step(B0{}, std::false_type{}, step);
  }
  };
  sweep();
  if constexpr (MULTI) {
    // the group's further tasks: dK and dV keep accumulating
    for (int k = 1; k < it.n_members; ++k) {
      __syncthreads();   // the previous task's last step may still be read from LDS
      task_idx = p.members[it.member0 + k];
      t = p.tasks[task_idx];
      delta = t.q_pos0 - t.kv_pos0;
      member();
      member_rows();
      sweep();
    }
  }

  // Epilogue: lane = key l32, channels c*32 + 8 (j/4) + 4 hh + j%4.
  if (!key_ok) return;
  if constexpr (MULTI) {
    if (it.slot >= 0) {
      // a split item: fp32 partials of its 128 keys, summed by kv_reduce_kernel
      const int64_t sb = ((int64_t)it.slot * 128 + (my_key - it.key0)) * D;
#pragma unroll
      for (int c = 0; c < NCB; ++c)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int ch = c * 32 + 8 * q4 + 4 * hh;
          const f32x16& a = dk_acc[c];
          const f32x16& b = dv_acc[c];
          *(float4*)(p.slot_k + sb + ch) = make_float4(a[4 * q4] * p.scale, a[4 * q4 + 1] * p.scale,
                                                       a[4 * q4 + 2] * p.scale, a[4 * q4 + 3] * p.scale);
          *(float4*)(p.slot_v + sb + ch) = make_float4(b[4 * q4], b[4 * q4 + 1], b[4 * q4 + 2], b[4 * q4 + 3]);
        }
      return;
    }
  }
  const int64_t base = (kv_row0 + my_key) * kv_stride + it.kv_head * D;
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int ch = c * 32 + 8 * q4 + 4 * hh;
      float k4[4], v4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        k4[j] = dk_acc[c][4 * q4 + j] * p.scale;
        v4[j] = dv_acc[c][4 * q4 + j];
      }
      if (p.accumulate) {
        float* ka = p.dKacc + base + ch;
        float* va = p.dVacc + base + ch;
        float4 ko = *(float4*)ka, vo = *(float4*)va;
        *(float4*)ka = make_float4(ko.x + k4[0], ko.y + k4[1], ko.z + k4[2], ko.w + k4[3]);
        *(float4*)va = make_float4(vo.x + v4[0], vo.y + v4[1], vo.z + v4[2], vo.w + v4[3]);
      } else {
        bf16x4 kb, vb;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          kb[j] = (__bf16)k4[j];
          vb[j] = (__bf16)v4[j];
        }
        *(bf16x4*)(p.dK + base + ch) = kb;
        *(bf16x4*)(p.dV + base + ch) = vb;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dQ: work items as in the forward (hpw heads x 8/hpw blocks of 32 rows),
// eight waves, two per SIMD: while one wave runs its exponentials and dS the
// other's MFMAs proceed.  That needs at most 256 registers per wave, so the
// dO^T operands stay in LDS (the wave's own rows, read per tile) instead of
// registers; each tile runs one body, operands read as the MFMAs need them:
// the S^T chain, then the dP^T chain with S's exponentials under it (0.6-0.9 %
// faster than the two chains interleaved), then dS and dQ.  One wave per SIMD
// with every operand in registers and a fixed issue order was 4-5 % slower on
// the 512K and CA-task backward.
// ---------------------------------------------------------------------------
template <int D, bool PAGED, bool MULTI>
__global__ __launch_bounds__(512, 1) void bwd_q_kernel(BwdParams p) {
  constexpr int NWQ = 8;          // waves
  constexpr int BN = 64;
  constexpr int KS = D + 32;      // K row stride: rows rotated by (row / 4) % 4 chunks (below)
  constexpr int VS = D + 8;       // V is read row-wise only
  constexpr int NCB = D / 32;
  constexpr int NKS = D / 16;
  constexpr int CH = D / 8;
  constexpr int RPP = 64 * NWQ / CH;
  constexpr int PASSES = BN / RPP;
  __shared__ __attribute__((aligned(16))) __bf16 lds_k[2][BN * KS];
  __shared__ __attribute__((aligned(16))) __bf16 lds_v[2][BN * VS];
  // K tile rows are read row-wise (16 lanes, one 16-byte chunk each) and by
  // transpose reads (4 rows x 4 chunks per 16 lanes); a stride of D + 32 and
  // a rotation of (row / 4) % 4 chunks keep both free of bank conflicts, and
  // every address a lane constant plus an immediate.
  auto krot = [](int row) { return ((row >> 2) & 3) * 8; };
  constexpr int DS = D + 8;       // dO row stride in LDS (elements)
  __shared__ __attribute__((aligned(16))) __bf16 lds_do[NWQ * 32 * DS];   // each wave's dO rows

  const FwdItem it = p.qitems[blockIdx.x];
  // The item's query shard: tasks it.task .. it.task + n_seg - 1 share the
  // query rows; t is the context being swept (the only one unless MULTI).
  ca_task t = p.tasks[it.task];
  int task_idx = it.task;
  const int tid = threadIdx.x;
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int hpw = p.hpw;
  const int head = it.kv_head * p.group + it.head_sub * hpw + (wave_u % hpw);
  const int wrow0 = it.row0 + (wave_u / hpw) * 32;
  const int rt = 32 * (NWQ / hpw);
  const int wg_last = min(it.row0 + rt, t.q_len) - 1;
  const int w_last = min(wrow0 + 32, t.q_len) - 1;
  int64_t delta;
  int kv_len, kv_hi, w_kv_hi, w_full;
  auto context = [&]() __attribute__((always_inline)) {
    delta = t.q_pos0 - t.kv_pos0;
    kv_len = t.kv_len;
    kv_hi = (int)clamp64((int64_t)wg_last + delta + 1, 0, kv_len);
    w_kv_hi = (w_last < wrow0) ? 0 : (int)clamp64((int64_t)w_last + delta + 1, 0, kv_len);
    w_full = (int)clamp64(((int64_t)wrow0 + delta + 1) / BN, 0, (kv_len / BN));
  };
  context();

  const int qrow = wrow0 + l32;
  const bool qvalid = qrow < t.q_len;
  const int64_t q_stride = (int64_t)p.hq * D;
  bf16x8 qf[NKS];
  // dO^T operands: this lane's query row, channels 16 s + 8 hh .. + 7, in
  // the wave's own LDS rows (no barrier: written and read by the same wave).
  const int do_off = (wave_u * 32 + l32) * DS + 8 * hh;
  {
    const __bf16* qp = p.Q + (t.q_off + qrow) * q_stride + head * D + 8 * hh;
    const __bf16* op = p.dO + (t.o_off + qrow) * q_stride + head * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      qf[s] = qvalid ? *(const bf16x8*)(qp + 16 * s) : bf16x8_zero();
      *(bf16x8*)(&lds_do[do_off + 16 * s]) = qvalid ? *(const bf16x8*)(op + 16 * s) : bf16x8_zero();
    }
  }
  const float lse2 = qvalid ? lse_log2(p.LSE[(t.o_off + qrow) * p.hq + head]) : INFINITY;
  const float dval = qvalid ? p.Dvec[(t.o_off + qrow) * p.hq + head] : 0.f;

  f32x16 dq_acc[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) dq_acc[c] = f32x16_zero();

  int n_tiles = (kv_hi + BN - 1) / BN;
  const int64_t kv_stride = (int64_t)p.hkv * D;
  const uint32_t row_bytes = (uint32_t)(kv_stride * 2);
  const __bf16* kbase = p.K + it.kv_head * D;
  const __bf16* vbase = p.V + it.kv_head * D;
  const int ld_row = tid / CH;
  const int ld_chunk = tid % CH;
  const uint32_t ld_voff = (uint32_t)ld_row * row_bytes + (uint32_t)ld_chunk * 16;
  uint4 kreg[PASSES], vreg[PASSES];
  // Paged K/V: a tile's physical page is read one tile ahead (vector load,
  // waited on in order with the tile loads) and moved to a scalar register
  // where the loads need it; 64-key tiles lie inside one page.
  const __amdgpu_buffer_rsrc_t prs = make_rsrc(p.pages, p.page_bytes);
  auto tile_page = [&](int tile) -> int {
    if constexpr (PAGED) {
      const int64_t v = t.kv_off + (int64_t)tile * BN;
      return __builtin_amdgcn_raw_buffer_load_b32(prs, (uint32_t)(v >> p.page_shift) * 4u, 0, 0);
    } else {
      return 0;
    }
  };
  // rows >= kv_hi read as zeros; nothing past the context is read
  auto gload = [&](int tile, int page) {
    int64_t r0 = t.kv_off + (int64_t)tile * BN;
    if constexpr (PAGED) {
      const int64_t pg = __builtin_amdgcn_readfirstlane(page);
      r0 = (pg << p.page_shift) | (r0 & ((int64_t(1) << p.page_shift) - 1));
    }
    const int n = min(BN, kv_hi - tile * BN);
    const __amdgpu_buffer_rsrc_t krs = rows_rsrc(kbase + r0 * kv_stride, n, row_bytes);
    const __amdgpu_buffer_rsrc_t vrs = rows_rsrc(vbase + r0 * kv_stride, n, row_bytes);
#pragma unroll
    for (int r = 0; r < PASSES; ++r) {
      kreg[r] = buffer_load_16(krs, ld_voff + (uint32_t)(r * RPP) * row_bytes, 0);
      vreg[r] = buffer_load_16(vrs, ld_voff + (uint32_t)(r * RPP) * row_bytes, 0);
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int r = 0; r < PASSES; ++r) {
      const int row = r * RPP + ld_row;
      *(uint4*)(&lds_k[buf][row * KS + ld_chunk * 8 + krot(row)]) = kreg[r];
      *(uint4*)(&lds_v[buf][row * VS + ld_chunk * 8]) = vreg[r];
    }
  };
  const int k_row_off = l32 * KS + 8 * hh + krot(l32);   // A of S^T  (key l32, ch 16 s + 8 hh)
  const int v_row_off = l32 * VS + 8 * hh;       // A of dP^T (key l32, ch 16 s + 8 hh)
  const int g16 = lane >> 4;
  const int j16 = lane & 15;
  // K^T reads: rows kb + j16 / 4 + 4 hh (kb a multiple of 16), rotated by hh
  // chunks; the second read, 8 rows on, by hh + 2
  const int kt_off = ((j16 >> 2) + 4 * hh) * KS + 16 * (g16 & 1) + 4 * (j16 & 3) + 8 * hh;

  // Sink + sliding-window mask (win > 0): as in the forward, the workgroup
  // visits the sink tiles [0, t_a) and the window tiles [t_b, n_tiles).
  int win, sj, t_a, t_b, n_visit;
  int64_t w_lo_first, w_lo_last;
  auto context_tiles = [&]() __attribute__((always_inline)) {
    win = 0;
    sj = 0;
    if (p.masks) {
      win = p.masks[task_idx].window;
      if (win > 0) sj = (int)clamp64((int64_t)p.masks[task_idx].sink - t.kv_pos0, 0, kv_len);
    }
    w_lo_first = (int64_t)wrow0 + delta - win + 1;
    w_lo_last = (int64_t)w_last + delta - win + 1;
    t_a = 0;
    t_b = 0;
    if (win > 0) {
      t_a = min((sj + BN - 1) / BN, n_tiles);
      t_b = min(max(t_a, (int)(clamp64((int64_t)it.row0 + delta - win + 1, 0, kv_len) / BN)), n_tiles);
    }
    n_visit = t_a + (n_tiles - t_b);
  };
  context_tiles();
  auto tile_of = [&](int k) { return k < t_a ? k : t_b + (k - t_a); };
  auto wave_sees = [&](int tile) {
    if (tile * BN >= w_kv_hi) return false;
    return win == 0 || tile * BN < sj || (int64_t)(tile + 1) * BN > w_lo_first;
  };
  auto needs_mask = [&](int tile) {
    if (tile >= w_full) return true;
    return win > 0 && !((tile + 1) * BN <= sj || (int64_t)tile * BN >= w_lo_last);
  };
  auto sweep = [&]() __attribute__((always_inline)) {
  auto body = [&](int buf, int tile) {
    const int k0 = tile * BN;
    if (!wave_sees(tile)) return;
    f32x16 s_acc[2], dp_acc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      s_acc[mb] = f32x16_zero();
      dp_acc[mb] = f32x16_zero();
    }
    int od = do_off;
    asm volatile("" : "+v"(od));   // dO^T read per tile, not hoisted into registers
#pragma unroll
    for (int s = 0; s < NKS; ++s)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const bf16x8 ka = *(const bf16x8*)(&lds_k[buf][k_row_off + mb * 32 * KS + 16 * s]);
        s_acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[s], s_acc[mb], 0, 0, 0);
      }
    __builtin_amdgcn_sched_barrier(0);
    float pv[2][16];
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const bf16x8 ob = *(const bf16x8*)(&lds_do[od + 16 * s]);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const bf16x8 va = *(const bf16x8*)(&lds_v[buf][v_row_off + mb * 32 * VS + 16 * s]);
        dp_acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, ob, dp_acc[mb], 0, 0, 0);
      }
      // exponentials of S under the dP chain: 4 per step
#pragma unroll
      for (int k = 0; k < 32 / NKS; ++k) {
        const int e = s * (32 / NKS) + k;
        pv[e >> 4][e & 15] = exp2_fast(fmaf(s_acc[e >> 4][e & 15], p.scale_log2, -lse2));
      }
    }
    if (needs_mask(tile)) {
      keep_branch();
      const int lim = (int)clamp64(min((int64_t)qrow + delta, (int64_t)kv_len - 1) - k0, -1, BN);
      const int wlo = win > 0 ? (int)clamp64((int64_t)qrow + delta - win + 1 - k0, -1, BN + 1) : -1;
      const int slim = (int)clamp64((int64_t)sj - k0, 0, BN);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int r = mb * 32 + 8 * (j >> 2) + 4 * hh + (j & 3);
          pv[mb][j] = (r <= lim && (r >= wlo || r < slim)) ? pv[mb][j] : 0.f;
        }
    }
    bf16x8 dsf[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) dsf[mb][j >> 3][j & 7] = (__bf16)(pv[mb][j] * (dp_acc[mb][j] - dval));
    // dQ^T += K^T dS^T (K^T through transpose reads, keys permuted like dS^T)
    const __bf16* kl = &lds_k[buf][kt_off];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int kb = mb * 32 + 16 * half;
#pragma unroll
        for (int c = 0; c < NCB; ++c) {
          const __bf16* a0 = kl + kb * KS + c * 32;
          const bf16x8 kt = concat_bf16x4(ds_read_tr16(a0), ds_read_tr16(a0 + 8 * KS + 16));
          dq_acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt, dsf[mb][half], dq_acc[c], 0, 0, 0);
        }
      }
    };

  int next_page = 0;
  // k indexes the visited tiles; tiles run in LDS-buffer pairs so that every
  // LDS address is a lane constant plus an immediate.
  auto do_tile = [&](auto buf_tag, int k) {
    constexpr int BUF = decltype(buf_tag)::value;
    swrite(BUF);
    __syncthreads();
    if (k + 1 < n_visit) {
      gload(tile_of(k + 1), next_page);
      if (k + 2 < n_visit) next_page = tile_page(tile_of(k + 2));
    }
    body(BUF, tile_of(k));
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  int k = 0;
  if (n_visit > 0) gload(tile_of(0), tile_page(tile_of(0)));
  if (n_visit > 1) next_page = tile_page(tile_of(1));
  for (; k + 1 < n_visit; k += 2) {
    do_tile(B0{}, k);
    do_tile(B1{}, k + 1);
  }
  if (k < n_visit) do_tile(B0{}, k);
  };
  sweep();
  if constexpr (MULTI) {
    // the shard's further contexts: dQ keeps accumulating
    for (int sg = 1; sg < it.n_seg; ++sg) {
      __syncthreads();   // the previous context's last tile may still be read from LDS
      task_idx = it.task + sg;
      t = p.tasks[task_idx];
      context();
      n_tiles = (kv_hi + BN - 1) / BN;
      context_tiles();
      sweep();
    }
  }

  if (!qvalid) return;
  if constexpr (MULTI) {
    if (it.stage_row >= 0) {
      // a key chunk of a split shard: fp32 partial dQ to staging, summed by
      // dq_reduce_kernel
      float* sq = p.stage_dQ + ((int64_t)it.stage_row + qrow) * q_stride + head * D;
#pragma unroll
      for (int c = 0; c < NCB; ++c)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *(float4*)(sq + c * 32 + 8 * q4 + 4 * hh) =
              make_float4(dq_acc[c][4 * q4] * p.scale, dq_acc[c][4 * q4 + 1] * p.scale,
                          dq_acc[c][4 * q4 + 2] * p.scale, dq_acc[c][4 * q4 + 3] * p.scale);
      return;
    }
  }
  const int64_t base = (t.q_off + qrow) * q_stride + head * D;
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int ch = c * 32 + 8 * q4 + 4 * hh;
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = dq_acc[c][4 * q4 + j] * p.scale;
      if (p.accumulate) {
        float* a = p.dQacc + base + ch;
        const float4 o = *(float4*)a;
        *(float4*)a = make_float4(o.x + v[0], o.y + v[1], o.z + v[2], o.w + v[3]);
      } else {
        bf16x4 b;
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = (__bf16)v[j];
        *(bf16x4*)(p.dQ + base + ch) = b;
      }
    }
  }
}

// dK, dV of split (tile, KV head) pairs: the sum of their partial slots,
// added in slot order (deterministic), written as bf16 or added into the
// fp32 accumulators.  One thread per (record, key, 4 channels).
template <int D>
__global__ __launch_bounds__(256) void kv_reduce_kernel(const KvReduce* recs, int32_t n_recs, const float* slot_k,
                                                        const float* slot_v, __bf16* dK, __bf16* dV, float* dKacc,
                                                        float* dVacc, int accumulate, int hkv) {
  constexpr int C4 = D / 4;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rec = g / (128 * C4);
  if (rec >= n_recs) return;
  const KvReduce r = recs[rec];
  const int key = (int)((g / C4) % 128);
  const int c4 = (int)(g % C4);
  if (key >= r.n_keys) return;
  float4 sk = make_float4(0.f, 0.f, 0.f, 0.f), sv = sk;
  for (int k = 0; k < r.n_slots; ++k) {
    const int64_t o = ((int64_t)(r.slot0 + k) * 128 + key) * D + 4 * c4;
    const float4 a = *(const float4*)(slot_k + o), b = *(const float4*)(slot_v + o);
    sk.x += a.x; sk.y += a.y; sk.z += a.z; sk.w += a.w;
    sv.x += b.x; sv.y += b.y; sv.z += b.z; sv.w += b.w;
  }
  const int64_t base = (r.row0 + key) * (int64_t)hkv * D + (int64_t)r.kv_head * D + 4 * c4;
  if (accumulate) {
    float4 ko = *(float4*)(dKacc + base), vo = *(float4*)(dVacc + base);
    *(float4*)(dKacc + base) = make_float4(ko.x + sk.x, ko.y + sk.y, ko.z + sk.z, ko.w + sk.w);
    *(float4*)(dVacc + base) = make_float4(vo.x + sv.x, vo.y + sv.y, vo.z + sv.z, vo.w + sv.w);
  } else {
    bf16x4 kb, vb;
    kb[0] = (__bf16)sk.x; kb[1] = (__bf16)sk.y; kb[2] = (__bf16)sk.z; kb[3] = (__bf16)sk.w;
    vb[0] = (__bf16)sv.x; vb[1] = (__bf16)sv.y; vb[2] = (__bf16)sv.z; vb[3] = (__bf16)sv.w;
    *(bf16x4*)(dK + base) = kb;
    *(bf16x4*)(dV + base) = vb;
  }
}

// dQ of split shards: the sum of the key chunks' partials, in chunk order
// (deterministic), written as bf16 or added into the fp32 accumulator.
// blockIdx.y = shard; one thread per (row, head, 4 channels).
template <int D>
__global__ __launch_bounds__(256) void dq_reduce_kernel(const ShardMerge* recs, const float* stage_dQ, __bf16* dQ,
                                                        float* dQacc, int accumulate, int hq) {
  constexpr int C4 = D / 4;
  const ShardMerge r = recs[blockIdx.y];
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= (int64_t)r.q_len * hq * C4) return;
  const int64_t pair = g / C4;                  // (row, head) of the shard
  const int c4 = (int)(g % C4);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k = 0; k < r.n_chunks; ++k) {
    const float4 v = *(const float4*)(stage_dQ + ((r.stage_row0 + (int64_t)k * r.q_len) * hq + pair) * D + 4 * c4);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  const int64_t at = (r.o_off * hq + pair) * D + 4 * c4;
  if (accumulate) {
    const float4 o = *(float4*)(dQacc + at);
    *(float4*)(dQacc + at) = make_float4(o.x + acc.x, o.y + acc.y, o.z + acc.z, o.w + acc.w);
  } else {
    bf16x4 b;
    b[0] = (__bf16)acc.x; b[1] = (__bf16)acc.y; b[2] = (__bf16)acc.z; b[3] = (__bf16)acc.w;
    *(bf16x4*)(dQ + at) = b;
  }
}

hipError_t launch_dq_reduce(const ShardMerge* recs, int32_t n_recs, int32_t max_q_len, const float* stage_dQ,
                            __bf16* dQ, float* dQacc, int accumulate, int hq, int d, hipStream_t s) {
  if (n_recs <= 0) return hipSuccess;
  const int64_t threads = (int64_t)max_q_len * hq * (d / 4);
  const dim3 grid((unsigned)((threads + 255) / 256), (unsigned)n_recs);
  if (d == 128)
    hipLaunchKernelGGL(dq_reduce_kernel<128>, grid, dim3(256), 0, s, recs, stage_dQ, dQ, dQacc, accumulate, hq);
  else
    hipLaunchKernelGGL(dq_reduce_kernel<64>, grid, dim3(256), 0, s, recs, stage_dQ, dQ, dQacc, accumulate, hq);
  return hipGetLastError();
}

hipError_t launch_kv_reduce(const KvReduce* recs, int32_t n_recs, const float* slot_k, const float* slot_v,
                            __bf16* dK, __bf16* dV, float* dKacc, float* dVacc, int accumulate, int hkv, int d,
                            hipStream_t s) {
  if (n_recs <= 0) return hipSuccess;
  const int64_t threads = (int64_t)n_recs * 128 * (d / 4);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  if (d == 128)
    hipLaunchKernelGGL(kv_reduce_kernel<128>, dim3(blocks), dim3(256), 0, s, recs, n_recs, slot_k, slot_v, dK, dV,
                       dKacc, dVacc, accumulate, hkv);
  else
    hipLaunchKernelGGL(kv_reduce_kernel<64>, dim3(blocks), dim3(256), 0, s, recs, n_recs, slot_k, slot_v, dK, dV,
                       dKacc, dVacc, accumulate, hkv);
  return hipGetLastError();
}

__global__ void f32_to_bf16_kernel(const float* src, __bf16* dst, int64_t n) {
  const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i4 + 3 < n) {
    const float4 v = *(const float4*)(src + i4);
    bf16x4 b;
    b[0] = (__bf16)v.x; b[1] = (__bf16)v.y; b[2] = (__bf16)v.z; b[3] = (__bf16)v.w;
    *(bf16x4*)(dst + i4) = b;
  } else {
    for (int64_t i = i4; i < n; ++i) dst[i] = (__bf16)src[i];
  }
}

hipError_t launch_bwd_prep(const __bf16* O, const __bf16* dO, float* Dv, int64_t n_pairs, int d, hipStream_t s) {
  if (n_pairs <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n_pairs * 16 + 255) / 256);
  if (d == 128)
    hipLaunchKernelGGL(bwd_prep_kernel<128>, dim3(blocks), dim3(256), 0, s, O, dO, Dv, n_pairs);
  else
    hipLaunchKernelGGL(bwd_prep_kernel<64>, dim3(blocks), dim3(256), 0, s, O, dO, Dv, n_pairs);
  return hipGetLastError();
}

// MULTI: calls with query shards over several contexts or context groups of
// several tasks; all others run the single-task kernels.
template <int D, bool PAGED, bool WIN>
hipError_t launch_bwd_kv_dpw(const BwdParams& p, hipStream_t s) {
  if (p.multi)
    hipLaunchKernelGGL((bwd_kv_kernel<D, PAGED, WIN, true>), dim3(p.n_items), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((bwd_kv_kernel<D, PAGED, WIN, false>), dim3(p.n_items), dim3(256), 0, s, p);
  return hipGetLastError();
}

// WIN: the loop split for sink + sliding-window masks, taken when the call
// has masks; calls without masks run the variant without it.
template <int D, bool PAGED>
hipError_t launch_bwd_kv_dp(const BwdParams& p, hipStream_t s) {
  return p.masks ? launch_bwd_kv_dpw<D, PAGED, true>(p, s) : launch_bwd_kv_dpw<D, PAGED, false>(p, s);
}

template <int D>
hipError_t launch_bwd_kv_d(const BwdParams& p, hipStream_t s) {
  return p.pages ? launch_bwd_kv_dp<D, true>(p, s) : launch_bwd_kv_dp<D, false>(p, s);
}

template <int D, bool PAGED>
hipError_t launch_bwd_q_dp(const BwdParams& p, hipStream_t s) {
  if (p.multi)
    hipLaunchKernelGGL((bwd_q_kernel<D, PAGED, true>), dim3(p.n_qitems), dim3(512), 0, s, p);
  else
    hipLaunchKernelGGL((bwd_q_kernel<D, PAGED, false>), dim3(p.n_qitems), dim3(512), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_q_d(const BwdParams& p, hipStream_t s) {
  return p.pages ? launch_bwd_q_dp<D, true>(p, s) : launch_bwd_q_dp<D, false>(p, s);
}

hipError_t launch_bwd_kv(const BwdParams& p, int d, hipStream_t s) {
  if (p.n_items <= 0) return hipSuccess;
  return d == 128 ? launch_bwd_kv_d<128>(p, s) : launch_bwd_kv_d<64>(p, s);
}

hipError_t launch_bwd_q(const BwdParams& p, int d, hipStream_t s) {
  if (p.n_qitems <= 0) return hipSuccess;
  return d == 128 ? launch_bwd_q_d<128>(p, s) : launch_bwd_q_d<64>(p, s);
}

hipError_t launch_f32_to_bf16(const float* src, __bf16* dst, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n / 4 + 256) / 256);
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3(blocks), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}

}  // namespace ca
