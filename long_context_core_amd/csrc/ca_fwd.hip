// K1 — fused core-attention forward over a CA-task table (gfx950).
//
// A workgroup (8 waves, two per SIMD) runs a work item: 256 (query row, head)
// pairs that all read the same KV head — hpw heads x (8 / hpw) blocks of 32
// rows — so each K/V tile staged in LDS feeds eight MFMA streams.  Either one
// workgroup per item, or (PERSIST) one resident workgroup per compute unit
// claiming items from its XCD's share of the queue and loading the next
// item's Q and first tiles under the current item's epilogue.  Per 64-key
// tile a wave:
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
// Paged K/V (PAGED): K and V are stores of pages of 2^page_shift rows and a
// task's context rows are virtual; virtual row v lives in physical page
// pages[v >> page_shift] at the same row within the page (block tables:
// "DCP: Addressing Input Dynamism In Long-Context Training via Dynamic
// Context Parallelism", Executor Design, the Blockwise Attention
// instruction).  Pages hold a multiple of 128 rows and contexts start on a
// 128-row boundary, so every 64-key tile lies inside one page.
//
// Query shards over several contexts (MULTI): consecutive tasks with the
// same query rows are swept one after another by the same online softmax,
// so the item attends to the union of their keys (the causal-blockwise and
// shared-question masks of "DCP: Addressing Input Dynamism In Long-Context
// Training via Dynamic Context Parallelism", Section 2.4, Figure 6c / 6d).
//
// Outputs: O (bf16, or fp32 partials) and LSE = ln sum exp(scale q.k), the
// statistic that makes partials mergeable by Equation 4 ("Context Parallelism
// for Scalable Million-Token Inference", Section 3.4 Merge Attention).

#include "ca_internal.h"
#include "ca_kernel_util.h"

namespace ca {

// Row statistics are kept relative to a running max m2 that is only raised
// when some row's max grows by more than kRescaleLog2 (in log2 units); until
// then probabilities may reach 2^kRescaleLog2, which fp32 accumulators and
// bf16 operands hold exactly in range.  O and the row sum share the same
// reference, so the final O = acc / l and LSE = ln2 (m2 + log2 l) are exact
// regardless of when the reference moved.
constexpr float kRescaleLog2 = 8.0f;

template <int D, int NW, bool PAGED, bool MULTI, bool PERSIST>
__global__ __launch_bounds__(64 * NW, 8 / NW) void fwd_kernel(FwdParams p) {
  constexpr int NT = 64 * NW;     // threads
  constexpr int BN = 64;          // keys per tile
  constexpr int KS = D + 8;       // K row stride in LDS (elements): 16 B pad
  constexpr int VS = D + 32;      // V row stride in LDS (elements): 64 B pad, no transpose-read conflicts
  constexpr int NCB = D / 32;     // 32-channel output blocks
  constexpr int NKS = D / 16;     // 16-channel reduction steps of Q.K
  constexpr int CH = D / 8;       // 16-byte chunks per row
  constexpr int RPP = NT / CH;    // rows per load pass
  constexpr int PASSES = BN / RPP;

  __shared__ __attribute__((aligned(16))) __bf16 lds_k[2][BN * KS];
  __shared__ __attribute__((aligned(16))) __bf16 lds_v[2][BN * VS];

  // PERSIST: n_slots resident workgroups (a multiple of 8).  Workgroups are
  // dealt to the 8 XCDs in turn, so workgroup b runs on XCD x = b % 8; it
  // starts with item b and then claims, from XCD x's counter, the next
  // unclaimed item of x's share of the longest-first queue (items x, x + 8,
  // x + 16, ...: the share the one-item-per-workgroup launch also gives x,
  // which keeps each XCD's L2 on its own KV heads).  The claim for the next
  // item is taken when an item starts (its latency hides under the item), and
  // the claimed item's loads are issued before this item's epilogue.
  // Otherwise item b alone.  lds_next[parity]: the claimed item, written by
  // thread 0 and read by every wave after the item's last barrier.
  __shared__ int32_t lds_next[2];
  int parity = 0;
  const int tid = threadIdx.x;
  const int xcd = blockIdx.x & 7;
  uint32_t claim = 0;
  auto claimed_item = [&]() { return (int32_t)(xcd + 8 * (claim + (uint32_t)(p.n_slots >> 3))); };
  if constexpr (PERSIST) {
    if (tid == 0) claim = atomicAdd(p.counter + xcd, 1u);
  }
  FwdItem it = p.items[blockIdx.x];
  // The item's query shard: tasks it.task .. it.task + n_seg - 1 share the
  // query rows; t is the context being swept (the only one unless MULTI).
  ca_task t = p.tasks[it.task];
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;       // half-wave

  const int hpw = p.hpw;
  // wave-uniform values, kept in scalar registers
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int rt = 32 * (NW / hpw);
  int head, wrow0, wg_last, w_last;
  auto item_rows = [&]() __attribute__((always_inline)) {
    head = it.kv_head * p.group + it.head_sub * hpw + (wave_u % hpw);
    wrow0 = it.row0 + (wave_u / hpw) * 32;
    wg_last = min(it.row0 + rt, t.q_len) - 1;
    w_last = min(wrow0 + 32, t.q_len) - 1;
  };
  item_rows();

  // Per context: the key range of the workgroup and of this wave; tiles
  // [0, w_full) are visible to every row of the wave (no mask).  Sink +
  // sliding-window mask (win > 0): besides being causal, key j must lie
  // within the row's win latest positions (j > i + delta - win) or be one of
  // the sink keys [0, sj).  The workgroup visits the sink tiles [0, t_a) and
  // the window tiles [t_b, n_tiles); win == 0 visits [0, n_tiles).
  int64_t delta, w_lo_first, w_lo_last;   // window starts of the wave's first and last rows
  int kv_len, kv_hi, w_kv_hi, w_full, win, sj;
  auto context = [&](int task_idx) __attribute__((always_inline)) {
    delta = t.q_pos0 - t.kv_pos0;
    kv_len = t.kv_len;
    kv_hi = (int)clamp64((int64_t)wg_last + delta + 1, 0, kv_len);
    w_kv_hi = (w_last < wrow0) ? 0 : (int)clamp64((int64_t)w_last + delta + 1, 0, kv_len);
    w_full = (int)clamp64(((int64_t)wrow0 + delta + 1) / BN, 0, (kv_len / BN));
    win = 0;
    sj = 0;
    if (p.masks) {
      if constexpr (PERSIST) {
        const ca_task_mask mk = wave_uniform(p.masks[task_idx]);
        win = mk.window;
        if (win > 0) sj = (int)clamp64((int64_t)mk.sink - t.kv_pos0, 0, kv_len);
      } else {
        win = p.masks[task_idx].window;
        if (win > 0) sj = (int)clamp64((int64_t)p.masks[task_idx].sink - t.kv_pos0, 0, kv_len);
      }
    }
    w_lo_first = (int64_t)wrow0 + delta - win + 1;
    w_lo_last = (int64_t)w_last + delta - win + 1;
  };
  context(it.task);

  // Q^T operand: this lane's query row, channels 16 s + 8 hh .. + 7.
  int qrow;
  bool qvalid;
  bf16x8 qf[NKS];
  auto load_q = [&]() __attribute__((always_inline)) {
    qrow = wrow0 + l32;
    qvalid = qrow < t.q_len;
    const __bf16* qp = p.Q + (t.q_off + qrow) * (int64_t)(p.hq * D) + head * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < NKS; ++s) qf[s] = qvalid ? *(const bf16x8*)(qp + 16 * s) : bf16x8_zero();
  };
  load_q();

  f32x16 o_acc[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) o_acc[c] = f32x16_zero();
  float m2 = -INFINITY;   // reference max, log2 units
  float lsum = 0.f;       // sum of exp2(s * c - m2)

  int n_tiles, t_a, t_b, n_visit;
  auto context_tiles = [&]() __attribute__((always_inline)) {
    n_tiles = (kv_hi + BN - 1) / BN;
    t_a = 0;
    t_b = 0;
    if (win > 0) {
      t_a = min((sj + BN - 1) / BN, n_tiles);
      t_b = max(t_a, (int)(clamp64((int64_t)it.row0 + delta - win + 1, 0, kv_len) / BN));
      t_b = min(t_b, n_tiles);
    }
    n_visit = t_a + (n_tiles - t_b);
  };
  context_tiles();
  auto tile_of = [&](int k) { return k < t_a ? k : t_b + (k - t_a); };
  // Does this wave see any key of the tile, and does every row see all of it?
  auto wave_sees = [&](int tile) {
    if (tile * BN >= w_kv_hi) return false;
    return win == 0 || tile * BN < sj || (int64_t)(tile + 1) * BN > w_lo_first;
  };
  auto needs_mask = [&](int tile) {
    if (tile >= w_full) return true;
    return win > 0 && !((tile + 1) * BN <= sj || (int64_t)tile * BN >= w_lo_last);
  };
  const int64_t kv_stride = (int64_t)p.hkv * D;
  const uint32_t row_bytes = (uint32_t)(kv_stride * 2);
  const __bf16* kbase = p.K + it.kv_head * D;   // the item's KV head (PERSIST: reset per item)
  const __bf16* vbase = p.V + it.kv_head * D;
  const int ld_row = tid / CH;
  const int ld_chunk = tid % CH;
  const uint32_t ld_voff = (uint32_t)ld_row * row_bytes + (uint32_t)ld_chunk * 16;

  // Tile loads: rows >= kv_hi read as zeros (range-checked buffer loads over
  // the tile's own rows, so nothing past the context is ever read).  Paged
  // K/V: a tile starts at a multiple of 64 virtual rows and pages hold a
  // multiple of 128 rows, so each tile lies inside one page.
  // Two register sets: tile k + 2 is loaded while tile k is computed.
  uint4 kreg[2][PASSES], vreg[2][PASSES];
  // Paged K/V: the physical page of a tile is read one tile ahead of its
  // loads, through a vector load (waited on in order with the tile loads; a
  // load that had to complete at once would stall on the tile in flight),
  // and moved to a scalar register only where the loads need it.
  const __amdgpu_buffer_rsrc_t prs = make_rsrc(p.pages, p.page_bytes);
  auto tile_page = [&](int tile) -> int {
    if constexpr (PAGED) {
      const int64_t v = t.kv_off + (int64_t)tile * BN;
      return __builtin_amdgcn_raw_buffer_load_b32(prs, (uint32_t)(v >> p.page_shift) * 4u, 0, 0);
    } else {
      return 0;
    }
  };
  auto tile_row = [&](int tile, int page) -> int64_t {
    const int64_t v = t.kv_off + (int64_t)tile * BN;
    if constexpr (PAGED) {
      const int64_t pg = __builtin_amdgcn_readfirstlane(page);
      return (pg << p.page_shift) | (v & ((int64_t(1) << p.page_shift) - 1));
    } else {
      return v;
    }
  };
  // set: register set, a compile-time constant (registers are not indexable)
  auto gload = [&](auto set_tag, int tile, int64_t r0) __attribute__((always_inline)) {
    constexpr int SET = decltype(set_tag)::value;
    const int n = min(BN, kv_hi - tile * BN);
    const __amdgpu_buffer_rsrc_t krs = rows_rsrc(kbase + r0 * kv_stride, n, row_bytes);
    const __amdgpu_buffer_rsrc_t vrs = rows_rsrc(vbase + r0 * kv_stride, n, row_bytes);
#pragma unroll
    for (int r = 0; r < PASSES; ++r) {
      kreg[SET][r] = buffer_load_16(krs, ld_voff + (uint32_t)(r * RPP) * row_bytes, 0);
      vreg[SET][r] = buffer_load_16(vrs, ld_voff + (uint32_t)(r * RPP) * row_bytes, 0);
    }
  };
  auto swrite = [&](auto set_tag) __attribute__((always_inline)) {
    constexpr int SET = decltype(set_tag)::value;   // also the LDS buffer
#pragma unroll
    for (int r = 0; r < PASSES; ++r) {
      const int row = r * RPP + ld_row;
      *(uint4*)(&lds_k[SET][row * KS + ld_chunk * 8]) = kreg[SET][r];
      *(uint4*)(&lds_v[SET][row * VS + ld_chunk * 8]) = vreg[SET][r];
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
  const int v_lane_off = ((j16 >> 2) + 4 * hh) * VS + 16 * (g16 & 1) + 4 * (j16 & 3);

  // One key tile for this wave.
  bf16x8 pf[2][2];
  auto qk = [&](int buf, f32x16* s_acc) __attribute__((always_inline)) {
    // S^T chain with the K operands read KPF steps ahead (fixed by fences:
    // left alone, the schedule waits on each read right before its MFMA;
    // 2 steps measured best against 1, 3 and 4).
    constexpr int KPF = 2;
    const __bf16* kl = &lds_k[buf][k_lane_off];
    bf16x8 kf[NKS][2];
#pragma unroll
    for (int s = 0; s < KPF; ++s)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) kf[s][mb] = *(const bf16x8*)(kl + mb * 32 * KS + 16 * s);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        s_acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s][mb], qf[s], s == 0 ? f32x16_zero() : s_acc[mb],
                                                            0, 0, 0);
      if (s + KPF < NKS) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) kf[s + KPF][mb] = *(const bf16x8*)(kl + mb * 32 * KS + 16 * (s + KPF));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto softmax = [&](int tile, f32x16* s_acc) __attribute__((always_inline)) {
    const int k0 = tile * BN;
    // Mask only where the tile straddles the diagonal, the context end or a
    // window / sink edge: key k0 + r (r in [0, 64)) is visible iff r <= lim
    // and (no window, or r >= wlo, or r < slim).
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
          s_acc[mb][j] = (r <= lim && (r >= wlo || r < slim)) ? s_acc[mb][j] : -INFINITY;
        }
    }
    // Tile max of this row, both half-waves: one three-input max per two
    // scores, in two independent chains.
    float mx0 = fmaxf(s_acc[0][0], s_acc[0][1]);
    float mx1 = fmaxf(s_acc[1][0], s_acc[1][1]);
#pragma unroll
    for (int j = 2; j < 16; j += 2) {
      mx0 = fmaxf(fmaxf(mx0, s_acc[0][j]), s_acc[0][j + 1]);
      mx1 = fmaxf(fmaxf(mx1, s_acc[1][j]), s_acc[1][j + 1]);
    }
    float mx = max_halves(fmaxf(mx0, mx1));
    const float m_tile = mx * p.scale_log2;
    // Raise the reference only when some row of the wave outgrew it.
    if (__any(m_tile > m2 + kRescaleLog2)) {
      keep_branch();
      const float m_new = fmaxf(m2, m_tile);
      const float alpha = (m2 == -INFINITY) ? 0.f : exp2_fast(m2 - m_new);   // rows still empty: acc is 0
      lsum *= alpha;
#pragma unroll
      for (int c = 0; c < NCB; ++c)
#pragma unroll
        for (int j = 0; j < 16; ++j) o_acc[c][j] *= alpha;
      m2 = m_new;
    }
    const float m_use = (m2 == -INFINITY) ? 0.f : m2;
    // P^T fragments: registers 8*half .. 8*half+7 of score block mb; the row
    // sum is taken in fp32 before rounding (two independent add chains).
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float e = exp2_fast(fmaf(s_acc[mb][8 * half + i], p.scale_log2, -m_use));
          if (i & 1) rs1 += e; else rs0 += e;
          pf[mb][half][i] = (__bf16)e;
        }
    lsum += sum_halves(rs0 + rs1);
  };
  auto pv = [&](int buf) __attribute__((always_inline)) {
    const __bf16* vl = &lds_v[buf][v_lane_off];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int kb = mb * 32 + 16 * half;
#pragma unroll
        for (int c = 0; c < NCB; ++c) {
          const __bf16* a0 = vl + kb * VS + c * 32;
          const bf16x8 vf = concat_bf16x4(ds_read_tr16(a0), ds_read_tr16(a0 + 8 * VS));
          o_acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[mb][half], o_acc[c], 0, 0, 0);
        }
      }
    }
  };

  // Tile k sits in register set k & 1 from two steps ahead and in LDS
  // buffer k & 1 from one step ahead.  Step k: one barrier, S(k) from K
  // buffer k & 1, then tile k + 1 is staged into buffer (k + 1) & 1 and tile
  // k + 3 loaded into the freed set while the softmax of tile k runs, then
  // O += P(k) V(k).  The barrier at the start of step k + 1 orders the
  // staging before its reads; the buffer it overwrites held tile k - 1, read
  // in step k - 1, before the barrier of step k.
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  // A context's sweep in two parts: sweep_issue() starts the loads of its
  // first two tiles (registers only), sweep_run() stages them and runs the
  // steps; the next context's loads can thus be in flight while the current
  // one finishes (after its last step every register set is free).
  int next_page = 0;
  auto sweep_issue = [&]() __attribute__((always_inline)) {
  next_page = 0;
  if (n_visit > 0) gload(S0{}, tile_of(0), tile_row(tile_of(0), tile_page(tile_of(0))));
  if (n_visit > 1) gload(S1{}, tile_of(1), tile_row(tile_of(1), tile_page(tile_of(1))));
  if (n_visit > 2) next_page = tile_page(tile_of(2));
  };
  auto sweep_run = [&]() __attribute__((always_inline)) {
  if (n_visit > 0) swrite(S0{});
  if (n_visit > 2) {
    gload(S0{}, tile_of(2), tile_row(tile_of(2), next_page));
    if (n_visit > 3) next_page = tile_page(tile_of(3));
  }
  auto step = [&](auto kb_tag, int k) __attribute__((always_inline)) {
    constexpr int KB = decltype(kb_tag)::value;    // buffer of tile k; tile k + 1 is in set 1 - KB
    using SN = std::integral_constant<int, 1 - KB>;
    __syncthreads();
    const int tile = tile_of(k);
    const bool sees = wave_sees(tile);
    f32x16 s_acc[2];
    if (sees) qk(KB, s_acc);
    if (k + 1 < n_visit) swrite(SN{});
    if (k + 3 < n_visit) {
      gload(SN{}, tile_of(k + 3), tile_row(tile_of(k + 3), next_page));
      if (k + 4 < n_visit) next_page = tile_page(tile_of(k + 4));
    }
    if (sees) {
      softmax(tile, s_acc);
      pv(KB);
    }
  };
  for (int k = 0; k < n_visit; k += 2) {
    step(S0{}, k);
    if (k + 1 < n_visit) step(S1{}, k + 1);
  }
  };
  // Epilogue of one item: O = acc / l, LSE = ln 2 * (m2 + log2 l); empty
  // rows: 0, -inf.  Row orow of O / LSE, or staging row srow (>= 0) for a
  // key chunk of a split shard (fp32 partials, merged by Equation 4 later).
  auto epilogue = [&](bool valid, int e_head, int64_t orow, int64_t srow) __attribute__((always_inline)) {
    if (!valid) return;
    const float inv_l = lsum > 0.f ? 1.f / lsum : 0.f;
    if constexpr (MULTI) {
      if (srow >= 0) {
        if (hh == 0)
          p.stage_LSE[srow * p.hq + e_head] =
              lsum > 0.f ? (m2 + __log2f(lsum)) * 0.69314718055994530942f : -INFINITY;
        float* so = p.stage_O + srow * (int64_t)(p.hq * D) + e_head * D;
#pragma unroll
        for (int c = 0; c < NCB; ++c)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            *(float4*)(so + c * 32 + 8 * q4 + 4 * hh) =
                make_float4(o_acc[c][4 * q4] * inv_l, o_acc[c][4 * q4 + 1] * inv_l, o_acc[c][4 * q4 + 2] * inv_l,
                            o_acc[c][4 * q4 + 3] * inv_l);
        return;
      }
    }
    if (hh == 0) {
      p.LSE[orow * p.hq + e_head] = lsum > 0.f ? (m2 + __log2f(lsum)) * 0.69314718055994530942f : -INFINITY;
    }
    const int64_t obase = orow * (int64_t)(p.hq * D) + e_head * D;
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
  };

  sweep_issue();
  if constexpr (PERSIST) {
    if (tid == 0) lds_next[0] = claimed_item();   // after the loads above: waits for the claim only
  }
  for (;;) {
    sweep_run();
    if constexpr (MULTI) {
      // the shard's further contexts: the online softmax state carries over
      for (int sg = 1; sg < it.n_seg; ++sg) {
        if constexpr (PERSIST)
          t = wave_uniform(p.tasks[it.task + sg]);
        else
          t = p.tasks[it.task + sg];
        context(it.task + sg);
        context_tiles();
        sweep_issue();
        __syncthreads();   // the previous context's last tiles may still be read from LDS
        sweep_run();
      }
    }
    const int64_t orow = t.o_off + qrow;
    const int64_t srow = MULTI && it.stage_row >= 0 ? (int64_t)it.stage_row + qrow : -1;
    if constexpr (!PERSIST) {
      epilogue(qvalid, head, orow, srow);
      return;
    } else {
      // The claimed item: its Q and first tiles are loaded while this item's
      // outputs are written; the claim after it is taken at once.
      __syncthreads();   // this item's last tiles are read; the claim is visible
      // wave-uniform: keeps the item's fields, and everything derived from
      // them, in scalar registers
      const int nxt = __builtin_amdgcn_readfirstlane(lds_next[parity]);
      parity ^= 1;
      const bool more = nxt < p.n_items;
      const bool e_valid = qvalid;
      const int e_head = head;
      if (more) {
        if (tid == 0) claim = atomicAdd(p.counter + xcd, 1u);
        it = wave_uniform(p.items[nxt]);
        t = wave_uniform(p.tasks[it.task]);
        kbase = p.K + it.kv_head * D;
        vbase = p.V + it.kv_head * D;
        item_rows();
        context(it.task);
        load_q();
        context_tiles();
        sweep_issue();
      }
      epilogue(e_valid, e_head, orow, srow);
      if (!more) return;
      // lds_next[parity] was last read after the previous item's last
      // barrier, which every wave has passed since
      if (tid == 0) lds_next[parity] = claimed_item();
#pragma unroll
      for (int c = 0; c < NCB; ++c) o_acc[c] = f32x16_zero();
      m2 = -INFINITY;
      lsum = 0.f;
    }
  }
}

// MULTI: calls with query shards over several contexts; all others run the
// single-context kernel.
template <int D, int NW, bool PAGED>
hipError_t launch_forward_dp(const FwdParams& p, hipStream_t s) {
  if (p.counter) {
    if (p.multi)
      hipLaunchKernelGGL((fwd_kernel<D, NW, PAGED, true, true>), dim3(min(p.n_slots, p.n_items)), dim3(64 * NW), 0, s, p);
    else
      hipLaunchKernelGGL((fwd_kernel<D, NW, PAGED, false, true>), dim3(min(p.n_slots, p.n_items)), dim3(64 * NW), 0, s, p);
  } else {
    if (p.multi)
      hipLaunchKernelGGL((fwd_kernel<D, NW, PAGED, true, false>), dim3(p.n_items), dim3(64 * NW), 0, s, p);
    else
      hipLaunchKernelGGL((fwd_kernel<D, NW, PAGED, false, false>), dim3(p.n_items), dim3(64 * NW), 0, s, p);
  }
  return hipGetLastError();
}

template <int D, int NW>
hipError_t launch_forward_d(const FwdParams& p, hipStream_t s) {
  return p.pages ? launch_forward_dp<D, NW, true>(p, s) : launch_forward_dp<D, NW, false>(p, s);
}

hipError_t launch_forward(const FwdParams& p, int d, hipStream_t s) {
  if (p.n_items <= 0) return hipSuccess;
  return d == 128 ? launch_forward_d<128, 8>(p, s) : launch_forward_d<64, 8>(p, s);
}

}  // namespace ca
