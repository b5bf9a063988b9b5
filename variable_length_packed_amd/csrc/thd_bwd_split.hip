// Backward attention over packed variable-length ("thd") tensors (head dims
// 8 to 256, padded to 32, 64, 128 or 256 in registers): the gradients of TransformerEngine PR "Add per-sequence causal
// policy to packed THD attention" (Changes: Q/K/V gradient parity), in two
// passes that each own their outputs, so that no gradient is accumulated with
// atomics:
//   dq pass   : query-stationary, shaped like the forward: one workgroup per
//               (sequence, 128-row query tile, query head) walks the key tiles
//               its rows can see, recomputes S and dP and accumulates
//               dQ = scale dS K in registers; it also forms D = rowsum(dO * O)
//               from the stored output and leaves -D and -LSE/scale for
//               the second pass;
//   dk/dv pass: key-stationary: one workgroup per (sequence, key tile, kv
//               head), 32 keys per wave (128-key tiles of 4 waves for short
//               walks and for head dims above 128, 256-key tiles of 8 waves
//               for long ones), walks the
//               32-row query tiles of every query head of its GQA group
//               (from the last tile down, the group's heads innermost),
//               recomputes S and dP and accumulates dK^T and dV^T in
//               registers (thd_bwd_dkdv.hip).
// Textbook softmax-attention backward with the probabilities recomputed from
// the forward's log-sum-exp:
//   P = exp(scale Q K^T - LSE),  dV = P^T dO,  dP = dO V^T,
//   dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
// S and dP are formed twice (once per pass): 14 d instead of 10 d FLOPs per
// valid (query, key) pair.  In exchange nothing is added with atomics (a key
// tile's dQ atomics, 4,096 per query tile, ran at the device's memory-side
// atomic rate), no fp32 dq accumulator has to be cleared and converted, and dq
// is deterministic.
//
// Three launches: a pre pass (both passes' schedules, zeros on every pad row of
// dq, dk and dv), the dq pass, the dk/dv pass.
#include "thd_bwd_split.hpp"
#include "thd_launch.hpp"

namespace thd {

namespace {

using namespace split;

// dq pass schedule: query tile t of sequence b walks W = ceil(lk / BN) key
// tiles, or, with a causal mask type, those up to its last row's diagonal:
// W = clamp(a t + a + ceil(off / BN), 0, ceil(lk / BN)), a = BM / BN (the
// forward's model).
template <int BN>
struct DqSchedModel {
  static_assert(kDqBM % BN == 0, "whole key tiles per query tile");
  static constexpr int kSlope = kDqBM / BN;
  const SplitParams& p;
  __device__ SeqSummary seq(int b) const {
    const int lq = split_lq(p, b), lk = split_lk(p, b);
    const int mt = mask_type_of(p.causal, b);
    SeqSummary s;
    s.x = ceil_div_pos(lq, kDqBM);
    s.H = ceil_div_pos(lk, BN);
    s.causal = mask_is_causal(mt);
    s.c = kSlope + ceil_div(causal_offset(mt, lq, lk), BN);
    s.sq = (int)seq_start(p.cu_q, p.pad_q, b);
    s.sk = (int)seq_start(p.cu_kv, p.pad_kv, b);
    s.lq = lq;
    s.lk = lk;
    s.mtype = mt;
    return s;
  }
};

// dk/dv pass schedule: key tile kt walks W = ceil(lq / BQ) query tiles, or,
// with a causal mask type, those from the first one that sees key kt BK:
// W = clamp(ceil(lq / BQ) - (BK / BQ) kt + ceil(off / BQ), 0, ceil(lq / BQ)).
template <int BK>
struct KvSchedModel {
  static constexpr int kSlope = -BK / kKvBQ;
  const SplitParams& p;
  __device__ SeqSummary seq(int b) const {
    const int lq = split_lq(p, b), lk = split_lk(p, b);
    const int mt = mask_type_of(p.causal, b);
    SeqSummary s;
    s.x = ceil_div_pos(lk, BK);
    s.H = ceil_div_pos(lq, kKvBQ);
    s.causal = mask_is_causal(mt);
    s.c = s.H + ceil_div(causal_offset(mt, lq, lk), kKvBQ);
    s.sq = (int)seq_start(p.cu_q, p.pad_q, b);
    s.sk = (int)seq_start(p.cu_kv, p.pad_kv, b);
    s.lq = lq;
    s.lk = lk;
    s.mtype = mt;
    return s;
  }
};

// Zero the pad rows [r0, r0 + kPadRows) of a [T, h * d] output (rows outside
// every sequence, through cu / cu_padded).
__device__ void zero_pad_rows(const int32_t* cu, const int32_t* cu_pad, int batch, int64_t T,
                              int row_elems, int64_t r0, uint16_t* out0, uint16_t* out1) {
  __shared__ uint8_t invalid[kPadRows];
  const int tid = threadIdx.x;
  int mine = 0;
  if (tid < kPadRows) {
    const int64_t r = r0 + tid;
    const bool inv = r < T && !row_is_valid(cu, cu_pad, batch, r, T);
    invalid[tid] = inv;
    mine = inv;
  }
  if (!__syncthreads_or(mine)) return;
  const int chunks = row_elems / 8;
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int idx = tid; idx < kPadRows * chunks; idx += 256) {
    const int rr = idx / chunks;
    const int c = idx - rr * chunks;
    if (invalid[rr]) {
      const int64_t off = (r0 + rr) * (int64_t)row_elems + 8 * c;
      *(u32x4*)(out0 + off) = z;
      if (out1) *(u32x4*)(out1 + off) = z;
    }
  }
}

template <int DP, int BK>
__global__ __launch_bounds__(256) void thd_bwd_split_pre_kernel(SplitParams p) {
  int blk = blockIdx.x;
  const int wave = (int)(threadIdx.x >> 6);
  if (blk < p.n_qsched_wg) {
    build_schedule_by_sequence(DqSchedModel<DqTile<DP>::BN>{p}, p.batch, p.n_qtiles, p.qsched,
                               blk * 4 + wave);
    return;
  }
  blk -= p.n_qsched_wg;
  if (blk < p.n_ksched_wg) {
    build_schedule_by_sequence(KvSchedModel<BK>{p}, p.batch, p.n_ktiles, p.ksched, blk * 4 + wave);
    return;
  }
  blk -= p.n_ksched_wg;
  if (blk < p.n_qzero_wg) {
    zero_pad_rows(p.cu_q, p.pad_q, p.batch, p.T_q, p.h_q * p.d, (int64_t)blk * kPadRows, p.dq,
                  nullptr);
    return;
  }
  blk -= p.n_qzero_wg;
  zero_pad_rows(p.cu_kv, p.pad_kv, p.batch, p.T_kv, p.h_kv * p.d, (int64_t)blk * kPadRows, p.dk,
                p.dv);
}

// ---------------------------------------------------------------------------
// dq pass
// ---------------------------------------------------------------------------
// One workgroup = 4 waves = one (sequence, 128-row query tile, query head), in
// schedule order with the forward's head slots.  Wave w owns query rows
// 32w .. 32w+31.  The products run transposed, as in the forward, so that a
// lane owns one query row: S^T = K Q^T and dP^T = V dO^T (K and V rows from
// LDS, Q and dO held as operands), P^T = exp2(S^T scale log2e - LSE log2e),
// dS^T = P^T (dP^T - D), and dQ^T += K^T dS^T with K^T from transpose reads
// of the same K tile.  K and V tiles go straight from memory into LDS, row
// major with swizzled 16-byte chunks, as in the forward.
template <class DT, int DP>
__global__ __launch_bounds__(256, DP > 128 ? 1 : 2) void thd_bwd_dq_kernel(SplitParams p) {
  constexpr int BM = kDqBM, BN = DqTile<DP>::BN;
  constexpr int NT = BN / 32;      // 32-key S^T tiles per LDS tile
  constexpr int NKB = BN / 16;     // 16-key blocks (K steps of dQ^T)
  constexpr int NC = DP / 16;      // 16-wide d blocks (K steps of S^T, dP^T)
  constexpr int ND = DP / 32;      // 32-row d tiles of dQ^T
  constexpr int KCH = DP / 8;
  constexpr int TILE = BN * DP * 2;
  constexpr int BPW = TILE / 1024 / 4;
  static_assert(BPW >= 1 && BPW * 4096 == TILE, "tile splits into 1 KB blocks over 4 waves");
  static_assert(2 * BPW < 16, "loads of one tile fit the vmcnt field");
  // buffer j: K tile at 2j TILE, V tile at (2j + 1) TILE; then (DP = 128) a
  // [32][DP] tile per wave through which its Q and dO rows pass
  constexpr int ROWS = DP == 128 ? 32 * DP * 2 : 0;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * kDqBufs * TILE + 4 * ROWS];

  const int bid = blockIdx.x;
  const int rk = bid / p.h_q;
  const int slot = bid - rk * p.h_q;
  const int hq = (slot % p.h_kv) * p.group + slot / p.h_kv;
  SchedItem item;
  if (!load_sched_item(p.qsched, rk, item)) return;
  const int b = uniform(item.b);
  const int tile_in_seq = uniform(item.t);
  if (b < 0 || b >= p.batch || tile_in_seq < 0) return;

  const int tid = threadIdx.x;
  const int w = uniform(tid >> 6);
  const int l = tid & 63;
  const int r = l & 31;
  const int h = l >> 5;
  const int g16 = l & 15;
  const int grp = l >> 4;

  const uint32_t qrow_bytes = (uint32_t)p.h_q * p.d * 2;
  const uint32_t kvrow_bytes = (uint32_t)p.h_kv * p.d * 2;
  // the item's slot starts, lengths (split_lq / split_lk) and mask type
  const int64_t sq = uniform(item.sq);
  const int64_t sk = uniform(item.sk);
  const int lq = uniform(item.lq);
  const int lk = uniform(item.lk);
  const int mtype = uniform(item.mtype);
  const bool causal = mask_is_causal(mtype);
  const int off = causal_offset(mtype, lq, lk);
  const int hk = hq / p.group;
  const int q0 = tile_in_seq * BM;
  if (q0 >= lq) return;
  const int qw0 = q0 + w * 32;
  const int my_q = qw0 + r;

  int kv_end = lk;
  if (causal && q0 + BM + off < kv_end) kv_end = q0 + BM + off;
  const int n_kv_tiles = ceil_div_pos(kv_end, BN);

  const int64_t hoff = sq * (int64_t)p.h_q * p.d + (int64_t)hq * p.d;
  const rsrc_t q_rs = make_rsrc(p.q + hoff, (uint32_t)lq * qrow_bytes);
  const rsrc_t g_rs = make_rsrc(p.dout + hoff, (uint32_t)lq * qrow_bytes);
  const rsrc_t o_rs = make_rsrc(p.o + hoff, (uint32_t)lq * qrow_bytes);
  const rsrc_t dq_rs = make_rsrc(p.dq + hoff, (uint32_t)lq * qrow_bytes);
  const char* kbase = (const char*)(p.k + sk * (int64_t)p.h_kv * p.d + (int64_t)hk * p.d);
  const char* vbase = (const char*)(p.v + sk * (int64_t)p.h_kv * p.d + (int64_t)hk * p.d);

  uint32_t loff[BPW];
#pragma unroll
  for (int n = 0; n < BPW; ++n) {
    const int slot_ = 64 * (BPW * w + n) + l;
    const int row = slot_ / KCH;
    const int x = slot_ - row * KCH;
    const int gc = x ^ (int)((swz<DP>(row, 0) >> 4) & (KCH - 1));
    loff[n] = 8 * gc < p.d ? (uint32_t)row * kvrow_bytes + 16u * gc : kOobOffset;
  }
  auto load_tile = [&](int k0, int buf) {
    const uint32_t left = (uint32_t)(lk - k0);
    const u32x4 k_rs = rsrc_words(kbase + (int64_t)k0 * kvrow_bytes, left * kvrow_bytes);
    const u32x4 v_rs = rsrc_words(vbase + (int64_t)k0 * kvrow_bytes, left * kvrow_bytes);
    const uint32_t kt = lds_addr(smem) + (uint32_t)(2 * buf * TILE + 1024 * BPW * w);
#pragma unroll
    for (int n = 0; n < BPW; ++n) {
      buf_load_lds16(k_rs, kt + 1024 * n, loff[n]);
      buf_load_lds16(v_rs, kt + TILE + 1024 * n, loff[n]);
    }
  };
  // The first tiles go in flight before the row operands are read: they
  // need only the sequence's bounds.
#pragma unroll
  for (int t = 0; t < kDqBufs - 1; ++t)
    if (t < n_kv_tiles) load_tile(t * BN, t);


  // Q and dO as the B operands of S^T and dP^T: lane holds row my_q,
  // d 16c + 8h .. +7; D = rowsum(dO * O) over the same chunks of O, the two
  // halves of a row meeting across lanes r and r + 32.
  typename DT::vec8 qreg[NC], greg[NC];
  float Drow;
  if constexpr (DP == 128) {
    // Whole rows: load j of the wave covers rows RPI j .. RPI j + RPI - 1,
    // lane l the 16-byte chunk l % KCH of row RPI j + l / KCH.  (Loaded
    // straight into the operand layout, 32 bytes of each of 32 rows per load,
    // the pass took 0.178 against 0.175 ms on 16 causal sequences of
    // 64-2,048 tokens, h 16, d 128, and 0.543 against 0.520 ms on 64 padded
    // sequences of up to 1,024 tokens, h 32.)
    constexpr int RPI = 64 / KCH, NJ = 32 / RPI;
    unsigned char* st = smem + 2 * kDqBufs * TILE + w * ROWS;
    u32x4 qv[NJ], gv[NJ], ov[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int row = RPI * j + l / KCH, x = l % KCH;
      const uint32_t o = 8 * x < p.d ? (uint32_t)(qw0 + row) * qrow_bytes + 16u * x : kOobOffset;
      qv[j] = buf_load16(q_rs, o, 0);
      gv[j] = buf_load16(g_rs, o, 0);
      ov[j] = buf_load16(o_rs, o, 0);
    }
    // Q: rows into the tile, then lane (r, h) reads Q[r][16c + 8h ..]
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      *(u32x4*)(st + swz<DP>(RPI * j + l / KCH, 8 * (l % KCH))) = qv[j];
    asm volatile("" ::: "memory");
#pragma unroll
    for (int c = 0; c < NC; ++c) qreg[c] = as_vec8<DT>(*(const u32x4*)(st + swz<DP>(r, 16 * c + 8 * h)));
    asm volatile("" ::: "memory");
    // D = rowsum(dO * O): a row's KCH lanes sum their chunks; its sum goes to
    // word row of the tile (whose Q reads are done), where lanes r read it
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      float dp_ = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dp_ += DT::to_f32((uint16_t)(gv[j][e] & 0xffffu)) * DT::to_f32((uint16_t)(ov[j][e] & 0xffffu));
        dp_ += DT::to_f32((uint16_t)(gv[j][e] >> 16)) * DT::to_f32((uint16_t)(ov[j][e] >> 16));
      }
      dp_ = group_sum<KCH>(dp_);
      if (l % KCH == 0) ((float*)st)[RPI * j + l / KCH] = dp_;
    }
    asm volatile("" ::: "memory");
    Drow = ((const float*)st)[r];
    asm volatile("" ::: "memory");
    // dO: rows into the tile, then the operand reads as for Q
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      *(u32x4*)(st + swz<DP>(RPI * j + l / KCH, 8 * (l % KCH))) = gv[j];
    asm volatile("" ::: "memory");
#pragma unroll
    for (int c = 0; c < NC; ++c) greg[c] = as_vec8<DT>(*(const u32x4*)(st + swz<DP>(r, 16 * c + 8 * h)));
  } else {
    // Q and dO as the B operands of S^T and dP^T: lane holds row my_q,
    // d 16c + 8h .. +7; D = rowsum(dO * O) over the same chunks of O, the two
    // halves of a row meeting across lanes r and r + 32.
    float dpart = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int dd = 16 * c + 8 * h;
      const uint32_t o = dd < p.d ? (uint32_t)my_q * qrow_bytes + 2u * dd : kOobOffset;
      qreg[c] = as_vec8<DT>(buf_load16(q_rs, o, 0));
      const u32x4 gv = buf_load16(g_rs, o, 0);
      const u32x4 ov = buf_load16(o_rs, o, 0);
      greg[c] = as_vec8<DT>(gv);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dpart += DT::to_f32((uint16_t)(gv[j] & 0xffffu)) * DT::to_f32((uint16_t)(ov[j] & 0xffffu));
        dpart += DT::to_f32((uint16_t)(gv[j] >> 16)) * DT::to_f32((uint16_t)(ov[j] >> 16));
      }
    }
    Drow = wave_sum_halves(dpart);
  }
  float lse_row = 0.f;
  if (my_q < lq) lse_row = p.lse[(int64_t)hq * p.T_q + sq + my_q];
  // statistics of this row for the dk/dv pass
  if (h == 0 && my_q < lq) {
    p.dsum[(int64_t)hq * p.T_q + sq + my_q] = -Drow;
    p.lsum[(int64_t)hq * p.T_q + sq + my_q] = lse_row * (-1.0f / p.scale);
  }
  // a row that sees no key has LSE -inf and every score masked: P = 0
  const float lse2 = lse_row == -__builtin_inff() ? 0.f : lse_row * kLog2e;

  f32x16 acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc[i] = f32x16{};

  // Operand addresses inside a tile (as in the forward):
  //   K / V rows 32tt + r, chunk 2c + h:  (b_k ^ (c << 5)) + 32tt 2DP (+ TILE for V)
  //   K^T operand (dt, kb, j):            (b_t ^ tr_chunk(dt, j)) + tr_row(kb, j)
  const uint32_t b_k = swz<DP>(r, 8 * h);
  const uint32_t b_t = swz<DP>(4 * h + (g16 >> 2), 16 * (grp & 1) + 4 * (g16 & 3));
  const float c2 = p.c2;

  // Tiles this wave computes: with a causal mask type, the tiles past its
  // last row's diagonal are skipped, and so is every later tile.
  int n_act = qw0 < lq ? n_kv_tiles : 0;
  if (causal && n_act > 0) {
    const int last = qw0 + 31 + off;  // last key the wave's last row sees
    const int na = last < 0 ? 0 : last / BN + 1;
    n_act = na < n_act ? na : n_act;
  }

  // S^T and dP^T of the tile in buffer bi.
  auto sdp = [&](int bi, f32x16 (&s)[NT], f32x16 (&dp)[NT]) {
    const uint32_t a_k = opaque(b_k + (uint32_t)(2 * bi * TILE));
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      s[tt] = f32x16{};
      dp[tt] = f32x16{};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const uint32_t ad = (a_k ^ (uint32_t)(c << 5)) + 32 * tt * DP * 2;
        const u32x4 ka = *(const u32x4*)(smem + ad);
        const u32x4 va = *(const u32x4*)(smem + ad + TILE);
        s[tt] = DT::mfma(as_vec8<DT>(ka), qreg[c], s[tt]);
        dp[tt] = DT::mfma(as_vec8<DT>(va), greg[c], dp[tt]);
      }
    }
  };
  // Scores of keys this lane's row does not see to -inf.
  auto mask = [&](int k0, f32x16 (&s)[NT]) {
    const bool need_mask = (k0 + BN > lk) || (causal && k0 + BN - 1 > qw0 + off);
    if (need_mask) {
      const int lim = causal ? (my_q + 1 + off < lk ? my_q + 1 + off : lk) : lk;
#pragma unroll
      for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = k0 + 32 * tt + 8 * (i >> 2) + 4 * h + (i & 3);
          if (j >= lim) s[tt][i] = -__builtin_inff();
        }
    }
  };
  // The next tile's S^T and dP^T (buffer bn) interleaved with this tile's
  // dS^T (from s, dp) and then dQ^T += K^T dS^T (buffer bc).  The order is
  // fixed by scheduling fences: segment g issues the LDS reads of a later K
  // step, the two products of K step g and the dS of 16 / NC elements, so
  // that the matrix unit works while the vector unit forms the
  // probabilities.
  auto overlapped = [&](int bc, int bn, const f32x16 (&s)[NT], const f32x16 (&dp)[NT],
                        f32x16 (&sn)[NT], f32x16 (&dpn)[NT]) {
    constexpr int NSEG = NT * NC;      // K steps of the next tile's products
    constexpr int EPS = 16 * NT / NSEG;  // dS elements per segment
    static_assert(EPS * NSEG == 16 * NT && EPS >= 1, "whole elements per segment");
    const uint32_t a_k = opaque(b_k + (uint32_t)(2 * bn * TILE));
    const uint32_t a_t = opaque(b_t + (uint32_t)(2 * bc * TILE));
    auto kv_addr = [&](int g) {
      return (a_k ^ (uint32_t)((g % NC) << 5)) + 32 * (g / NC) * DP * 2;
    };
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      sn[tt] = f32x16{};
      dpn[tt] = f32x16{};
    }
    float tmp[16 * NT];
    typename DT::vec8 dsb[NKB];
    // LDS reads run kDqReadAhead K steps ahead of their products
    constexpr int RA = kDqReadAhead < NSEG ? kDqReadAhead : NSEG;
    u32x4 kr[RA + 1], vr[RA + 1];
#pragma unroll
    for (int g = 0; g < RA; ++g) {
      kr[g] = *(const u32x4*)(smem + kv_addr(g));
      vr[g] = *(const u32x4*)(smem + kv_addr(g) + TILE);
    }
#pragma unroll
    for (int g = 0; g < NSEG; ++g) {
      if (g + RA < NSEG) {
        kr[(g + RA) % (RA + 1)] = *(const u32x4*)(smem + kv_addr(g + RA));
        vr[(g + RA) % (RA + 1)] = *(const u32x4*)(smem + kv_addr(g + RA) + TILE);
      }
      const u32x4 ka = kr[g % (RA + 1)], va = vr[g % (RA + 1)];
      const int tt = g / NC, c = g % NC;
      sn[tt] = DT::mfma(as_vec8<DT>(ka), qreg[c], sn[tt]);
      dpn[tt] = DT::mfma(as_vec8<DT>(va), greg[c], dpn[tt]);
#pragma unroll
      for (int e = 0; e < EPS; ++e) {
        const int x = g * EPS + e;
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[x >> 4][x & 15], c2, -lse2));
        tmp[x] = pv * (dp[x >> 4][x & 15] - Drow);
        // pins the element's vector work to this segment (instruction
        // selection would otherwise move it next to its use)
        asm volatile("" : "+v"(tmp[x]));
      }
      if (((g + 1) * EPS) % 8 == 0) {
        const int kb = ((g + 1) * EPS) / 8 - 1;
        dsb[kb] = pack8<DT>(tmp + 8 * kb);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const u32x4 a =
            cat2(lds_read_tr(smem, (a_t ^ tr_chunk<DP>(dt, 0)) + tr_row<DP>(kb, 0)),
                 lds_read_tr(smem, (a_t ^ tr_chunk<DP>(dt, 1)) + tr_row<DP>(kb, 1)));
        acc[dt] = DT::mfma(as_vec8<DT>(a), dsb[kb], acc[dt]);
      }
  };
  // Iteration it: tiles it and it + 1 are in LDS (buffers it % B and
  // (it + 1) % B, B = kDqBufs), tile it + 2 is in flight, and tile it + B - 1
  // is loaded into the buffer tile it - 1 used.
  // S^T and dP^T of tile it + 1 are formed while the probabilities and dS of
  // tile it are (the two are independent, so the matrix products overlap the
  // vector work); the scores of tile it arrive in (s, dp) from the iteration
  // before.
  auto step = [&](int it, f32x16 (&s)[NT], f32x16 (&dp)[NT], f32x16 (&sn)[NT],
                  f32x16 (&dpn)[NT]) {
    if (it + kDqBufs - 1 < n_kv_tiles)
      load_tile((it + kDqBufs - 1) * BN, (it + kDqBufs - 1) % kDqBufs);
    if (it < n_act) {
      // (the products of the next tile are formed even past this wave's last
      // tile: its buffer is in LDS either way, and a branch would split the
      // block in which they overlap this tile's vector work)
      mask(it * BN, s);
      overlapped(it % kDqBufs, (it + 1) % kDqBufs, s, dp, sn, dpn);
    }
    // Tile it + 2 is in; the one loaded after it (2 BPW loads) may still be
    // in flight.  (The tile loads are not counted by the compiler; see the
    // forward.)
    if (kDqBufs > 3 && it + 3 < n_kv_tiles)
      __builtin_amdgcn_s_waitcnt(0x0f70 | (kDqBufs > 3 ? 2 * BPW : 0));
    else
      __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
  };

  // vmcnt(0): operands and the first tiles are in
  __builtin_amdgcn_s_waitcnt(0x0f70);
  __syncthreads();
  f32x16 s0[NT], dp0[NT], s1[NT], dp1[NT];
  if (n_act > 0) sdp(0, s0, dp0);
  for (int it = 0; it < n_kv_tiles; it += 2) {
    step(it, s0, dp0, s1, dp1);
    if (it + 1 < n_kv_tiles) step(it + 1, s1, dp1, s0, dp0);
  }

  // dq = scale dQ; rows past lq are dropped by the resource bound.
  if constexpr (DP != 64) {
    // Each wave stages its 32 rows (bf16, row-major, swizzled) in its own part
    // of the K/V tiles, which every wave is done with after the walk's last
    // barrier, then stores whole rows: each store covers 64 / KCH full rows.
    static_assert(4 * 32 * DP * 2 <= 2 * kDqBufs * TILE, "staging fits the K/V tiles");
    unsigned char* st = smem + (size_t)w * 32 * DP * 2;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = 32 * dt + 8 * g + 4 * h;
        u32x2 out;
        out[0] = (uint32_t)DT::bits(acc[dt][4 * g + 0] * p.scale) |
                 ((uint32_t)DT::bits(acc[dt][4 * g + 1] * p.scale) << 16);
        out[1] = (uint32_t)DT::bits(acc[dt][4 * g + 2] * p.scale) |
                 ((uint32_t)DT::bits(acc[dt][4 * g + 3] * p.scale) << 16);
        *(u32x2*)(st + swz<DP>(r, dd)) = out;
      }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < 32 * KCH / 64; ++j) {
      const int c = l + 64 * j;
      const int row = c / KCH, x = c - row * KCH;
      const u32x4 v = *(const u32x4*)(st + swz<DP>(row, 8 * x));
      // rows past lq are dropped by the resource bound
      buf_store16(v, dq_rs, 8 * x < p.d ? (uint32_t)(qw0 + row) * qrow_bytes + 16u * x : kOobOffset, 0);
    }
  } else {
    // At DP = 64 the staging's registers would cost the third wave per SIMD
    // (171 against 168 VGPRs; the pass took 0.102 against 0.097 ms at h 16 on
    // the same layout), so dq leaves straight from the accumulators, 8 bytes
    // per lane; rows past lq are dropped by the resource bound.
    const uint32_t orow = (uint32_t)my_q * qrow_bytes;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = 32 * dt + 8 * g + 4 * h;
        u32x2 out;
        out[0] = (uint32_t)DT::bits(acc[dt][4 * g + 0] * p.scale) |
                 ((uint32_t)DT::bits(acc[dt][4 * g + 1] * p.scale) << 16);
        out[1] = (uint32_t)DT::bits(acc[dt][4 * g + 2] * p.scale) |
                 ((uint32_t)DT::bits(acc[dt][4 * g + 3] * p.scale) << 16);
        if (dd < p.d) buf_store8(out, dq_rs, orow + 2u * dd, 0);
      }
  }
}

template <class DT, int DP>
hipError_t launch_split_t(const SplitParams& sp, int64_t n_pre, hipStream_t s,
                          hipEvent_t const* ev) {
  auto mark = [&](int i) -> hipError_t { return ev ? hipEventRecord(ev[i], s) : hipSuccess; };
  hipError_t e = mark(0);
  if (e != hipSuccess) return e;
  if (n_pre > 0) {
    if (sp.kv_bk == kKvBkLong)
      hipLaunchKernelGGL((thd_bwd_split_pre_kernel<DP, kKvBkLong>), dim3((unsigned)n_pre), dim3(256),
                         0, s, sp);
    else
      hipLaunchKernelGGL((thd_bwd_split_pre_kernel<DP, kKvBkShort>), dim3((unsigned)n_pre),
                         dim3(256), 0, s, sp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = mark(1)) != hipSuccess) return e;
  if (sp.batch > 0) {
    hipLaunchKernelGGL((thd_bwd_dq_kernel<DT, DP>), dim3((unsigned)(sp.n_qtiles * sp.h_q)),
                       dim3(256), 0, s, sp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = mark(2)) != hipSuccess) return e;
  if (sp.batch > 0 && (e = launch_dkdv<DT, DP>(sp, s)) != hipSuccess) return e;
  return mark(3);
}

size_t align256_s(size_t x) { return (x + 255) & ~(size_t)255; }

int64_t split_qtiles(const Problem& p) { return (p.T_q + kDqBM - 1) / kDqBM + p.batch; }
// Keys per dk/dv workgroup, from host scalars only: a key tile walks at most
// max_seqlen_q rows of each of the group's query heads.
int split_kv_bk(const Problem& p) {
  return p.d > 128 || (int64_t)p.max_q * (p.h_q / p.h_kv) <= kKvShortWalkRows ? kKvBkShort : kKvBkLong;
}
int64_t split_ktiles(const Problem& p) {
  const int bk = split_kv_bk(p);
  return (p.T_kv + bk - 1) / bk + p.batch;
}

}  // namespace

// -D and -LSE/scale ([h_q][T_q] fp32 each), then the dq pass's schedule
// (sched_bytes of the query-tile bound) and the dk/dv pass's (of the
// key-tile bound).
size_t bwd_workspace_bytes(const Problem& p) {
  const size_t stats = align256_s((size_t)p.T_q * p.h_q * 2 * sizeof(float));
  const size_t qs = align256_s(sched_bytes(split_qtiles(p)));
  const size_t ks = align256_s(sched_bytes(split_ktiles(p)));
  return stats + qs + ks;
}

hipError_t launch_bwd(const Problem& p, const void* q, const void* k, const void* v,
                      const void* o, const void* dout, const float* lse, void* dq, void* dk,
                      void* dv, void* workspace, hipStream_t s, hipEvent_t const* ev) {
  SplitParams sp;
  sp.q = (const uint16_t*)q;
  sp.k = (const uint16_t*)k;
  sp.v = (const uint16_t*)v;
  sp.o = (const uint16_t*)o;
  sp.dout = (const uint16_t*)dout;
  sp.lse = lse;
  sp.dq = (uint16_t*)dq;
  sp.dk = (uint16_t*)dk;
  sp.dv = (uint16_t*)dv;
  const size_t stats = align256_s((size_t)p.T_q * p.h_q * 2 * sizeof(float));
  sp.dsum = (float*)workspace;
  sp.lsum = sp.dsum + (size_t)p.T_q * p.h_q;
  sp.qsched = (int32_t*)((char*)workspace + stats);
  sp.ksched = (int32_t*)((char*)workspace + stats +
                         align256_s(sched_bytes(split_qtiles(p))));
  sp.cu_q = p.cu_q;
  sp.cu_kv = p.cu_kv;
  sp.pad_q = p.pad_q;
  sp.pad_kv = p.pad_kv;
  sp.causal = p.causal;
  sp.T_q = p.T_q;
  sp.T_kv = p.T_kv;
  sp.batch = p.batch;
  sp.h_q = p.h_q;
  sp.h_kv = p.h_kv;
  sp.group = p.h_q / p.h_kv;
  sp.d = p.d;
  sp.scale = p.scale;
  sp.c2 = p.scale * kLog2e;
  sp.n_qtiles = (int)split_qtiles(p);
  sp.n_ktiles = (int)split_ktiles(p);
  sp.kv_bk = split_kv_bk(p);
  const int n_sched = p.batch > 0 ? (p.batch + 3) / 4 : 0;
  sp.n_qsched_wg = n_sched;
  sp.n_ksched_wg = n_sched;
  sp.n_qzero_wg = (int)((p.T_q + kPadRows - 1) / kPadRows);
  sp.n_kzero_wg = (int)((p.T_kv + kPadRows - 1) / kPadRows);
  const int64_t n_pre =
      (int64_t)sp.n_qsched_wg + sp.n_ksched_wg + sp.n_qzero_wg + sp.n_kzero_wg;
  if (p.d <= 32)
    return p.bf16 ? launch_split_t<Bf16, 32>(sp, n_pre, s, ev) : launch_split_t<Fp16, 32>(sp, n_pre, s, ev);
  if (p.d <= 64)
    return p.bf16 ? launch_split_t<Bf16, 64>(sp, n_pre, s, ev) : launch_split_t<Fp16, 64>(sp, n_pre, s, ev);
  if (p.d <= 128)
    return p.bf16 ? launch_split_t<Bf16, 128>(sp, n_pre, s, ev) : launch_split_t<Fp16, 128>(sp, n_pre, s, ev);
  return p.bf16 ? launch_split_t<Bf16, 256>(sp, n_pre, s, ev) : launch_split_t<Fp16, 256>(sp, n_pre, s, ev);
}

}  // namespace thd
