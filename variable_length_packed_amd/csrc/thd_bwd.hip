// Backward attention over packed variable-length ("thd") tensors, head dims
// above 128 (136 .. 256; smaller head dims take the two-pass backward of
// thd_bwd_split.hip).
//
// Gradients of sum(O * dO) w.r.t. Q, K and V for the forward in thd_fwd.hip
// (TransformerEngine PR "Add per-sequence causal policy to packed THD
// attention", Changes: Q/K/V gradient parity with the scalar-policy path).
// Textbook softmax-attention backward with the probabilities recomputed from
// the forward's log-sum-exp:
//   P = exp(scale * Q K^T - LSE),  dV = P^T dO,  dP = dO V^T,
//   dS = P * (dP - D) with D = rowsum(dO * O),
//   dQ = scale * dS K,  dK = scale * dS^T Q.
//
// Three launches, correct first and not tuned:
//   pre  : -D per (row, head), -LSE/scale, zeroing of the fp32 dQ
//          accumulator, and the main kernel's schedule (key tiles grouped by
//          sequence, each sequence's largest first);
//   main : one workgroup of 4 waves per (sequence, 64-key tile, kv head); dK
//          and dV of a tile in registers, dQ of each query tile added to the
//          accumulator with fp32 atomics;
//   post : dQ accumulator -> storage dtype, zeros on pad rows of dK and dV.
#include <type_traits>

#include "thd_common.hpp"
#include "thd_launch.hpp"

namespace thd {

namespace {

constexpr int kBwdBQ = 32;   // query rows per step
constexpr int kWideBK = 64;  // keys per workgroup
constexpr int kZeroRowsB = 64;

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* dq_acc;  // [T_q, h_q, DP], row-major like dq
  float* dsum;    // [h_q, T_q], holds -D
  float* lsum;    // [h_q, T_q], holds -LSE / scale
  int32_t* sched; // item count, then the items by rank (build_schedule_by_sequence)
  const int32_t* cu_q;
  const int32_t* cu_kv;
  const int32_t* pad_q;
  const int32_t* pad_kv;
  const uint8_t* causal;
  int64_t T_q, T_kv;
  int batch, h_q, h_kv, group, d;
  float scale, c2;
  int n_kv_tiles;  // key tiles per kv head (upper bound)
  int n_main;      // n_kv_tiles * h_kv
  int n_sched;     // leading workgroups of the pre pass that build the schedule
};

// ---------------------------------------------------------------------------
// pre: -D = -rowsum(dO * O) in fp32, -LSE / scale, and dq_acc = 0; DP / 8 lanes
// per (row, head).
// ---------------------------------------------------------------------------
// Schedule of the main kernel (grouped by sequence, largest tile first, see
// build_schedule_by_sequence): key tile
// kt of sequence b walks W = ceil(lq / BQ) query tiles, or, with a causal
// mask type, those from the first one that sees key kt * BK:
// W = clamp(ceil(lq / BQ) - (BK / BQ) kt + ceil(off / BQ), 0, ceil(lq / BQ)),
// with the main kernel's clamping of the lengths.
template <int BK>
struct BwdSchedModel {
  static_assert(BK % kBwdBQ == 0, "work model assumes whole query tiles per key tile");
  static constexpr int kSlope = -BK / kBwdBQ;
  const BwdParams& p;
  int64_t acc_row_bytes;  // accumulator row: the main kernel's clamp of lq
  __device__ SeqSummary seq(int b) const {
    const int64_t sq = seq_start(p.cu_q, p.pad_q, b);
    const int64_t sk = seq_start(p.cu_kv, p.pad_kv, b);
    const int lq =
        clamp_rows(sq, seq_len_clamped(p.cu_q, b, p.T_q), p.T_q, acc_row_bytes);
    const int lk =
        clamp_rows(sk, seq_len_clamped(p.cu_kv, b, p.T_kv), p.T_kv, (int64_t)p.h_kv * p.d * 2);
    const int mt = mask_type_of(p.causal, b);
    SeqSummary s;
    s.x = ceil_div_pos(lk, BK);
    s.H = ceil_div_pos(lq, kBwdBQ);
    s.causal = mask_is_causal(mt);
    s.c = s.H + ceil_div(causal_offset(mt, lq, lk), kBwdBQ);
    s.sq = (int)sq;
    s.sk = (int)sk;
    s.lq = lq;
    s.lk = lk;
    s.mtype = mt;
    return s;
  }
};

// Keys per workgroup of the main kernel.
template <int DP>
constexpr int kMainBK = kWideBK;

// (row, head) pairs per pre / post workgroup: KCH = DP / 8 lanes per pair
// (one 16-byte chunk each), 256 / KCH lane groups, two pairs per group.
template <int DP>
constexpr int kPairsPerBlock = 2 * 256 / (DP / 8);

template <class DT, int DP>
__global__ __launch_bounds__(256) void thd_bwd_pre_kernel(BwdParams p) {
  if ((int)blockIdx.x < p.n_sched) {
    build_schedule_by_sequence(BwdSchedModel<kMainBK<DP>>{p, (int64_t)p.h_q * DP * 4}, p.batch,
                               p.n_kv_tiles, p.sched,
                   blockIdx.x * 4 + (int)(threadIdx.x >> 6));
    return;
  }
  // A workgroup covers PB consecutive rows of one head; consecutive
  // workgroups take the heads of one row block in turn, so that together
  // they stream the block's rows of o, dout and the accumulator, and each
  // writes its rows' statistics ([h_q][T_q]) as one contiguous run.
  constexpr int KCH = DP / 8, PB = kPairsPerBlock<DP>;
  const int64_t pairs = p.T_q * p.h_q;
  const int64_t bb = (int64_t)((int)blockIdx.x - p.n_sched);
  const int64_t rb = bb / p.h_q;
  const int head = (int)(bb - rb * p.h_q);
  const int g = threadIdx.x / KCH;
  const int c = threadIdx.x % KCH;
  // Every row is processed, pad rows included: the main kernel reads -D and
  // -LSE/scale only at rows inside a sequence (through range-limited
  // resources), and the accumulator of a pad row receives no atomics, so it
  // stays zero and converts to the +0 the pad rows of dq need.
  int64_t pr[2], si[2];
  u32x4 a[2], gr[2];
  float lse_v[2] = {0.f, 0.f};
  // All loads first (the LSE too), so that each wave has them in flight at once.
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int64_t row = rb * PB + g + t * (PB / 2);
    pr[t] = row < p.T_q ? row * p.h_q + head : pairs;  // pairs: past the end
    si[t] = (int64_t)head * p.T_q + row;              // statistics: [h_q][T_q]
    a[t] = gr[t] = u32x4{0u, 0u, 0u, 0u};
    if (pr[t] < pairs && 8 * c < p.d) {
      const int64_t off = pr[t] * p.d + 8 * c;  // o, dout: [T_q][h_q][d]
      a[t] = *(const u32x4*)(p.o + off);
      gr[t] = *(const u32x4*)(p.dout + off);
    }
    if (pr[t] < pairs && c == 1) lse_v[t] = p.lse[si[t]];
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (pr[t] < pairs) {
      float* dst = p.dq_acc + pr[t] * DP + 8 * c;
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      *(f32x4*)dst = z;
      *(f32x4*)(dst + 4) = z;
    }
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc += DT::to_f32((uint16_t)(a[t][w] & 0xffffu)) * DT::to_f32((uint16_t)(gr[t][w] & 0xffffu));
      acc += DT::to_f32((uint16_t)(a[t][w] >> 16)) * DT::to_f32((uint16_t)(gr[t][w] >> 16));
    }
    acc = group_sum<KCH>(acc);
    if (pr[t] < pairs && c < 2) {
      if (c == 0) p.dsum[si[t]] = -acc;                     // -D
      else p.lsum[si[t]] = lse_v[t] * (-1.0f / p.scale);   // -LSE / scale
    }
  }
}

// ---------------------------------------------------------------------------
// main, head dims above 128 (DP = 256)
// ---------------------------------------------------------------------------
// One workgroup of 4 waves per (sequence, 64-key tile, kv head).  Wave w owns
// keys 32 (w & 1) .. +31 of the tile and the half 128 (w >> 1) .. +127 of the
// head dim for its dK^T / dV^T accumulators (the 256-wide accumulators of 32
// keys would not fit one wave's registers); the two waves of a key group both
// form S and dP over the whole head dim.  dQ of a query tile comes from dS
// staged in LDS: wave w takes d columns 64w .. 64w+63 over the 64 keys.  The
// same textbook gradients as the kernel above.
//
// LDS: K 32K, V 32K, Q 16K, dO 16K (row-major, swizzled 16-byte chunks as in
// the kernel above) and dS 4K = 100K.  Q and dO of the next query tile go
// straight into LDS once every wave is done with the current ones.
template <class DT>
__global__ __launch_bounds__(256, 1) void thd_bwd_main_wide_kernel(BwdParams p) {
  constexpr int DP = 256, BK = kWideBK, BQ = kBwdBQ;
  constexpr int NC = DP / 16;      // K steps of S and dP
  constexpr int NDH = 4;           // 32-column d tiles of a wave's half
  constexpr int KCH = DP / 8;      // 16-byte chunks per row
  constexpr int OFF_K = 0;
  constexpr int OFF_V = OFF_K + BK * DP * 2;
  constexpr int OFF_Q = OFF_V + BK * DP * 2;
  constexpr int OFF_DO = OFF_Q + BQ * DP * 2;
  constexpr int OFF_DS = OFF_DO + BQ * DP * 2;
  constexpr int SMEM = OFF_DS + BQ * BK * 2;
  static_assert(SMEM <= 163840, "LDS budget of one workgroup");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[SMEM];
  unsigned char* Kt = smem + OFF_K;
  unsigned char* Vt = smem + OFF_V;
  unsigned char* Qb = smem + OFF_Q;
  unsigned char* Ob = smem + OFF_DO;
  unsigned char* dSs = smem + OFF_DS;

  const int bid = blockIdx.x;
  const int rk = bid / p.h_kv;
  const int hk = bid - rk * p.h_kv;
  SchedItem item;
  if (!load_sched_item(p.sched, rk, item)) return;
  const int b = uniform(item.b);
  const int tile_in_seq = uniform(item.t);
  if (b < 0 || b >= p.batch || tile_in_seq < 0) return;

  const int tid = threadIdx.x;
  const int w = uniform(tid >> 6);
  const int kg = w & 1;   // key group: keys 32 kg .. 32 kg + 31 of the tile
  const int dh = w >> 1;  // accumulator half: d 128 dh .. 128 dh + 127
  const int l = tid & 63;
  const int r = l & 31;
  const int h = l >> 5;
  const int g16 = l & 15;
  const int grp = l >> 4;

  const uint32_t qrow_bytes = (uint32_t)p.h_q * p.d * 2;
  const uint32_t kvrow_bytes = (uint32_t)p.h_kv * p.d * 2;
  const uint32_t accrow_bytes = (uint32_t)p.h_q * DP * 4;
  // the item's slot starts, lengths (clamped as BwdSchedModel clamps them)
  // and mask type
  const int64_t sq = uniform(item.sq);
  const int64_t sk = uniform(item.sk);
  const int lq = uniform(item.lq);
  const int lk = uniform(item.lk);
  const int mtype = uniform(item.mtype);
  const bool causal = mask_is_causal(mtype);
  const int off = causal_offset(mtype, lq, lk);
  const int k0 = tile_in_seq * BK;
  if (k0 >= lk) return;
  const int kw0 = k0 + 32 * kg;
  const int my_k = kw0 + r;

  // A row-major tile of `rows` rows goes from memory straight into LDS: load
  // i of wave w fills 1 KB block 4i + w, lane l the 16-byte slot
  // 64 (4i + w) + l (row slot / KCH, swizzled chunk position slot % KCH,
  // holding the row's memory chunk (slot % KCH) ^ f(row)); chunks past d
  // read as zeros, and so do rows past the resource.
  auto tile_to_lds = [&](const u32x4& rs, uint32_t lds, uint32_t row_bytes, int rows) {
    for (int i = 0; i < rows * KCH / 256; ++i) {
      const int slot = 64 * (4 * i + w) + l;
      const int row = slot / KCH;
      const int x = slot - row * KCH;
      const int gc = x ^ (int)((swz<DP>(row, 0) >> 4) & (KCH - 1));
      const uint32_t o = 8 * gc < p.d ? (uint32_t)row * row_bytes + 16u * gc : kOobOffset;
      buf_load_lds16(rs, lds + 1024u * (4 * i + w), o);
    }
  };
  {
    const uint16_t* kbase = p.k + (sk + k0) * (int64_t)p.h_kv * p.d + (int64_t)hk * p.d;
    const uint16_t* vbase = p.v + (sk + k0) * (int64_t)p.h_kv * p.d + (int64_t)hk * p.d;
    const uint32_t kv_bytes = (uint32_t)(lk - k0) * kvrow_bytes;
    tile_to_lds(rsrc_words(kbase, kv_bytes), lds_addr(Kt), kvrow_bytes, BK);
    tile_to_lds(rsrc_words(vbase, kv_bytes), lds_addr(Vt), kvrow_bytes, BK);
  }
  // Query rows q0 .. q0+31 of head hq (Q and dO) into LDS.
  auto qtile_to_lds = [&](int hq_, int q0_) {
    const int64_t hoff = sq * (int64_t)p.h_q * p.d + (int64_t)hq_ * p.d + (int64_t)q0_ * p.h_q * p.d;
    const uint32_t left = (uint32_t)(lq - q0_) * qrow_bytes;
    tile_to_lds(rsrc_words(p.q + hoff, left), lds_addr(Qb), qrow_bytes, BQ);
    tile_to_lds(rsrc_words(p.dout + hoff, left), lds_addr(Ob), qrow_bytes, BQ);
  };

  const int q_start = causal ? max(floor_div(k0 - off, BQ), 0) * BQ : 0;
  const int n_qt = (lq > q_start) ? (lq - q_start + BQ - 1) / BQ : 0;
  const int n_iter = p.group * n_qt;

  f32x16 dk_acc[NDH], dv_acc[NDH];
#pragma unroll
  for (int i = 0; i < NDH; ++i) {
    dk_acc[i] = f32x16{};
    dv_acc[i] = f32x16{};
  }
  const float c2 = p.c2;
  const uint32_t b_q = swz<DP>(r, 8 * h);
  const uint32_t b_k = swz<DP>(32 * kg + r, 8 * h);
  const uint32_t b_t = swz<DP>(4 * h + (g16 >> 2), 16 * (grp & 1) + 4 * (g16 & 3));
  // dS tile [BQ][BK]: key j of a 16-key block sits at position
  // (j & 3) | ((j >> 3) & 1) << 2 | ((j >> 2) & 1) << 3, so that the 8 keys a
  // transposed K operand row group holds ({4h .. 4h+3, 8+4h .. 8+4h+3}) are
  // one 16-byte chunk; chunks XOR-swizzled by row & 7.
  auto ds_off = [](int q, int key) -> uint32_t {
    const int pos = (key & ~15) | (key & 3) | (((key >> 3) & 1) << 2) | (((key >> 2) & 1) << 3);
    return (uint32_t)q * (BK * 2) + ((uint32_t)((pos >> 3) ^ (q & 7)) << 4) + (uint32_t)(pos & 7) * 2;
  };

  int hq = hk * p.group, q0 = q_start;
  if (n_iter > 0) qtile_to_lds(hq, q0);
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): K, V and the first query tile are in LDS
  __syncthreads();
  for (int iter = 0; iter < n_iter; ++iter) {
    // Row statistics of this lane's query rows q0 + 8m + 4h + e (register
    // 4m + e): S starts from -LSE/scale and dP from -D.
    f32x16 s, dp;
    {
      const int64_t roff = (int64_t)hq * p.T_q + sq;
      const rsrc_t l_rs = make_rsrc(p.lsum + roff, (uint32_t)lq * 4u);
      const rsrc_t d_rs = make_rsrc(p.dsum + roff, (uint32_t)lq * 4u);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t so = (uint32_t)(q0 + 8 * m + 4 * h) * 4u;
        const f32x4 lv = __builtin_bit_cast(f32x4, buf_load16(l_rs, so, 0));
        const f32x4 dv = __builtin_bit_cast(f32x4, buf_load16(d_rs, so, 0));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[4 * m + e] = lv[e];
          dp[4 * m + e] = dv[e];
        }
      }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint32_t cx = (uint32_t)c << 5;
      const u32x4 qa = *(const u32x4*)(Qb + (b_q ^ cx));
      const u32x4 ka = *(const u32x4*)(Kt + (b_k ^ cx));
      const u32x4 oa = *(const u32x4*)(Ob + (b_q ^ cx));
      const u32x4 va = *(const u32x4*)(Vt + (b_k ^ cx));
      s = DT::mfma(as_vec8<DT>(qa), as_vec8<DT>(ka), s);
      dp = DT::mfma(as_vec8<DT>(oa), as_vec8<DT>(va), dp);
    }
    {
      const int lim_lo = causal ? my_k - q0 - off : -1;
      const int row_hi = my_k < lk ? lq - q0 : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qi = 8 * (i >> 2) + 4 * h + (i & 3);
        if (!(qi >= lim_lo && qi < row_hi)) s[i] = -__builtin_inff();
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float pv = __builtin_amdgcn_exp2f(s[i] * c2);
      s[i] = pv;
      dp[i] = pv * dp[i];
    }
    typename DT::vec8 pb[2], db[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float tp[8], td[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        tp[j] = s[8 * kb + j];
        td[j] = dp[8 * kb + j];
      }
      pb[kb] = pack8<DT>(tp);
      db[kb] = pack8<DT>(td);
    }
    // dV^T += dO^T P and dK^T += Q^T dS over this wave's half of the head dim
#pragma unroll
    for (int dt = 0; dt < NDH; ++dt)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int dg = 4 * dh + dt;  // 32-column d tile of the whole head dim
        const uint32_t t0 = b_t ^ tr_xor<DP>(dg, kb, 0);
        const uint32_t t1 = b_t ^ tr_xor<DP>(dg, kb, 1);
        const u32x4 to = cat2(lds_read_tr(Ob, t0), lds_read_tr(Ob, t1));
        const u32x4 tq = cat2(lds_read_tr(Qb, t0), lds_read_tr(Qb, t1));
        dv_acc[dt] = DT::mfma(as_vec8<DT>(to), pb[kb], dv_acc[dt]);
        dk_acc[dt] = DT::mfma(as_vec8<DT>(tq), db[kb], dk_acc[dt]);
      }
    // dS (query-major) for the dQ product; the two waves of a key group hold
    // the same values, the first one writes them.
    if (dh == 0) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 words = __builtin_bit_cast(u32x4, db[kb]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = 8 * kb + j;
          const int qi = 8 * (i >> 2) + 4 * h + (i & 3);
          *(uint16_t*)(dSs + ds_off(qi, 32 * kg + r)) = (uint16_t)(words[j >> 1] >> (16 * (j & 1)));
        }
      }
    }
    __syncthreads();  // dS complete; every wave is done with this tile's Q and dO

    int hq_n = hq, q0_n = q0 + BQ;
    if (q0_n >= lq) {
      q0_n = q_start;
      ++hq_n;
    }
    if (iter + 1 < n_iter) qtile_to_lds(hq_n, q0_n);

    // dQ[q][64w + 32nt + n] = sum over the tile's keys of dS[q][key] K[key][.]:
    // A = dS rows (one 16-byte chunk, keys in the order the transposed K
    // operand holds them), B = K^T from transpose reads of the K tile.
    f32x16 dq[2] = {f32x16{}, f32x16{}};
    int kv_act = lk - k0;
    if (kv_act > BK) kv_act = BK;
#pragma unroll
    for (int kb = 0; kb < BK / 16; ++kb) {
      if (16 * kb >= kv_act) break;
      const u32x4 da = *(const u32x4*)(dSs + ds_off(r, 16 * kb + 4 * h));
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int dg = 2 * w + nt;
        const u32x4 kt = cat2(lds_read_tr(Kt, b_t ^ tr_xor<DP>(dg, kb, 0)),
                              lds_read_tr(Kt, b_t ^ tr_xor<DP>(dg, kb, 1)));
        dq[nt] = DT::mfma(as_vec8<DT>(da), as_vec8<DT>(kt), dq[nt]);
      }
    }
    {
      // lane (r, h) holds dQ[q0 + 8(i/4) + 4h + (i%4)][64w + 32nt + r]; rows
      // past lq and columns past d fall outside the resource / are skipped.
      const rsrc_t acc_rs =
          make_rsrc(p.dq_acc + (sq * p.h_q + hq) * DP, (uint32_t)lq * accrow_bytes);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int col = 64 * w + 32 * nt + r;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = q0 + 8 * (i >> 2) + 4 * h + (i & 3);
          const uint32_t o = col < p.d ? (uint32_t)row * accrow_bytes + 4u * col : kOobOffset;
          buf_atomic_add(dq[nt][i], acc_rs, o, 0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // the next query tile is in LDS
    __syncthreads();                     // and every wave is done with dS
    hq = hq_n;
    q0 = q0_n;
  }

  const uint32_t kv_bytes = (uint32_t)(lk - k0) * kvrow_bytes;
  const rsrc_t dk_rs = make_rsrc(p.dk + (sk + k0) * (int64_t)p.h_kv * p.d + (int64_t)hk * p.d,
                                 kv_bytes);
  const rsrc_t dv_rs = make_rsrc(p.dv + (sk + k0) * (int64_t)p.h_kv * p.d + (int64_t)hk * p.d,
                                 kv_bytes);
  const uint32_t krow = (uint32_t)(32 * kg + r) * kvrow_bytes;
#pragma unroll
  for (int dt = 0; dt < NDH; ++dt)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int dd = 128 * dh + 32 * dt + 8 * gq + 4 * h;
      if (dd < p.d) {
        u32x2 ok, ov;
        ok[0] = (uint32_t)DT::bits(dk_acc[dt][4 * gq + 0] * p.scale) |
                ((uint32_t)DT::bits(dk_acc[dt][4 * gq + 1] * p.scale) << 16);
        ok[1] = (uint32_t)DT::bits(dk_acc[dt][4 * gq + 2] * p.scale) |
                ((uint32_t)DT::bits(dk_acc[dt][4 * gq + 3] * p.scale) << 16);
        ov[0] = (uint32_t)DT::bits(dv_acc[dt][4 * gq + 0]) |
                ((uint32_t)DT::bits(dv_acc[dt][4 * gq + 1]) << 16);
        ov[1] = (uint32_t)DT::bits(dv_acc[dt][4 * gq + 2]) |
                ((uint32_t)DT::bits(dv_acc[dt][4 * gq + 3]) << 16);
        buf_store8(ok, dk_rs, krow + 2u * dd, 0);
        buf_store8(ov, dv_rs, krow + 2u * dd, 0);
      }
    }
}

// ---------------------------------------------------------------------------
// post: dq = scale * dq_acc in the storage dtype; zero pad rows of dk / dv.
// ---------------------------------------------------------------------------
template <class DT, int DP>
__global__ __launch_bounds__(256) void thd_bwd_post_kernel(BwdParams p, int n_zero_wg) {
  const int tid = threadIdx.x;
  // The pad-row workgroups come first: each starts with a dependent search of
  // the sequence starts, whose latency the conversion stream behind it covers.
  if ((int)blockIdx.x >= n_zero_wg) {
    // (row, head) pairs in row-major order, like the pre pass: pair pr sits
    // at pr * DP in the accumulator and at pr * d in dq, so each thread reads
    // and writes chunk c of two pairs of one stream each.
    constexpr int KCH = DP / 8, PB = kPairsPerBlock<DP>;
    const int64_t pairs = p.T_q * p.h_q;
    const int64_t p0 = (int64_t)((int)blockIdx.x - n_zero_wg) * PB;
    const int g = tid / KCH;
    const int c = tid % KCH;
    if (8 * c >= p.d) return;
    f32x4 v[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t pr = p0 + g + t * (PB / 2);
      if (pr < pairs) {
        const float* src = p.dq_acc + pr * DP + 8 * c;
        v[t][0] = *(const f32x4*)src;
        v[t][1] = *(const f32x4*)(src + 4);
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t pr = p0 + g + t * (PB / 2);
      if (pr < pairs) {
        u32x4 out;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const f32x4& x = v[t][k >> 1];
          out[k] = (uint32_t)DT::bits(x[2 * (k & 1)] * p.scale) |
                   ((uint32_t)DT::bits(x[2 * (k & 1) + 1] * p.scale) << 16);
        }
        *(u32x4*)(p.dq + pr * p.d + 8 * c) = out;
      }
    }
    return;
  }
  __shared__ uint8_t invalid[kZeroRowsB];
  const int64_t r0 = (int64_t)blockIdx.x * kZeroRowsB;
  int mine = 0;
  if (tid < kZeroRowsB) {
    const int64_t rr = r0 + tid;
    const bool inv = rr < p.T_kv && !row_is_valid(p.cu_kv, p.pad_kv, p.batch, rr, p.T_kv);
    invalid[tid] = inv;
    mine = inv;
  }
  if (!__syncthreads_or(mine)) return;
  const int chunks = p.h_kv * p.d / 8;
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int idx = tid; idx < kZeroRowsB * chunks; idx += 256) {
    const int rr = idx / chunks;
    const int c = idx - rr * chunks;
    if (invalid[rr]) {
      const int64_t off = (r0 + rr) * (int64_t)(p.h_kv * p.d) + 8 * c;
      *(u32x4*)(p.dk + off) = z;
      *(u32x4*)(p.dv + off) = z;
    }
  }
}

template <class DT, int DP>
hipError_t launch_bwd_t(const BwdParams& bp, hipStream_t s, hipEvent_t const* ev) {
  auto mark = [&](int i) -> hipError_t {
    return ev ? hipEventRecord(ev[i], s) : hipSuccess;
  };
  hipError_t em = mark(0);
  if (em != hipSuccess) return em;
  const int64_t n_pair_blocks = (bp.T_q * bp.h_q + kPairsPerBlock<DP> - 1) / kPairsPerBlock<DP>;
  const int64_t n_pre =
      bp.n_sched + (bp.T_q + kPairsPerBlock<DP> - 1) / kPairsPerBlock<DP> * bp.h_q;
  if (n_pre > 0) {
    hipLaunchKernelGGL((thd_bwd_pre_kernel<DT, DP>), dim3((unsigned)n_pre), dim3(256), 0, s, bp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((em = mark(1)) != hipSuccess) return em;
  if (bp.n_main > 0) {
    static_assert(DP == 256, "head dims up to 128 take the two-pass backward");
    hipLaunchKernelGGL((thd_bwd_main_wide_kernel<DT>), dim3(bp.n_main), dim3(256), 0, s, bp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((em = mark(2)) != hipSuccess) return em;
  const int64_t n_conv = n_pair_blocks;
  const int64_t n_zero = (bp.T_kv + kZeroRowsB - 1) / kZeroRowsB;
  if (n_conv + n_zero > 0) {
    hipLaunchKernelGGL((thd_bwd_post_kernel<DT, DP>), dim3((unsigned)(n_conv + n_zero)), dim3(256), 0,
                       s, bp, (int)n_zero);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return mark(3);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int padded_dim(int d) { return d <= 32 ? 32 : d <= 64 ? 64 : d <= 128 ? 128 : 256; }

}  // namespace

static int64_t kv_tile_bound(const Problem& p) { return (p.T_kv + kWideBK - 1) / kWideBK + p.batch; }

// Head dims up to 128: the two-pass backward's workspace.  Above: the fp32 dq
// accumulator [T_q][h_q][256], then -D = -rowsum(dO * O) and -LSE / scale (each [h_q][T_q]), then
// the main kernel's schedule (sched_bytes of the key-tile bound).
static bool use_split(const Problem& p) { return p.d <= 128; }

size_t bwd_workspace_bytes(const Problem& p) {
  if (use_split(p)) return split_bwd_workspace_bytes(p);
  const size_t acc = align256((size_t)p.T_q * p.h_q * padded_dim(p.d) * sizeof(float));
  const size_t dsum = align256((size_t)p.T_q * p.h_q * 2 * sizeof(float));
  const size_t sched = align256(sched_bytes(kv_tile_bound(p)));
  return acc + dsum + sched;
}

hipError_t launch_bwd(const Problem& p, const void* q, const void* k, const void* v,
                      const void* o, const void* dout, const float* lse, void* dq, void* dk,
                      void* dv, void* workspace, hipStream_t s, hipEvent_t const* ev) {
  if (use_split(p))
    return launch_bwd_split(p, q, k, v, o, dout, lse, dq, dk, dv, workspace, s, ev);
  BwdParams bp;
  bp.q = (const uint16_t*)q;
  bp.k = (const uint16_t*)k;
  bp.v = (const uint16_t*)v;
  bp.o = (const uint16_t*)o;
  bp.dout = (const uint16_t*)dout;
  bp.lse = lse;
  bp.dq = (uint16_t*)dq;
  bp.dk = (uint16_t*)dk;
  bp.dv = (uint16_t*)dv;
  bp.dq_acc = (float*)workspace;
  const size_t acc_bytes = align256((size_t)p.T_q * p.h_q * padded_dim(p.d) * sizeof(float));
  bp.dsum = (float*)((char*)workspace + acc_bytes);
  bp.lsum = bp.dsum + (size_t)p.T_q * p.h_q;
  bp.sched = (int32_t*)((char*)workspace + acc_bytes +
                        align256((size_t)p.T_q * p.h_q * 2 * sizeof(float)));
  bp.cu_q = p.cu_q;
  bp.cu_kv = p.cu_kv;
  bp.pad_q = p.pad_q;
  bp.pad_kv = p.pad_kv;
  bp.causal = p.causal;
  bp.T_q = p.T_q;
  bp.T_kv = p.T_kv;
  bp.batch = p.batch;
  bp.h_q = p.h_q;
  bp.h_kv = p.h_kv;
  bp.group = p.h_q / p.h_kv;
  bp.d = p.d;
  bp.scale = p.scale;
  bp.c2 = p.scale * kLog2e;
  const int64_t n_kv_tiles = kv_tile_bound(p);
  bp.n_kv_tiles = (int)n_kv_tiles;
  bp.n_main = (p.batch > 0) ? (int)(n_kv_tiles * p.h_kv) : 0;
  bp.n_sched = (p.batch > 0) ? (p.batch + 3) / 4 : 0;
  return p.bf16 ? launch_bwd_t<Bf16, 256>(bp, s, ev) : launch_bwd_t<Fp16, 256>(bp, s, ev);
}

}  // namespace thd
