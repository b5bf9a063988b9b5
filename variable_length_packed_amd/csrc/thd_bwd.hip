// Backward attention over packed variable-length ("thd") tensors.
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
// Three launches:
//   pre  : D per (row, head) and zeroing of the fp32 dQ accumulator;
//   main : one workgroup per (sequence, 128-key tile, kv head); each wave
//          owns 32 keys and keeps K, V, dK^T and dV^T in registers while it
//          walks the 32-row query tiles (from the diagonal when causal) of
//          every query head of its GQA group.  dQ of a query tile is
//          computed by the whole workgroup from dS staged in LDS (wave w
//          takes d columns 32w..32w+31) and added to the accumulator with
//          fp32 atomics;
//   post : dQ accumulator -> storage dtype, zeros on pad rows of dK and dV.
#include <type_traits>

#include "thd_common.hpp"
#include "thd_launch.hpp"

namespace thd {

namespace {

constexpr int kBwdBK = 128;  // keys per workgroup
constexpr int kBwdBQ = 32;   // query rows per step
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
  float* dq_acc;  // [T_q, h_q, d]
  float* dsum;    // [h_q, T_q]
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
};

// ---------------------------------------------------------------------------
// pre: D = rowsum(dO * O) in fp32, and dq_acc = 0.  16 lanes per (row, head).
// ---------------------------------------------------------------------------
template <class DT, int DP>
__global__ __launch_bounds__(256) void thd_bwd_pre_kernel(BwdParams p) {
  const int64_t pair = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int c = threadIdx.x & 15;
  if (pair >= p.T_q * p.h_q) return;  // whole 16-lane groups leave together
  const int64_t row = pair / p.h_q;
  const int hh = (int)(pair - row * p.h_q);
  const bool valid = row_is_valid(p.cu_q, p.pad_q, p.batch, row, p.T_q);
  const int64_t off = row * (int64_t)p.h_q * p.d + (int64_t)hh * p.d + 8 * c;
  float acc = 0.f;
  if (8 * c < p.d) {
    if (valid) {
      const u32x4 a = *(const u32x4*)(p.o + off);
      const u32x4 g = *(const u32x4*)(p.dout + off);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc += DT::to_f32((uint16_t)(a[w] & 0xffffu)) * DT::to_f32((uint16_t)(g[w] & 0xffffu));
        acc += DT::to_f32((uint16_t)(a[w] >> 16)) * DT::to_f32((uint16_t)(g[w] >> 16));
      }
    }
  }
  if (8 * c < DP) {
    // accumulator layout [h_q][T_q][DP]
    float* acc = p.dq_acc + ((int64_t)hh * p.T_q + row) * DP + 8 * c;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    *(f32x4*)acc = z;
    *(f32x4*)(acc + 4) = z;
  }
  acc += __shfl_xor(acc, 8, 16);
  acc += __shfl_xor(acc, 4, 16);
  acc += __shfl_xor(acc, 2, 16);
  acc += __shfl_xor(acc, 1, 16);
  if (c == 0) p.dsum[(int64_t)hh * p.T_q + row] = valid ? acc : 0.f;
}

// ---------------------------------------------------------------------------
// main
// ---------------------------------------------------------------------------
// One workgroup of 8 waves per (sequence, 128-key tile, kv head).  The waves
// form two halves of 4; wave w of a half owns keys 32w .. 32w+31 and keeps
// dK^T / dV^T for them in registers.  The halves share the K and V tiles in
// LDS and take alternate query tiles (items 2j + half of the list
// "every query head of the GQA group x every 32-row query tile from the
// diagonal"), each with its own double-buffered Q / dO / LSE / D tiles and dS
// tile, so two waves share each SIMD.  At the end the halves' dK and dV are
// summed through LDS.
//
// LDS (bytes, DP = 128): K 32K, V 32K, per half 2 x (Q 8K + dO 8K) + LSE/D
// 512 + dS 8.5K.  Q, dO, K and V are row-major with swizzled 16-byte chunks;
// Q^T, dO^T and K^T operands come from transpose reads.
template <class DT, int DP>
__global__ __launch_bounds__(512, 1) void thd_bwd_main_kernel(BwdParams p) {
  constexpr int BK = kBwdBK, BQ = kBwdBQ;
  constexpr int NC = DP / 16;
  constexpr int ND = DP / 32;
  constexpr int KCH = DP / 8;
  constexpr int SST = BK + 8;   // dS row stride (elements)
  constexpr int TILE = BQ * DP * 2;
  constexpr int OFF_K = 0;
  constexpr int OFF_V = OFF_K + BK * DP * 2;
  constexpr int OFF_HALF = OFF_V + BK * DP * 2;
  // half-local layout
  constexpr int H_Q = 0;
  constexpr int H_DO = H_Q + 2 * TILE;
  constexpr int H_LSE = H_DO + 2 * TILE;
  constexpr int H_D = H_LSE + 2 * BQ * 4;
  constexpr int H_DS = H_D + 2 * BQ * 4;
  constexpr int HALF_BYTES = H_DS + BQ * SST * 2;
  constexpr int SMEM = OFF_HALF + 2 * HALF_BYTES;
  static_assert(2 * 4 * 64 * ND * 16 * 4 <= SMEM, "dK/dV reduction must fit the LDS");
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  unsigned char* Kt = smem + OFF_K;
  unsigned char* Vt = smem + OFF_V;

  const int bid = blockIdx.x;
  const int logical = xcd_remap(bid, p.n_main);
  const int hk = logical / p.n_kv_tiles;
  const int t = logical - hk * p.n_kv_tiles;
  int tile_in_seq = 0;
  const int b = uniform(find_tile(p.cu_kv, p.batch, p.T_kv, BK, t, p.n_kv_tiles, &tile_in_seq));
  if (b < 0) return;
  tile_in_seq = uniform(tile_in_seq);

  const int tid = threadIdx.x;
  const int wg = uniform(tid >> 6);  // wave in the workgroup, 0..7
  const int half = wg >> 2;
  const int w = wg & 3;              // wave in its half: keys 32w .. 32w+31
  const int ltid = tid & 255;        // thread in its half
  const int l = tid & 63;
  const int r = l & 31;
  const int h = l >> 5;
  const int g16 = l & 15;            // lane inside its 16-lane group
  const int grp = l >> 4;            // 16-lane group of the wave
  unsigned char* hbase = smem + OFF_HALF + half * HALF_BYTES;
  uint16_t* dSs = (uint16_t*)(hbase + H_DS);

  const uint32_t qrow_bytes = (uint32_t)p.h_q * p.d * 2;
  const uint32_t kvrow_bytes = (uint32_t)p.h_kv * p.d * 2;
  const uint32_t accrow_bytes = (uint32_t)p.h_q * p.d * 4;
  const int64_t sq = seq_start(p.cu_q, p.pad_q, b);
  const int64_t sk = seq_start(p.cu_kv, p.pad_kv, b);
  const int lq = uniform(clamp_rows(sq, seq_len_clamped(p.cu_q, b, p.T_q), p.T_q, accrow_bytes));
  const int lk = uniform(clamp_rows(sk, seq_len_clamped(p.cu_kv, b, p.T_kv), p.T_kv, kvrow_bytes));
  const bool causal = p.causal ? (p.causal[b] != 0) : false;
  const int k0 = tile_in_seq * BK;
  if (k0 >= lk) return;
  const int kw0 = k0 + 32 * w;
  const int my_k = kw0 + r;

  // Keys [k0, lk) of kv head hk; rows past lk read as zeros.
  const uint16_t* kbase = p.k + (sk + k0) * (int64_t)p.h_kv * p.d + (int64_t)hk * p.d;
  const uint16_t* vbase = p.v + (sk + k0) * (int64_t)p.h_kv * p.d + (int64_t)hk * p.d;
  const uint32_t kv_bytes = (uint32_t)(lk - k0) * kvrow_bytes;
  {
    const rsrc_t k_rs = make_rsrc(kbase, kv_bytes);
    const rsrc_t v_rs = make_rsrc(vbase, kv_bytes);
#pragma unroll
    for (int i = 0; i < BK * KCH / 512; ++i) {
      const int cid = tid + 512 * i;
      const int row = cid / KCH;
      const int x = cid - row * KCH;
      const uint32_t off = 8 * x < p.d ? (uint32_t)row * kvrow_bytes + 16u * x : kOobOffset;
      *(u32x4*)(Kt + swz<DP>(row, 8 * x)) = buf_load16(k_rs, off, 0);
      *(u32x4*)(Vt + swz<DP>(row, 8 * x)) = buf_load16(v_rs, off, 0);
    }
  }

  // Query tiles: from the first tile that can see key k0 when causal.
  const int q_start = causal ? (k0 / BQ) * BQ : 0;
  const int n_qt = (lq > q_start) ? (lq - q_start + BQ - 1) / BQ : 0;
  const int n_iter = p.group * n_qt;
  const int n_rounds = (n_iter + 1) / 2;

  // Staging of one query tile by the 256 threads of a half: BQ*KCH chunks of
  // Q and of dO; threads 256-BQ .. 255 of the half also fetch LSE and D.
  constexpr int QLOADS = (BQ * KCH + 255) / 256;
  const int st_lane = ltid - (256 - BQ);
  u32x4 qreg[QLOADS], oreg[QLOADS];
  float lse_r = 0.f, d_r = 0.f;

  auto load_q = [&](int hq, int q0) {
    const int64_t hoff = sq * (int64_t)p.h_q * p.d + (int64_t)hq * p.d;
    const rsrc_t q_rs = make_rsrc(p.q + hoff, (uint32_t)lq * qrow_bytes);
    const rsrc_t o_rs = make_rsrc(p.dout + hoff, (uint32_t)lq * qrow_bytes);
#pragma unroll
    for (int i = 0; i < QLOADS; ++i) {
      const int cid = ltid + 256 * i;
      const int row = cid / KCH;
      const int x = cid - row * KCH;
      const uint32_t off = (cid < BQ * KCH && 8 * x < p.d)
                               ? (uint32_t)(q0 + row) * qrow_bytes + 16u * x
                               : kOobOffset;
      qreg[i] = buf_load16(q_rs, off, 0);
      oreg[i] = buf_load16(o_rs, off, 0);
    }
    if (st_lane >= 0) {
      const int qi = q0 + st_lane;
      if (qi < lq) {
        const int64_t idx = (int64_t)hq * p.T_q + sq + qi;
        lse_r = p.lse[idx] * kLog2e;
        d_r = p.dsum[idx];
      } else {
        lse_r = __builtin_inff();  // rows past the sequence get P = 0
        d_r = 0.f;
      }
    }
  };

  auto store_q = [&](int buf) {
    unsigned char* Qb = hbase + H_Q + buf * TILE;
    unsigned char* Ob = hbase + H_DO + buf * TILE;
#pragma unroll
    for (int i = 0; i < QLOADS; ++i) {
      const int cid = ltid + 256 * i;
      const int row = cid / KCH;
      const int x = cid - row * KCH;
      if (cid < BQ * KCH) {
        *(u32x4*)(Qb + swz<DP>(row, 8 * x)) = qreg[i];
        *(u32x4*)(Ob + swz<DP>(row, 8 * x)) = oreg[i];
      }
    }
    if (st_lane >= 0) {
      ((float*)(hbase + H_LSE))[buf * BQ + st_lane] = lse_r;
      ((float*)(hbase + H_D))[buf * BQ + st_lane] = d_r;
    }
  };

  // A half without an item (last round, odd count) still runs the products
  // on its buffers with everything masked: start them as finite zeros.
  for (int i = ltid; i < (2 * TILE * 2 + 4 * BQ * 4) / 16; i += 256)
    ((u32x4*)hbase)[i] = u32x4{0u, 0u, 0u, 0u};

  f32x16 dk_acc[ND], dv_acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) {
    dk_acc[i] = f32x16{};
    dv_acc[i] = f32x16{};
  }

  // Transpose-read addressing: lane s of a 16-lane group reads row
  // R0 + s/4, columns C0 + 4*(s%4) .. +3.
  const int tr_row = g16 >> 2;
  const int tr_col = 4 * (g16 & 3);
  const float c2 = p.c2;
  const int dcol = 32 * w + r;  // d column of this lane in the dQ product

  // Item it -> (query head, first query row); a half walks it = half, +2, ...
  auto item = [&](int it, int& hq_, int& q0_) {
    const int hi = it / n_qt;
    hq_ = hk * p.group + hi;
    q0_ = q_start + (it - hi * n_qt) * BQ;
  };
  int it = half;
  int hq = 0, q0 = 0;
  if (it < n_iter) item(it, hq, q0);
  __syncthreads();  // K / V tiles and zeroed buffers visible
  if (it < n_iter) {
    load_q(hq, q0);
    store_q(0);
  }
  __syncthreads();
  for (int round = 0; round < n_rounds; ++round, it += 2) {
    const int buf = round & 1;
    const bool live = it < n_iter;
    const bool more = it + 2 < n_iter;
    int hq_n = 0, q0_n = 0;
    if (more) {
      item(it + 2, hq_n, q0_n);
      load_q(hq_n, q0_n);
    }

    const unsigned char* Qb = hbase + H_Q + buf * TILE;
    const unsigned char* Ob = hbase + H_DO + buf * TILE;
    const float* lse2s = (const float*)(hbase + H_LSE) + buf * BQ;
    const float* dds = (const float*)(hbase + H_D) + buf * BQ;

    // Every wave runs the products, also when none of its keys is visible to
    // this query tile or its half has no item (then the mask zeroes P and
    // dS): the accumulators are updated unconditionally and stay in the MFMA
    // registers across iterations.
    {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const u32x4 qa = *(const u32x4*)(Qb + swz<DP>(r, 16 * c + 8 * h));
        const u32x4 ka = *(const u32x4*)(Kt + swz<DP>(32 * w + r, 16 * c + 8 * h));
        const u32x4 oa = *(const u32x4*)(Ob + swz<DP>(r, 16 * c + 8 * h));
        const u32x4 va = *(const u32x4*)(Vt + swz<DP>(32 * w + r, 16 * c + 8 * h));
        s = DT::mfma(as_vec8<DT>(qa), as_vec8<DT>(ka), s);
        dp = DT::mfma(as_vec8<DT>(oa), as_vec8<DT>(va), dp);
      }
      const bool need_mask = !live || (kw0 + 32 > lk) || (causal && kw0 + 31 > q0);
      const int lim_lo = causal ? my_k - q0 : -1;  // visible iff qi >= my_k - q0
      const bool key_ok = live && my_k < lk;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qi = 8 * (i >> 2) + 4 * h + (i & 3);
        float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c2, -lse2s[qi]));
        if (need_mask) pv = (key_ok && qi >= lim_lo) ? pv : 0.f;
        s[i] = pv;
        dp[i] = pv * (dp[i] - dds[qi]);
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
      // dV^T += dO^T P and dK^T += Q^T dS.  A operand lane (r, h) needs
      // column d = 32dt + r at query slots q = 16kb + {4h..4h+3, 8+4h..8+4h+3},
      // the order in which P / dS hold them: two transpose reads.
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        const int c0 = 32 * dt + 16 * (grp & 1) + tr_col;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int r0 = 16 * kb + 4 * h + tr_row;
          const u32x4 to =
              cat2(lds_read_tr(Ob, swz<DP>(r0, c0)), lds_read_tr(Ob, swz<DP>(r0 + 8, c0)));
          const u32x4 tq =
              cat2(lds_read_tr(Qb, swz<DP>(r0, c0)), lds_read_tr(Qb, swz<DP>(r0 + 8, c0)));
          dv_acc[dt] = DT::mfma(as_vec8<DT>(to), pb[kb], dv_acc[dt]);
          dk_acc[dt] = DT::mfma(as_vec8<DT>(tq), db[kb], dk_acc[dt]);
        }
      }
      // dS (query-major) for the dQ product of this half; elements are taken
      // from the packed 32-bit words (element j sits in word j/2, half j&1).
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 words = __builtin_bit_cast(u32x4, db[kb]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = 8 * kb + j;
          const int qi = 8 * (i >> 2) + 4 * h + (i & 3);
          dSs[qi * SST + 32 * w + r] = (uint16_t)(words[j >> 1] >> (16 * (j & 1)));
        }
      }
    }
    __syncthreads();  // dS complete; every wave is done with this query buffer
    if (more) store_q(buf ^ 1);

    if (live && w < ND) {
      // dQ[q][32w + r] = sum_kv dS[q][kv] K[kv][32w + r]; B operand lane
      // (r, h) needs K rows 16kb + 8h + 0..7 at column 32w + r.
      int kv_act = lk - k0;
      if (kv_act > BK) kv_act = BK;
      if (causal && q0 + BQ - k0 < kv_act) kv_act = q0 + BQ - k0;
      const int nkb = (kv_act + 15) / 16;
      const int c0 = 32 * w + 16 * (grp & 1) + tr_col;
      f32x16 dq = f32x16{};
#pragma unroll
      for (int kb = 0; kb < BK / 16; ++kb) {
        if (kb < nkb) {
          const u32x4 da = *(const u32x4*)(&dSs[r * SST + 16 * kb + 8 * h]);
          const int r0 = 16 * kb + 8 * h + tr_row;
          const u32x4 kt =
              cat2(lds_read_tr(Kt, swz<DP>(r0, c0)), lds_read_tr(Kt, swz<DP>(r0 + 4, c0)));
          dq = DT::mfma(as_vec8<DT>(da), as_vec8<DT>(kt), dq);
        }
      }
      // rows past lq fall outside the resource and are dropped; accumulator
      // layout [h_q][T_q][DP], so the 4 rows of a group are immediate offsets
      const rsrc_t acc_rs = make_rsrc(p.dq_acc + ((int64_t)hq * p.T_q + sq) * DP,
                                      (uint32_t)lq * (DP * 4));
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t base =
            dcol < p.d ? (uint32_t)((q0 + 8 * g + 4 * h) * DP + dcol) * 4u : kOobOffset;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          buf_atomic_add(dq[4 * g + e], acc_rs,
                         base == kOobOffset ? kOobOffset : base + e * DP * 4, 0);
      }
    }
    __syncthreads();  // next query buffers visible; dS reads done
    hq = hq_n;
    q0 = q0_n;
  }

  // Sum the halves: half 1 parks its dK, half 0 its dV in LDS (element-major,
  // lane-contiguous), then half 0 writes dK and half 1 writes dV.
  float* red = (float*)smem;
  constexpr int PER = 4 * 64;  // lanes of one half
  const int slot = w * 64 + l;
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float x = half ? dk_acc[dt][i] : dv_acc[dt][i];
      red[(half * ND * 16 + dt * 16 + i) * PER + slot] = x;
    }
  __syncthreads();
  f32x16 out[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float other = red[((1 - half) * ND * 16 + dt * 16 + i) * PER + slot];
      out[dt][i] = (half ? dv_acc[dt][i] : dk_acc[dt][i]) + other;
    }
  const float mul = half ? 1.f : p.scale;  // dK carries the softmax scale
  uint16_t* dst = half ? p.dv : p.dk;
  const rsrc_t o_rs = make_rsrc(dst + (sk + k0) * (int64_t)p.h_kv * p.d + (int64_t)hk * p.d,
                                kv_bytes);
  const uint32_t krow = (uint32_t)(32 * w + r) * kvrow_bytes;
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int dd = 32 * dt + 8 * gq + 4 * h;
      if (dd < p.d) {
        u32x2 ov;
        ov[0] = (uint32_t)DT::bits(out[dt][4 * gq + 0] * mul) |
                ((uint32_t)DT::bits(out[dt][4 * gq + 1] * mul) << 16);
        ov[1] = (uint32_t)DT::bits(out[dt][4 * gq + 2] * mul) |
                ((uint32_t)DT::bits(out[dt][4 * gq + 3] * mul) << 16);
        buf_store8(ov, o_rs, krow + 2u * dd, 0);
      }
    }
}

// ---------------------------------------------------------------------------
// post: dq = scale * dq_acc in the storage dtype; zero pad rows of dk / dv.
// ---------------------------------------------------------------------------
template <class DT, int DP>
__global__ __launch_bounds__(256) void thd_bwd_post_kernel(BwdParams p, int64_t n_chunks,
                                                           int n_conv_wg) {
  const int tid = threadIdx.x;
  if ((int)blockIdx.x < n_conv_wg) {
    // chunk idx = ((hq * T_q) + row) * (d/8) + c: reads the head-major
    // accumulator in order, writes dq[row][hq][8c .. 8c+7]
    const int64_t idx = (int64_t)blockIdx.x * 256 + tid;
    if (idx >= n_chunks) return;
    const int cpr = p.d / 8;
    const int64_t hr = idx / cpr;
    const int c8 = (int)(idx - hr * cpr) * 8;
    const int64_t hq = hr / p.T_q;
    const int64_t row = hr - hq * p.T_q;
    const float* src = p.dq_acc + hr * DP + c8;
    const f32x4 a = *(const f32x4*)src;
    const f32x4 c = *(const f32x4*)(src + 4);
    u32x4 out;
    out[0] = (uint32_t)DT::bits(a[0] * p.scale) | ((uint32_t)DT::bits(a[1] * p.scale) << 16);
    out[1] = (uint32_t)DT::bits(a[2] * p.scale) | ((uint32_t)DT::bits(a[3] * p.scale) << 16);
    out[2] = (uint32_t)DT::bits(c[0] * p.scale) | ((uint32_t)DT::bits(c[1] * p.scale) << 16);
    out[3] = (uint32_t)DT::bits(c[2] * p.scale) | ((uint32_t)DT::bits(c[3] * p.scale) << 16);
    *(u32x4*)(p.dq + (row * p.h_q + hq) * p.d + c8) = out;
    return;
  }
  __shared__ uint8_t invalid[kZeroRowsB];
  const int64_t r0 = (int64_t)(blockIdx.x - n_conv_wg) * kZeroRowsB;
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
  const int64_t pairs = bp.T_q * bp.h_q;
  if (pairs > 0) {
    hipLaunchKernelGGL((thd_bwd_pre_kernel<DT, DP>), dim3((unsigned)((pairs + 15) / 16)), dim3(256),
                       0, s, bp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((em = mark(1)) != hipSuccess) return em;
  if (bp.n_main > 0) {
    hipLaunchKernelGGL((thd_bwd_main_kernel<DT, DP>), dim3(bp.n_main), dim3(512), 0, s, bp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((em = mark(2)) != hipSuccess) return em;
  const int64_t n_chunks = bp.T_q * bp.h_q * bp.d / 8;
  const int64_t n_conv = (n_chunks + 255) / 256;
  const int64_t n_zero = (bp.T_kv + kZeroRowsB - 1) / kZeroRowsB;
  if (n_conv + n_zero > 0) {
    hipLaunchKernelGGL((thd_bwd_post_kernel<DT, DP>), dim3((unsigned)(n_conv + n_zero)), dim3(256), 0,
                       s, bp, n_chunks, (int)n_conv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return mark(3);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int padded_dim(int d) { return d <= 32 ? 32 : d <= 64 ? 64 : 128; }

}  // namespace

// fp32 dq accumulator [h_q][T_q][DP] (DP = head_dim rounded up to 32, 64 or
// 128) followed by D = rowsum(dO * O) [h_q][T_q].
size_t bwd_workspace_bytes(const Problem& p) {
  const size_t acc = align256((size_t)p.T_q * p.h_q * padded_dim(p.d) * sizeof(float));
  const size_t dsum = align256((size_t)p.T_q * p.h_q * sizeof(float));
  return acc + dsum;
}

hipError_t launch_bwd(const Problem& p, const void* q, const void* k, const void* v,
                      const void* o, const void* dout, const float* lse, void* dq, void* dk,
                      void* dv, void* workspace, hipStream_t s, hipEvent_t const* ev) {
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
  bp.dsum = (float*)((char*)workspace +
                     align256((size_t)p.T_q * p.h_q * padded_dim(p.d) * sizeof(float)));
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
  const int64_t n_kv_tiles = (p.T_kv + kBwdBK - 1) / kBwdBK + p.batch;
  bp.n_kv_tiles = (int)n_kv_tiles;
  bp.n_main = (p.batch > 0) ? (int)(n_kv_tiles * p.h_kv) : 0;
  if (p.d <= 32) return p.bf16 ? launch_bwd_t<Bf16, 32>(bp, s, ev) : launch_bwd_t<Fp16, 32>(bp, s, ev);
  if (p.d <= 64) return p.bf16 ? launch_bwd_t<Bf16, 64>(bp, s, ev) : launch_bwd_t<Fp16, 64>(bp, s, ev);
  return p.bf16 ? launch_bwd_t<Bf16, 128>(bp, s, ev) : launch_bwd_t<Fp16, 128>(bp, s, ev);
}

}  // namespace thd
