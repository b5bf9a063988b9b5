// dk/dv pass of the backward (see thd_bwd_split.hip
// for the whole backward and its sources).
//
// One workgroup per (sequence, key tile of BK = 256 or 128 keys, kv head), in
// schedule order, kv heads minor.  Each wave owns NB blocks of 32 keys and keeps dK^T and dV^T for
// them in registers (K and V sit in LDS) while the workgroup walks the 32-row
// query tiles its keys can see (down to the diagonal when causal), from the
// last one down, every query head of its GQA group at each tile.  Per query tile and key block: S = Q K^T and dP = dO V^T
// (accumulators starting from -LSE/scale and -D), P = exp2(S scale log2e),
// dS = P dP, dV^T += dO^T P and dK^T += Q^T dS (Q^T, dO^T from transpose
// reads).  With NB > 1 a wave's operand reads of Q, dO, Q^T and dO^T serve
// every one of its key blocks.
//
// LDS (bytes, DP = 128, BK = 256): Q and dO of two query tiles (double
// buffered, 32K), K 64K and V 64K (resident) = 160K; the next tile's Q and dO
// are loaded into registers while the current one is computed and stored to
// the other buffer at the end, and one barrier per query tile publishes it.
// BK = 128: one query tile (16K), K 32K, V 32K = 80K, two workgroups per CU;
// the next tile is stored after a barrier that ends every wave's reads of the
// current one, and a second barrier publishes it.  DP = 256 takes BK = 128
// only: 32K + 64K + 64K = 160K, one workgroup per CU.  Tiles are row-major with
// swizzled 16-byte chunks (see swz).
#include "thd_bwd_split.hpp"

namespace thd {
namespace split {

namespace {

// Key blocks of 32 per wave.  Two (four waves, one per SIMD, 256
// accumulators per lane kept in the accumulation registers by assembly
// products) was parity-green and halved the operand reads per product, but
// ran the benchmark workload's pass in 292 against 255 us and the GQA
// workload's in 16.1 against 14.3 ms: with one wave per SIMD nothing overlaps
// its softmax and its waits.
constexpr int kDkdvBlocks = 1;

template <class DT, int DP, int NB, int BK>
__global__ __launch_bounds__(64 * BK / (32 * NB), DP > 128 ? 1 : 256 * NB / BK)
void thd_bwd_dkdv_kernel(SplitParams p) {
  constexpr int BQ = kKvBQ, NQB = kKvQBufs<BK>;
  constexpr int NW = BK / (32 * NB);  // waves per workgroup
  constexpr int NTH = 64 * NW;      // threads per workgroup
  constexpr int NC = DP / 16;
  constexpr int ND = DP / 32;
  constexpr int KCH = DP / 8;
  constexpr int TILE = BQ * DP * 2;
  constexpr int OFF_Q = 0;          // Q of buffer j at 2j TILE, dO at (2j + 1) TILE
  constexpr int OFF_K = 2 * NQB * TILE;
  constexpr int OFF_V = OFF_K + BK * DP * 2;
  constexpr int SMEM = OFF_V + BK * DP * 2;
  constexpr int NSTAGE = (BQ * KCH + NTH - 1) / NTH;  // Q / dO chunks per thread
  static_assert(SMEM <= 163840, "LDS budget of one workgroup");
  static_assert(OFF_K < 65536, "tiles read through the offset field start below 64K");
  static_assert(BK == 32 * NB * NW, "the waves' key blocks cover the tile");
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  unsigned char* Kt = smem + OFF_K;
  unsigned char* Vt = smem + OFF_V;

  const int bid = blockIdx.x;
  const int rk = bid / p.h_kv;
  const int hk = bid - rk * p.h_kv;
  SchedItem item;
  if (!load_sched_item(p.ksched, rk, item)) return;
  const int b = uniform(item.b);
  const int tile_in_seq = uniform(item.t);
  if (b < 0 || b >= p.batch || tile_in_seq < 0) return;

  const int tid = threadIdx.x;
  const int w = uniform(tid >> 6);  // key blocks NB w .. NB w + NB - 1
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
  const int k0 = tile_in_seq * BK;
  if (k0 >= lk) return;
  const int kw0 = k0 + 32 * NB * w;  // first key of this wave

  // Keys [k0, lk) of kv head hk -> LDS, straight from memory: load i of wave
  // w fills 1 KB block NW i + w of each tile, lane l the 16-byte slot
  // 64 (NW i + w) + l (row slot / KCH, swizzled chunk position slot % KCH,
  // holding memory chunk (slot % KCH) ^ f(row)); rows past lk read as zeros.
  // Waited for before the first barrier.
  const uint16_t* kbase = p.k + (sk + k0) * (int64_t)p.h_kv * p.d + (int64_t)hk * p.d;
  const uint16_t* vbase = p.v + (sk + k0) * (int64_t)p.h_kv * p.d + (int64_t)hk * p.d;
  const uint32_t kv_bytes = (uint32_t)(lk - k0) * kvrow_bytes;
  {
    static_assert(BK * KCH % (64 * NW) == 0, "whole 1 KB blocks per wave");
    const u32x4 k_rs = rsrc_words(kbase, kv_bytes);
    const u32x4 v_rs = rsrc_words(vbase, kv_bytes);
    const uint32_t k_lds = lds_addr(Kt), v_lds = lds_addr(Vt);
#pragma unroll
    for (int i = 0; i < BK * KCH / (64 * NW); ++i) {
      const int slot = 64 * (NW * i + w) + l;
      const int row = slot / KCH;
      const int x = slot - row * KCH;
      const int gc = x ^ (int)((swz<DP>(row, 0) >> 4) & (KCH - 1));
      const uint32_t o = 8 * gc < p.d ? (uint32_t)row * kvrow_bytes + 16u * gc : kOobOffset;
      buf_load_lds16(k_rs, k_lds + 1024u * (NW * i + w), o);
      buf_load_lds16(v_rs, v_lds + 1024u * (NW * i + w), o);
    }
  }

  const int q_start = causal ? max(floor_div(k0 - off, BQ), 0) * BQ : 0;
  const int n_qt = (lq > q_start) ? (lq - q_start + BQ - 1) / BQ : 0;
  const int n_iter = p.group * n_qt;

  // Staging of a query tile: BQ KCH chunks each of Q and dO, thread tid takes
  // chunks tid + NTH j.
  u32x4 qreg[NSTAGE], oreg[NSTAGE];
  uint32_t s_off[NSTAGE], s_lds[NSTAGE];
#pragma unroll
  for (int j = 0; j < NSTAGE; ++j) {
    const int ch = tid + NTH * j;
    const int row = ch / KCH, x = ch - row * KCH;
    const bool ld = ch < BQ * KCH;
    s_off[j] = (ld && 8 * x < p.d) ? (uint32_t)row * qrow_bytes + 16u * x : kOobOffset;
    s_lds[j] = ld ? swz<DP>(row, 8 * x) : 0xffffffffu;
    qreg[j] = oreg[j] = u32x4{0u, 0u, 0u, 0u};
  }
  auto load_q = [&](int hq_, int q0_, bool real) {
    const int64_t hoff = sq * (int64_t)p.h_q * p.d + (int64_t)hq_ * p.d;
    const rsrc_t q_rs = make_rsrc(p.q + hoff, (uint32_t)lq * qrow_bytes);
    const rsrc_t o_rs = make_rsrc(p.dout + hoff, (uint32_t)lq * qrow_bytes);
#pragma unroll
    for (int j = 0; j < NSTAGE; ++j) {
      const uint32_t o =
          (s_off[j] == kOobOffset || !real) ? kOobOffset : s_off[j] + (uint32_t)q0_ * qrow_bytes;
      qreg[j] = buf_load16(q_rs, o, 0);
      oreg[j] = buf_load16(o_rs, o, 0);
    }
  };
  auto store_q = [&](int qb) {
#pragma unroll
    for (int j = 0; j < NSTAGE; ++j)
      if (s_lds[j] != 0xffffffffu) {
        *(u32x4*)(smem + OFF_Q + 2 * qb * TILE + s_lds[j]) = qreg[j];
        *(u32x4*)(smem + OFF_Q + (2 * qb + 1) * TILE + s_lds[j]) = oreg[j];
      }
  };

  f32x16 dk_acc[NB][ND], dv_acc[NB][ND];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      dk_acc[nb][i] = f32x16{};
      dv_acc[nb][i] = f32x16{};
    }

  const float c2 = p.c2;
  // address bases: Q / dO rows r, chunk 2c + h; K / V rows of key block nb
  // (32 (NB w + nb) + r, whose swizzle equals row r's: the block offset is
  // added); transpose reads as in the other kernels
  const uint32_t b_q = swz<DP>(r, 8 * h);
  const uint32_t b_k = swz<DP>(32 * NB * w + r, 8 * h);
  const uint32_t b_t = swz<DP>(4 * h + (g16 >> 2), 16 * (grp & 1) + 4 * (g16 & 3));

  // Walk order: from the last query tile down to the first one the keys
  // see, every query head of the group at each tile before the next tile.
  // The key tiles of a sequence and kv head that run together (on one XCD)
  // then read the same Q / dO rows at about the same time.
  const int hq_first = hk * p.group, hq_last = hq_first + p.group - 1;
  const int q_last = n_qt > 0 ? q_start + (n_qt - 1) * BQ : q_start;
  int hq = hq_first, q0 = q_last;
  auto advance = [&](int& hq_, int& q0_) {
    if (hq_ < hq_last) {
      ++hq_;
    } else {
      hq_ = hq_first;
      q0_ -= BQ;
    }
  };

  // Row statistics of this lane's query rows q0 + 8m + 4h + e (register
  // 4m + e of the C layout), loaded one query tile ahead: -LSE/scale (the
  // initial S, so that P = exp2(S scale log2 e)) and -D (the initial dP, so
  // that dS = P dP); the load past the last tile goes out of range.
  f32x16 st_l, st_d;
  rsrc_t l_rs, d_rs;
  uint32_t st_off = kOobOffset;
  auto setup_stats = [&](int hq_, int q0_, bool real) {
    const int64_t roff = real ? (int64_t)hq_ * p.T_q + sq : 0;
    l_rs = make_rsrc(p.lsum + roff, (uint32_t)lq * 4u);
    d_rs = make_rsrc(p.dsum + roff, (uint32_t)lq * 4u);
    st_off = real ? (uint32_t)(q0_ + 4 * h) * 4u : kOobOffset;
  };
  auto load_stat = [&](int j) {
    const int m = j >> 1;
    const uint32_t o = st_off == kOobOffset ? kOobOffset : st_off + 32u * m;
    const f32x4 v = __builtin_bit_cast(f32x4, buf_load16((j & 1) ? d_rs : l_rs, o, 0));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (j & 1)
        st_d[4 * m + e] = v[e];
      else
        st_l[4 * m + e] = v[e];
    }
  };

  if (n_iter > 0) {
    setup_stats(hq, q0, true);
#pragma unroll
    for (int j = 0; j < 8; ++j) load_stat(j);
    load_q(hq, q0, true);
    store_q(0);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // K, V blocks in LDS (not counted by the compiler)
  __syncthreads();
  for (int iter = 0; iter < n_iter; ++iter) {
    const int qb = NQB == 2 ? iter & 1 : 0;
    const bool more = iter + 1 < n_iter;
    int hq_n = hq, q0_n = q0;
    advance(hq_n, q0_n);
    load_q(hq_n, q0_n, more);
    const uint32_t qbase = (uint32_t)(OFF_Q + 2 * qb * TILE);
    f32x16 s[NB], dp[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      s[nb] = st_l;
      dp[nb] = st_d;
    }
    setup_stats(hq_n, q0_n, more);
    {
      // Software pipelined: the operands of step c + 1 are read before the
      // products of step c, and the scheduler is kept from undoing it.
      const uint32_t a_q = opaque(b_q + qbase), a_k = opaque(b_k + OFF_K),
                     a_v = opaque(b_k + OFF_V);
      u32x4 qa[2], oa[2], ka[2][NB], va[2][NB];
      auto ld_s = [&](int c, int sl) {
        const uint32_t cx = (uint32_t)c << 5;
        qa[sl] = *(const u32x4*)(smem + (a_q ^ cx));
        oa[sl] = *(const u32x4*)(smem + (a_q ^ cx) + TILE);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          ka[sl][nb] = *(const u32x4*)(smem + (a_k ^ cx) + 32 * nb * DP * 2);
          va[sl][nb] = *(const u32x4*)(smem + (a_v ^ cx) + 32 * nb * DP * 2);
        }
      };
      ld_s(0, 0);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if (c + 1 < NC) ld_s(c + 1, (c + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          s[nb] = DT::mfma(as_vec8<DT>(qa[c & 1]), as_vec8<DT>(ka[c & 1][nb]), s[nb]);
          dp[nb] = DT::mfma(as_vec8<DT>(oa[c & 1]), as_vec8<DT>(va[c & 1][nb]), dp[nb]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    typename DT::vec8 pb[NB][2], db[NB][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      // mask: key past lk, query row past lq, or (causal) key after the row;
      // only blocks on the diagonal or at a sequence's end need it
      const int kb0 = kw0 + 32 * nb;
      const int my_k = kb0 + r;
      const bool need_mask =
          (kb0 + 32 > lk) || (q0 + BQ > lq) || (causal && kb0 + 31 > q0 + off);
      if (__builtin_expect(need_mask, 0)) {
        const int lim_lo = causal ? my_k - q0 - off : -1;
        const int row_hi = my_k < lk ? lq - q0 : 0;
        // the rows' offset formed here: hoisted out of the walk, the 16 row
        // indices held 15 more VGPRs (at d = 64 the third wave per SIMD)
        const int h4 = (int)opaque(4u * h);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qi = 8 * (i >> 2) + h4 + (i & 3);
          if (!(qi >= lim_lo && qi < row_hi)) s[nb][i] = -__builtin_inff();
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = __builtin_amdgcn_exp2f(s[nb][i] * c2);
        s[nb][i] = pv;
        dp[nb][i] = pv * dp[nb][i];
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float tp[8], td[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          tp[j] = s[nb][8 * kb + j];
          td[j] = dp[nb][8 * kb + j];
        }
        pb[nb][kb] = pack8<DT>(tp);
        db[nb][kb] = pack8<DT>(td);
      }
    }
    {
      // dV^T += dO^T P and dK^T += Q^T dS: each transposed operand read serves
      // every key block; the next tile's statistics are loaded meanwhile
      const uint32_t a_t = opaque(b_t + qbase);
      u32x4 to[2], tq[2];
      auto ld_t = [&](int i, int sl) {
        const int dt = i >> 1, kb = i & 1;
        const uint32_t t0 = (a_t ^ tr_chunk<DP>(dt, 0)) + tr_row<DP>(kb, 0);
        const uint32_t t1 = (a_t ^ tr_chunk<DP>(dt, 1)) + tr_row<DP>(kb, 1);
        to[sl] = cat2(lds_read_tr(smem + TILE, t0), lds_read_tr(smem + TILE, t1));
        tq[sl] = cat2(lds_read_tr(smem, t0), lds_read_tr(smem, t1));
      };
      constexpr int kSteps = 2 * ND;  // statistics loads spread over the steps
      ld_t(0, 0);
#pragma unroll
      for (int i = 0; i < 2 * ND; ++i) {
        const int dt = i >> 1, kb = i & 1;
        if (i + 1 < 2 * ND) ld_t(i + 1, (i + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          dv_acc[nb][dt] = DT::mfma(as_vec8<DT>(to[i & 1]), pb[nb][kb], dv_acc[nb][dt]);
          dk_acc[nb][dt] = DT::mfma(as_vec8<DT>(tq[i & 1]), db[nb][kb], dk_acc[nb][dt]);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if ((j * kSteps) / 8 == i) load_stat(j);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (NQB == 2) {
      // The next tile goes into the other buffer, which every wave left at
      // the barrier ending the previous iteration.
      if (more) store_q(qb ^ 1);
      __syncthreads();
    } else {
      __syncthreads();  // every wave is done with this tile's Q and dO
      if (more) store_q(0);
      __syncthreads();
    }
    hq = hq_n;
    q0 = q0_n;
  }

  const rsrc_t dk_rs = make_rsrc(p.dk + (sk + k0) * (int64_t)p.h_kv * p.d + (int64_t)hk * p.d,
                                 kv_bytes);
  const rsrc_t dv_rs = make_rsrc(p.dv + (sk + k0) * (int64_t)p.h_kv * p.d + (int64_t)hk * p.d,
                                 kv_bytes);
  // Each wave stages its key blocks' dK and dV (bf16, row-major, swizzled) in
  // its own part of the K/V tiles, free once the walk is over, then stores
  // whole rows: each store covers 64 / KCH full rows.  (Stored straight from
  // the accumulators, 8 bytes per lane and 32 rows per store, the pass took
  // 0.247 against 0.229 ms on 16 causal sequences of 64-2,048 tokens, h 16,
  // d 128, and 0.96 against 0.78 ms on 32 cross-attention pairs.)
  static_assert(2 * NB * 32 * DP * 2 * NW <= 2 * BK * DP * 2, "staging fits the K/V tiles");
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    unsigned char* st_k = smem + OFF_K + (size_t)(2 * (NB * w + nb)) * 32 * DP * 2;
    unsigned char* st_v = st_k + 32 * DP * 2;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int dd = 32 * dt + 8 * gq + 4 * h;
        u32x2 ok, ov;
        ok[0] = (uint32_t)DT::bits(dk_acc[nb][dt][4 * gq + 0] * p.scale) |
                ((uint32_t)DT::bits(dk_acc[nb][dt][4 * gq + 1] * p.scale) << 16);
        ok[1] = (uint32_t)DT::bits(dk_acc[nb][dt][4 * gq + 2] * p.scale) |
                ((uint32_t)DT::bits(dk_acc[nb][dt][4 * gq + 3] * p.scale) << 16);
        ov[0] = (uint32_t)DT::bits(dv_acc[nb][dt][4 * gq + 0]) |
                ((uint32_t)DT::bits(dv_acc[nb][dt][4 * gq + 1]) << 16);
        ov[1] = (uint32_t)DT::bits(dv_acc[nb][dt][4 * gq + 2]) |
                ((uint32_t)DT::bits(dv_acc[nb][dt][4 * gq + 3]) << 16);
        *(u32x2*)(st_k + swz<DP>(r, dd)) = ok;
        *(u32x2*)(st_v + swz<DP>(r, dd)) = ov;
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < 32 * KCH / 64; ++j) {
      const int c = l + 64 * j;
      const int row = c / KCH, x = c - row * KCH;
      const u32x4 vk = *(const u32x4*)(st_k + swz<DP>(row, 8 * x));
      const u32x4 vv = *(const u32x4*)(st_v + swz<DP>(row, 8 * x));
      const uint32_t o = 8 * x < p.d ? (uint32_t)(32 * (NB * w + nb) + row) * kvrow_bytes + 16u * x
                                     : kOobOffset;
      buf_store16(vk, dk_rs, o, 0);
      buf_store16(vv, dv_rs, o, 0);
    }
  }
}

}  // namespace

template <class DT, int DP>
hipError_t launch_dkdv(const SplitParams& p, hipStream_t s) {
  const dim3 grid((unsigned)(p.n_ktiles * p.h_kv));
  if constexpr (DP <= 128) {
    if (p.kv_bk == kKvBkLong) {
      hipLaunchKernelGGL((thd_bwd_dkdv_kernel<DT, DP, kDkdvBlocks, kKvBkLong>), grid,
                         dim3(64 * kKvBkLong / (32 * kDkdvBlocks)), 0, s, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((thd_bwd_dkdv_kernel<DT, DP, kDkdvBlocks, kKvBkShort>), grid,
                     dim3(64 * kKvBkShort / (32 * kDkdvBlocks)), 0, s, p);
  return hipGetLastError();
}

template hipError_t launch_dkdv<Bf16, 32>(const SplitParams&, hipStream_t);
template hipError_t launch_dkdv<Fp16, 32>(const SplitParams&, hipStream_t);
template hipError_t launch_dkdv<Bf16, 64>(const SplitParams&, hipStream_t);
template hipError_t launch_dkdv<Fp16, 64>(const SplitParams&, hipStream_t);
template hipError_t launch_dkdv<Bf16, 128>(const SplitParams&, hipStream_t);
template hipError_t launch_dkdv<Fp16, 128>(const SplitParams&, hipStream_t);
template hipError_t launch_dkdv<Bf16, 256>(const SplitParams&, hipStream_t);
template hipError_t launch_dkdv<Fp16, 256>(const SplitParams&, hipStream_t);

}  // namespace split
}  // namespace thd
