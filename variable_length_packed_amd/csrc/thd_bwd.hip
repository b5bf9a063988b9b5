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

__device__ __forceinline__ int tr_group_pos(int g4) {
  return (g4 == 1) ? 2 : (g4 == 2) ? 1 : g4;
}

// ---------------------------------------------------------------------------
// pre: D = rowsum(dO * O) in fp32, and dq_acc = 0.  16 lanes per (row, head).
// ---------------------------------------------------------------------------
template <class DT>
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
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    *(f32x4*)(p.dq_acc + off) = z;
    *(f32x4*)(p.dq_acc + off + 4) = z;
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
template <class DT, int DP>
__global__ __launch_bounds__(256) void thd_bwd_main_kernel(BwdParams p) {
  constexpr int BK = kBwdBK, BQ = kBwdBQ;
  constexpr int NC = DP / 16;
  constexpr int ND = DP / 32;
  constexpr int RST = DP + 8;   // row-major Q / dO / K-staging stride
  constexpr int TST = BQ + 8;   // transposed Q / dO stride
  constexpr int SST = BK + 8;   // dS stride
  constexpr int KCH = DP / 8;
  constexpr int OFF_QS = 0;
  constexpr int OFF_DOS = OFF_QS + BQ * RST * 2;
  constexpr int OFF_QT = OFF_DOS + BQ * RST * 2;
  constexpr int OFF_DOT = OFF_QT + DP * TST * 2;
  constexpr int OFF_DS = OFF_DOT + DP * TST * 2;
  constexpr int OFF_LSE = OFF_DS + BQ * SST * 2;
  constexpr int OFF_D = OFF_LSE + BQ * 4;
  constexpr int SMEM = OFF_D + BQ * 4;
  constexpr int KSTAGE = BK * RST * 2;
  static_assert(KSTAGE <= OFF_DS, "K staging must fit below the dS region");
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  uint16_t* Qs = (uint16_t*)(smem + OFF_QS);
  uint16_t* dOs = (uint16_t*)(smem + OFF_DOS);
  uint16_t* Qt = (uint16_t*)(smem + OFF_QT);
  uint16_t* dOt = (uint16_t*)(smem + OFF_DOT);
  uint16_t* dSs = (uint16_t*)(smem + OFF_DS);
  float* lse2s = (float*)(smem + OFF_LSE);
  float* dds = (float*)(smem + OFF_D);
  uint16_t* Kst = (uint16_t*)smem;  // aliases the query-tile buffers at start

  const int bid = blockIdx.x;
  const int logical = xcd_remap(bid, p.n_main);
  const int hk = logical / p.n_kv_tiles;
  const int t = logical - hk * p.n_kv_tiles;
  int tile_in_seq = 0;
  const int b = find_tile(p.cu_kv, p.batch, p.T_kv, BK, t, p.n_kv_tiles, &tile_in_seq);
  if (b < 0) return;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  const int r = l & 31;
  const int h = l >> 5;

  const int lq = seq_len_clamped(p.cu_q, b, p.T_q);
  const int lk = seq_len_clamped(p.cu_kv, b, p.T_kv);
  const int64_t sq = seq_start(p.cu_q, p.pad_q, b);
  const int64_t sk = seq_start(p.cu_kv, p.pad_kv, b);
  const bool causal = p.causal ? (p.causal[b] != 0) : false;
  const int k0 = tile_in_seq * BK;
  const int kw0 = k0 + 32 * w;
  const int my_k = kw0 + r;
  const int64_t q_stride = (int64_t)p.h_q * p.d;
  const int64_t kv_stride = (int64_t)p.h_kv * p.d;

  // K and V of this lane's key as B operands (S = Q K^T, dP = dO V^T).
  typename DT::vec8 kB[NC], vB[NC];
  {
    const int64_t g = sk + my_k;
    const bool ok = my_k < lk && g >= 0 && g < p.T_kv;
    const uint16_t* ks = p.k + g * kv_stride + (int64_t)hk * p.d;
    const uint16_t* vs = p.v + g * kv_stride + (int64_t)hk * p.d;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int dd = 16 * c + 8 * h;
      u32x4 xk = {0u, 0u, 0u, 0u}, xv = {0u, 0u, 0u, 0u};
      if (ok && dd < p.d) {
        xk = *(const u32x4*)(ks + dd);
        xv = *(const u32x4*)(vs + dd);
      }
      kB[c] = as_vec8<DT>(xk);
      vB[c] = as_vec8<DT>(xv);
    }
  }

  // K of the whole tile as the B operand of dQ = dS K for d columns
  // 32w .. 32w+31: lane holds K[16kb + 8h + j][32w + r], staged via LDS.
  typename DT::vec8 kA[BK / 16];
  {
#pragma unroll
    for (int i = 0; i < BK * KCH / 256; ++i) {
      const int cid = tid + 256 * i;
      const int row = cid / KCH;
      const int c = cid - row * KCH;
      const int j = k0 + row;
      const int64_t g = sk + j;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (j < lk && g >= 0 && g < p.T_kv && 8 * c < p.d)
        x = *(const u32x4*)(p.k + g * kv_stride + (int64_t)hk * p.d + 8 * c);
      *(u32x4*)(&Kst[row * RST + 8 * c]) = x;
    }
    __syncthreads();
    if (w < ND) {
#pragma unroll
      for (int kb = 0; kb < BK / 16; ++kb) {
        uint16_t e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e[j] = Kst[(16 * kb + 8 * h + j) * RST + 32 * w + r];
        u32x4 x;
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = (uint32_t)e[2 * j] | ((uint32_t)e[2 * j + 1] << 16);
        kA[kb] = as_vec8<DT>(x);
      }
    }
  }

  // Query tiles: from the first tile that can see key k0 when causal.
  const int q_start = causal ? (k0 / BQ) * BQ : 0;
  const int n_qt = (lq > q_start) ? (lq - q_start + BQ - 1) / BQ : 0;
  const int n_iter = p.group * n_qt;

  // Staging of one query tile: thread t < DP loads 4 rows x 8 d of Q and dO;
  // threads 224..255 load LSE and D.
  const int s_grp = tid & 7;    // group of 4 query rows
  const int s_chunk = tid >> 3; // 8-wide d chunk
  u32x4 qreg[4], oreg[4];
  float lse_r = 0.f, d_r = 0.f;

  auto load_q = [&](int iter) {
    const int hq = hk * p.group + iter / n_qt;
    const int q0 = q_start + (iter % n_qt) * BQ;
    if (tid < DP) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int qi = q0 + 4 * s_grp + i;
        const int64_t g = sq + qi;
        u32x4 xq = {0u, 0u, 0u, 0u}, xo = {0u, 0u, 0u, 0u};
        if (qi < lq && g >= 0 && g < p.T_q && 8 * s_chunk < p.d) {
          const int64_t off = g * q_stride + (int64_t)hq * p.d + 8 * s_chunk;
          xq = *(const u32x4*)(p.q + off);
          xo = *(const u32x4*)(p.dout + off);
        }
        qreg[i] = xq;
        oreg[i] = xo;
      }
    }
    if (tid >= 256 - BQ) {
      const int qi = q0 + tid - (256 - BQ);
      const int64_t g = sq + qi;
      if (qi < lq && g >= 0 && g < p.T_q) {
        lse_r = p.lse[(int64_t)hq * p.T_q + g] * kLog2e;
        d_r = p.dsum[(int64_t)hq * p.T_q + g];
      } else {
        lse_r = __builtin_inff();
        d_r = 0.f;
      }
    }
  };

  auto store_transposed = [&](uint16_t* dstT, const u32x4* src) {
    const int pos = 16 * (s_grp >> 2) + 4 * tr_group_pos(s_grp & 3);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int word = e >> 1;
      const uint32_t x0 = src[0][word], x1 = src[1][word], x2 = src[2][word], x3 = src[3][word];
      u32x2 out;
      if (!(e & 1)) {
        out[0] = (x0 & 0xffffu) | (x1 << 16);
        out[1] = (x2 & 0xffffu) | (x3 << 16);
      } else {
        out[0] = (x0 >> 16) | (x1 & 0xffff0000u);
        out[1] = (x2 >> 16) | (x3 & 0xffff0000u);
      }
      *(u32x2*)(&dstT[(8 * s_chunk + e) * TST + pos]) = out;
    }
  };

  auto store_q = [&]() {
    if (tid < DP) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *(u32x4*)(&Qs[(4 * s_grp + i) * RST + 8 * s_chunk]) = qreg[i];
        *(u32x4*)(&dOs[(4 * s_grp + i) * RST + 8 * s_chunk]) = oreg[i];
      }
      store_transposed(Qt, qreg);
      store_transposed(dOt, oreg);
    }
    if (tid >= 256 - BQ) {
      lse2s[tid - (256 - BQ)] = lse_r;
      dds[tid - (256 - BQ)] = d_r;
    }
  };

  f32x16 dk_acc[ND], dv_acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) {
    dk_acc[i] = f32x16{};
    dv_acc[i] = f32x16{};
  }

  __syncthreads();  // K staging fully consumed before the buffers are reused
  if (n_iter > 0) load_q(0);
  for (int iter = 0; iter < n_iter; ++iter) {
    const int hq = hk * p.group + iter / n_qt;
    const int q0 = q_start + (iter % n_qt) * BQ;
    __syncthreads();
    store_q();
    __syncthreads();
    if (iter + 1 < n_iter) load_q(iter + 1);

    const bool active = (kw0 < lk) && (!causal || q0 + BQ - 1 >= kw0);
    if (active) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const u32x4 a = *(const u32x4*)(&Qs[r * RST + 16 * c + 8 * h]);
        s = DT::mfma(as_vec8<DT>(a), kB[c], s);
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const u32x4 a = *(const u32x4*)(&dOs[r * RST + 16 * c + 8 * h]);
        dp = DT::mfma(as_vec8<DT>(a), vB[c], dp);
      }
      const bool need_mask = (kw0 + 32 > lk) || (causal && kw0 + 31 > q0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qi = 8 * (i >> 2) + 4 * h + (i & 3);
        float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], p.c2, -lse2s[qi]));
        if (need_mask) {
          const bool vis = (my_k < lk) && (!causal || my_k <= q0 + qi);
          if (!vis) pv = 0.f;
        }
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
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x4 ao = *(const u32x4*)(&dOt[(32 * dt + r) * TST + 16 * kb + 8 * h]);
          dv_acc[dt] = DT::mfma(as_vec8<DT>(ao), pb[kb], dv_acc[dt]);
          const u32x4 aq = *(const u32x4*)(&Qt[(32 * dt + r) * TST + 16 * kb + 8 * h]);
          dk_acc[dt] = DT::mfma(as_vec8<DT>(aq), db[kb], dk_acc[dt]);
        }
      // dS (query-major) for the workgroup-wide dQ product; elements are taken
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
    __syncthreads();

    int kv_act = lk - k0;
    if (kv_act > BK) kv_act = BK;
    if (causal && q0 + BQ - k0 < kv_act) kv_act = q0 + BQ - k0;
    if (w < ND && kv_act > 0) {
      const int nkb = (kv_act + 15) / 16;
      f32x16 dq = f32x16{};
#pragma unroll
      for (int kb = 0; kb < BK / 16; ++kb) {
        if (kb < nkb) {
          const u32x4 a = *(const u32x4*)(&dSs[r * SST + 16 * kb + 8 * h]);
          dq = DT::mfma(as_vec8<DT>(a), kA[kb], dq);
        }
      }
      const int dcol = 32 * w + r;
      if (dcol < p.d) {
        float* base = p.dq_acc + (int64_t)hq * p.d + dcol;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qi = q0 + 8 * (i >> 2) + 4 * h + (i & 3);
          const int64_t g = sq + qi;
          if (qi < lq && g >= 0 && g < p.T_q) unsafeAtomicAdd(base + g * q_stride, dq[i]);
        }
      }
    }
  }

  // Epilogue: this lane's key row of dK (scaled) and dV.
  if (my_k < lk) {
    const int64_t g = sk + my_k;
    if (g >= 0 && g < p.T_kv) {
      uint16_t* dkp = p.dk + g * kv_stride + (int64_t)hk * p.d;
      uint16_t* dvp = p.dv + g * kv_stride + (int64_t)hk * p.d;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int dd = 32 * dt + 8 * gq + 4 * h;
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
            *(u32x2*)(dkp + dd) = ok;
            *(u32x2*)(dvp + dd) = ov;
          }
        }
    }
  }
}

// ---------------------------------------------------------------------------
// post: dq = scale * dq_acc in the storage dtype; zero pad rows of dk / dv.
// ---------------------------------------------------------------------------
template <class DT>
__global__ __launch_bounds__(256) void thd_bwd_post_kernel(BwdParams p, int64_t n_chunks,
                                                           int n_conv_wg) {
  const int tid = threadIdx.x;
  if ((int)blockIdx.x < n_conv_wg) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + tid;
    if (idx >= n_chunks) return;
    const f32x4 a = *(const f32x4*)(p.dq_acc + 8 * idx);
    const f32x4 c = *(const f32x4*)(p.dq_acc + 8 * idx + 4);
    u32x4 out;
    out[0] = (uint32_t)DT::bits(a[0] * p.scale) | ((uint32_t)DT::bits(a[1] * p.scale) << 16);
    out[1] = (uint32_t)DT::bits(a[2] * p.scale) | ((uint32_t)DT::bits(a[3] * p.scale) << 16);
    out[2] = (uint32_t)DT::bits(c[0] * p.scale) | ((uint32_t)DT::bits(c[1] * p.scale) << 16);
    out[3] = (uint32_t)DT::bits(c[2] * p.scale) | ((uint32_t)DT::bits(c[3] * p.scale) << 16);
    *(u32x4*)(p.dq + 8 * idx) = out;
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
    hipLaunchKernelGGL((thd_bwd_pre_kernel<DT>), dim3((unsigned)((pairs + 15) / 16)), dim3(256),
                       0, s, bp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((em = mark(1)) != hipSuccess) return em;
  if (bp.n_main > 0) {
    hipLaunchKernelGGL((thd_bwd_main_kernel<DT, DP>), dim3(bp.n_main), dim3(256), 0, s, bp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((em = mark(2)) != hipSuccess) return em;
  const int64_t n_chunks = bp.T_q * bp.h_q * bp.d / 8;
  const int64_t n_conv = (n_chunks + 255) / 256;
  const int64_t n_zero = (bp.T_kv + kZeroRowsB - 1) / kZeroRowsB;
  if (n_conv + n_zero > 0) {
    hipLaunchKernelGGL((thd_bwd_post_kernel<DT>), dim3((unsigned)(n_conv + n_zero)), dim3(256), 0,
                       s, bp, n_chunks, (int)n_conv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return mark(3);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t bwd_workspace_bytes(const Problem& p) {
  const size_t acc = align256((size_t)p.T_q * p.h_q * p.d * sizeof(float));
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
  bp.dsum = (float*)((char*)workspace + align256((size_t)p.T_q * p.h_q * p.d * sizeof(float)));
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
