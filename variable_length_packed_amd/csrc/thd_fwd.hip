// Forward attention over packed variable-length ("thd") tensors.
//
// Computes, per sequence and query head, softmax(scale * Q K^T + mask) V with
// the per-sequence causal flag of TransformerEngine PR "Add per-sequence
// causal policy to packed THD attention" (Description; top-left causal), the
// padded slot starts of that PR's two-call example (maintainer review), and
// pad rows written as zeros.  The mask of sequence b is derived inline from
// cu_seqlens (key j visible iff j < lk_b, and j <= i when causal), so no mask
// tensor is read and the host never synchronises.
//
// One workgroup = 4 waves = one (sequence, 128-row query tile, query head)
// work item, decoded on the device from cu_seqlens_q.  Each wave owns 32
// query rows.  Scores are computed transposed, S^T = K Q^T, so that a lane
// owns one query row: the row max needs one exchange between wave halves and
// the probabilities land directly in the B-operand layout of O^T = V^T P^T.
// K tiles are staged in LDS row-major, V tiles transposed (with the K-slot
// permutation that matches the accumulator layout of S^T).  Extra workgroups
// at the end of the grid write zeros to pad rows of O and -inf to their LSE.
#include "thd_common.hpp"
#include "thd_launch.hpp"

namespace thd {

namespace {

constexpr int kFwdBM = 128;  // query rows per workgroup
constexpr int kFwdBN = 64;   // keys per LDS tile
constexpr int kWaveM = 32;   // query rows per wave
constexpr int kZeroRows = 64;

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int32_t* cu_q;
  const int32_t* cu_kv;
  const int32_t* pad_q;
  const int32_t* pad_kv;
  const uint8_t* causal;
  int64_t T_q, T_kv;
  int batch, h_q, h_kv, group, d;
  float scale, c2;  // c2 = scale * log2(e)
  int n_tiles;      // query tiles per head (upper bound over all layouts)
  int n_attn;       // n_tiles * h_q workgroups doing attention
};

// Position of key group g4 (4 keys) inside a 16-key block of the transposed
// V tile: groups 1 and 2 trade places, so that lane half h reads keys
// {4h..4h+3, 8+4h..8+4h+3} of the block as 8 contiguous elements, which is
// the order in which the S^T accumulator holds them.
__device__ __forceinline__ int vt_group_pos(int g4) {
  return (g4 == 1) ? 2 : (g4 == 2) ? 1 : g4;
}

// Zero the pad rows [r0, r0 + kZeroRows) of O and set their LSE to -inf.
__device__ void fwd_zero_pad_rows(const FwdParams& p, int zb) {
  __shared__ uint8_t invalid[kZeroRows];
  const int tid = threadIdx.x;
  const int64_t r0 = (int64_t)zb * kZeroRows;
  int mine = 0;
  if (tid < kZeroRows) {
    const int64_t r = r0 + tid;
    const bool inv = r < p.T_q && !row_is_valid(p.cu_q, p.pad_q, p.batch, r, p.T_q);
    invalid[tid] = inv;
    mine = inv;
  }
  if (!__syncthreads_or(mine)) return;
  const int chunks = p.h_q * p.d / 8;  // 16-byte chunks per row
  const int total = kZeroRows * chunks;
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int idx = tid; idx < total; idx += blockDim.x) {
    const int rr = idx / chunks;
    const int c = idx - rr * chunks;
    if (invalid[rr]) *(u32x4*)(p.o + (r0 + rr) * (int64_t)(p.h_q * p.d) + 8 * c) = z;
  }
  for (int idx = tid; idx < kZeroRows * p.h_q; idx += blockDim.x) {
    const int hh = idx / kZeroRows;
    const int rr = idx - hh * kZeroRows;
    if (invalid[rr]) p.lse[(int64_t)hh * p.T_q + r0 + rr] = -__builtin_inff();
  }
}

template <class DT, int DP>
__global__ __launch_bounds__(256) void thd_fwd_kernel(FwdParams p) {
  constexpr int BM = kFwdBM, BN = kFwdBN;
  constexpr int KST = DP + 8;      // LDS row stride of K (elements)
  constexpr int VST = BN + 8;      // LDS row stride of V^T (elements)
  constexpr int NC = DP / 16;      // 16-wide d blocks (MFMA K steps of S^T)
  constexpr int ND = DP / 32;      // 32-row d tiles of O^T
  constexpr int KCH = DP / 8;      // 16-byte chunks per K row
  constexpr int KLOADS = BN * KCH / 256;
  constexpr int VTHREADS = 2 * DP; // 16 key groups x DP/8 chunks
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BN * KST];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[DP * VST];

  const int bid = blockIdx.x;
  if (bid >= p.n_attn) {
    fwd_zero_pad_rows(p, bid - p.n_attn);
    return;
  }
  const int logical = xcd_remap(bid, p.n_attn);
  const int hq = logical / p.n_tiles;
  const int t = logical - hq * p.n_tiles;
  int tile_in_seq = 0;
  const int b = find_tile(p.cu_q, p.batch, p.T_q, BM, t, p.n_tiles, &tile_in_seq);
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
  const int hk = hq / p.group;
  const int q0 = tile_in_seq * BM;
  const int qw0 = q0 + w * kWaveM;
  const int my_q = qw0 + r;
  const int64_t q_stride = (int64_t)p.h_q * p.d;
  const int64_t kv_stride = (int64_t)p.h_kv * p.d;

  int kv_end = lk;
  if (causal && q0 + BM < kv_end) kv_end = q0 + BM;
  const int n_kv_tiles = (kv_end + BN - 1) / BN;

  // Q as the B operand of S^T = K Q^T: lane holds Q[my_q][16c + 8h .. +7].
  typename DT::vec8 qreg[NC];
  {
    const int64_t row = sq + my_q;
    const bool ok = my_q < lq && row >= 0 && row < p.T_q;
    const uint16_t* src = p.q + row * q_stride + (int64_t)hq * p.d;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int dd = 16 * c + 8 * h;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (ok && dd < p.d) x = *(const u32x4*)(src + dd);
      qreg[c] = as_vec8<DT>(x);
    }
  }

  f32x16 acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc[i] = f32x16{};
  float m_run = -__builtin_inff();
  float l_run = 0.f;

  // Global -> register staging of one K/V tile.
  u32x4 kreg[KLOADS];
  u32x4 vreg[4];
  const int v_grp = tid & 15;   // key group of 4 keys
  const int v_chunk = tid >> 4; // 8-wide d chunk
  const uint16_t* kbase = p.k + (int64_t)hk * p.d;
  const uint16_t* vbase = p.v + (int64_t)hk * p.d;

  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
      const int cid = tid + 256 * i;
      const int row = cid / KCH;
      const int c = cid - row * KCH;
      const int j = k0 + row;
      const int64_t g = sk + j;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (j < lk && g >= 0 && g < p.T_kv && 8 * c < p.d) x = *(const u32x4*)(kbase + g * kv_stride + 8 * c);
      kreg[i] = x;
    }
    if (tid < VTHREADS) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = k0 + 4 * v_grp + i;
        const int64_t g = sk + j;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (j < lk && g >= 0 && g < p.T_kv && 8 * v_chunk < p.d)
          x = *(const u32x4*)(vbase + g * kv_stride + 8 * v_chunk);
        vreg[i] = x;
      }
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
      const int cid = tid + 256 * i;
      const int row = cid / KCH;
      const int c = cid - row * KCH;
      *(u32x4*)(&Ks[row * KST + 8 * c]) = kreg[i];
    }
    if (tid < VTHREADS) {
      // 4 keys x 8 d  ->  8 rows of V^T with 4 keys each
      const int pos = 16 * (v_grp >> 2) + 4 * vt_group_pos(v_grp & 3);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int word = e >> 1;
        const bool hi = e & 1;
        uint32_t x0 = vreg[0][word], x1 = vreg[1][word], x2 = vreg[2][word], x3 = vreg[3][word];
        u32x2 out;
        if (!hi) {
          out[0] = (x0 & 0xffffu) | (x1 << 16);
          out[1] = (x2 & 0xffffu) | (x3 << 16);
        } else {
          out[0] = (x0 >> 16) | (x1 & 0xffff0000u);
          out[1] = (x2 >> 16) | (x3 & 0xffff0000u);
        }
        *(u32x2*)(&Vt[(8 * v_chunk + e) * VST + pos]) = out;
      }
    }
  };

  if (n_kv_tiles > 0) load_tile(0);
  for (int it = 0; it < n_kv_tiles; ++it) {
    const int k0 = it * BN;
    __syncthreads();
    store_tile();
    __syncthreads();
    if (it + 1 < n_kv_tiles) load_tile(k0 + BN);

    const bool active = (qw0 < lq) && (!causal || k0 <= qw0 + kWaveM - 1);
    if (!active) continue;

    // S^T tiles: rows = keys k0 + 32*tt + (C row), columns = this wave's queries
    f32x16 s[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      s[tt] = f32x16{};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const u32x4 a = *(const u32x4*)(&Ks[(32 * tt + r) * KST + 16 * c + 8 * h]);
        s[tt] = DT::mfma(as_vec8<DT>(a), qreg[c], s[tt]);
      }
    }

    const bool need_mask = (k0 + BN > lk) || (causal && k0 + BN - 1 > qw0);
    if (need_mask) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = k0 + 32 * tt + 8 * (i >> 2) + 4 * h + (i & 3);
          const bool vis = (j < lk) && (!causal || j <= my_q);
          if (!vis) s[tt][i] = -__builtin_inff();
        }
    }

    float mt = -__builtin_inff();
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[tt][i]);
    mt = fmaxf(mt, wave_swap_halves(mt));
    const float m_new = fmaxf(m_run, mt);
    const float mc = (m_new == -__builtin_inff()) ? 0.f : m_new * p.c2;
    const float alpha = __builtin_amdgcn_exp2f(m_run * p.c2 - mc);
    float ps = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[tt][i], p.c2, -mc));
        s[tt][i] = e;
        ps += e;
      }
    l_run = l_run * alpha + ps;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;

    typename DT::vec8 pb[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float tmp[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) tmp[j] = s[kb >> 1][8 * (kb & 1) + j];
      pb[kb] = pack8<DT>(tmp);
    }
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const u32x4 a = *(const u32x4*)(&Vt[(32 * dt + r) * VST + 16 * kb + 8 * h]);
        acc[dt] = DT::mfma(as_vec8<DT>(a), pb[kb], acc[dt]);
      }
  }

  // Epilogue: O = acc / l, LSE = m * scale + ln(l).
  const float lt = l_run + wave_swap_halves(l_run);
  if (my_q < lq) {
    const int64_t row = sq + my_q;
    if (row >= 0 && row < p.T_q) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      uint16_t* dst = p.o + row * q_stride + (int64_t)hq * p.d;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int dd = 32 * dt + 8 * g + 4 * h;
          if (dd < p.d) {
            u32x2 out;
            out[0] = (uint32_t)DT::bits(acc[dt][4 * g + 0] * inv) |
                     ((uint32_t)DT::bits(acc[dt][4 * g + 1] * inv) << 16);
            out[1] = (uint32_t)DT::bits(acc[dt][4 * g + 2] * inv) |
                     ((uint32_t)DT::bits(acc[dt][4 * g + 3] * inv) << 16);
            *(u32x2*)(dst + dd) = out;
          }
        }
      if (h == 0)
        p.lse[(int64_t)hq * p.T_q + row] =
            lt > 0.f ? m_run * p.scale + __logf(lt) : -__builtin_inff();
    }
  }
}

template <class DT, int DP>
hipError_t launch_fwd_t(const FwdParams& fp, int grid, hipStream_t s) {
  hipLaunchKernelGGL((thd_fwd_kernel<DT, DP>), dim3(grid), dim3(256), 0, s, fp);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const Problem& p, const void* q, const void* k, const void* v, void* o,
                      float* lse, hipStream_t s) {
  FwdParams fp;
  fp.q = (const uint16_t*)q;
  fp.k = (const uint16_t*)k;
  fp.v = (const uint16_t*)v;
  fp.o = (uint16_t*)o;
  fp.lse = lse;
  fp.cu_q = p.cu_q;
  fp.cu_kv = p.cu_kv;
  fp.pad_q = p.pad_q;
  fp.pad_kv = p.pad_kv;
  fp.causal = p.causal;
  fp.T_q = p.T_q;
  fp.T_kv = p.T_kv;
  fp.batch = p.batch;
  fp.h_q = p.h_q;
  fp.h_kv = p.h_kv;
  fp.group = p.h_q / p.h_kv;
  fp.d = p.d;
  fp.scale = p.scale;
  fp.c2 = p.scale * kLog2e;
  const int64_t n_tiles = (p.T_q + kFwdBM - 1) / kFwdBM + p.batch;
  fp.n_tiles = (int)n_tiles;
  fp.n_attn = (p.batch > 0) ? (int)(n_tiles * p.h_q) : 0;
  const int64_t n_zero = (p.T_q + kZeroRows - 1) / kZeroRows;
  const int64_t grid = fp.n_attn + n_zero;
  if (grid == 0) return hipSuccess;
  if (p.d <= 32) return p.bf16 ? launch_fwd_t<Bf16, 32>(fp, (int)grid, s) : launch_fwd_t<Fp16, 32>(fp, (int)grid, s);
  if (p.d <= 64) return p.bf16 ? launch_fwd_t<Bf16, 64>(fp, (int)grid, s) : launch_fwd_t<Fp16, 64>(fp, (int)grid, s);
  return p.bf16 ? launch_fwd_t<Bf16, 128>(fp, (int)grid, s) : launch_fwd_t<Fp16, 128>(fp, (int)grid, s);
}

}  // namespace thd
