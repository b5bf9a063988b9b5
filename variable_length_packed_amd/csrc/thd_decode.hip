// Split-KV forward for packed sequences with few query rows each (the
// KV-cache / decode shape: a handful of new tokens against a long key/value
// history).  Same attention and mask types as thd_fwd.hip; only the work
// split differs.
//
// The regular forward gives one workgroup a 128-row query tile and walks all
// of its keys; with 1-4 query rows per sequence that leaves most of the tile
// idle and each sequence's keys serial.  Here the rows of a GQA group --
// group query heads x query positions, at most 32 -- fill the 32 columns of
// one MFMA tile, and the keys of a sequence are split into chunks handled by
// separate single-wave workgroups.  Each writes an unnormalised partial
// (O, running max, row sum) for its chunk; a merge pass combines the chunks
// of a row through their log-sum-exp:
//   M = max_c m_c,  L = sum_c l_c 2^(m_c - M),  O = sum_c O_c 2^(m_c - M) / L,
//   LSE = (M + log2 L) ln 2   (m in log2 units of the scaled scores).
//
// Per 32-key step a wave loads the step's 32 K and V rows whole (each load
// instruction covers four 256-byte rows of its kv head), stages K in its own
// LDS tile and reads the A operand of S^T = K Q^T (keys x query rows) from
// it, applies the mask and the online softmax, stages V in a second tile and
// adds V^T P^T, whose A operand comes from transpose reads of that tile.
// Workgroups run kv heads minor, so the heads of one (sequence, chunk) read
// the same packed K/V rows at the same time.  Chunks past a sequence's last
// visible key write nothing; the merge reads only the chunks below it.
// (On 64 decode sequences against 256-16,384 keys, GQA 32/8, d = 128: K loaded
// straight into the A operand -- 32 B of each of 32 rows per instruction --
// 0.603 ms; K staged whole 0.556; both with heads minor 0.525; and without
// the empty chunks' writes 0.505.  A copy of the pass that only loads its
// K/V takes 0.492 ms.)
#include <limits.h>

#include "thd_common.hpp"
#include "thd_launch.hpp"

namespace thd {

namespace {

constexpr int kDecRows = 32;  // query rows per wave (GQA group x query positions)
constexpr int kDecStep = 32;  // keys per step

struct DecParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  // per (row, chunk); chunks past a sequence's last visible key stay unwritten
  float* part_o;   // [rows * n_split][DP]: unnormalised partial outputs
  float* part_ml;  // [rows * n_split][2]: max (log2 units) and row sum
  const int32_t* cu_q;
  const int32_t* cu_kv;
  const int32_t* pad_q;
  const int32_t* pad_kv;
  const uint8_t* mask_type;
  int64_t T_q, T_kv;
  int batch, h_q, h_kv, group, d;
  float scale, c2;
  int lq_max;   // query rows per sequence covered (the host bound)
  int ck;       // keys per split, a multiple of kDecStep
  int n_split;  // splits per (sequence, kv head)
};

// ---------------------------------------------------------------------------
// split: one wave per (sequence, key chunk, kv head), kv heads minor
// ---------------------------------------------------------------------------
template <class DT, int DP>
__global__ __launch_bounds__(64) void thd_decode_split_kernel(DecParams p) {
  constexpr int NC = DP / 16;
  constexpr int ND = DP / 32;
  constexpr int KCH = DP / 8;
  __shared__ __attribute__((aligned(16))) unsigned char Vs[kDecStep * DP * 2];
  __shared__ __attribute__((aligned(16))) unsigned char Ks[kDecStep * DP * 2];

  const int hk = blockIdx.x % p.h_kv;
  const int rest = blockIdx.x / p.h_kv;
  const int split = rest % p.n_split;
  const int b = rest / p.n_split;
  const int l = threadIdx.x;
  const int r = l & 31;
  const int h = l >> 5;
  const int g16 = l & 15;
  const int grp = l >> 4;
  const int tr_row = g16 >> 2;
  const int tr_col = 4 * (g16 & 3);

  const uint32_t qrow_bytes = (uint32_t)p.h_q * p.d * 2;
  const uint32_t kvrow_bytes = (uint32_t)p.h_kv * p.d * 2;
  const int64_t sq = seq_start(p.cu_q, p.pad_q, b);
  const int64_t sk = seq_start(p.cu_kv, p.pad_kv, b);
  const int lq = uniform(clamp_rows(sq, seq_len_clamped(p.cu_q, b, p.T_q), p.T_q, qrow_bytes));
  const int lk = uniform(clamp_rows(sk, seq_len_clamped(p.cu_kv, b, p.T_kv), p.T_kv, kvrow_bytes));
  const int mtype = mask_type_of(p.mask_type, b);
  const bool causal = mask_is_causal(mtype);
  const int off = causal_offset(mtype, lq, lk);  // key j visible to query i iff j <= i + off

  // Column r of the tile: query head hk*group + r / lq_max, position r % lq_max.
  const int hql = r / p.lq_max;
  const int qi = r - hql * p.lq_max;
  const bool row_ok = hql < p.group && qi < lq;
  const int hq = hk * p.group + hql;
  int lim = lk;  // keys j < lim visible to this row
  if (causal && qi + 1 + off < lim) lim = qi + 1 + off;
  if (!row_ok) lim = INT_MIN;

  // Keys of this split; causal sequences stop at the last row's diagonal.
  const int k_lo = split * p.ck;
  int k_hi = min(k_lo + p.ck, lk);
  if (causal && lq + off < k_hi) k_hi = lq + off;
  if (k_lo >= k_hi) return;  // no key of this chunk is visible: nothing to merge
  const int lim_r = min(lim, k_hi);

  // Q as the B operand of S^T = K Q^T: lane (r, h) holds Q[row r][16c + 8h ..].
  const rsrc_t q_rs = make_rsrc(p.q + sq * (int64_t)p.h_q * p.d, (uint32_t)lq * qrow_bytes);
  typename DT::vec8 qreg[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int dd = 16 * c + 8 * h;
    const uint32_t off_q = (row_ok && dd < p.d)
                               ? (uint32_t)qi * qrow_bytes + (uint32_t)hq * p.d * 2 + 2u * dd
                               : kOobOffset;
    qreg[c] = as_vec8<DT>(buf_load16(q_rs, off_q, 0));
  }

  const char* kbase = (const char*)(p.k + sk * (int64_t)p.h_kv * p.d + (int64_t)hk * p.d);
  const char* vbase = (const char*)(p.v + sk * (int64_t)p.h_kv * p.d + (int64_t)hk * p.d);
  const rsrc_t k_rs = make_rsrc(kbase, (uint32_t)lk * kvrow_bytes);
  const rsrc_t v_rs = make_rsrc(vbase, (uint32_t)lk * kvrow_bytes);

  f32x16 acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc[i] = f32x16{};
  float m_run = -__builtin_inff();  // running max of the raw scores
  float l_run = 0.f;                // this lane's share of the row sum
  const float c2 = p.c2;

  constexpr int NV = kDecStep * KCH / 64;
  for (int j0 = k_lo; j0 < k_hi; j0 += kDecStep) {
    // K and V rows j0 .. j0+31, KCH 16-byte chunks each: lane l takes chunks
    // l + 64u; rows past lk read as zeros
    u32x4 kr[NV], vr[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int cid = l + 64 * u;
      const int row = cid / KCH;
      const int x = cid - row * KCH;
      const uint32_t o = 8 * x < p.d ? (uint32_t)(j0 + row) * kvrow_bytes + 16u * x : kOobOffset;
      kr[u] = buf_load16(k_rs, o, 0);
      vr[u] = buf_load16(v_rs, o, 0);
    }
    // K tile -> LDS, then the A operand of S^T = K Q^T: lane (r, h) reads
    // K[row r][16c + 8h ..]
    __syncthreads();  // the previous step's K reads are done
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int cid = l + 64 * u;
      const int row = cid / KCH;
      const int x = cid - row * KCH;
      *(u32x4*)(Ks + swz<DP>(row, 8 * x)) = kr[u];
    }
    __syncthreads();  // K tile complete
    u32x4 ka[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) ka[c] = *(const u32x4*)(Ks + swz<DP>(r, 16 * c + 8 * h));
    f32x16 s = f32x16{};
#pragma unroll
    for (int c = 0; c < NC; ++c) s = DT::mfma(as_vec8<DT>(ka[c]), qreg[c], s);

    // register i holds key j0 + 8(i/4) + 4h + i%4 of query row r
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = j0 + 8 * (i >> 2) + 4 * h + (i & 3);
      if (j >= lim_r) s[i] = -__builtin_inff();
    }
    float mt = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[i]);
    mt = wave_max_halves(mt);
    const float m_new = fmaxf(m_run, mt);
    if (m_new != -__builtin_inff() && m_new != m_run) {
      const float alpha = m_run == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f((m_run - m_new) * c2);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;
      m_run = m_new;
    }
    const float mc = m_run == -__builtin_inff() ? 0.f : m_run * c2;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c2, -mc));
      s[i] = e;
      l_run += e;
    }
    typename DT::vec8 pb[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float tp[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) tp[i] = s[8 * kb + i];
      pb[kb] = pack8<DT>(tp);
    }

    __syncthreads();  // the previous step's tile reads are done
#pragma unroll
    for (int u = 0; u < kDecStep * KCH / 64; ++u) {
      const int cid = l + 64 * u;
      const int row = cid / KCH;
      const int x = cid - row * KCH;
      *(u32x4*)(Vs + swz<DP>(row, 8 * x)) = vr[u];
    }
    __syncthreads();  // tile complete
    // O^T += V^T P^T: A lane (r, h) = V[keys 16kb + {4h..4h+3, 8+4h..8+4h+3}][d = 32dt + r]
    // (two transpose reads), the key order in which P holds them.
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int r0 = 16 * kb + 4 * h + tr_row;
        const int c0 = 32 * dt + 16 * (grp & 1) + tr_col;
        const u32x4 a = cat2(lds_read_tr(Vs, swz<DP>(r0, c0)), lds_read_tr(Vs, swz<DP>(r0 + 8, c0)));
        acc[dt] = DT::mfma(as_vec8<DT>(a), pb[kb], acc[dt]);
      }
  }

  // Partial of this chunk for query row r: acc holds O^T[32dt + 8g + 4h + e][r].
  const float lt = wave_sum_halves(l_run);  // every lane still active here
  if (!row_ok) return;
  const int64_t idx = (((int64_t)b * p.h_q + hq) * p.lq_max + qi) * p.n_split + split;
  float* po = p.part_o + idx * DP;
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = acc[dt][4 * g + e];
      *(f32x4*)(po + 32 * dt + 8 * g + 4 * h) = v4;
    }
  if (h == 0) {
    p.part_ml[2 * idx] = m_run == -__builtin_inff() ? -__builtin_inff() : m_run * c2;
    p.part_ml[2 * idx + 1] = lt;
  }
}

// ---------------------------------------------------------------------------
// merge: one wave per (sequence, query head, query position)
// ---------------------------------------------------------------------------
template <class DT, int DP>
__global__ __launch_bounds__(256) void thd_decode_merge_kernel(DecParams p) {
  const int64_t row_id = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  const int64_t n_rows = (int64_t)p.batch * p.h_q * p.lq_max;
  if (row_id >= n_rows) return;
  const int qi = (int)(row_id % p.lq_max);
  const int64_t t = row_id / p.lq_max;
  const int hq = (int)(t % p.h_q);
  const int b = (int)(t / p.h_q);
  const uint32_t qrow_bytes = (uint32_t)p.h_q * p.d * 2;
  const int64_t sq = seq_start(p.cu_q, p.pad_q, b);
  const int lq = clamp_rows(sq, seq_len_clamped(p.cu_q, b, p.T_q), p.T_q, qrow_bytes);
  if (qi >= lq) return;  // past the sequence: a pad row, or a row of the next one
  // the chunks the split pass wrote: those below the sequence's last visible key
  const uint32_t kvrow_bytes = (uint32_t)p.h_kv * p.d * 2;
  const int64_t sk = seq_start(p.cu_kv, p.pad_kv, b);
  const int lk = clamp_rows(sk, seq_len_clamped(p.cu_kv, b, p.T_kv), p.T_kv, kvrow_bytes);
  const int mtype = mask_type_of(p.mask_type, b);
  int k_end = lk;
  if (mask_is_causal(mtype)) k_end = min(k_end, lq + causal_offset(mtype, lq, lk));
  const int n_valid = k_end > 0 ? min(p.n_split, (k_end + p.ck - 1) / p.ck) : 0;

  // Lane l takes chunks l, l + 64, ...: the maximum, then the weighted row
  // sum; the chunks' outputs are then added with every lane on its columns.
  // No step waits on the previous chunk's loads (a loop that branched on each
  // chunk's maximum before loading its output took 33 against 17 us on 64 decode
  // sequences against 256-16,384 keys).
  const int64_t base = row_id * p.n_split;
  float M = -__builtin_inff();
  for (int s = l; s < n_valid; s += 64) M = fmaxf(M, p.part_ml[2 * (base + s)]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  float L = 0.f;
  if (M != -__builtin_inff())
    for (int s = l; s < n_valid; s += 64) {
      const float ms = p.part_ml[2 * (base + s)];
      if (ms != -__builtin_inff()) L += p.part_ml[2 * (base + s) + 1] * __builtin_amdgcn_exp2f(ms - M);
    }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o, 64);

  constexpr int PER = DP / 64 > 0 ? DP / 64 : 1;  // output columns per lane
  float accv[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) accv[e] = 0.f;
  if (M != -__builtin_inff()) {
    // a chunk with no visible key for this row holds zeros and weighs 0
#pragma unroll 4
    for (int s = 0; s < n_valid; ++s) {
      const float ms = p.part_ml[2 * (base + s)];
      const float wgt = ms == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(ms - M);
      const float* po = p.part_o + (base + s) * DP;
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int dd = PER * l + e;
        if (dd < DP) accv[e] += po[dd] * wgt;
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* orow = p.o + (sq + qi) * (int64_t)p.h_q * p.d + (int64_t)hq * p.d;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int dd = PER * l + e;
    if (dd < p.d) orow[dd] = DT::bits(accv[e] * inv);
  }
  if (l == 0)
    p.lse[(int64_t)hq * p.T_q + sq + qi] =
        L > 0.f ? (M + __log2f(L)) * kLn2 : -__builtin_inff();
}

struct DecodeShape {
  int ck, n_split;
};

DecodeShape decode_shape(const Problem& p) {
  // enough single-wave workgroups to fill the chip several times over, with
  // chunks of at least two steps
  int ck = 2048;
  const int64_t units = (int64_t)p.batch * p.h_kv;
  while (ck > 2 * kDecStep && units * ((p.max_kv + ck - 1) / ck) < 16384) ck /= 2;
  DecodeShape ds;
  ds.ck = ck;
  ds.n_split = p.max_kv > 0 ? (p.max_kv + ck - 1) / ck : 1;
  return ds;
}

int padded_dim(int d) { return d <= 32 ? 32 : d <= 64 ? 64 : 128; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

template <class DT, int DP>
hipError_t launch_decode_t(const DecParams& dp, hipStream_t s) {
  const int64_t n_split_wg = (int64_t)dp.batch * dp.h_kv * dp.n_split;
  hipLaunchKernelGGL((thd_decode_split_kernel<DT, DP>), dim3((unsigned)n_split_wg), dim3(64), 0, s,
                     dp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n_rows = (int64_t)dp.batch * dp.h_q * dp.lq_max;
  hipLaunchKernelGGL((thd_decode_merge_kernel<DT, DP>), dim3((unsigned)((n_rows + 3) / 4)), dim3(256),
                     0, s, dp);
  return hipGetLastError();
}

}  // namespace

bool decode_applies(const Problem& p) {
  const int group = p.h_q / p.h_kv;
  // head dims above 128 take the tiled forward
  if (!(p.batch > 0 && p.max_q >= 1 && (int64_t)p.max_q * group <= kDecRows && p.max_kv > 0 &&
        p.d <= 128))
    return false;
  const DecodeShape ds = decode_shape(p);
  const int64_t wgs = (int64_t)p.batch * p.h_kv * ds.n_split;
  return wgs < ((int64_t)1 << 31) && (int64_t)p.batch * p.h_q * p.max_q < ((int64_t)1 << 31);
}

// Partial outputs [B * h_q * max_q * n_split][DP] fp32, then their max and
// sum [same][2].
size_t decode_workspace_bytes(const Problem& p) {
  const DecodeShape ds = decode_shape(p);
  const size_t n = (size_t)p.batch * p.h_q * p.max_q * ds.n_split;
  return align256(n * padded_dim(p.d) * sizeof(float)) + align256(n * 2 * sizeof(float));
}

hipError_t launch_decode(const Problem& p, const void* q, const void* k, const void* v, void* o,
                         float* lse, void* workspace, hipStream_t s) {
  hipError_t e = launch_fwd_pad_rows(p, o, lse, s);
  if (e != hipSuccess) return e;
  const DecodeShape ds = decode_shape(p);
  DecParams dp;
  dp.q = (const uint16_t*)q;
  dp.k = (const uint16_t*)k;
  dp.v = (const uint16_t*)v;
  dp.o = (uint16_t*)o;
  dp.lse = lse;
  const size_t n = (size_t)p.batch * p.h_q * p.max_q * ds.n_split;
  dp.part_o = (float*)workspace;
  dp.part_ml = (float*)((char*)workspace + align256(n * padded_dim(p.d) * sizeof(float)));
  dp.cu_q = p.cu_q;
  dp.cu_kv = p.cu_kv;
  dp.pad_q = p.pad_q;
  dp.pad_kv = p.pad_kv;
  dp.mask_type = p.causal;
  dp.T_q = p.T_q;
  dp.T_kv = p.T_kv;
  dp.batch = p.batch;
  dp.h_q = p.h_q;
  dp.h_kv = p.h_kv;
  dp.group = p.h_q / p.h_kv;
  dp.d = p.d;
  dp.scale = p.scale;
  dp.c2 = p.scale * kLog2e;
  dp.lq_max = p.max_q;
  dp.ck = ds.ck;
  dp.n_split = ds.n_split;
  if (p.d <= 32) return p.bf16 ? launch_decode_t<Bf16, 32>(dp, s) : launch_decode_t<Fp16, 32>(dp, s);
  if (p.d <= 64) return p.bf16 ? launch_decode_t<Bf16, 64>(dp, s) : launch_decode_t<Fp16, 64>(dp, s);
  return p.bf16 ? launch_decode_t<Bf16, 128>(dp, s) : launch_decode_t<Fp16, 128>(dp, s);
}

}  // namespace thd
