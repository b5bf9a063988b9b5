// Forward attention over packed variable-length ("thd") tensors.
//
// Computes, per sequence and query head, softmax(scale * Q K^T + mask) V with
// the per-sequence causal policy of TransformerEngine PR "Add per-sequence
// causal policy to packed THD attention" (Description; the mask types of its
// maintainer review: padding, top-left and bottom-right causal), the padded
// slot starts of that PR's two-call example, and pad rows written as zeros.
// The mask of sequence b is derived inline from cu_seqlens (key j visible iff
// j < lk_b and, when causal, j <= i + off with off = 0 or lk_b - lq_b), so no
// mask tensor is read and the host never synchronises.
//
// One workgroup = 4 waves = one (sequence, 128-row query tile, query head)
// work item.  A pre pass orders the (sequence, query tile) items by sequence
// (sequences by the key tiles their largest item walks, largest first) and,
// within a sequence, largest item first; the attention workgroups take them
// in that order, query heads minor, so that all query tiles of a sequence and
// head run together and share its K and V in L2.  Each wave owns 32
// query rows.  Scores are computed transposed, S^T = K Q^T, so that a lane
// owns one query row: the row max needs one exchange between wave halves and
// the probabilities land directly in the B-operand layout of O^T = V^T P^T.
// K and V tiles go from memory straight into LDS (no register staging),
// row-major with swizzled 16-byte chunks, double buffered; the V^T operand of
// the PV product comes from transpose reads.  The pre pass also writes zeros
// to pad rows of O and -inf to their LSE.
#include "thd_common.hpp"
#include "thd_launch.hpp"

namespace thd {

namespace {

constexpr int kFwdBM = 128;  // query rows per workgroup
// Keys per LDS tile and tiles in flight.  At d > 32 the tiles hold 32 keys,
// and three workgroups (three waves per SIMD) share a CU.  At d = 128 two
// stages (32 KB per workgroup) ran the forward about 1 % faster than three
// (48 KB) on short and long causal sequences alike, and 64-key tiles in two
// stages (two workgroups per CU) about 4.5 % slower; d = 64 keeps three
// stages.  At d <= 32 a 32-key tile would be smaller than one 1 KB load per
// wave, and 64-key tiles in two stages are kept.  Head dims above 128 (DP =
// 256) take 32-key tiles in two stages (64 KB per workgroup) and two
// workgroups per CU: their Q operand and accumulators need about 230
// registers per lane.
template <int DP>
struct FwdTile {
  static constexpr int BN = DP > 32 ? 32 : 64;
  static constexpr int NS = DP >= 128 ? 2 : DP > 32 ? 3 : 2;
  static constexpr int WG_PER_CU = DP > 128 ? 2 : DP > 32 ? 3 : 2;
};
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
  int n_sched;      // workgroups of the pre pass building the schedule
  int32_t* sched;   // item count, then the items by rank (build_schedule_by_sequence)
};

// Schedule of the attention workgroups (grouped by sequence, largest tile
// first, see build_schedule_by_sequence):
// query tile t of sequence b walks W = ceil(lk / BN) key tiles, or, with a
// causal mask type, the tiles up to its last row's diagonal:
// W = ceil(clamp(min(lk, (t + 1) BM + off), 0) / BN) = clamp(a t + a + ceil(off / BN), 0, ceil(lk / BN))
// with a = BM / BN, and the kernel's clamping of the lengths.
template <int BN>
struct FwdSchedModel {
  static_assert(kFwdBM % BN == 0, "work model assumes whole key tiles per query tile");
  static constexpr int kSlope = kFwdBM / BN;
  const FwdParams& p;
  __device__ SeqSummary seq(int b) const {
    const int64_t sq = seq_start(p.cu_q, p.pad_q, b);
    const int64_t sk = seq_start(p.cu_kv, p.pad_kv, b);
    const int lq =
        clamp_rows(sq, seq_len_clamped(p.cu_q, b, p.T_q), p.T_q, (int64_t)p.h_q * p.d * 2);
    const int lk =
        clamp_rows(sk, seq_len_clamped(p.cu_kv, b, p.T_kv), p.T_kv, (int64_t)p.h_kv * p.d * 2);
    const int mt = mask_type_of(p.causal, b);
    SeqSummary s;
    s.x = ceil_div_pos(lq, kFwdBM);
    s.H = ceil_div_pos(lk, BN);
    s.causal = mask_is_causal(mt);
    s.c = kSlope + ceil_div(causal_offset(mt, lq, lk), BN);
    s.sq = (int)sq;
    s.sk = (int)sk;
    s.lq = lq;
    s.lk = lk;
    s.mtype = mt;
    return s;
  }
};

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

// pre: schedule of the attention workgroups (key tiles of BN keys), then
// zeros on pad rows.
template <int BN>
__global__ __launch_bounds__(256) void thd_fwd_pre_kernel(FwdParams p) {
  if ((int)blockIdx.x < p.n_sched) {
    build_schedule_by_sequence(FwdSchedModel<BN>{p}, p.batch, p.n_tiles, p.sched,
                   blockIdx.x * 4 + (int)(threadIdx.x >> 6));
    return;
  }
  fwd_zero_pad_rows(p, blockIdx.x - p.n_sched);
}

// Threshold (log2 units) by which a row maximum must grow before the running
// maximum is moved and the accumulator rescaled; below it the stale maximum
// stays, probabilities may reach 2^8, which fp32 sums and 16-bit P hold.
constexpr float kRescaleLog2 = 8.0f;

template <class DT, int DP>
__global__ __launch_bounds__(256, FwdTile<DP>::WG_PER_CU) void thd_fwd_kernel(FwdParams p) {
  constexpr int BM = kFwdBM, BN = FwdTile<DP>::BN, NS = FwdTile<DP>::NS;
  constexpr int NT = BN / 32;      // 32-key S^T tiles per LDS tile
  constexpr int NKB = BN / 16;     // 16-key blocks (MFMA K steps of O^T)
  constexpr int NC = DP / 16;      // 16-wide d blocks (MFMA K steps of S^T)
  constexpr int ND = DP / 32;      // 32-row d tiles of O^T
  constexpr int KCH = DP / 8;      // 16-byte chunks per K row
  constexpr int TILE = BN * DP * 2;  // bytes of one K or V tile
  constexpr int BPW = TILE / 1024 / 4;  // 1 KB blocks (one load each) per wave per tile
  static_assert(BPW >= 1 && BPW * 4096 == TILE, "tile splits into 1 KB blocks over 4 waves");
  static_assert(2 * BPW < 16, "loads of one tile fit the vmcnt field");
  // buffer j: K tile at 2j * TILE, V tile at (2j + 1) * TILE
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * NS * TILE];

  // Workgroups in schedule order, heads minor.  Slot s of a rank takes kv
  // head s % h_kv and query head (s % h_kv) * group + s / h_kv of its group:
  // with h_kv a multiple of 8, every query head of kv head hk then lands on
  // XCD hk % 8 (the workgroup id modulo 8), whose L2 holds that head's K and
  // V for all of them.  (Without GQA this is query head s.)
  const int bid = blockIdx.x;
  const int rk = bid / p.h_q;
  const int slot = bid - rk * p.h_q;
  const int hq = (slot % p.h_kv) * p.group + slot / p.h_kv;
  SchedItem item;
  if (!load_sched_item(p.sched, rk, item)) return;
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
  // the item's slot starts, lengths (clamped as FwdSchedModel clamps them)
  // and mask type
  const int64_t sq = uniform(item.sq);
  const int64_t sk = uniform(item.sk);
  const int lq = uniform(item.lq);
  const int lk = uniform(item.lk);
  const int mtype = uniform(item.mtype);
  const bool causal = mask_is_causal(mtype);
  const int off = causal_offset(mtype, lq, lk);  // key j visible to query i iff j <= i + off
  const int hk = hq / p.group;
  const int q0 = tile_in_seq * BM;
  if (q0 >= lq) return;
  const int qw0 = q0 + w * kWaveM;
  const int my_q = qw0 + r;

  int kv_end = lk;
  if (causal && q0 + BM + off < kv_end) kv_end = q0 + BM + off;
  const int n_kv_tiles = ceil_div_pos(kv_end, BN);  // 0: every row sees no key

  // Resources: this sequence's rows of head hq (q, o) and of head hk (k, v).
  const uint16_t* qbase = p.q + sq * (int64_t)p.h_q * p.d + (int64_t)hq * p.d;
  uint16_t* obase = p.o + sq * (int64_t)p.h_q * p.d + (int64_t)hq * p.d;
  const rsrc_t q_rs = make_rsrc(qbase, (uint32_t)lq * qrow_bytes);
  const rsrc_t o_rs = make_rsrc(obase, (uint32_t)lq * qrow_bytes);
  const char* kbase = (const char*)(p.k + sk * (int64_t)p.h_kv * p.d + (int64_t)hk * p.d);
  const char* vbase = (const char*)(p.v + sk * (int64_t)p.h_kv * p.d + (int64_t)hk * p.d);

  // Q as the B operand of S^T = K Q^T: lane holds Q[my_q][16c + 8h .. +7].
  typename DT::vec8 qreg[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int dd = 16 * c + 8 * h;
    const uint32_t off = dd < p.d ? (uint32_t)my_q * qrow_bytes + 2u * dd : kOobOffset;
    qreg[c] = as_vec8<DT>(buf_load16(q_rs, off, 0));
  }

  f32x16 acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc[i] = f32x16{};
  float m_run = -__builtin_inff();  // running max of the raw scores (stale up to 2^8)
  float l_run = 0.f;                // this lane's share of the row sum

  // Tile staging: load n of wave w fills 1 KB block BPW * w + n of a tile,
  // lane l the 16-byte slot 64 * block + l, i.e. row slot / KCH, swizzled
  // chunk x = slot % KCH, which holds memory chunk x ^ f(row).  The same
  // offsets (relative to the tile's first row) serve K and V; chunks past d
  // and rows past lk read as zeros.
  uint32_t loff[BPW];
#pragma unroll
  for (int n = 0; n < BPW; ++n) {
    const int slot = 64 * (BPW * w + n) + l;
    const int row = slot / KCH;
    const int x = slot - row * KCH;
    const int gc = x ^ (int)((swz<DP>(row, 0) >> 4) & (KCH - 1));
    loff[n] = 8 * gc < p.d ? (uint32_t)row * kvrow_bytes + 16u * gc : kOobOffset;
  }
  auto load_tile = [&](int k0, int buf) {
    const uint32_t left = (uint32_t)(lk - k0);  // >= 1 for every tile we visit
    const u32x4 k_rs = rsrc_words(kbase + (int64_t)k0 * kvrow_bytes, left * kvrow_bytes);
    const u32x4 v_rs = rsrc_words(vbase + (int64_t)k0 * kvrow_bytes, left * kvrow_bytes);
    const uint32_t kt = lds_addr(smem) + (uint32_t)(2 * buf * TILE + 1024 * BPW * w);
#pragma unroll
    for (int n = 0; n < BPW; ++n) {
      buf_load_lds16(k_rs, kt + 1024 * n, loff[n]);
      buf_load_lds16(v_rs, kt + TILE + 1024 * n, loff[n]);
    }
  };
  // Operand addresses inside a tile (see swz and tr_xor); row parts set bits
  // that are zero in the base and are added, so they ride in the offset
  // field, as do the buffer's K / V choice:
  //   K rows 32tt + r, chunk 2c + h:  (b_k ^ (c << 5)) + 32tt * 2DP
  //   V^T operand (dt, kb, j):        (b_t ^ tr_chunk(dt, j)) + tr_row(kb, j)
  const uint32_t b_k = swz<DP>(r, 8 * h);
  const uint32_t b_t = swz<DP>(4 * h + (g16 >> 2), 16 * (grp & 1) + 4 * (g16 & 3));

  const float c2 = p.c2;
  // Tiles 0 .. NS-2 go in flight before the loop; iteration it issues tile
  // it + NS - 1 into the buffer that iteration it - 1 read.
#pragma unroll
  for (int t = 0; t < NS - 1; ++t)
    if (t < n_kv_tiles) load_tile(t * BN, t);
  // vmcnt(0): the Q operand and the first tiles are in.  The full wait (once
  // per workgroup) also tells the compiler, which does not count the tile
  // loads, that the Q loads are done; otherwise it would treat them as
  // pending at the loop head and wait, inside the S products, for every load.
  __builtin_amdgcn_s_waitcnt(0x0f70);
  __syncthreads();
  int buf = 0, lbuf = NS - 1;  // buffer read by this iteration, buffer it loads
  for (int it = 0; it < n_kv_tiles; ++it) {
    const int k0 = it * BN;
    // The buffer loaded here was last read in the previous iteration, which
    // every wave has left (barrier below).
    if (it + NS - 1 < n_kv_tiles) load_tile(k0 + (NS - 1) * BN, lbuf);

    const bool active = (qw0 < lq) && (!causal || k0 <= qw0 + kWaveM - 1 + off);
    if (active) {
      // per-iteration bases (kept opaque so that the XORs are formed here and
      // not hoisted into one register per address)
      const uint32_t bo = (uint32_t)(2 * buf * TILE);
      const uint32_t a_k = opaque(b_k + bo), a_t = opaque(b_t + bo);
      // S^T tiles: rows = keys k0 + 32*tt + (C row), columns = this wave's queries
      f32x16 s[NT];
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        s[tt] = f32x16{};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const u32x4 a = *(const u32x4*)(smem + ((a_k ^ (uint32_t)(c << 5)) + 32 * tt * DP * 2));
          s[tt] = DT::mfma(as_vec8<DT>(a), qreg[c], s[tt]);
        }
      }

      const bool need_mask = (k0 + BN > lk) || (causal && k0 + BN - 1 > qw0 + off);
      if (need_mask) {
        // keys j < lim visible (lim <= 0: none)
        const int lim = causal ? (my_q + 1 + off < lk ? my_q + 1 + off : lk) : lk;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int j = k0 + 32 * tt + 8 * (i >> 2) + 4 * h + (i & 3);
            if (j >= lim) s[tt][i] = -__builtin_inff();
          }
      }

      float mt = -__builtin_inff();
#pragma unroll
      for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[tt][i]);
      mt = wave_max_halves(mt);
      // Move the running max only when it grew by more than 2^8 in exp2 units.
      const bool grow = mt != -__builtin_inff() &&
                        (m_run == -__builtin_inff() || (mt - m_run) * c2 > kRescaleLog2);
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float m_new = grow ? mt : m_run;
        const float alpha = grow ? __builtin_amdgcn_exp2f((m_run - m_new) * c2) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;
        m_run = m_new;
      }
      const float mc = m_run == -__builtin_inff() ? 0.f : m_run * c2;
#pragma unroll
      for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[tt][i], c2, -mc));
          s[tt][i] = e;
          l_run += e;
        }

      typename DT::vec8 pb[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        float tmp[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) tmp[j] = s[kb >> 1][8 * (kb & 1) + j];
        pb[kb] = pack8<DT>(tmp);
      }
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const u32x4 a =
              cat2(lds_read_tr(smem, (a_t ^ tr_chunk<DP>(dt, 0)) + TILE + tr_row<DP>(kb, 0)),
                   lds_read_tr(smem, (a_t ^ tr_chunk<DP>(dt, 1)) + TILE + tr_row<DP>(kb, 1)));
          acc[dt] = DT::mfma(as_vec8<DT>(a), pb[kb], acc[dt]);
        }
    }
    // This wave's part of tile it + 1 is in LDS: the loads of later tiles
    // (NS - 2 of them at most, 2 BPW loads each) may still be pending.
    if (NS > 2 && it + 2 < n_kv_tiles)
      __builtin_amdgcn_s_waitcnt(0x0f70 | (NS > 2 ? 2 * BPW : 0));
    else
      __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    buf = buf + 1 == NS ? 0 : buf + 1;
    lbuf = lbuf + 1 == NS ? 0 : lbuf + 1;
  }

  // Epilogue: O = acc / l, LSE = m * scale + ln(l).  Rows past lq are dropped
  // by the resource bound.
  const float lt = wave_sum_halves(l_run);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  // Each wave stages its 32 rows (bf16, row-major, swizzled) in its own part
  // of the K/V tiles, which every wave is done with after the walk's last
  // barrier, then stores whole rows: each store covers 64 / KCH full rows.
  static_assert(4 * 32 * DP * 2 <= 2 * NS * TILE, "staging fits the K/V tiles");
  unsigned char* st = smem + (size_t)w * 32 * DP * 2;
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dd = 32 * dt + 8 * g + 4 * h;
      u32x2 out;
      out[0] = (uint32_t)DT::bits(acc[dt][4 * g + 0] * inv) |
               ((uint32_t)DT::bits(acc[dt][4 * g + 1] * inv) << 16);
      out[1] = (uint32_t)DT::bits(acc[dt][4 * g + 2] * inv) |
               ((uint32_t)DT::bits(acc[dt][4 * g + 3] * inv) << 16);
      *(u32x2*)(st + swz<DP>(r, dd)) = out;
    }
  asm volatile("" ::: "memory");
#pragma unroll
  for (int j = 0; j < 32 * KCH / 64; ++j) {
    const int c = l + 64 * j;
    const int row = c / KCH, x = c - row * KCH;
    const u32x4 v = *(const u32x4*)(st + swz<DP>(row, 8 * x));
    // rows past lq are dropped by the resource bound
    buf_store16(v, o_rs, 8 * x < p.d ? (uint32_t)(qw0 + row) * qrow_bytes + 16u * x : kOobOffset, 0);
  }
  if (h == 0 && my_q < lq)
    p.lse[(int64_t)hq * p.T_q + sq + my_q] =
        lt > 0.f ? m_run * p.scale + __logf(lt) : -__builtin_inff();
}

// Pre pass (schedule for this head dim's key tiles, pad rows), then attention.
template <class DT, int DP>
hipError_t launch_fwd_t(const FwdParams& fp, int64_t n_pre, hipStream_t s) {
  if (n_pre > 0) {
    hipLaunchKernelGGL((thd_fwd_pre_kernel<FwdTile<DP>::BN>), dim3((unsigned)n_pre), dim3(256), 0,
                       s, fp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (fp.n_attn == 0) return hipSuccess;
  hipLaunchKernelGGL((thd_fwd_kernel<DT, DP>), dim3(fp.n_attn), dim3(256), 0, s, fp);
  return hipGetLastError();
}

int64_t fwd_tile_bound(const Problem& p) { return (p.T_q + kFwdBM - 1) / kFwdBM + p.batch; }

}  // namespace

// The attention workgroups' schedule (sched_bytes of the query-tile bound); or,
// for few query rows per sequence, the split-KV partials.
size_t fwd_workspace_bytes(const Problem& p) {
  if (decode_applies(p)) return decode_workspace_bytes(p);
  return p.batch > 0 ? sched_bytes(fwd_tile_bound(p)) : 0;
}

static FwdParams pad_params(const Problem& p, void* o, float* lse) {
  FwdParams fp = {};
  fp.o = (uint16_t*)o;
  fp.lse = lse;
  fp.cu_q = p.cu_q;
  fp.pad_q = p.pad_q;
  fp.T_q = p.T_q;
  fp.batch = p.batch;
  fp.h_q = p.h_q;
  fp.d = p.d;
  fp.n_sched = 0;
  return fp;
}

hipError_t launch_fwd_pad_rows(const Problem& p, void* o, float* lse, hipStream_t s) {
  const int64_t n_zero = (p.T_q + kZeroRows - 1) / kZeroRows;
  if (n_zero == 0) return hipSuccess;
  // no schedule (n_sched = 0): any key tile size
  hipLaunchKernelGGL(thd_fwd_pre_kernel<FwdTile<128>::BN>, dim3((unsigned)n_zero), dim3(256), 0, s,
                     pad_params(p, o, lse));
  return hipGetLastError();
}

hipError_t launch_fwd(const Problem& p, const void* q, const void* k, const void* v, void* o,
                      float* lse, void* workspace, hipStream_t s) {
  if (decode_applies(p)) return launch_decode(p, q, k, v, o, lse, workspace, s);
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
  const int64_t n_tiles = fwd_tile_bound(p);
  fp.n_tiles = (int)n_tiles;
  fp.n_attn = (p.batch > 0) ? (int)(n_tiles * p.h_q) : 0;
  fp.n_sched = (p.batch > 0) ? (p.batch + 3) / 4 : 0;
  fp.sched = (int32_t*)workspace;
  const int64_t n_zero = (p.T_q + kZeroRows - 1) / kZeroRows;
  const int64_t n_pre = fp.n_sched + n_zero;
  if (p.d <= 32)
    return p.bf16 ? launch_fwd_t<Bf16, 32>(fp, n_pre, s) : launch_fwd_t<Fp16, 32>(fp, n_pre, s);
  if (p.d <= 64)
    return p.bf16 ? launch_fwd_t<Bf16, 64>(fp, n_pre, s) : launch_fwd_t<Fp16, 64>(fp, n_pre, s);
  if (p.d <= 128)
    return p.bf16 ? launch_fwd_t<Bf16, 128>(fp, n_pre, s) : launch_fwd_t<Fp16, 128>(fp, n_pre, s);
  return p.bf16 ? launch_fwd_t<Bf16, 256>(fp, n_pre, s) : launch_fwd_t<Fp16, 256>(fp, n_pre, s);
}

}  // namespace thd
