// Shared device helpers for the packed-thd attention kernels (gfx950 only).
//
// MFMA used throughout: v_mfma_f32_32x32x16_{bf16,f16}.  Operand layout for a
// wave of 64 lanes, lane l, half h = l / 32, r = l % 32:
//   A (32 x 16, M x K): lane holds A[r][8h .. 8h+7]
//   B (16 x 32, K x N): lane holds B[8h .. 8h+7][r]
//   C (32 x 32, M x N): lane holds C[8*(i/4) + 4h + (i%4)][r], i = 0..15
// The K index only has to agree between A and B, so a kernel may feed any
// fixed permutation of the 16 K values to both operands.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace thd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element traits: storage is 16-bit, arithmetic in fp32, MFMA in the type.
struct Bf16 {
  typedef __bf16 elem;
  typedef bf16x8 vec8;
  static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // 16x16x32: A lane l holds A[l%16][8(l/16) .. +7], B lane l holds
  // B[8(l/16) .. +7][l%16], C lane l holds C[4(l/16) + i][l%16], i = 0..3.
  static __device__ __forceinline__ f32x4_t mfma16(vec8 a, vec8 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint16_t bits(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
  }
  static __device__ __forceinline__ float to_f32(uint16_t b) {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
  }
};

struct Fp16 {
  typedef _Float16 elem;
  typedef f16x8 vec8;
  static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t mfma16(vec8 a, vec8 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint16_t bits(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  }
  static __device__ __forceinline__ float to_f32(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
  }
};

template <class DT>
__device__ __forceinline__ typename DT::vec8 as_vec8(u32x4 v) {
  return __builtin_bit_cast(typename DT::vec8, v);
}

// Pack 8 fp32 values into 8 16-bit elements (round to nearest even).
template <class DT>
__device__ __forceinline__ typename DT::vec8 pack8(const float* x) {
  typename DT::vec8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (typename DT::elem)x[i];
  return r;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Max and sum of x over lanes l and l ^ 32, in every lane.  v_permlane32_swap
// exchanges lanes 32-63 of its first register with lanes 0-31 of its second,
// so with x in both, each lane ends up holding its own value in one register
// and its partner's in the other: a symmetric combination of the two needs no
// lane select, and no LDS round trip as a bpermute would.  Written as
// assembly with both registers as in/out operands (the compiler builtin,
// given the same value twice, was folded as if the swap were a no-op); the
// s_nop covers the wait states between the VALU writes of the copies and the
// permlane's reads.  Every lane of the wave must be active.
__device__ __forceinline__ void halves_pair(float x, float& a, float& b) {
  a = x;
  b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float wave_max_halves(float x) {
  float a, b;
  halves_pair(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float wave_sum_halves(float x) {
  float a, b;
  halves_pair(x, a, b);
  return a + b;
}

// Sum of x over each aligned group of N lanes (N = 4, 8, 16 or 32), in every
// lane of the group, by DPP row operations (no LDS round trip): exchanges
// within pairs and within quads (quad permutes [1,0,3,2] and [2,3,0,1]), then
// with the mirrored lane of the half row (8 lanes) and of the row (16 lanes);
// groups of 32 add the other row's sum with one lane shuffle.
// Each step adds two partial sums in either order, so all lanes of a group
// end with the same value.  Every lane of the wave must be active.
template <int CTRL>
__device__ __forceinline__ float add_dpp(float v) {
  const int o = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false);
  return v + __builtin_bit_cast(float, o);
}
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32, "groups of 4 to 32 lanes");
  x = add_dpp<0xB1>(x);                   // quad_perm [1,0,3,2]
  x = add_dpp<0x4E>(x);                   // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x = add_dpp<0x141>(x);   // row_half_mirror
  if constexpr (N >= 16) x = add_dpp<0x140>(x);  // row_mirror
  if constexpr (N >= 32) x += __shfl_xor(x, 16, 64);  // the neighbouring DPP row
  return x;
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// ---------------------------------------------------------------------------
// Raw buffer access.  A buffer resource covers one sequence's rows of one
// head: base = its first element, num_records = rows * row_bytes.  Loads past
// num_records return zeros and stores / atomics past it are dropped, which is
// how rows beyond a sequence's length are handled without per-access checks.
// Offsets are 32-bit, so every resource is kept below 2^31 bytes.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // gfx9 raw buffer format word
constexpr uint32_t kOobOffset = 0x80000000u;  // any offset >= num_records reads 0

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}

__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

// The four descriptor words make_rsrc builds (stride 0), made wave-uniform,
// for use as an assembly operand.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  u32x4 w;
  w[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  w[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
  w[2] = __builtin_amdgcn_readfirstlane(bytes);
  w[3] = (uint32_t)kRsrcWord3;
  return w;
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16 bytes per lane from a buffer straight into LDS: lane i of the wave
// writes LDS byte lds_wave + 16 i (lds_wave is made wave-uniform; it goes to
// M0); a lane whose offset is out of range writes zeros.  The wave's vmcnt
// counts the load until its data is in LDS: the caller waits for it and
// synchronises the workgroup before the tile is read.  Written as assembly:
// the compiler cannot tell the tile being filled from the tiles being read
// and would otherwise wait for the load before every transpose read of LDS.
// M0 is otherwise unused by these kernels (no compiler-generated instruction
// reads or writes it; checked in the generated code), so the clobber is safe.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void buf_load_lds16(u32x4 rs, uint32_t lds_wave, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_wave)), "v"(voff), "s"(rs)
               : "m0", "memory");
}
#pragma clang diagnostic pop

// 8 or 16 bytes per lane (outputs leave as whole rows staged in LDS, 16 bytes
// per lane; the 8-byte form stores straight from MFMA accumulators)
__device__ __forceinline__ void buf_store8(u32x2 v, rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ void buf_store16(u32x4 v, rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)voff, (int)soff, 0);
}

// ---------------------------------------------------------------------------
// LDS tiles.  A [rows][DP] tile of 16-bit elements is stored row-major with
// its 16-byte chunks XOR-swizzled per row by f(row).  For DP = 128, f is a
// bijection on 16 consecutive rows (MFMA operand rows read at one logical
// chunk hit 16 distinct 16-byte bank groups), its bits 1-2 and bits 2-3 are
// each distinct on 4 consecutive rows starting at a multiple of 4 (transpose
// reads of 4 rows x 2 or 4 neighbouring chunks), and its bits 0-2 are a
// bijection on 8 consecutive rows -- conflict-free for both a 32- and a
// 64-bank view of LDS.
// ---------------------------------------------------------------------------
template <int DP>
__device__ __forceinline__ uint32_t swz(int row, int elem) {
  constexpr int KCH = DP / 8;
  const int f = (((0xAC60 >> (4 * (row & 3))) & 15) ^ ((row >> 2) & 1) ^ (((row >> 3) & 1) << 3)) &
                (KCH - 1);
  return (uint32_t)row * (DP * 2) + ((uint32_t)((elem >> 3) ^ f) << 4) + (uint32_t)(elem & 7) * 2;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// i%4 of the 8-byte rows addressed by lanes i/4, i/4+4, i/4+8, i/4+12 of the
// group (in that order).  With lane s addressing row R0 + s/4 at column
// C0 + 4*(s%4), lane i gets column C0 + i of rows R0 .. R0+3.
__device__ __forceinline__ u32x2 lds_read_tr(const unsigned char* lds, uint32_t byte_off) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds + byte_off));
  return __builtin_bit_cast(u32x2, v);
}

// Transpose-read operand of a 32x32x16 product whose contraction runs over
// tile rows: A lane (r, h) takes column C + 32dt (C = 16(grp & 1) + 4(g16 & 3),
// read through the transpose) of rows 16kb + 4h + {0..3} (j = 0) and
// 16kb + 8 + 4h + {0..3} (j = 1).  With R = 4h + (g16 >> 2) < 8,
//   swz(R + 16kb + 8j, C + 32dt) = swz(R, C) ^ tr_xor(dt, kb, j):
// the row offset is a multiple of 8 added to R < 8, f sees only its bit 3
// (as chunk bit 3, kept when DP >= 128), and 4dt lies above C's chunk bits.
// The row part only sets row bits that are zero in swz(R, C), so it may also
// be added (and then ride in an instruction's offset field).
template <int DP>
__device__ __forceinline__ uint32_t tr_row(int kb, int j) {
  return (uint32_t)((16 * kb + 8 * j) * DP * 2);
}
template <int DP>
__device__ __forceinline__ uint32_t tr_chunk(int dt, int j) {
  return (uint32_t)(4 * dt ^ (DP >= 128 ? 8 * j : 0)) << 4;
}
template <int DP>
__device__ __forceinline__ uint32_t tr_xor(int dt, int kb, int j) {
  return tr_row<DP>(kb, j) ^ tr_chunk<DP>(dt, j);
}

// Makes v opaque to the optimiser: values derived from it are formed where
// they are used instead of being hoisted out of the loop into registers.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ u32x4 cat2(u32x2 a, u32x2 b) {
  u32x4 r;
  r[0] = a[0];
  r[1] = a[1];
  r[2] = b[0];
  r[3] = b[1];
  return r;
}

// Rows of a sequence that may be touched: [start, start + n) intersected with
// [0, T), and few enough that n * row_bytes stays below 2^31.
__device__ __forceinline__ int clamp_rows(int64_t start, int len, int64_t T, int64_t row_bytes) {
  if (start < 0 || start >= T || len <= 0) return 0;
  int64_t n = len;
  if (n > T - start) n = T - start;
  const int64_t cap = ((int64_t)1 << 31) / row_bytes - 1;
  if (n > cap) n = cap;
  return (int)n;
}

// Length of sequence b as the int32 difference of a cumulative buffer,
// clamped to [0, cap] so that garbage metadata stays memory-safe.
__device__ __forceinline__ int seq_len_clamped(const int32_t* cu, int b, int64_t cap) {
  int64_t n = (int64_t)cu[b + 1] - (int64_t)cu[b];
  if (n < 0) n = 0;
  if (n > cap) n = cap;
  return (int)n;
}

__device__ __forceinline__ int64_t seq_start(const int32_t* cu, const int32_t* cu_padded, int b) {
  return (int64_t)(cu_padded ? cu_padded[b] : cu[b]);
}

// True when row r lies inside some sequence: the last sequence whose start is
// <= r (starts non-decreasing) must also cover r.
__device__ __forceinline__ bool row_is_valid(const int32_t* cu, const int32_t* cu_padded,
                                             int batch, int64_t r, int64_t cap) {
  int lo = 0, hi = batch - 1, found = -1;
  while (lo <= hi) {
    const int mid = (lo + hi) >> 1;
    if (seq_start(cu, cu_padded, mid) <= r) {
      found = mid;
      lo = mid + 1;
    } else {
      hi = mid - 1;
    }
  }
  if (found < 0) return false;
  return r < seq_start(cu, cu_padded, found) + seq_len_clamped(cu, found, cap);
}

// ---------------------------------------------------------------------------
// Per-sequence mask types (one uint8 per sequence): key j of a sequence is
// visible to its query i when j < lk and, for the causal types, j <= i + off
// with off = 0 (top-left) or lk - lq (bottom-right).  Other values: padding.
// ---------------------------------------------------------------------------
constexpr int kMaskPadding = 0;
constexpr int kMaskCausal = 1;
constexpr int kMaskCausalBottomRight = 2;

__device__ __forceinline__ int mask_type_of(const uint8_t* types, int b) {
  return types ? (int)types[b] : kMaskPadding;
}
__device__ __forceinline__ bool mask_is_causal(int mt) {
  return mt == kMaskCausal || mt == kMaskCausalBottomRight;
}
__device__ __forceinline__ int causal_offset(int mt, int lq, int lk) {
  return mt == kMaskCausalBottomRight ? lk - lq : 0;
}

__device__ __forceinline__ int floor_div(int a, int b) {  // b > 0
  const int q = a / b;
  return (a % b != 0 && a < 0) ? q - 1 : q;
}
__device__ __forceinline__ int ceil_div(int a, int b) {  // b > 0
  const int q = a / b;
  return (a % b != 0 && a > 0) ? q + 1 : q;
}
__device__ __forceinline__ int ceil_div_pos(int a, int b) { return a > 0 ? (a + b - 1) / b : 0; }
__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// ---------------------------------------------------------------------------
// Work schedules.  The tiles (sequence b, tile t) of a kernel have work W(t)
// in closed form from the lengths and the mask type: W(t) = H for all x
// tiles of a sequence (no causal mask) or W(t) = clamp(a t + c, 0, H) with
// the model's slope a (causal).  A Model gives md.seq(b) = {x, c, H, causal}
// and kSlope.  The schedule lists the tiles grouped by sequence, sequences
// in decreasing order of their largest tile's work (ties in sequence order),
// each sequence's tiles largest first; rank r is run by the workgroups
// r * heads .. r * heads + heads - 1.  The longest tiles still start first
// and short ones fill in behind them, and every tile of a sequence and head
// runs at about the same time on the XCD that the head fixes, so tiles that
// walk the same rows of the other operand share them in L2.
// Output: sched[0] = number of tiles kept (at most cap); the item of rank r
// at sched + kSchedHeader + kSchedWords r: the tile and everything its
// workgroup needs to start (sequence, tile, slot starts, clamped lengths,
// mask type), so that the workgroup reads one 32-byte record and no
// sequence metadata.  One wave per sequence (wave_id = b); its lanes take
// t = lane, lane + 64, ...; the wave of sequence 0 also writes sched[0].
// ---------------------------------------------------------------------------
struct SeqSummary {
  int x;        // tiles of the sequence
  int c, H;     // W(t) = clamp(a t + c, 0, H) when causal, else H; H < 2^30
  bool causal;
  int sq, sk;   // first rows of the sequence's query and key slots
  int lq, lk;   // lengths as the pass's kernel clamps them
  int mtype;    // mask type
};

constexpr int kSchedHeader = 8;  // int32 words before the first item
constexpr int kSchedWords = 8;   // int32 words per item
struct SchedItem {
  int32_t b, t;     // sequence, tile within it
  int32_t sq, sk;   // first rows of its query and key slots
  int32_t lq, lk;   // clamped lengths
  int32_t mtype;    // mask type
  int32_t unused;
};
static_assert(sizeof(SchedItem) == 4 * kSchedWords, "one item per kSchedWords words");

// Bytes of a schedule of at most cap items.
inline size_t sched_bytes(int64_t cap) {
  return (size_t)(kSchedHeader + kSchedWords * cap) * sizeof(int32_t);
}

// The item of `rank` (rank < the schedule's capacity, so the read stays in
// the buffer) and whether the schedule kept it: the count and the item are
// loaded together, one round trip.  The item of a rank past the count is
// stale and must not be used.
__device__ __forceinline__ bool load_sched_item(const int32_t* sched, int rank, SchedItem& it) {
  const int n = sched[0];
  it = *(const SchedItem*)(sched + kSchedHeader + kSchedWords * rank);
  // Uses the item before the count is tested: without it the compiler sinks
  // the item's loads below that branch, one round trip each.
  asm volatile("" ::"s"(it.b), "s"(it.t), "s"(it.sq), "s"(it.sk), "s"(it.lq), "s"(it.lk),
               "s"(it.mtype));
  return rank < n;
}

// Work of a sequence's largest tile (-1 for a sequence without tiles).
template <class Model>
__device__ __forceinline__ int seq_max_work(const SeqSummary& s) {
  if (s.x <= 0) return -1;
  if (!s.causal) return s.H;
  return clampi(Model::kSlope > 0 ? Model::kSlope * (s.x - 1) + s.c : s.c, 0, s.H);
}

// Sum of v over the 64 lanes of the wave, in every lane (all lanes active).
__device__ __forceinline__ int wave_sum_int(int v) {
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// The schedule described above; sequence b's wave counts the tiles of the
// sequences ahead of b and writes b's tiles after them.
template <class Model>
__device__ void build_schedule_by_sequence(const Model& md, int batch, int cap, int32_t* sched,
                                           int wave_id) {
  const int lane = lane_id();
  const int b = uniform(wave_id);
  if (b >= batch) return;
  const SeqSummary sb = md.seq(b);
  const int wb = seq_max_work<Model>(sb);
  int before = 0, total = 0;  // tiles of the sequences ahead of b; all tiles
  for (int c0 = 0; c0 < batch; c0 += 64) {
    const int j = c0 + lane;
    SeqSummary sj = {0, 0, 0, false};
    if (j < batch) sj = md.seq(j);
    const int wj = seq_max_work<Model>(sj);
    const bool ahead = j < batch && (wj > wb || (wj == wb && j < b));
    before += wave_sum_int(ahead ? sj.x : 0);
    total += wave_sum_int(sj.x);
  }
  const bool descending = sb.causal && Model::kSlope > 0;
  for (int t = lane; t < sb.x; t += 64) {
    const int rank = before + (descending ? sb.x - 1 - t : t);
    if (rank < cap) {
      int4 e0, e1;
      e0.x = b;
      e0.y = t;
      e0.z = sb.sq;
      e0.w = sb.sk;
      e1.x = sb.lq;
      e1.y = sb.lk;
      e1.z = sb.mtype;
      e1.w = 0;
      int4* dst = (int4*)(sched + kSchedHeader + kSchedWords * rank);
      dst[0] = e0;
      dst[1] = e1;
    }
  }
  if (b == 0 && lane == 0) sched[0] = min(total, cap);
}

}  // namespace thd
