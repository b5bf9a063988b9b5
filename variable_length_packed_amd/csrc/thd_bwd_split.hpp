// Internal interface between the two sources of the backward
// (thd_bwd_split.hip: pre pass, dq pass and launch;
// thd_bwd_dkdv.hip: the dk/dv pass, built with its own compiler options).
#pragma once

#include "thd_common.hpp"

namespace thd {
namespace split {

constexpr int kDqBM = 128;   // query rows per dq workgroup (4 waves of 32 rows)
// The dk/dv pass's two shapes, chosen on the host from the length of its
// walks (max_seqlen_q times the GQA group); above head dim 128 always the
// short one (the long one's LDS would not fit):
//   long walks : 256 keys (8 waves), Q and dO of two query tiles in LDS
//                (160 KB, one workgroup per CU, one barrier per query tile);
//   short walks: 128 keys (4 waves), one query tile in LDS (80 KB, two
//                workgroups per CU, two barriers per query tile), so that one
//                workgroup's K/V prologue and barriers overlap the other's work.
constexpr int kKvBkLong = 256;
constexpr int kKvBkShort = 128;
constexpr int kKvShortWalkRows = 4096;  // max_seqlen_q * group up to this: short
template <int BK>
constexpr int kKvQBufs = BK == kKvBkLong ? 2 : 1;  // query tiles a workgroup holds in LDS
constexpr int kKvBQ = 32;    // query rows per dk/dv step
constexpr int kPadRows = 64; // rows per pad-zeroing workgroup

// Key tiles of the dq pass: as the forward's (32 keys at d > 32, 64 at
// d <= 32); three buffers, two tiles resident and one loading.
template <int DP>
struct DqTile {
  static constexpr int BN = DP > 32 ? 32 : 64;
};
constexpr int kDqBufs = 3;
constexpr int kDqReadAhead = 1;  // K steps between an LDS read and its product

struct SplitParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* dsum;      // [h_q, T_q]: -D, written by the dq pass
  float* lsum;      // [h_q, T_q]: -LSE / scale, written by the dq pass
  int32_t* qsched;  // item count, then (sequence, query tile) items by rank
  int32_t* ksched;  // item count, then (sequence, key tile) items by rank
  const int32_t* cu_q;
  const int32_t* cu_kv;
  const int32_t* pad_q;
  const int32_t* pad_kv;
  const uint8_t* causal;
  int64_t T_q, T_kv;
  int batch, h_q, h_kv, group, d;
  float scale, c2;   // c2 = scale * log2(e)
  int n_qtiles;      // query tiles per head (upper bound)
  int n_ktiles;      // key tiles per kv head (upper bound)
  int kv_bk;         // keys per dk/dv workgroup: kKvBkLong or kKvBkShort
  int n_qsched_wg;   // pre-pass workgroups building the dq schedule
  int n_ksched_wg;   // ... and the dk/dv schedule
  int n_qzero_wg;    // ... zeroing pad rows of dq (kPadRows rows each)
  int n_kzero_wg;    // ... zeroing pad rows of dk and dv
};

// Both passes clamp a sequence's rows the same way (32-bit offsets per
// sequence), and so do the work models of their schedules.
__device__ __forceinline__ int split_lq(const SplitParams& p, int b) {
  const int64_t sq = seq_start(p.cu_q, p.pad_q, b);
  return clamp_rows(sq, seq_len_clamped(p.cu_q, b, p.T_q), p.T_q, (int64_t)p.h_q * p.d * 2);
}
__device__ __forceinline__ int split_lk(const SplitParams& p, int b) {
  const int64_t sk = seq_start(p.cu_kv, p.pad_kv, b);
  return clamp_rows(sk, seq_len_clamped(p.cu_kv, b, p.T_kv), p.T_kv, (int64_t)p.h_kv * p.d * 2);
}

// Launch the dk/dv pass (grid n_ktiles * h_kv, key tiles of p.kv_bk) on
// stream s.
template <class DT, int DP>
hipError_t launch_dkdv(const SplitParams& p, hipStream_t s);

}  // namespace split
}  // namespace thd
