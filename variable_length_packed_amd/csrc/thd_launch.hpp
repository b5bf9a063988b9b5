// Host-side launchers shared between the C ABI layer and the kernel files.
// All arguments have been validated by the caller; launchers only size grids
// and enqueue kernels on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace thd {

struct Problem {
  const int32_t* cu_q;
  const int32_t* cu_kv;
  const int32_t* pad_q;   // may be null
  const int32_t* pad_kv;  // may be null
  const uint8_t* causal;  // per-sequence mask type (thd_mask_type); may be null
  int batch;
  int max_q, max_kv;      // host bounds on the sequence lengths
  int64_t T_q, T_kv;
  int h_q, h_kv, d;
  float scale;
  bool bf16;
};

hipError_t launch_padding_mask(const int32_t* cu, int batch, int max_seqlen, uint8_t* mask,
                               hipStream_t s);

size_t fwd_workspace_bytes(const Problem& p);

// Zeros on the pad rows of o and -inf on their LSE (the forward's pad pass).
hipError_t launch_fwd_pad_rows(const Problem& p, void* o, float* lse, hipStream_t s);

// Split-KV forward for few query rows per sequence (see thd_decode.hip).
bool decode_applies(const Problem& p);
size_t decode_workspace_bytes(const Problem& p);
hipError_t launch_decode(const Problem& p, const void* q, const void* k, const void* v, void* o,
                         float* lse, void* workspace, hipStream_t s);

hipError_t launch_fwd(const Problem& p, const void* q, const void* k, const void* v, void* o,
                      float* lse, void* workspace, hipStream_t s);

size_t bwd_workspace_bytes(const Problem& p);

// `events` is null or four events recorded on `s` before the pre pass, before
// the main kernel, before the post pass and after it.
hipError_t launch_bwd(const Problem& p, const void* q, const void* k, const void* v,
                      const void* o, const void* dout, const float* lse, void* dq, void* dk,
                      void* dv, void* workspace, hipStream_t s,
                      hipEvent_t const* events = nullptr);

// Context parallelism, one rank's share (see thd_cp.hip).  side 0: the view
// of rank `rank`'s queries for the step that reads rank `peer`'s keys; side 1:
// the view of rank `peer`'s keys for that step.
struct CpLayoutArgs {
  const int32_t* cu_seqlens;   // global valid lengths, batch + 1 entries
  const uint8_t* mask_type;    // per sequence; may be null (padding)
  int batch, n, rank, peer, side;
  int32_t* out_cu;             // batch + 1, may be null
  int32_t* out_padded;         // batch + 1, may be null
  int32_t* out_global_padded;  // batch + 1, may be null
  uint8_t* out_mask;           // batch, may be null
};

struct CpGatherArgs {
  const int32_t* cu_seqlens;     // global valid lengths
  const int32_t* local_padded;   // the rank's local slot starts (side 0 view of step peer = rank)
  const int32_t* global_padded;  // global slot starts
  int batch, n, rank;
  const void* src;
  int64_t total_global;
  void* dst;
  int64_t total_local;
  int row_bytes;                 // multiple of 16
};

struct MergeArgs {
  const void* o_part;   // [total, h, d] storage dtype
  const float* lse_part;  // [h, total]
  float* o_acc;         // [total, h, d]
  float* lse_acc;       // [h, total]
  void* o_out;          // may be null
  int64_t total;
  int h, d;
  int first;
};

struct AccumulateArgs {
  const void* src;  // n elements, storage dtype
  float* acc;       // n elements
  void* out;        // may be null
  int64_t n;        // multiple of 8
  int first;
};

hipError_t launch_accumulate(const AccumulateArgs& a, bool bf16, hipStream_t s);

// One pass over up to kMaxParts partials: their log-sum-exp merge, or their sum.
constexpr int kMaxParts = 8;
struct MergeNArgs {
  const void* o[kMaxParts];      // [total, h, d] storage dtype
  const float* lse[kMaxParts];   // [h, total]
  int n;
  void* o_out;                   // [total, h, d] storage dtype
  float* lse_out;                // [h, total]; may be null
  int64_t total;
  int h, d;
};
struct SumNArgs {
  const void* x[kMaxParts];  // count elements, storage dtype
  int n;
  void* out;                 // count elements, storage dtype
  int64_t count;             // multiple of 8
};
hipError_t launch_lse_merge_n(const MergeNArgs& a, bool bf16, hipStream_t s);
hipError_t launch_sum_n(const SumNArgs& a, bool bf16, hipStream_t s);
hipError_t launch_cp_layout(const CpLayoutArgs& a, hipStream_t s);
hipError_t launch_cp_gather(const CpGatherArgs& a, hipStream_t s);
hipError_t launch_lse_merge(const MergeArgs& a, bool bf16, hipStream_t s);

}  // namespace thd
