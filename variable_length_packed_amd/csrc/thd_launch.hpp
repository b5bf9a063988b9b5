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
hipError_t launch_padding_masks(const int32_t* cu_q, const int32_t* cu_kv, int batch,
                                int max_q, int max_kv, uint8_t* mask_q, uint8_t* mask_kv,
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

// The backward as a dq pass and a dk/dv pass (thd_bwd_split.hip, thd_bwd_dkdv.hip).
// `events` is null or four events recorded on `s` before the pre pass, before
// the dq pass, before the dk/dv pass and after it.
size_t bwd_workspace_bytes(const Problem& p);
hipError_t launch_bwd(const Problem& p, const void* q, const void* k, const void* v,
                      const void* o, const void* dout, const float* lse, void* dq, void* dk,
                      void* dv, void* workspace, hipStream_t s,
                      hipEvent_t const* events = nullptr);

}  // namespace thd
