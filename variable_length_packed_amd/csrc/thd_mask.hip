// Padding mask from cumulative sequence lengths, built on the device.
//
// TransformerEngine PR "[PyTorch] Build the attention padding mask without
// host syncs", Description: the mask is positions >= seqlens with seqlens the
// first `batch` differences of cu_seqlens (Changes: later entries of a longer
// buffer are ignored).  One elementwise kernel, no host round-trip.
#include "thd_common.hpp"
#include "thd_launch.hpp"

namespace thd {

// Each thread writes four consecutive mask bytes of one row.
__global__ __launch_bounds__(256) void padding_mask_kernel(const int32_t* __restrict__ cu,
                                                           int batch, int max_seqlen,
                                                           int quads_per_row,
                                                           uint8_t* __restrict__ mask) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)batch * quads_per_row;
  if (idx >= total) return;
  const int b = (int)(idx / quads_per_row);
  const int s0 = (int)(idx - (int64_t)b * quads_per_row) * 4;
  // int32 difference with two's-complement wrap, compared as a wider integer
  const int32_t len = (int32_t)((uint32_t)cu[b + 1] - (uint32_t)cu[b]);
  uint8_t* row = mask + (int64_t)b * max_seqlen;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int s = s0 + e;
    if (s < max_seqlen) row[s] = (uint8_t)((int64_t)s >= (int64_t)len);
  }
}

hipError_t launch_padding_mask(const int32_t* cu, int batch, int max_seqlen, uint8_t* mask,
                               hipStream_t s) {
  if (batch == 0 || max_seqlen == 0) return hipSuccess;
  const int quads = (max_seqlen + 3) / 4;
  const int64_t total = (int64_t)batch * quads;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(padding_mask_kernel, dim3((unsigned)blocks), dim3(256), 0, s, cu, batch,
                     max_seqlen, quads, mask);
  return hipGetLastError();
}

}  // namespace thd
