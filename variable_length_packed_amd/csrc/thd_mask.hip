// Padding mask from cumulative sequence lengths, built on the device.
//
// TransformerEngine PR "[PyTorch] Build the attention padding mask without
// host syncs", Description: the mask is positions >= seqlens with seqlens the
// first `batch` differences of cu_seqlens (Changes: later entries of a longer
// buffer are ignored).  One elementwise kernel, no host round-trip.
#include "thd_common.hpp"
#include "thd_launch.hpp"

namespace thd {

// One mask to build: rows of max_seqlen bytes, quads = ceil(max_seqlen / 4)
// groups of four bytes per row, blocks of 256 threads (one group each).
struct MaskJob {
  const int32_t* cu;
  uint8_t* mask;
  int max_seqlen;
  int quads;
  int64_t groups;  // batch * quads
};

// Each thread writes four consecutive mask bytes of one row; blocks
// [0, blocks_a) build mask a, the rest mask b (empty for a single mask).
__global__ __launch_bounds__(256) void padding_mask_kernel(MaskJob a, MaskJob b, int batch,
                                                           int blocks_a) {
  const bool first = (int)blockIdx.x < blocks_a;
  const MaskJob& j = first ? a : b;
  const int64_t idx = (int64_t)(first ? blockIdx.x : blockIdx.x - blocks_a) * blockDim.x + threadIdx.x;
  if (idx >= j.groups) return;
  const int row = (int)(idx / j.quads);
  const int s0 = (int)(idx - (int64_t)row * j.quads) * 4;
  // int32 difference with two's-complement wrap, compared as a wider integer
  const int32_t len = (int32_t)((uint32_t)j.cu[row + 1] - (uint32_t)j.cu[row]);
  uint8_t* out = j.mask + (int64_t)row * j.max_seqlen;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int s = s0 + e;
    if (s < j.max_seqlen) out[s] = (uint8_t)((int64_t)s >= (int64_t)len);
  }
}

namespace {
MaskJob mask_job(const int32_t* cu, int batch, int max_seqlen, uint8_t* mask) {
  MaskJob j;
  j.cu = cu;
  j.mask = mask;
  j.max_seqlen = max_seqlen;
  j.quads = (max_seqlen + 3) / 4;
  j.groups = (int64_t)batch * j.quads;
  return j;
}
int64_t mask_blocks(const MaskJob& j) { return (j.groups + 255) / 256; }
}  // namespace

hipError_t launch_padding_mask(const int32_t* cu, int batch, int max_seqlen, uint8_t* mask,
                               hipStream_t s) {
  return launch_padding_masks(cu, nullptr, batch, max_seqlen, 0, mask, nullptr, s);
}

// Both masks of a query / key pair in one launch; a mask with no bytes is
// skipped.
hipError_t launch_padding_masks(const int32_t* cu_q, const int32_t* cu_kv, int batch,
                                int max_q, int max_kv, uint8_t* mask_q, uint8_t* mask_kv,
                                hipStream_t s) {
  const MaskJob a = mask_job(cu_q, batch, max_q, mask_q);
  const MaskJob b = mask_job(cu_kv, batch, max_kv, mask_kv);
  const int64_t ba = mask_blocks(a), bb = mask_blocks(b);
  if (ba + bb == 0) return hipSuccess;
  hipLaunchKernelGGL(padding_mask_kernel, dim3((unsigned)(ba + bb)), dim3(256), 0, s, a, b, batch,
                     (int)ba);
  return hipGetLastError();
}

}  // namespace thd
