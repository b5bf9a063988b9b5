// C ABI of libthdattn.so (declared in include/thd_attn.h).
//
// Host code only validates host-visible scalars and pointers, derives the
// grid sizes from them and enqueues kernels; it never reads device memory
// and never synchronises, following the no-host-sync requirement of
// TransformerEngine PR "[PyTorch] Build the attention padding mask without
// host syncs" (Description, Changes).
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "thd_attn.h"
#include "thd_launch.hpp"

namespace {

constexpr int64_t kMaxRows = (int64_t)1 << 31;  // row indices fit int32 offsets per head

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// Kernels address a sequence's rows with 32-bit byte offsets from its first
// row, so max_seqlen rows of every buffer they address per sequence must
// stay below 2^31 bytes: q / o / dq rows (h_q * head_dim * 2 bytes) and
// k / v / dk / dv rows (h_kv * head_dim * 2).
int check_sizes(const thd_varlen_args* a) {
  const int64_t lim = (int64_t)1 << 31;
  const int64_t q_row = (int64_t)a->h_q * a->head_dim * 2;
  const int64_t kv_row = (int64_t)a->h_kv * a->head_dim * 2;
  if ((int64_t)a->max_seqlen_q * q_row >= lim || (int64_t)a->max_seqlen_kv * kv_row >= lim)
    return THD_ERR_SHAPE;
  return THD_OK;
}

int to_problem(const thd_varlen_args* a, thd::Problem* p) {
  if (!a) return THD_ERR_NULL;
  if (a->batch < 0 || a->max_seqlen_q < 0 || a->max_seqlen_kv < 0 || a->total_q < 0 ||
      a->total_kv < 0)
    return THD_ERR_SHAPE;
  if (a->h_q <= 0 || a->h_kv <= 0 || a->h_q % a->h_kv != 0) return THD_ERR_SHAPE;
  if (a->total_q >= kMaxRows || a->total_kv >= kMaxRows) return THD_ERR_SHAPE;
  if (a->dtype != THD_FP16 && a->dtype != THD_BF16) return THD_ERR_UNSUPPORTED;
  if (a->head_dim < 8 || a->head_dim > 256 || a->head_dim % 8 != 0) return THD_ERR_UNSUPPORTED;
  if (a->batch > 0 && (!a->cu_seqlens_q || !a->cu_seqlens_kv)) return THD_ERR_NULL;
  // grid bounds: query/key tiles times heads must fit a 32-bit grid
  const int64_t tiles_q = (a->total_q + 127) / 128 + a->batch;
  const int64_t tiles_kv = (a->total_kv + 127) / 128 + a->batch;
  if (tiles_q * a->h_q >= ((int64_t)1 << 31) || tiles_kv * a->h_kv >= ((int64_t)1 << 31))
    return THD_ERR_SHAPE;
  if (int st = check_sizes(a)) return st;
  p->cu_q = a->cu_seqlens_q;
  p->cu_kv = a->cu_seqlens_kv;
  p->pad_q = a->cu_seqlens_q_padded;
  p->pad_kv = a->cu_seqlens_kv_padded;
  p->causal = a->mask_type;
  p->batch = a->batch;
  p->max_q = a->max_seqlen_q;
  p->max_kv = a->max_seqlen_kv;
  p->T_q = a->total_q;
  p->T_kv = a->total_kv;
  p->h_q = a->h_q;
  p->h_kv = a->h_kv;
  p->d = a->head_dim;
  float s = a->softmax_scale;
  if (!(s > 0.f) || isinf(s)) s = 1.0f / sqrtf((float)a->head_dim);
  p->scale = s;
  p->bf16 = a->dtype == THD_BF16;
  return THD_OK;
}

int check_tensor(const void* ptr, int64_t rows) {
  if (rows == 0) return THD_OK;
  if (!ptr) return THD_ERR_NULL;
  if (!aligned16(ptr)) return THD_ERR_UNSUPPORTED;
  return THD_OK;
}

// Host-visible checks of a forward call: the problem plus its tensors.
int fwd_problem(const thd_varlen_args* args, const void* q, const void* k, const void* v,
                const void* o, const float* lse, thd::Problem* p) {
  int st = to_problem(args, p);
  if (st != THD_OK) return st;
  const int64_t Tq = p->T_q, Tk = p->T_kv;
  if ((st = check_tensor(q, Tq)) || (st = check_tensor(o, Tq)) || (st = check_tensor(k, Tk)) ||
      (st = check_tensor(v, Tk)))
    return st;
  if (Tq > 0 && !lse) return THD_ERR_NULL;
  return THD_OK;
}

// The forward's workspace for callers that cannot allocate
// (thd_attn_fwd_noalloc): a fixed array in device memory, one copy per
// device, held until the process ends.
constexpr size_t kNoAllocScratchBytes = (size_t)THD_FWD_NOALLOC_MAX_WORKSPACE;
constexpr int kMaxDevices = 256;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's copy of `scratch`, looked up once
// per device with that device current.  On the host the array's name is
// only a stand-in for the symbol, never a device address: kernels and copies
// get this pointer instead.
int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return THD_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return THD_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return THD_OK;
}

}  // namespace

extern "C" {

int thd_version(void) { return 100; }

const char* thd_status_string(int status) {
  switch (status) {
    case THD_OK: return "THD_OK";
    case THD_ERR_NULL: return "THD_ERR_NULL: a required pointer is NULL";
    case THD_ERR_SHAPE: return "THD_ERR_SHAPE: a size is negative or inconsistent";
    case THD_ERR_UNSUPPORTED: return "THD_ERR_UNSUPPORTED: head_dim, dtype or alignment not supported";
    case THD_ERR_WORKSPACE: return "THD_ERR_WORKSPACE: workspace missing, too small or misaligned";
    case THD_ERR_HIP: return "THD_ERR_HIP: the HIP runtime refused a launch";
    default: return "unknown thd_status";
  }
}

int thd_padding_mask(const int32_t* cu_seqlens, int32_t batch, int32_t max_seqlen,
                     uint8_t* mask, void* stream) {
  if (batch < 0 || max_seqlen < 0) return THD_ERR_SHAPE;
  if ((int64_t)batch * max_seqlen == 0) return THD_OK;
  if (!cu_seqlens || !mask) return THD_ERR_NULL;
  hipError_t e = thd::launch_padding_mask(cu_seqlens, batch, max_seqlen, mask,
                                          (hipStream_t)stream);
  return e == hipSuccess ? THD_OK : THD_ERR_HIP;
}

int thd_padding_masks(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, int32_t batch,
                      int32_t max_seqlen_q, int32_t max_seqlen_kv, uint8_t* mask_q,
                      uint8_t* mask_kv, void* stream) {
  if (batch < 0 || max_seqlen_q < 0 || max_seqlen_kv < 0) return THD_ERR_SHAPE;
  const bool any_q = (int64_t)batch * max_seqlen_q > 0;
  const bool any_kv = (int64_t)batch * max_seqlen_kv > 0;
  if ((any_q && (!cu_seqlens_q || !mask_q)) || (any_kv && (!cu_seqlens_kv || !mask_kv)))
    return THD_ERR_NULL;
  hipError_t e = thd::launch_padding_masks(cu_seqlens_q, cu_seqlens_kv, batch,
                                           any_q ? max_seqlen_q : 0, any_kv ? max_seqlen_kv : 0,
                                           mask_q, mask_kv, (hipStream_t)stream);
  return e == hipSuccess ? THD_OK : THD_ERR_HIP;
}

size_t thd_attn_fwd_workspace_size(const thd_varlen_args* args) {
  thd::Problem p;
  if (to_problem(args, &p) != THD_OK) return 0;
  return thd::fwd_workspace_bytes(p);
}

int thd_attn_fwd(const thd_varlen_args* args, const void* q, const void* k, const void* v,
                 void* o, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  thd::Problem p;
  int st = fwd_problem(args, q, k, v, o, lse, &p);
  if (st != THD_OK) return st;
  const size_t need = thd::fwd_workspace_bytes(p);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return THD_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return THD_ERR_WORKSPACE;
  }
  hipError_t e = thd::launch_fwd(p, q, k, v, o, lse, workspace, (hipStream_t)stream);
  return e == hipSuccess ? THD_OK : THD_ERR_HIP;
}

int thd_attn_fwd_noalloc(const thd_varlen_args* args, const void* q, const void* k,
                         const void* v, void* o, float* lse, void* stream) {
  thd::Problem p;
  int st = fwd_problem(args, q, k, v, o, lse, &p);
  if (st != THD_OK) return st;
  const size_t need = thd::fwd_workspace_bytes(p);
  if (need > kNoAllocScratchBytes) return THD_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0 && (st = scratch_of_current_device(&ws)) != THD_OK) return st;
  hipError_t e = thd::launch_fwd(p, q, k, v, o, lse, ws, (hipStream_t)stream);
  return e == hipSuccess ? THD_OK : THD_ERR_HIP;
}

size_t thd_attn_bwd_workspace_size(const thd_varlen_args* args) {
  thd::Problem p;
  if (to_problem(args, &p) != THD_OK) return 0;
  return thd::bwd_workspace_bytes(p);
}

static int attn_bwd_impl(const thd_varlen_args* args, const void* q, const void* k,
                         const void* v, const void* o, const void* dout, const float* lse,
                         void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                         void* stream, void* const* events) {
  thd::Problem p;
  int st = to_problem(args, &p);
  if (st != THD_OK) return st;
  const int64_t Tq = p.T_q, Tk = p.T_kv;
  if ((st = check_tensor(q, Tq)) || (st = check_tensor(o, Tq)) ||
      (st = check_tensor(dout, Tq)) || (st = check_tensor(dq, Tq)) ||
      (st = check_tensor(k, Tk)) || (st = check_tensor(v, Tk)) || (st = check_tensor(dk, Tk)) ||
      (st = check_tensor(dv, Tk)))
    return st;
  if (Tq > 0 && !lse) return THD_ERR_NULL;
  const size_t need = thd::bwd_workspace_bytes(p);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return THD_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return THD_ERR_WORKSPACE;
  }
  hipError_t e = thd::launch_bwd(p, q, k, v, o, dout, lse, dq, dk, dv, workspace,
                                 (hipStream_t)stream, (hipEvent_t const*)events);
  return e == hipSuccess ? THD_OK : THD_ERR_HIP;
}

int thd_attn_bwd(const thd_varlen_args* args, const void* q, const void* k, const void* v,
                 const void* o, const void* dout, const float* lse, void* dq, void* dk,
                 void* dv, void* workspace, size_t workspace_bytes, void* stream) {
  return attn_bwd_impl(args, q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes,
                       stream, nullptr);
}

int thd_attn_bwd_timed(const thd_varlen_args* args, const void* q, const void* k,
                       const void* v, const void* o, const void* dout, const float* lse,
                       void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                       void* stream, void* const* events) {
  if (!events || !events[0] || !events[1] || !events[2] || !events[3]) return THD_ERR_NULL;
  return attn_bwd_impl(args, q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes,
                       stream, events);
}

}  // extern "C"
