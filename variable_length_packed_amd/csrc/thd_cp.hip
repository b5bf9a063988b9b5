// Context parallelism, the part one GPU runs: the shard of one rank and the
// merge of its partial attention outputs.
//
// Megatron-LM issue "How to pad sequences that cannot be evenly split in
// context parallelism (CP)?" (question and repro) splits one sequence across
// devices; its length must first be padded to a multiple of 2n (n ranks), with
// the pad marked by cu_seqlens_padded.  The split used here is the
// load-balanced one: sequence b (valid length len_b) is padded to
// P_b = 2n * C_b rows, C_b = ceil(len_b / 2n), cut into 2n chunks of C_b rows,
// and rank r holds chunks r and 2n-1-r, in that order, as one local slot of
// 2 C_b rows.  Pads sit at the end of a sequence, so a rank's valid rows are a
// prefix of its slot (if its first chunk holds a pad, its second holds only
// pads).
//
// Rank r attends its local queries to the keys of every rank t (the KV ring);
// with a causal sequence, chunk order decides what is visible:
//   t == r: the local slots against each other, causal (top-left: chunk r
//           precedes chunk 2n-1-r in both);
//   t <  r: every local query sees chunk t of rank t (the first half of t's
//           slot) and nothing of chunk 2n-1-t;
//   t >  r: only the second local chunk (2n-1-r) sees rank t, all of it.
// A padding-mask sequence sees all of every rank.  Each step is one call of
// the attention forward on sub-views described by (cu_seqlens,
// cu_seqlens_padded) pairs; rows a step does not cover come out as zeros with
// LSE = -inf, which the merge ignores.  The merge folds the partial outputs by
// their log-sum-exp in fp32.
#include <math.h>

#include "thd_common.hpp"
#include "thd_launch.hpp"

namespace thd {

namespace {

struct CpChunks {
  int C;      // chunk rows
  int v1;     // valid rows of the first local chunk
  int v2;     // valid rows of the second local chunk
};

__device__ __forceinline__ CpChunks cp_chunks(int len, int n, int r) {
  CpChunks c;
  c.C = len > 0 ? (len + 2 * n - 1) / (2 * n) : 0;
  const int a = len - r * c.C, b = len - (2 * n - 1 - r) * c.C;
  c.v1 = a < 0 ? 0 : (a > c.C ? c.C : a);
  c.v2 = b < 0 ? 0 : (b > c.C ? c.C : b);
  return c;
}

__device__ __forceinline__ int seq_len_of(const int32_t* cu, int b) {
  const int l = cu[b + 1] - cu[b];
  return l > 0 ? l : 0;
}

// The view of sequence b for one (rank, peer, side): valid rows, offset of
// its first row inside the owner's local slot, slot rows, global slot rows.
struct CpView {
  int valid, start, slot;
  int64_t gslot;
};

__device__ __forceinline__ CpView cp_view(const CpLayoutArgs& a, int b) {
  const int owner = a.side == 0 ? a.rank : a.peer;  // whose local slots the view is in
  const int len = seq_len_of(a.cu_seqlens, b);
  const CpChunks c = cp_chunks(len, a.n, owner);
  const bool causal = a.mask_type != nullptr && mask_is_causal(a.mask_type[b]);
  CpView v;
  v.valid = c.v1 + c.v2;
  v.start = 0;
  if (causal && a.side == 0 && a.peer > a.rank) {  // only the second query chunk
    v.valid = c.v2;
    v.start = c.C;
  } else if (causal && a.side == 1 && a.peer < a.rank) {  // only the first key chunk
    v.valid = c.v1;
  }
  v.slot = 2 * c.C;
  v.gslot = 2 * (int64_t)a.n * c.C;
  return v;
}

// One workgroup: per-thread runs of sequences, a scan of the run totals, then
// the exclusive prefixes written out (entry `batch` holds the totals).
__global__ __launch_bounds__(256) void thd_cp_layout_kernel(CpLayoutArgs a) {
  __shared__ int64_t sv[256], ss[256], sg[256];
  const int tid = threadIdx.x;
  const int per = (a.batch + 255) / 256;
  const int b0 = min(tid * per, a.batch), b1 = min(b0 + per, a.batch);
  int64_t v = 0, sl = 0, g = 0;
  for (int b = b0; b < b1; ++b) {
    const CpView w = cp_view(a, b);
    v += w.valid;
    sl += w.slot;
    g += w.gslot;
  }
  sv[tid] = v;
  ss[tid] = sl;
  sg[tid] = g;
  __syncthreads();
  if (tid == 0) {
    int64_t pv = 0, ps = 0, pg = 0;
    for (int i = 0; i < 256; ++i) {
      const int64_t tv = sv[i], ts = ss[i], tg = sg[i];
      sv[i] = pv;
      ss[i] = ps;
      sg[i] = pg;
      pv += tv;
      ps += ts;
      pg += tg;
    }
    if (a.out_cu) a.out_cu[a.batch] = (int32_t)pv;
    if (a.out_padded) a.out_padded[a.batch] = (int32_t)ps;
    if (a.out_global_padded) a.out_global_padded[a.batch] = (int32_t)pg;
  }
  __syncthreads();
  v = sv[tid];
  sl = ss[tid];
  g = sg[tid];
  for (int b = b0; b < b1; ++b) {
    const CpView w = cp_view(a, b);
    if (a.out_cu) a.out_cu[b] = (int32_t)v;
    if (a.out_padded) a.out_padded[b] = (int32_t)(sl + w.start);
    if (a.out_global_padded) a.out_global_padded[b] = (int32_t)g;
    if (a.out_mask) {
      const bool causal = a.mask_type != nullptr && mask_is_causal(a.mask_type[b]);
      a.out_mask[b] = (uint8_t)(a.peer == a.rank && causal ? kMaskCausal : kMaskPadding);
    }
    v += w.valid;
    sl += w.slot;
    g += w.gslot;
  }
}

// Local row l of rank r: the sequence whose slot holds it (binary search over
// the local slot starts), then its chunk and the global row.  16 bytes per
// thread; rows outside every slot are left alone.
__global__ __launch_bounds__(256) void thd_cp_gather_kernel(CpGatherArgs a) {
  if (a.batch == 0) return;
  const int chunks = a.row_bytes / 16;
  const int64_t total = a.total_local * chunks;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t l = i / chunks;
    const int c16 = (int)(i - l * chunks);
    // last b with local_padded[b] <= l: the non-empty slot holding l (empty
    // slots start where the next one does)
    int lo = 0, hi = a.batch;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.local_padded[mid] <= l) lo = mid;
      else hi = mid;
    }
    const int b = lo;
    const int64_t off = l - a.local_padded[b];
    const CpChunks c = cp_chunks(seq_len_of(a.cu_seqlens, b), a.n, a.rank);
    if (off < 0 || off >= 2 * (int64_t)c.C) continue;
    const int chunk = off < c.C ? a.rank : 2 * a.n - 1 - a.rank;
    const int64_t g = a.global_padded[b] + (int64_t)chunk * c.C + (off % c.C);
    if (g < 0 || g >= a.total_global) continue;
    const u32x4 v = *(const u32x4*)((const char*)a.src + g * a.row_bytes + 16 * c16);
    *(u32x4*)((char*)a.dst + l * a.row_bytes + 16 * c16) = v;
  }
}

// (row, head) pairs, d / 8 lanes each: fold one partial (o_part, lse_part)
// into the fp32 accumulator (o_acc, lse_acc); with `first` the accumulator
// is taken as empty, with o_out the merged result is also written in the
// storage dtype.
template <class DT>
__global__ __launch_bounds__(256) void thd_lse_merge_kernel(MergeArgs a) {
  const int kch = a.d / 8;
  const int64_t pairs = a.total * a.h;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t pr = i / kch;
  const int c = (int)(i - pr * kch);
  if (pr >= pairs) return;
  const int64_t row = pr / a.h;
  const int hh = (int)(pr - row * a.h);
  const int64_t li = (int64_t)hh * a.total + row;
  const float lb = a.lse_part[li];
  const float la = a.first ? -INFINITY : a.lse_acc[li];
  const float m = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f, lse = -INFINITY;
  if (m != -INFINITY) {
    wa = la == -INFINITY ? 0.f : expf(la - m);
    wb = lb == -INFINITY ? 0.f : expf(lb - m);
    lse = m + logf(wa + wb);
    const float inv = 1.f / (wa + wb);
    wa *= inv;
    wb *= inv;
  }
  f32x4* acc = (f32x4*)(a.o_acc + pr * a.d + 8 * c);
  const u32x4 pv = *(const u32x4*)((const uint16_t*)a.o_part + pr * a.d + 8 * c);
  f32x4 y[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  if (!a.first) {
    y[0] = acc[0];
    y[1] = acc[1];
  }
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = DT::to_f32((uint16_t)(pv[e >> 1] >> (16 * (e & 1))));
    o[e] = wa * y[e >> 2][e & 3] + wb * x;
  }
  acc[0] = f32x4{o[0], o[1], o[2], o[3]};
  acc[1] = f32x4{o[4], o[5], o[6], o[7]};
  if (a.o_out) {
    u32x4 out;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      out[k] = (uint32_t)DT::bits(o[2 * k]) | ((uint32_t)DT::bits(o[2 * k + 1]) << 16);
    *(u32x4*)((uint16_t*)a.o_out + pr * a.d + 8 * c) = out;
  }
  if (c == 0) a.lse_acc[li] = lse;
}

// acc (+)= src elementwise in fp32 (first: =), 8 elements per thread; with
// out, the sum is also written in the storage dtype.
template <class DT>
__global__ __launch_bounds__(256) void thd_accumulate_kernel(AccumulateArgs a) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= a.n) return;
  const u32x4 v = *(const u32x4*)((const uint16_t*)a.src + i);
  f32x4* acc = (f32x4*)(a.acc + i);
  f32x4 y[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  if (!a.first) {
    y[0] = acc[0];
    y[1] = acc[1];
  }
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    o[e] = y[e >> 2][e & 3] + DT::to_f32((uint16_t)(v[e >> 1] >> (16 * (e & 1))));
  acc[0] = f32x4{o[0], o[1], o[2], o[3]};
  acc[1] = f32x4{o[4], o[5], o[6], o[7]};
  if (a.out) {
    u32x4 w;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = (uint32_t)DT::bits(o[2 * k]) | ((uint32_t)DT::bits(o[2 * k + 1]) << 16);
    *(u32x4*)((uint16_t*)a.out + i) = w;
  }
}

// (row, head) pairs, d / 8 lanes each: the log-sum-exp merge of n partials
// in one pass.  With m = max_k lse_k and w_k = exp(lse_k - m):
// lse = m + log(sum_k w_k), o = sum_k (w_k / sum_j w_j) o_k, in fp32; a pair
// whose partials are all -inf gets lse -inf and o = 0.
template <class DT>
__global__ __launch_bounds__(256) void thd_lse_merge_n_kernel(MergeNArgs a) {
  const int kch = a.d / 8;
  const int64_t pairs = a.total * a.h;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t pr = i / kch;
  const int c = (int)(i - pr * kch);
  if (pr >= pairs) return;
  const int64_t row = pr / a.h;
  const int hh = (int)(pr - row * a.h);
  const int64_t li = (int64_t)hh * a.total + row;
  float l[kMaxParts];
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < kMaxParts; ++k) {
    l[k] = k < a.n ? a.lse[k][li] : -INFINITY;
    m = fmaxf(m, l[k]);
  }
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float lse = -INFINITY;
  if (m != -INFINITY) {
    float wsum = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxParts; ++k) {
      l[k] = l[k] == -INFINITY ? 0.f : expf(l[k] - m);  // weight (0 for k >= n)
      wsum += l[k];
    }
    lse = m + logf(wsum);
    const float inv = 1.f / wsum;
#pragma unroll
    for (int k = 0; k < kMaxParts; ++k) {
      if (k >= a.n || l[k] == 0.f) continue;
      const float wk = l[k] * inv;
      const u32x4 pv = *(const u32x4*)((const uint16_t*)a.o[k] + pr * a.d + 8 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        o[e] += wk * DT::to_f32((uint16_t)(pv[e >> 1] >> (16 * (e & 1))));
    }
  }
  u32x4 out;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    out[k] = (uint32_t)DT::bits(o[2 * k]) | ((uint32_t)DT::bits(o[2 * k + 1]) << 16);
  *(u32x4*)((uint16_t*)a.o_out + pr * a.d + 8 * c) = out;
  if (a.lse_out && c == 0) a.lse_out[li] = lse;
}

// Sum of n partials, 8 elements per thread, in fp32 (partials added in
// order), written once in the storage dtype.
template <class DT>
__global__ __launch_bounds__(256) void thd_sum_n_kernel(SumNArgs a) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= a.count) return;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < kMaxParts; ++k) {
    if (k >= a.n) break;
    const u32x4 v = *(const u32x4*)((const uint16_t*)a.x[k] + i);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] += DT::to_f32((uint16_t)(v[e >> 1] >> (16 * (e & 1))));
  }
  u32x4 w;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    w[k] = (uint32_t)DT::bits(o[2 * k]) | ((uint32_t)DT::bits(o[2 * k + 1]) << 16);
  *(u32x4*)((uint16_t*)a.out + i) = w;
}

}  // namespace

hipError_t launch_lse_merge_n(const MergeNArgs& a, bool bf16, hipStream_t s) {
  const int64_t work = a.total * a.h * (a.d / 8);
  if (work == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((work + 255) / 256);
  if (bf16)
    hipLaunchKernelGGL(thd_lse_merge_n_kernel<Bf16>, dim3(blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(thd_lse_merge_n_kernel<Fp16>, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sum_n(const SumNArgs& a, bool bf16, hipStream_t s) {
  if (a.count == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((a.count / 8 + 255) / 256);
  if (bf16)
    hipLaunchKernelGGL(thd_sum_n_kernel<Bf16>, dim3(blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(thd_sum_n_kernel<Fp16>, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_accumulate(const AccumulateArgs& a, bool bf16, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((a.n / 8 + 255) / 256);
  if (bf16)
    hipLaunchKernelGGL(thd_accumulate_kernel<Bf16>, dim3(blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(thd_accumulate_kernel<Fp16>, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_cp_layout(const CpLayoutArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(thd_cp_layout_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_cp_gather(const CpGatherArgs& a, hipStream_t s) {
  if (a.total_local == 0) return hipSuccess;
  const int64_t work = a.total_local * (a.row_bytes / 16);
  const int64_t blocks = (work + 255) / 256;
  hipLaunchKernelGGL(thd_cp_gather_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_lse_merge(const MergeArgs& a, bool bf16, hipStream_t s) {
  const int64_t work = a.total * a.h * (a.d / 8);
  if (work == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((work + 255) / 256);
  if (bf16)
    hipLaunchKernelGGL(thd_lse_merge_kernel<Bf16>, dim3(blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(thd_lse_merge_kernel<Fp16>, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace thd
