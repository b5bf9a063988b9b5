/*
 * thd_attn.h -- C ABI of libthdattn.so: scaled-dot-product attention over
 * packed variable-length ("thd") tensors on AMD Instinct MI355X (gfx950).
 *
 * Definitions follow three pages:
 *   [I]  Megatron-LM issue "How to pad sequences that cannot be evenly split in
 *        context parallelism (CP)?" -- packed thd q/k/v of shape [T, h, d],
 *        int32 cu_seqlens, max_seqlen, the "padding" mask type, pad tokens
 *        that hold garbage and must not be attended.
 *   [C]  TransformerEngine PR "Add per-sequence causal policy to packed THD
 *        attention" -- Description/Changes: one causal flag per packed
 *        sequence ("padding_causal" vs "padding"); maintainer review: the
 *        two-call example with cu_seqlens_padded, whose pad positions are
 *        written as zeros.
 *   [M]  TransformerEngine PR "[PyTorch] Build the attention padding mask
 *        without host syncs" -- Description: mask = positions >= seqlens;
 *        Changes: cu_seqlens may be longer than batch+1 (extra entries are
 *        ignored), no host synchronisation.
 *
 * Conventions common to every entry point
 *   - Every tensor pointer is a DEVICE pointer; the caller allocates and owns
 *     all memory, the library allocates and frees nothing and keeps no state
 *     besides its loaded code objects and the fixed per-device workspace
 *     array of thd_attn_fwd_noalloc (with its per-device address).
 *   - Tensors are dense and row-major: q, o, dq, dout are [total_q, h_q, d];
 *     k, v, dk, dv are [total_kv, h_kv, d]; row stride h*d elements.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream).  No call reads device memory from the host, copies device to
 *     host or synchronises, so every call may be captured in a HIP graph.
 *   - Only host-visible arguments are validated; an invalid one returns a
 *     negative status before anything is launched.  Device metadata
 *     (cu_seqlens*, mask_type) is never validated: for malformed values every
 *     row index is clamped into range, so the kernels stay memory-safe, but
 *     the result is unspecified.
 *   - Size limits (THD_ERR_SHAPE otherwise): total_q, total_kv < 2^31; a
 *     sequence's rows are addressed with 32-bit byte offsets, so
 *     max_seqlen_q * h_q * head_dim * 2 and max_seqlen_kv * h_kv * head_dim * 2
 *     must be below 2^31.  max_seqlen_* must bound the true lengths: a
 *     longer sequence is clamped as above.
 *   - No C++ exception crosses this interface.
 *
 * Sequence placement [I], [C]
 *   Sequence b (0 <= b < batch) has lq_b = cu_seqlens_q[b+1] - cu_seqlens_q[b]
 *   valid query rows starting at row sq_b = cu_seqlens_q_padded[b] (or
 *   cu_seqlens_q[b] when no padded offsets are given); likewise for keys and
 *   values with cu_seqlens_kv / cu_seqlens_kv_padded.  Every other row of
 *   [0, total) -- slot tails, gaps, rows before the first slot or after the
 *   last -- is a pad row: it is never read for attention and every output
 *   written for it is +0.0 (bit pattern 0).
 *
 * Mask [C] (Description; maintainer review: one mask type per sequence)
 *   Query i of sequence b (0-based inside the sequence) attends key j iff
 *   j < lk_b and, by mask_type[b]:
 *     THD_MASK_PADDING (0)                 every such key;
 *     THD_MASK_CAUSAL (1)                  j <= i ("padding_causal", top-left);
 *     THD_MASK_CAUSAL_BOTTOM_RIGHT (2)     j <= i + lk_b - lq_b
 *                                          ("padding_causal_bottom_right");
 *   any other value is taken as THD_MASK_PADDING, and a 0/1 causal flag per
 *   sequence is a valid mask_type array.  A query row with no visible key
 *   (lk_b == 0, or the first lq_b - lk_b rows under bottom-right alignment)
 *   gets output 0 and log-sum-exp -inf, and has zero gradient.
 *
 * Head mapping: query head hq reads key/value head hq / (h_q / h_kv).
 */
#ifndef THD_ATTN_H
#define THD_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  THD_OK = 0,
  THD_ERR_NULL = -1,        /* a required pointer is NULL                     */
  THD_ERR_SHAPE = -2,       /* a size is negative or inconsistent             */
  THD_ERR_UNSUPPORTED = -3, /* head_dim or dtype outside what is built        */
  THD_ERR_WORKSPACE = -4,   /* workspace missing, too small or misaligned     */
  THD_ERR_HIP = -5          /* the HIP runtime refused a launch               */
} thd_status;

typedef enum { THD_FP16 = 0, THD_BF16 = 1 } thd_dtype;

typedef enum {
  THD_MASK_PADDING = 0,
  THD_MASK_CAUSAL = 1,
  THD_MASK_CAUSAL_BOTTOM_RIGHT = 2
} thd_mask_type;

/* Problem description shared by the attention entry points.  The pointers
 * are DEVICE pointers to int32/uint8 metadata and are read only by kernels. */
typedef struct {
  const int32_t* cu_seqlens_q;         /* >= batch+1 entries; later ones ignored   */
  const int32_t* cu_seqlens_kv;        /* self attention: may alias cu_seqlens_q   */
  const int32_t* cu_seqlens_q_padded;  /* NULL => row starts are cu_seqlens_q      */
  const int32_t* cu_seqlens_kv_padded; /* NULL => row starts are cu_seqlens_kv     */
  const uint8_t* mask_type;            /* [batch] thd_mask_type; NULL => padding   */
  int32_t batch;                       /* >= 0; 0 writes zeros everywhere          */
  int32_t max_seqlen_q;                /* >= 0; bound on lq_b (host scalar, [I])   */
  int32_t max_seqlen_kv;               /* >= 0; bound on lk_b                      */
  int64_t total_q;                     /* rows of q / o / dq / dout                */
  int64_t total_kv;                    /* rows of k / v / dk / dv                  */
  int32_t h_q;                         /* query heads, >= 1                        */
  int32_t h_kv;                        /* key/value heads, h_q % h_kv == 0         */
  int32_t head_dim;                    /* multiple of 8, 8..256                    */
  float softmax_scale;                 /* <= 0 or NaN => 1/sqrt(head_dim)          */
  int32_t dtype;                       /* thd_dtype of q/k/v/o/dout/dq/dk/dv       */
} thd_varlen_args;

/* Padding mask [M] (Description): for b < batch and s < max_seqlen,
 *   mask[b*max_seqlen + s] = (s >= (int32)(cu_seqlens[b+1] - cu_seqlens[b]))
 * written as uint8 0/1 (1 = pad), i.e. the bool [batch,1,1,max_seqlen] mask
 * of the page flattened.  The difference wraps as int32 arithmetic does, so
 * the result is defined for every input; entries of cu_seqlens past batch+1
 * are never read.  One kernel, no host synchronisation.
 * Errors: THD_ERR_NULL (cu_seqlens or mask NULL while batch*max_seqlen > 0),
 * THD_ERR_SHAPE (batch < 0 or max_seqlen < 0). */
int thd_padding_mask(const int32_t* cu_seqlens, int32_t batch, int32_t max_seqlen,
                     uint8_t* mask, void* stream);

/* The query and key/value padding masks [M] (Changes: attention_mask_q and
 * attention_mask_kv) in one launch: mask_q as thd_padding_mask(cu_seqlens_q,
 * batch, max_seqlen_q) and mask_kv as thd_padding_mask(cu_seqlens_kv, batch,
 * max_seqlen_kv), byte for byte.  A mask with batch * max_seqlen = 0 is not
 * written and its pointers may be NULL.
 * Errors: THD_ERR_SHAPE (batch or a max_seqlen < 0), THD_ERR_NULL (a
 * cu_seqlens or mask NULL for a mask with bytes to write). */
int thd_padding_masks(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, int32_t batch,
                      int32_t max_seqlen_q, int32_t max_seqlen_kv, uint8_t* mask_q,
                      uint8_t* mask_kv, void* stream);

/* Bytes of device workspace thd_attn_fwd needs for these arguments (the
 * order in which its workgroups take the query tiles, a few bytes per tile),
 * 0 if the arguments are invalid or the batch is empty.  The workspace needs
 * no initialisation. */
size_t thd_attn_fwd_workspace_size(const thd_varlen_args* args);

/* Forward [I], [C]: o = softmax(scale * q k^T + mask) v per sequence and head.
 *   o   [total_q, h_q, head_dim]  output, every pad row written as +0;
 *   lse [h_q, total_q] fp32       natural-log log-sum-exp of the scaled
 *                                 scores per query row (-inf on pad rows and
 *                                 rows that see no key); needed by backward.
 * q, k, v are read only at valid rows.  workspace must be a device buffer of
 * at least thd_attn_fwd_workspace_size(args) bytes, 256-byte aligned, used by
 * this call only (it may be NULL when that size is 0).  Errors: THD_ERR_NULL,
 * THD_ERR_SHAPE, THD_ERR_UNSUPPORTED, THD_ERR_WORKSPACE, THD_ERR_HIP. */
int thd_attn_fwd(const thd_varlen_args* args, const void* q, const void* k,
                 const void* v, void* o, float* lse, void* workspace,
                 size_t workspace_bytes, void* stream);

/* Largest forward workspace (bytes) thd_attn_fwd_noalloc can provide. */
#define THD_FWD_NOALLOC_MAX_WORKSPACE (16u << 20)

/* thd_attn_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same validation, kernels and results as thd_attn_fwd, with the
 * workspace taken from a fixed device array of THD_FWD_NOALLOC_MAX_WORKSPACE
 * bytes inside the library (one per device, held until the process ends)
 * instead of a caller buffer.  The caller still passes every input and
 * output.  The call allocates and frees nothing; its first call on a device
 * looks up that device's array (call it once before a graph capture), with
 * the stream's device current.  Every call on one device shares that
 * device's array, and nothing in it needs to start at zero; calls that
 * overlap in time on one device (several streams or host threads) race on it
 * and their results are undefined.  Errors: as thd_attn_fwd, and
 * THD_ERR_WORKSPACE when thd_attn_fwd_workspace_size(args) exceeds
 * THD_FWD_NOALLOC_MAX_WORKSPACE (returned before anything is launched). */
int thd_attn_fwd_noalloc(const thd_varlen_args* args, const void* q, const void* k,
                         const void* v, void* o, float* lse, void* stream);

/* Bytes of device workspace thd_attn_bwd needs for these arguments (per-row
 * fp32 statistics and the order of the work items, a few bytes per row),
 * 0 if the arguments are invalid.  The workspace needs no initialisation. */
size_t thd_attn_bwd_workspace_size(const thd_varlen_args* args);

/* Backward: gradients of sum(o * dout) w.r.t. q, k and v [C] (Changes: Q/K/V
 * gradient parity).  o and lse are the forward's outputs for the same
 * inputs (D = rowsum(dout * o) is formed from o as given); dout is read only
 * at valid query rows.  Nothing is accumulated with atomics, so dq, dk and
 * dv are deterministic.  dq, dk, dv have the shapes
 * of q, k, v; every pad row is written as +0, key/value gradients of a GQA
 * group are summed over its query heads.  workspace must be a device buffer
 * of at least thd_attn_bwd_workspace_size(args) bytes, 256-byte aligned,
 * used by this call only.  Errors: as thd_attn_fwd. */
int thd_attn_bwd(const thd_varlen_args* args, const void* q, const void* k,
                 const void* v, const void* o, const void* dout, const float* lse,
                 void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                 void* stream);

/* thd_attn_bwd with timing marks: the same validation and launches, plus
 * hipEventRecord of events[0..3] (four hipEvent_t created by the caller) on
 * `stream` around its three launches -- before the pre pass, before the dq
 * pass, before the dk/dv pass and after it -- so that a caller can time
 * each kernel on the stream it runs on.  Errors: as thd_attn_bwd, THD_ERR_NULL if
 * an event is missing, THD_ERR_HIP if recording fails. */
int thd_attn_bwd_timed(const thd_varlen_args* args, const void* q, const void* k,
                       const void* v, const void* o, const void* dout, const float* lse,
                       void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                       void* stream, void* const* events);

/* Static string naming a status code. */
const char* thd_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int thd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* THD_ATTN_H */
