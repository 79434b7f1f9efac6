/*
 * mla.h -- C ABI of the MI355X (gfx950) weight-absorbed MLA decode library.
 *
 * The operation is Multi-Head Latent Attention decode in its weight-absorbed
 * ("MQA decode") form over a compressed KV cache, as described on the pages
 * "DeepSeek-V3.2-Exp . KV cache" (decode view: the cache-write excerpt and the
 * "MQA decode" excerpt) and "DeepSeek MLA Architecture: How Multi-Head Latent
 * Attention Cuts KV Cache by 93%" (section 3, decoupled RoPE; section 4, the
 * absorption identities).  Each cached position holds a 512-wide normalised
 * latent c_KV and a 64-wide rotary key k_R shared by all heads.
 *
 * Conventions for every entry point
 *  - Tensor arguments are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or keeps them.  bf16 tensors are raw 16-bit
 *    patterns.  All tensors are dense row-major with the shapes given below.
 *    Pointers to bf16/uint8 tensors must be 16-byte aligned; int32/fp32
 *    tensors 4-byte aligned.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    work is enqueued asynchronously on it; no call synchronises the device,
 *    calls hipMalloc/hipMemset, or blocks the host.  The calls are safe to
 *    record into a HIP graph.
 *  - Host-side argument checks run before any HIP call; on failure nothing is
 *    enqueued and the status says why (mla_last_error() gives a detail text
 *    for the calling thread).  A launch failure returns MLA_ERR_HIP; the
 *    status is that launch's own, not an error an earlier HIP call left on
 *    the thread.  A call that launches several kernels (mla_decode,
 *    mla_decode_step) and fails at its k-th launch leaves kernels 0..k-1
 *    enqueued on the stream: the output is then undefined, and the caller
 *    should treat the stream as failed.
 *  - Calls from several host threads are safe; calls that write the same
 *    buffers must be ordered by the caller (same stream or events).
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 2: adds mla_decode_latent, mla_output_projection and mla_decode_noalloc;
 * the entry points and mla_params of version 1 are unchanged. */
#define MLA_ABI_VERSION 2

/* Fixed widths of the DeepSeek-V3 MLA layer (checked in mla_params). */
#define MLA_KV_LORA_RANK 512 /* latent width C */
#define MLA_QK_ROPE_DIM 64   /* rotary key width R */
#define MLA_QK_NOPE_DIM 128  /* per-head non-rotary query/key width Dn */
#define MLA_V_HEAD_DIM 128   /* per-head value width Dv */
#define MLA_FP8_BLOCK 128    /* latent elements per FP8 scale */
#define MLA_MAX_HEADS 128

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size or dimension */
  MLA_ERR_UNSUPPORTED = 2, /* a valid request this build does not implement */
  MLA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  MLA_ERR_HIP = 4          /* the HIP runtime reported an error */
} mla_status;

typedef enum mla_kv_dtype {
  MLA_KV_BF16 = 0,         /* latent cache holds bf16 values */
  MLA_KV_FP8_E4M3_B128 = 1 /* latent cache holds OCP E4M3FN codes, one fp32
                              scale per 128 contiguous latent elements */
} mla_kv_dtype;

/*
 * Problem description, passed by pointer (host memory, read during the call).
 *   batch         B >= 0 sequences (B == 0 is a no-op)
 *   seqlen_q      s: new rows per sequence for mla_cache_write (>= 0);
 *                 query tokens per sequence for mla_decode / mla_decode_step
 *                 (>= 1, batch * s <= 65535): the s tokens are the last s
 *                 cached positions of the sequence, and token i (0-based)
 *                 sees the rows up to its own, t < end_b - (s - 1 - i).
 *                 With a dense selection and s * num_heads <= 128 the s
 *                 tokens share the reads and the score work of each cache
 *                 tile
 *   num_heads     H, 1..128 (the local heads of this GPU)
 *   max_seq_len   T: second dimension of every cache buffer, >= 1
 *   kv_lora_rank, qk_nope_dim, qk_rope_dim, v_head_dim: must be 512, 128, 64, 128
 *   kv_dtype      an mla_kv_dtype
 *   topk          0: dense attention over [0, cache_lens[b]);
 *                 k > 0: entries per sequence of topk_idx (k <= T)
 *   softmax_scale multiplier of the logits, finite and > 0 (1/sqrt(192) for
 *                 DeepSeek-V3; a YaRN correction is folded in by the caller)
 *   trace_events  optional instrumentation, normally NULL.  Otherwise an array
 *                 of hipEvent_t (as void*, created with timing enabled):
 *                 events[2k] and events[2k+1] receive the start and end time
 *                 of mla_decode's k-th kernel (k = 0 absorb, 1 attention,
 *                 2 combine, 3 up-projection; 8 events), stamped by the kernel
 *                 dispatch itself (hipExtLaunchKernel), so their elapsed time
 *                 is the kernel's duration; mla_cache_write uses events[0]
 *                 and events[1] for its kernel.
 */
typedef struct mla_params {
  int32_t batch;
  int32_t seqlen_q;
  int32_t num_heads;
  int32_t max_seq_len;
  int32_t kv_lora_rank;
  int32_t qk_nope_dim;
  int32_t qk_rope_dim;
  int32_t v_head_dim;
  int32_t kv_dtype;
  int32_t topk;
  float softmax_scale;
  int32_t reserved;
  void* const* trace_events;
} mla_params;

/*
 * mla_cache_write -- store new rows in the latent and rotary caches.
 *
 * Follows the cache-write excerpt of "DeepSeek-V3.2-Exp . KV cache": rows
 * [start_pos, start_pos + s) of each sequence receive the new latent and
 * rotary rows.  With MLA_KV_FP8_E4M3_B128 the latent is stored in the form the
 * page says deployment uses: per block of 128 contiguous latent elements,
 *   scale = max|x| / 448            (fp32, IEEE division)
 *   code  = E4M3FN(x / scale)       (fp32 IEEE division, round to nearest
 *                                    even, saturating to +-448, sign of zero
 *                                    kept; a block with scale 0 gets code 0)
 * and the page's decode-side value is bf16(float(code) * scale).
 *
 *   kv_new     bf16 [B][s][512]
 *   pe_new     bf16 [B][s][64]
 *   start_pos  int32 [B] (device)
 *   kv_cache   bf16 [>=B][T][512], or uint8 E4M3FN codes [>=B][T][512]
 *   kv_scale   fp32 [>=B][T][4] for the FP8 cache; must be NULL for bf16
 *   pe_cache   bf16 [>=B][T][64]
 * Rows whose index falls outside [0, T) are dropped (nothing is stored).
 */
mla_status mla_cache_write(const mla_params* p, const void* kv_new, const void* pe_new,
                           const int32_t* start_pos, void* kv_cache, float* kv_scale,
                           void* pe_cache, void* stream);

/*
 * mla_decode_workspace_size -- bytes of device workspace mla_decode needs for
 * these parameters (a pure host computation; no device is touched).
 */
mla_status mla_decode_workspace_size(const mla_params* p, size_t* bytes);

/*
 * mla_decode -- one decode step of weight-absorbed MLA for every sequence.
 *
 * Follows the "MQA decode" excerpt of "DeepSeek-V3.2-Exp . KV cache" (whose
 * einsums carry the query-token dimension s) and sections 3-4 of the MLA
 * article, per sequence b, query token i < s and head h:
 *   1. absorb:  qa[c]   = sum_d q_nope[b,i,h,d] * wkv_b[h,d,c]          (d < 128)
 *   2. score:   S[t]    = (qa . c_KV[b,t] + q_pe[b,i,h] . k_R[b,t]) * softmax_scale
 *   3. softmax over the selected positions t (dense: t < e; top-k: the set
 *      of entries of topk_idx[b,i] inside [0, e))
 *   4. reduce:  o[c]    = sum_t p[t] * c_KV[b,t,c]
 *   5. up-project: out[b,i,h,d] = sum_c o[c] * wkv_b[h,128+d,c]
 * with end_b = min(max(cache_lens[b], 0), T) and e = end_b - (s - 1 - i)
 * (e = end_b for one query token).  c_KV is the bf16 latent, or for the FP8
 * cache bf16(float(code) * scale).
 *
 *   q_nope     bf16 [B][s][H][128]
 *   q_pe       bf16 [B][s][H][64] (already rotated)
 *   wkv_b      bf16 [H][256][512]: rows 0..127 the key half W_UK, rows
 *              128..255 the value half W_UV of each head
 *   kv_cache, kv_scale, pe_cache: as for mla_cache_write
 *   cache_lens int32 [B] (device): rows 0..cache_lens[b]-1 are valid
 *   topk_idx   int32 [B][s][topk] (device) when topk > 0, else NULL: one row
 *              per query token.  Entries outside [0, e) (e.g. -1 padding)
 *              are skipped; the valid entries of a row must be distinct.
 *   out        bf16 [B][s][H][128]
 *   workspace  device scratch of at least mla_decode_workspace_size() bytes,
 *              16-byte aligned; its contents are undefined after the call.
 * A query token with no selected position gets an output row of zeros.
 */
mla_status mla_decode(const mla_params* p, const void* q_nope, const void* q_pe,
                      const void* wkv_b, const void* kv_cache, const float* kv_scale,
                      const void* pe_cache, const int32_t* cache_lens, const int32_t* topk_idx,
                      void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_decode_step -- the fused decode step: store each sequence's new latent
 * and rotary row, then attend with it included.
 *
 * A decoding token's own compressed row joins the cache before its query
 * attends ("DeepSeek-V3.2-Exp . KV cache", the cache-write and "MQA decode"
 * excerpts; MLA article section 3, the cached latent per token).  The result
 * equals mla_cache_write with the same s and start_pos[b] = cache_lens[b] - s,
 * followed by mla_decode with the same arguments, but needs no extra launch:
 * the row stores run in spare workgroups of the absorb kernel.
 *
 *   kv_new     bf16 [B][s][512]: new latent rows c_KV of each sequence
 *   pe_new     bf16 [B][s][64]:  new rotary rows k_R (already rotated)
 *   kv_cache, kv_scale, pe_cache: as for mla_cache_write, written at rows
 *              cache_lens[b] - s .. cache_lens[b] - 1 of sequence b (rows
 *              outside [0, T) are not written), then read as for mla_decode
 *   every other argument, the workspace size and the trace events: as for
 *   mla_decode (the row stores are part of kernel 0's time)
 * Checks, errors and a rejected call enqueue nothing, as for mla_decode.  Two
 * sequences must not share cache rows.
 */
mla_status mla_decode_step(const mla_params* p, const void* kv_new, const void* pe_new,
                           const void* q_nope, const void* q_pe, const void* wkv_b,
                           void* kv_cache, float* kv_scale, void* pe_cache,
                           const int32_t* cache_lens, const int32_t* topk_idx, void* out,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_decode_latent -- mla_decode without its last step: the output is the
 * latent attention output of each head, before the value up-projection.
 *
 * Steps 1-4 of mla_decode (the MLA article, section 4: the attention weights
 * multiply the cached 512-wide latents directly, and W_UV is applied after,
 * or fused offline into the output projection as W_OV = W_O W_UV):
 *   o_lat[b,i,h,c] = sum_t p[t] * c_KV[b,t,c]
 *   o_lat      bf16 [B][s][H][512] (replaces `out`)
 * Every other argument, the checks, the workspace size and the errors are
 * those of mla_decode (trace events: kernels 0-2; no kernel 3 is launched).
 */
mla_status mla_decode_latent(const mla_params* p, const void* q_nope, const void* q_pe,
                             const void* wkv_b, const void* kv_cache, const float* kv_scale,
                             const void* pe_cache, const int32_t* cache_lens, const int32_t* topk_idx,
                             void* o_lat, void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_output_projection -- the layer's output projection after the decode,
 * for the batch * seqlen_q query tokens m (MLA article, section 5: the
 * heads' outputs, concatenated, go through W_O; section 4: W_UV fused into it
 * offline, W_OV[:, 512 h .. 512 h + 511] = W_O[:, 128 h .. 128 h + 127] W_UV[h]):
 *   y[m][n] = sum_k x[m][k] * w[n][k],  n < d_model
 *   kind MLA_OPROJ_WO:  x = mla_decode's out [B][s][H][128] (k = 128 h + d),
 *                       w = W_O bf16 [d_model][H * 128]
 *   kind MLA_OPROJ_WOV: x = mla_decode_latent's o_lat [B][s][H][512]
 *                       (k = 512 h + c), w = W_OV bf16 [d_model][H * 512]
 *   y          bf16 [B][s][d_model] (fp32 accumulation, one rounding)
 * p gives batch, seqlen_q and num_heads (the other fields are checked as for
 * mla_decode); 1 <= d_model <= 2^20.  No workspace; trace events 0 and 1
 * time its one kernel.  Deterministic: the same inputs give the same bits.
 */
#define MLA_OPROJ_WO 0
#define MLA_OPROJ_WOV 1
mla_status mla_output_projection(const mla_params* p, int32_t d_model, int32_t kind, const void* x,
                                 const void* w, void* y, void* stream);

/*
 * mla_decode_noalloc -- mla_decode without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, results, checks and errors as mla_decode, minus workspace
 * and workspace_bytes.  The workspace is a static device array of
 * MLA_NOALLOC_SCRATCH_BYTES inside the library: each GPU the call runs on
 * holds one copy from the first call on it until the process ends.  The call
 * allocates nothing (no hipMalloc, no hipFree, no allocating library
 * routine); its first call on a device looks the array's address up
 * (hipGetSymbolAddress), preferably outside graph capture.
 *   - A call whose mla_decode_workspace_size exceeds the scratch size is
 *     rejected with MLA_ERR_WORKSPACE and enqueues nothing.
 *   - Every call on one GPU shares that GPU's scratch: two calls that may
 *     overlap on one GPU (concurrent streams, or host threads without an
 *     ordering between them) race and give undefined outputs.  Calls on one
 *     stream, or otherwise ordered, are safe.  The scratch keeps the last
 *     call's contents; no call relies on them.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (64u << 20) /* 64 MiB per GPU */
mla_status mla_decode_noalloc(const mla_params* p, const void* q_nope, const void* q_pe,
                              const void* wkv_b, const void* kv_cache, const float* kv_scale,
                              const void* pe_cache, const int32_t* cache_lens,
                              const int32_t* topk_idx, void* out, void* stream);

/* Static text for a status code. */
const char* mla_status_string(mla_status s);

/* Detail text of the last failing call on the calling thread ("" if none). */
const char* mla_last_error(void);

/* MLA_ABI_VERSION of the loaded library. */
int mla_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MLA_H */
