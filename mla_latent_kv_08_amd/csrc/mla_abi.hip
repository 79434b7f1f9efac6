// mla_abi.hip -- the extern "C" entry points declared in include/mla.h:
// host-side argument checks, workspace sizing and status reporting.  Every
// check runs before the first HIP call, so a rejected call enqueues nothing.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "mla.h"
#include "mla_launch.hpp"
#include "mla_plan.hpp"

// Static device scratch of mla_decode_noalloc: the workspace of one call, in
// a file-scope device array each GPU holds from the library's first use on it
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: its device address on each GPU comes from
// hipGetSymbolAddress (once per device, with that device current) and only
// that address is ever passed to a kernel.
static __device__ __align__(256) char scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_last_error[256] = "";

mla_status fail(mla_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

mla_status ok() {
  g_last_error[0] = '\0';
  return MLA_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Checks shared by both entry points.
mla_status check_params(const mla_params* p) {
  if (!p) return fail(MLA_ERR_INVALID_ARG, "params is NULL");
  if (p->kv_lora_rank != MLA_KV_LORA_RANK || p->qk_nope_dim != MLA_QK_NOPE_DIM ||
      p->qk_rope_dim != MLA_QK_ROPE_DIM || p->v_head_dim != MLA_V_HEAD_DIM)
    return fail(MLA_ERR_UNSUPPORTED,
                "widths (kv_lora_rank, qk_nope, qk_rope, v) = (%d, %d, %d, %d); this build "
                "implements (512, 128, 64, 128)",
                p->kv_lora_rank, p->qk_nope_dim, p->qk_rope_dim, p->v_head_dim);
  if (p->batch < 0) return fail(MLA_ERR_INVALID_ARG, "batch = %d < 0", p->batch);
  if (p->max_seq_len < 1) return fail(MLA_ERR_INVALID_ARG, "max_seq_len = %d < 1", p->max_seq_len);
  if (p->kv_dtype != MLA_KV_BF16 && p->kv_dtype != MLA_KV_FP8_E4M3_B128)
    return fail(MLA_ERR_INVALID_ARG, "unknown kv_dtype %d", p->kv_dtype);
  // cache element offsets must fit the kernels' 64-bit row arithmetic and a
  // 32-bit row index per sequence
  if ((long long)p->batch * p->max_seq_len > (1LL << 40))
    return fail(MLA_ERR_INVALID_ARG, "batch * max_seq_len too large");
  return MLA_OK;
}

// Checks of the decode shape, shared by mla_decode_workspace_size and the
// decode entry points (the plan is only formed for shapes that pass them).
mla_status check_decode_shape(const mla_params* p) {
  if (p->seqlen_q < 1) return fail(MLA_ERR_INVALID_ARG, "seqlen_q = %d < 1", p->seqlen_q);
  if (p->num_heads < 1 || p->num_heads > MLA_MAX_HEADS)
    return fail(MLA_ERR_INVALID_ARG, "num_heads = %d outside 1..128", p->num_heads);
  if (p->topk < 0 || p->topk > p->max_seq_len)
    return fail(MLA_ERR_INVALID_ARG, "topk = %d outside 0..max_seq_len", p->topk);
  if ((long long)p->batch * p->seqlen_q > 65535)
    return fail(MLA_ERR_UNSUPPORTED, "batch * seqlen_q > 65535 query tokens");
  return MLA_OK;
}

}  // namespace

extern "C" {

const char* mla_status_string(mla_status s) {
  // A C caller may pass any int: read the argument's bits as an int, since
  // loading an out-of-range value as the C++ enum would be undefined.
  int v;
  memcpy(&v, &s, sizeof v);
  switch (v) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG: invalid argument";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: not implemented by this build";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace missing or too small";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: HIP runtime error";
  }
  return "unknown mla_status";
}

const char* mla_last_error(void) { return g_last_error; }

int mla_abi_version(void) { return MLA_ABI_VERSION; }

mla_status mla_cache_write(const mla_params* p, const void* kv_new, const void* pe_new,
                           const int32_t* start_pos, void* kv_cache, float* kv_scale,
                           void* pe_cache, void* stream) {
  mla_status st = check_params(p);
  if (st != MLA_OK) return st;
  if (p->seqlen_q < 0) return fail(MLA_ERR_INVALID_ARG, "seqlen_q = %d < 0", p->seqlen_q);
  if (p->batch == 0 || p->seqlen_q == 0) return ok();
  if ((long long)p->batch * p->seqlen_q > 0x7FFFFFFFLL)
    return fail(MLA_ERR_INVALID_ARG, "batch * seqlen_q exceeds 2^31 - 1 rows");
  const bool fp8 = p->kv_dtype == MLA_KV_FP8_E4M3_B128;
  if (!kv_new || !pe_new || !start_pos || !kv_cache || !pe_cache)
    return fail(MLA_ERR_INVALID_ARG, "a required tensor pointer is NULL");
  if (fp8 != (kv_scale != nullptr))
    return fail(MLA_ERR_INVALID_ARG, fp8 ? "FP8 cache needs kv_scale" : "kv_scale must be NULL for a bf16 cache");
  if (!aligned(kv_new, 16) || !aligned(pe_new, 16) || !aligned(kv_cache, 16) || !aligned(pe_cache, 16))
    return fail(MLA_ERR_INVALID_ARG, "bf16/uint8 tensors must be 16-byte aligned");
  if (!aligned(start_pos, 4) || (kv_scale && !aligned(kv_scale, 4)))
    return fail(MLA_ERR_INVALID_ARG, "int32/fp32 tensors must be 4-byte aligned");
  mla::CacheWriteArgs c{kv_new, pe_new, start_pos, kv_cache, kv_scale, pe_cache};
  const hipError_t e = mla::launch_cache_write(*p, c, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "HIP: %s", hipGetErrorString(e));
  return ok();
}

mla_status mla_decode_workspace_size(const mla_params* p, size_t* bytes) {
  mla_status st = check_params(p);
  if (st != MLA_OK) return st;
  if (!bytes) return fail(MLA_ERR_INVALID_ARG, "bytes is NULL");
  st = check_decode_shape(p);
  if (st != MLA_OK) return st;
  const mla::DecodePlan plan = mla::make_decode_plan(*p);
  if (plan.max_groups > 0x7FFFFFFFLL || plan.max_groups * plan.heads_padded > (1LL << 40))
    return fail(MLA_ERR_UNSUPPORTED, "too many attention workgroups for this batch and top-k");
  *bytes = plan.bytes;
  return ok();
}

}  // extern "C"

namespace {

// Checks of mla_decode's arguments (also those of the fused step); on success
// *plan holds the split of the call.  MLA_OK with batch == 0 means no-op.
mla_status check_decode(const mla_params* p, const void* q_nope, const void* q_pe,
                        const void* wkv_b, const void* kv_cache, const float* kv_scale,
                        const void* pe_cache, const int32_t* cache_lens, const int32_t* topk_idx,
                        void* out, void* workspace, size_t workspace_bytes, mla::DecodePlan* plan) {
  mla_status st = check_params(p);
  if (st != MLA_OK) return st;
  st = check_decode_shape(p);
  if (st != MLA_OK) return st;
  if (!(p->softmax_scale > 0.0f) || !isfinite(p->softmax_scale))
    return fail(MLA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (p->batch == 0) return MLA_OK;
  const bool fp8 = p->kv_dtype == MLA_KV_FP8_E4M3_B128;
  if (!q_nope || !q_pe || !wkv_b || !kv_cache || !pe_cache || !cache_lens || !out)
    return fail(MLA_ERR_INVALID_ARG, "a required tensor pointer is NULL");
  if (fp8 != (kv_scale != nullptr))
    return fail(MLA_ERR_INVALID_ARG, fp8 ? "FP8 cache needs kv_scale" : "kv_scale must be NULL for a bf16 cache");
  if ((p->topk > 0) != (topk_idx != nullptr))
    return fail(MLA_ERR_INVALID_ARG, p->topk > 0 ? "topk > 0 needs topk_idx" : "topk_idx given with topk = 0");
  if (!aligned(q_nope, 16) || !aligned(q_pe, 16) || !aligned(wkv_b, 16) || !aligned(kv_cache, 16) ||
      !aligned(pe_cache, 16) || !aligned(out, 16))
    return fail(MLA_ERR_INVALID_ARG, "bf16/uint8 tensors must be 16-byte aligned");
  if (!aligned(cache_lens, 4) || (kv_scale && !aligned(kv_scale, 4)) || (topk_idx && !aligned(topk_idx, 4)))
    return fail(MLA_ERR_INVALID_ARG, "int32/fp32 tensors must be 4-byte aligned");
  *plan = mla::make_decode_plan(*p);
  if (plan->max_groups > 0x7FFFFFFFLL || plan->max_groups * plan->heads_padded > (1LL << 40))
    return fail(MLA_ERR_UNSUPPORTED, "too many attention workgroups for this batch and top-k");
  if (!workspace || workspace_bytes < plan->bytes)
    return fail(MLA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", plan->bytes,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 16)) return fail(MLA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  return MLA_OK;
}

constexpr size_t kScratchBytes = (size_t)MLA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of `scratch` on the current device (looked up on the first
// call on that device); NULL with the status in *st on failure.
void* scratch_on_current_device(mla_status* st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *st = fail(MLA_ERR_HIP, "HIP: %s", hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *st = fail(MLA_ERR_UNSUPPORTED, "device %d: the static scratch covers devices 0..%d", dev,
               kMaxDevices - 1);
    return nullptr;
  }
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!ptr) {
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      *st = fail(MLA_ERR_HIP, "HIP: hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

}  // namespace

extern "C" {

mla_status mla_decode(const mla_params* p, const void* q_nope, const void* q_pe,
                      const void* wkv_b, const void* kv_cache, const float* kv_scale,
                      const void* pe_cache, const int32_t* cache_lens, const int32_t* topk_idx,
                      void* out, void* workspace, size_t workspace_bytes, void* stream) {
  mla::DecodePlan plan;
  mla_status st = check_decode(p, q_nope, q_pe, wkv_b, kv_cache, kv_scale, pe_cache, cache_lens,
                               topk_idx, out, workspace, workspace_bytes, &plan);
  if (st != MLA_OK || p->batch == 0) return st == MLA_OK ? ok() : st;
  mla::DecodeArgs d{q_nope, q_pe, wkv_b, kv_cache, kv_scale, pe_cache, cache_lens, topk_idx, out, workspace};
  const hipError_t e = mla::launch_decode(*p, d, nullptr, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "HIP: %s", hipGetErrorString(e));
  return ok();
}

mla_status mla_decode_step(const mla_params* p, const void* kv_new, const void* pe_new,
                           const void* q_nope, const void* q_pe, const void* wkv_b,
                           void* kv_cache, float* kv_scale, void* pe_cache,
                           const int32_t* cache_lens, const int32_t* topk_idx, void* out,
                           void* workspace, size_t workspace_bytes, void* stream) {
  mla::DecodePlan plan;
  mla_status st = check_decode(p, q_nope, q_pe, wkv_b, kv_cache, kv_scale, pe_cache, cache_lens,
                               topk_idx, out, workspace, workspace_bytes, &plan);
  if (st != MLA_OK || p->batch == 0) return st == MLA_OK ? ok() : st;
  if (!kv_new || !pe_new) return fail(MLA_ERR_INVALID_ARG, "a required tensor pointer is NULL");
  if (!aligned(kv_new, 16) || !aligned(pe_new, 16))
    return fail(MLA_ERR_INVALID_ARG, "bf16/uint8 tensors must be 16-byte aligned");
  mla::DecodeArgs d{q_nope, q_pe, wkv_b, kv_cache, kv_scale, pe_cache, cache_lens, topk_idx, out, workspace};
  mla::CacheWriteArgs c{kv_new, pe_new, nullptr, kv_cache, kv_scale, pe_cache};
  const hipError_t e = mla::launch_decode(*p, d, &c, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "HIP: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

extern "C" {

mla_status mla_decode_latent(const mla_params* p, const void* q_nope, const void* q_pe,
                             const void* wkv_b, const void* kv_cache, const float* kv_scale,
                             const void* pe_cache, const int32_t* cache_lens, const int32_t* topk_idx,
                             void* o_lat, void* workspace, size_t workspace_bytes, void* stream) {
  mla::DecodePlan plan;
  mla_status st = check_decode(p, q_nope, q_pe, wkv_b, kv_cache, kv_scale, pe_cache, cache_lens,
                               topk_idx, o_lat, workspace, workspace_bytes, &plan);
  if (st != MLA_OK || p->batch == 0) return st == MLA_OK ? ok() : st;
  mla::DecodeArgs d{q_nope, q_pe, wkv_b, kv_cache, kv_scale, pe_cache, cache_lens, topk_idx, nullptr, workspace};
  const hipError_t e = mla::launch_decode(*p, d, nullptr, (hipStream_t)stream, o_lat);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "HIP: %s", hipGetErrorString(e));
  return ok();
}

mla_status mla_output_projection(const mla_params* p, int32_t d_model, int32_t kind, const void* x,
                                 const void* w, void* y, void* stream) {
  mla_status st = check_params(p);
  if (st != MLA_OK) return st;
  st = check_decode_shape(p);
  if (st != MLA_OK) return st;
  if (kind != MLA_OPROJ_WO && kind != MLA_OPROJ_WOV)
    return fail(MLA_ERR_INVALID_ARG, "unknown output projection kind %d", kind);
  if (d_model < 1 || d_model > (1 << 20))
    return fail(MLA_ERR_INVALID_ARG, "d_model = %d outside 1..2^20", d_model);
  if (p->batch == 0) return ok();
  if (!x || !w || !y) return fail(MLA_ERR_INVALID_ARG, "a required tensor pointer is NULL");
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16))
    return fail(MLA_ERR_INVALID_ARG, "bf16 tensors must be 16-byte aligned");
  const int M = p->batch * p->seqlen_q;
  const int K = p->num_heads * (kind == MLA_OPROJ_WO ? MLA_V_HEAD_DIM : MLA_KV_LORA_RANK);
  const hipError_t e = mla::launch_output_projection(x, w, y, M, d_model, K, (hipStream_t)stream,
                                                     (hipEvent_t const*)p->trace_events);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "HIP: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

extern "C" {

mla_status mla_decode_noalloc(const mla_params* p, const void* q_nope, const void* q_pe,
                              const void* wkv_b, const void* kv_cache, const float* kv_scale,
                              const void* pe_cache, const int32_t* cache_lens,
                              const int32_t* topk_idx, void* out, void* stream) {
  // validate against the scratch size first (no HIP call for a rejected call);
  // any non-null 16-byte aligned value stands for the scratch in this check
  mla::DecodePlan plan;
  mla_status st = check_decode(p, q_nope, q_pe, wkv_b, kv_cache, kv_scale, pe_cache, cache_lens,
                               topk_idx, out, (void*)(uintptr_t)256, kScratchBytes, &plan);
  if (st == MLA_ERR_WORKSPACE)
    return fail(MLA_ERR_WORKSPACE, "this call needs %zu bytes of scratch; the static scratch holds %zu",
                plan.bytes, kScratchBytes);
  if (st != MLA_OK || p->batch == 0) return st == MLA_OK ? ok() : st;
  void* ws = scratch_on_current_device(&st);
  if (!ws) return st;
  mla::DecodeArgs d{q_nope, q_pe, wkv_b, kv_cache, kv_scale, pe_cache, cache_lens, topk_idx, out, ws};
  const hipError_t e = mla::launch_decode(*p, d, nullptr, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "HIP: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
