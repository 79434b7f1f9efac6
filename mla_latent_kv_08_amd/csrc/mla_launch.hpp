// mla_launch.hpp -- internal interface between the C ABI (argument checks)
// and the kernel launchers.  Arguments reaching here have been validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla.h"

namespace mla {

struct DecodeArgs {
  const void* q_nope;
  const void* q_pe;
  const void* wkv_b;
  const void* kv_cache;
  const float* kv_scale;
  const void* pe_cache;
  const int32_t* cache_lens;
  const int32_t* topk_idx;
  void* out;
  void* workspace;
};

struct CacheWriteArgs {
  const void* kv_new;
  const void* pe_new;
  const int32_t* start_pos;
  void* kv_cache;
  float* kv_scale;
  void* pe_cache;
};

hipError_t launch_decode(const mla_params& p, const DecodeArgs& d, hipStream_t stream);
hipError_t launch_cache_write(const mla_params& p, const CacheWriteArgs& c, hipStream_t stream);

}  // namespace mla
