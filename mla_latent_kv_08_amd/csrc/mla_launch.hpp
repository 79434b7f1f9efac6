// mla_launch.hpp -- internal interface between the C ABI (argument checks)
// and the kernel launchers.  Arguments reaching here have been validated.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>

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

// With `write` non-null (the fused decode step) the new row of each sequence is
// stored at position cache_lens[b] - 1 before the attention reads the caches.
// With `latent_out` non-null the combine writes the latent output
// [B][s][H][512] there and the up-projection is not launched (d.out unused).
hipError_t launch_decode(const mla_params& p, const DecodeArgs& d, const CacheWriteArgs* write,
                         hipStream_t stream, void* latent_out = nullptr);

// y[m][n] = sum_k x[m][k] w[n][k], bf16 in and out (fp32 accumulation);
// K a multiple of 64.
hipError_t launch_output_projection(const void* x, const void* w, void* y, int M, int N, int K,
                                    hipStream_t stream, hipEvent_t const* ev);

// Launch `kernel` on `stream` and return the launch's own status (not the
// thread's last error, which an earlier unrelated HIP call may have left).
// With `ev` non-null the start and end of the dispatch are stamped into ev[0]
// and ev[1] by the dispatch itself (no extra queue packets, so the elapsed
// time is the kernel's own duration).
template <typename... KArgs, typename... Args>
hipError_t launch_kernel_lds(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds_bytes,
                             hipStream_t stream, hipEvent_t const* ev, Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count of the kernel");
  // each argument converted to the kernel's parameter type, then passed by address
  std::tuple<KArgs...> vals{static_cast<KArgs>(args)...};
  return std::apply(
      [&](auto&... v) -> hipError_t {
        void* ptrs[] = {(void*)&v...};
        if (ev)
          return hipExtLaunchKernel((const void*)kernel, grid, block, ptrs, lds_bytes, stream, ev[0],
                                    ev[1], 0);
        return hipLaunchKernel((const void*)kernel, grid, block, ptrs, lds_bytes, stream);
      },
      vals);
}
template <typename... KArgs, typename... Args>
hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                         hipEvent_t const* ev, Args... args) {
  return launch_kernel_lds(kernel, grid, block, 0, stream, ev, args...);
}
hipError_t launch_cache_write(const mla_params& p, const CacheWriteArgs& c, hipStream_t stream);

}  // namespace mla
