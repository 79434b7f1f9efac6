// hbm_probe.hip -- attainable HBM read bandwidth of this GPU, for the
// benchmark's reference rate (not part of the decode library).
//
// Every workgroup streams its own contiguous slice of the buffer with 16-byte
// loads, four in flight per thread, and folds what it read into one word per
// wavefront (so no load is dead).  Read-only: no write traffic competes with
// the reads, unlike a device copy.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((__vector_size__(16)));

__global__ __launch_bounds__(256) void hbm_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                       size_t per_group, uint32_t* __restrict__ sink) {
  const size_t lo = (size_t)blockIdx.x * per_group;
  const size_t hi = lo + per_group < n16 ? lo + per_group : n16;
  uint32_t acc = 0;
  size_t i = lo + threadIdx.x;
  for (; i + 3 * 256 < hi; i += 4 * 256) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + 256);
    const u32x4 c = __builtin_nontemporal_load(src + i + 512);
    const u32x4 d = __builtin_nontemporal_load(src + i + 768);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3];
    acc ^= c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^ d[3];
  }
  for (; i < hi; i += 256) {
    const u32x4 a = src[i];
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) sink[4 * blockIdx.x + (threadIdx.x >> 6)] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16, 16-byte aligned) from `src` on `stream`,
// spread over `groups` workgroups of 256 threads; `sink` (4 * groups words
// of device memory) receives one word per wavefront.  Returns the launch
// status.
extern "C" int hbm_read_probe(const void* src, size_t bytes, int groups, uint32_t* sink, void* stream) {
  if (!src || !sink || groups < 1 || bytes % 16 || (uintptr_t)src % 16) return 1;
  const size_t n16 = bytes / 16;
  size_t per = (n16 + groups - 1) / groups;
  per = (per + 1023) / 1024 * 1024;
  void* args[] = {(void*)&src, (void*)&n16, (void*)&per, (void*)&sink};
  return (int)hipLaunchKernel((const void*)hbm_read_kernel, dim3(groups), dim3(256), args, 0,
                              (hipStream_t)stream);
}
