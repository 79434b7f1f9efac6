// mla_cache_store.hpp -- storing one new cache row (cache-write excerpt of
// "DeepSeek-V3.2-Exp . KV cache"): the bf16 copy, and the FP8 form with one
// fp32 scale per 128 latent elements.  Used by the cache-write kernels and by
// the write step of the fused decode step.
#pragma once
#include "mla_device.hpp"

namespace mla {

// bf16 cache: 16-byte chunk ch (0..63 latent, 64..71 rotary) of new row bi
// (input row index) into cache row `row`.
__device__ __forceinline__ void store_row_chunk_bf16(const uint16_t* kv_new, const uint16_t* pe_new,
                                                     uint16_t* kv, uint16_t* pe, size_t bi,
                                                     size_t row, int ch) {
  if (ch < 64) {
    *(u32x4*)(kv + row * kC + ch * 8) = *(const u32x4*)(kv_new + bi * kC + ch * 8);
  } else {
    *(u32x4*)(pe + row * kR + (ch - 64) * 8) = *(const u32x4*)(pe_new + bi * kR + (ch - 64) * 8);
  }
}

// FP8 cache: 128-element block blk of new row bi, one wavefront (each lane
// quantises two elements).  scale = amax / 448 and x / scale are IEEE fp32
// divisions; the encoder rounds to nearest even and saturates; a zero block
// gets scale 0 and codes 0.  Block 0 also copies the rotary row.
__device__ __forceinline__ void store_row_block_fp8(const uint16_t* kv_new, const uint16_t* pe_new,
                                                    uint8_t* kv, float* kv_scale, uint16_t* pe,
                                                    size_t bi, size_t row, int blk, int lane) {
  const uint32_t x2 = *(const uint32_t*)(kv_new + bi * kC + blk * kBlk + 2 * lane);
  const float x0 = bf_lo(x2), x1 = bf_hi(x2);
  const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
  const float scale = amax / 448.0f;
  uint32_t c0 = 0, c1 = 0;
  if (scale != 0.0f) {
    c0 = f32_to_e4m3fn(x0 / scale);
    c1 = f32_to_e4m3fn(x1 / scale);
  }
  *(uint16_t*)(kv + row * kC + blk * kBlk + 2 * lane) = (uint16_t)(c0 | (c1 << 8));
  if (lane == 0) kv_scale[row * 4 + blk] = scale;
  if (blk == 0 && lane < 8) *(u32x4*)(pe + row * kR + lane * 8) = *(const u32x4*)(pe_new + bi * kR + lane * 8);
}

}  // namespace mla
