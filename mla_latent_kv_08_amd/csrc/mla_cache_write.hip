// mla_cache_write.hip -- store new latent and rotary rows in the caches
// (cache-write excerpt of "DeepSeek-V3.2-Exp . KV cache"), optionally as
// E4M3FN codes with one fp32 scale per 128 latent elements.
#include "mla_cache_store.hpp"
#include "mla_device.hpp"
#include "mla_launch.hpp"

namespace mla {

// bf16 cache: one thread per 16-byte chunk of a new row (64 latent + 8 rotary).
__global__ __launch_bounds__(256) void cache_write_bf16_kernel(
    const uint16_t* __restrict__ kv_new, const uint16_t* __restrict__ pe_new,
    const int32_t* __restrict__ start_pos, uint16_t* __restrict__ kv, uint16_t* __restrict__ pe,
    int B, int s, int T) {
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long total = (long long)B * s * 72;
  if (gid >= total) return;
  const int ch = (int)(gid % 72);
  const long long bi = gid / 72;
  const int b = (int)(bi / s), i = (int)(bi % s);
  const long long r = (long long)start_pos[b] + i;
  if (r < 0 || r >= T) return;
  store_row_chunk_bf16(kv_new, pe_new, kv, pe, (size_t)bi, (size_t)b * T + (size_t)r, ch);
}

// FP8 cache: one wavefront per (sequence, new row, 128-element block).
__global__ __launch_bounds__(256) void cache_write_fp8_kernel(
    const uint16_t* __restrict__ kv_new, const uint16_t* __restrict__ pe_new,
    const int32_t* __restrict__ start_pos, uint8_t* __restrict__ kv, float* __restrict__ kv_scale,
    uint16_t* __restrict__ pe, int B, int s, int T) {
  const long long wid = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const long long total = (long long)B * s * 4;
  if (wid >= total) return;
  const int blk = (int)(wid & 3);
  const long long bi = wid >> 2;
  const int b = (int)(bi / s), i = (int)(bi % s);
  const long long r = (long long)start_pos[b] + i;
  if (r < 0 || r >= T) return;  // uniform per wave
  store_row_block_fp8(kv_new, pe_new, kv, kv_scale, pe, (size_t)bi, (size_t)b * T + (size_t)r, blk, lane);
}

hipError_t launch_cache_write(const mla_params& p, const CacheWriteArgs& c, hipStream_t stream) {
  const int B = p.batch, s = p.seqlen_q, T = p.max_seq_len;
  hipEvent_t const* ev = (hipEvent_t const*)p.trace_events;
  if (p.kv_dtype == MLA_KV_FP8_E4M3_B128) {
    const long long waves = (long long)B * s * 4;
    const unsigned blocks = (unsigned)((waves + 3) / 4);
    return launch_kernel(cache_write_fp8_kernel, dim3(blocks), dim3(256), stream, ev,
                         (const uint16_t*)c.kv_new, (const uint16_t*)c.pe_new, c.start_pos,
                         (uint8_t*)c.kv_cache, c.kv_scale, (uint16_t*)c.pe_cache, B, s, T);
  }
  const long long threads = (long long)B * s * 72;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  return launch_kernel(cache_write_bf16_kernel, dim3(blocks), dim3(256), stream, ev,
                       (const uint16_t*)c.kv_new, (const uint16_t*)c.pe_new, c.start_pos,
                       (uint16_t*)c.kv_cache, (uint16_t*)c.pe_cache, B, s, T);
}

}  // namespace mla
