// mla_cache_write.hip -- store new latent and rotary rows in the caches
// (cache-write excerpt of "DeepSeek-V3.2-Exp . KV cache"), optionally as
// E4M3FN codes with one fp32 scale per 128 latent elements.
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
  const size_t row = (size_t)b * T + (size_t)r;
  if (ch < 64) {
    *(u32x4*)(kv + row * kC + ch * 8) = *(const u32x4*)(kv_new + (size_t)bi * kC + ch * 8);
  } else {
    *(u32x4*)(pe + row * kR + (ch - 64) * 8) = *(const u32x4*)(pe_new + (size_t)bi * kR + (ch - 64) * 8);
  }
}

// FP8 cache: one wavefront per (sequence, new row, 128-element block); each lane
// quantises two elements.  scale = amax / 448 and x / scale are IEEE fp32
// divisions; the encoder rounds to nearest even and saturates.
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
  const size_t row = (size_t)b * T + (size_t)r;
  const uint32_t x2 = *(const uint32_t*)(kv_new + (size_t)bi * kC + blk * kBlk + 2 * lane);
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
  if (blk == 0 && lane < 8)
    *(u32x4*)(pe + row * kR + lane * 8) = *(const u32x4*)(pe_new + (size_t)bi * kR + lane * 8);
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
