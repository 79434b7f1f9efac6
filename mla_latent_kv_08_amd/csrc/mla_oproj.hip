// mla_oproj.hip -- the output projection that follows the decode on gfx950:
// y[m][n] = sum_k x[m][k] w[n][k] for the decode batch's tokens m.
//
// With x the heads' up-projected outputs (feature 128 h + d) and w = W_O it is
// the layer output of the MLA article's section 5 (W_O after the value
// up-projection); with x the latent outputs (feature 512 h + c) and w the
// fused W_OV = W_O W_UV of its section 4, the same output without the
// up-projection.  A decode batch has few tokens, so the kernel streams the
// weight once from HBM: HBM-bound, M x N x K x 2 FLOPs being negligible next
// to its N x K x 2 bytes.
#include "mla_device.hpp"
#include "mla_launch.hpp"

namespace mla {

constexpr int kOpWaves = 8;      // waves per workgroup (two per SIMD)
constexpr int kOpChunk = 64;     // k per chunk: four 16-wide MFMA steps
constexpr int kOpUnroll = 4;     // chunks whose loads a wave issues before their MFMAs

// grid (ceil(N / 32), ceil(M / 32)), 512 threads.  Workgroup (i, j) computes
// the 32 x 32 block y[32 j ..][32 i ..]: wave w takes the k chunks w, w + 8,
// ... and accumulates A = w rows (lane l: row 32 i + l % 32, 8 consecutive k
// at 16 step + 8 (l / 32)) times B = x rows (the same k of token 32 j + l %
// 32) in one 32 x 32 block (D[n][m]); the eight partial blocks are summed in
// LDS and rounded to bf16 once.  K is a multiple of 64; rows past N and
// tokens past M read the last row instead and are not stored.
__global__ __launch_bounds__(64 * kOpWaves) void oproj_kernel(const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ w,
                                                              uint16_t* __restrict__ y, int M, int N,
                                                              int K) {
  __shared__ float red[kOpWaves][16][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * 32, m0 = blockIdx.y * 32;
  const int r = lane & 31, g = lane >> 5;
  const int wrow = min(n0 + r, N - 1), xrow = min(m0 + r, M - 1);
  const uint16_t* wp = w + (size_t)wrow * K + 8 * g;
  const uint16_t* xp = x + (size_t)xrow * K + 8 * g;
  const int nc = K / kOpChunk;
  f32x16 acc = {};
  for (int c0 = wave; c0 < nc; c0 += kOpWaves * kOpUnroll) {
    u32x4 a[kOpUnroll][4], b[kOpUnroll][4];
#pragma unroll
    for (int u = 0; u < kOpUnroll; ++u) {
      const int c = c0 + kOpWaves * u;
      if (c < nc) {  // wave-uniform
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          a[u][s] = __builtin_nontemporal_load((const u32x4*)(wp + (size_t)c * kOpChunk + 16 * s));
          b[u][s] = *(const u32x4*)(xp + (size_t)c * kOpChunk + 16 * s);
        }
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) a[u][s] = b[u][s] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < kOpUnroll; ++u) {
#pragma unroll
      for (int s = 0; s < 4; ++s) acc = mfma32(a[u][s], b[u][s], acc);
    }
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) red[wave][e][lane] = acc[e];
  __syncthreads();
  // output (e, l): token m0 + l % 32, row n0 + 8 (e / 4) + 4 (l / 32) + e % 4
  for (int o = tid; o < 16 * 64; o += 64 * kOpWaves) {
    const int e = o >> 6, l = o & 63;
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < kOpWaves; ++k) v += red[k][e][l];
    const int m = m0 + (l & 31), n = n0 + 8 * (e >> 2) + 4 * (l >> 5) + (e & 3);
    if (m < M && n < N) y[(size_t)m * N + n] = (uint16_t)f2bf(v);
  }
}

hipError_t launch_output_projection(const void* x, const void* w, void* y, int M, int N, int K,
                                    hipStream_t stream, hipEvent_t const* ev) {
  const dim3 grid((unsigned)((N + 31) / 32), (unsigned)((M + 31) / 32));
  return launch_kernel(oproj_kernel, grid, dim3(64 * kOpWaves), stream, ev, (const uint16_t*)x,
                       (const uint16_t*)w, (uint16_t*)y, M, N, K);
}

}  // namespace mla
