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

constexpr int kOpWaves = 4;      // waves per workgroup, one per SIMD
constexpr int kOpKT = 64;        // k per tile: four 16-wide MFMA steps, 128 bytes per row
constexpr int kOpSlots = 4;      // tiles in each wave's ring (three in flight)
constexpr int kOpOperand = 32 * kOpKT * 2;   // 4 KB: 32 rows x 64 k, bf16
constexpr int kOpSlot = 2 * kOpOperand;      // w tile then x tile

// grid (ceil(N / 32), ceil(M / 32)), 256 threads.  Workgroup (i, j) computes
// the 32 x 32 block y[32 j ..][32 i ..].  The k range is cut into tiles of 64;
// wave v takes tiles v, v + 4, ... and streams each one (32 rows of w, 32
// tokens of x) into its own ring of LDS slots with direct-to-LDS loads, three
// tiles ahead: every 1 KB load covers 8 rows x 128 contiguous bytes.  In LDS a
// row's 16-byte chunk c sits at c ^ ((row >> 1) & 7), so the MFMA operand
// reads (16 rows per LDS cycle, one chunk each) hit distinct banks.  Per
// tile: four 32x32x16 MFMAs with A = w rows (lane l: row l % 32, 8 k at
// 16 step + 8 (l / 32)) and B = x rows (the same k of token l % 32) into
// one 32 x 32 block D[n][m].  No wave waits for another until the four
// partial blocks are summed in LDS and rounded to bf16 once.  K is a multiple
// of 64; rows past N and tokens past M read the last row and are not stored.
__global__ __launch_bounds__(64 * kOpWaves) void oproj_kernel(const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ w,
                                                              uint16_t* __restrict__ y, int M, int N,
                                                              int K) {
  __shared__ __attribute__((aligned(16))) char lds[kOpWaves][kOpSlots][kOpSlot];  // 128 KB
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * 32, m0 = blockIdx.y * 32;
  const int nt = K / kOpKT;
  const int mine = nt > wave ? (nt - wave + kOpWaves - 1) / kOpWaves : 0;  // tiles of this wave
  // Load q (0..3) of an operand tile covers rows 8 q .. 8 q + 7: lane l takes
  // row 8 q + l / 8 and stores LDS chunk l % 8, i.e. global chunk
  // (l % 8) ^ ((row >> 1) & 7) of that row.
  const int lr = lane >> 3, lc = lane & 7;
  const uint16_t* wsrc[4];
  const uint16_t* xsrc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 8 * q + lr, gc = lc ^ ((r >> 1) & 7);
    wsrc[q] = w + (size_t)min(n0 + r, N - 1) * K + 8 * gc;
    xsrc[q] = x + (size_t)min(m0 + r, M - 1) * K + 8 * gc;
  }
  auto issue = [&](int i) {  // the wave's i-th tile (global tile wave + 4 i) into slot i % 4
    const size_t k0 = (size_t)(wave + kOpWaves * i) * kOpKT;
    uint32_t base = lds_addr(lds[wave][i % kOpSlots]);
    base = __builtin_amdgcn_readfirstlane(base);
    lds_dma16<0>(wsrc[0] + k0, base);
    lds_dma16<1024>(wsrc[1] + k0, base);
    lds_dma16<2048>(wsrc[2] + k0, base);
    lds_dma16<3072>(wsrc[3] + k0, base);
    lds_dma16<kOpOperand>(xsrc[0] + k0, base);
    lds_dma16<kOpOperand + 1024>(xsrc[1] + k0, base);
    lds_dma16<kOpOperand + 2048>(xsrc[2] + k0, base);
    lds_dma16<kOpOperand + 3072>(xsrc[3] + k0, base);
  };
  // operand read offsets (bytes in a slot) of the four k-steps
  const int r = lane & 31, g = lane >> 5;
  int roff[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) roff[st] = r * (kOpKT * 2) + (((2 * st + g) ^ ((r >> 1) & 7)) << 4);

  f32x16 acc = {};
  const int pre = mine < kOpSlots - 1 ? mine : kOpSlots - 1;
  for (int i = 0; i < pre; ++i) issue(i);
  for (int i = 0; i < mine; ++i) {
    // tile i has landed once at most the loads of the tiles issued after it remain
    const int after = min(mine - 1, i + kOpSlots - 2) - i;  // 0, 1 or 2 tiles
    if (after >= 2) MLA_WAIT_VMCNT(16);
    else if (after == 1) MLA_WAIT_VMCNT(8);
    else MLA_WAIT_VMCNT(0);
    const char* slot = lds[wave][i % kOpSlots];
    u32x4 a[4], b[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      a[st] = *(const u32x4*)(slot + roff[st]);
      b[st] = *(const u32x4*)(slot + kOpOperand + roff[st]);
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) acc = mfma32(a[st], b[st], acc);
    // the slot refilled next held tile i - 1, whose operands are in registers
    if (i + kOpSlots - 1 < mine) issue(i + kOpSlots - 1);
  }
  __syncthreads();  // every wave's ring is drained and read: reuse the LDS
  float(*red)[16][64] = (float(*)[16][64])lds;
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
