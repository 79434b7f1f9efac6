// mla_decode.hip -- the four kernels of one weight-absorbed MLA decode step on
// gfx950, and their launcher.
//
//   absorb     qa[b,h,:] = q_nope[b,h,:] . W_UK[h]     ("MQA decode" excerpt,
//              first einsum; MLA article section 4, absorbed query)
//   attention  split-T flash decoding: scores against the latent and rotary
//              rows (second/third einsums), masked online softmax, latent
//              reduction (fourth einsum), one partial (O, m, l) per split
//   combine    log-sum-exp merge of the split partials into o[b,h,:]
//   uproj      out[b,h,:] = W_UV[h] . o[b,h,:]          (last einsum)
#include <math.h>

#include "mla_device.hpp"
#include "mla_launch.hpp"
#include "mla_plan.hpp"

namespace mla {

// ---------------------------------------------------------------------------
// absorb: grid (heads_padded, 4 column blocks of 128), 256 threads.
// Thread (cq = tid%16, dq = tid/16) keeps W_UK[h][8dq..8dq+7][c0..c0+7] in
// registers and accumulates over its 8 rows of d for every sequence; the 16
// partial sums per column are added through LDS.  Output row layout of qt:
// [absorbed q (512) | q_pe (64)] in bf16; padded heads are zero.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void absorb_kernel(const uint16_t* __restrict__ q_nope,
                                                     const uint16_t* __restrict__ q_pe,
                                                     const uint16_t* __restrict__ wkv_b,
                                                     uint16_t* __restrict__ qt, int B, int H,
                                                     int Hp) {
  const int h = blockIdx.x, cblk = blockIdx.y, tid = threadIdx.x;
  const int cq = tid & 15, dq = tid >> 4;
  const int c0 = cblk * 128 + cq * 8;
  if (h >= H) {  // padding heads: zero rows (the attention waves read them)
    for (int b = 0; b < B; ++b) {
      uint16_t* row = qt + ((size_t)b * Hp + h) * kQK;
      if (tid < 16) *(u32x4*)(row + cblk * 128 + tid * 8) = u32x4{0, 0, 0, 0};
      if (cblk == 0 && tid >= 16 && tid < 24) *(u32x4*)(row + kC + (tid - 16) * 8) = u32x4{0, 0, 0, 0};
    }
    return;
  }
  __shared__ float red[16][128 + 4];
  float w[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const u32x4 v = *(const u32x4*)(wkv_b + ((size_t)h * (kDN + kDV) + dq * 8 + i) * kC + c0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w[i][2 * j] = bf_lo(v[j]);
      w[i][2 * j + 1] = bf_hi(v[j]);
    }
  }
  for (int b = 0; b < B; ++b) {
    const u32x4 qv = *(const u32x4*)(q_nope + ((size_t)b * H + h) * kDN + dq * 8);
    float q[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      q[2 * j] = bf_lo(qv[j]);
      q[2 * j + 1] = bf_hi(qv[j]);
    }
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) s = fmaf(q[i], w[i][e], s);
      acc[e] = s;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[dq][cq * 8 + e] = acc[e];
    __syncthreads();
    if (tid < 128) {
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) s += red[k][tid];
      qt[((size_t)b * Hp + h) * kQK + cblk * 128 + tid] = (uint16_t)f2bf(s);
    }
    __syncthreads();
  }
  if (cblk == 0) {  // copy q_pe rows (8 x 16 B per sequence)
    for (int i = tid; i < 8 * B; i += 256) {
      const int b = i >> 3, part = i & 7;
      *(u32x4*)(qt + ((size_t)b * Hp + h) * kQK + kC + part * 8) =
          *(const u32x4*)(q_pe + ((size_t)b * H + h) * kR + part * 8);
    }
  }
}

// ---------------------------------------------------------------------------
// attention (split-T flash decoding)
//
// grid (num_splits, B), 256 threads = 4 waves.  Workgroup (split, b) walks its
// chunk of the selection in tiles of 32 cache rows held in LDS row-major
// ([t][576]: 512 latent then 64 rotary values), in a ring of kStages tiles.
//   scores  S^T = K . Qa^T    A operand: 16-byte row reads of the tile
//   update  O^T += V^T . P^T  A operand: ds_read_tr16_b64 transposing reads of
//                             the same tile (V = its first 512 columns)
// Wave w owns heads 32w..32w+31: Qa for them lives in registers (B operand,
// 36 k-steps of 16), O^T (512 x 32 fp32) in 16 accumulator blocks.  The S^T
// accumulator gives every lane one head (l%32) and 16 of the 32 rows (the
// other 16 sit in lane l^32), so the per-head softmax needs one cross-lane
// exchange, and the probabilities feed the update as its B operand in place:
// element e of the S^T block is row 8(e/4) + 4(l/32) + e%4, which is exactly
// the row order the two transposing reads deliver for k-step e/8.
//
// bf16 cache: the tiles are filled by direct global->LDS loads
// (global_load_lds_dwordx4, no staging registers), kStages-1 tiles ahead.
// FP8 cache: codes and scales go through registers one tile ahead and are
// dequantised to bf16(float(code) * scale) when stored.
//
// LDS swizzle: logical 16-byte chunk ch of row t sits at chunk ch ^ F(t),
// F(t) = 2(t&3) + ((t>>2)&1).  Eight consecutive rows read the same logical
// chunk from eight different bank groups, and each 16-lane group of a
// transposing read touches 16 distinct 8-byte bank slots.
// ---------------------------------------------------------------------------
constexpr int kTT = kTileRows;              // rows per tile
constexpr int kStages = 4;                  // tiles in the LDS ring
constexpr int kTileElems = kTT * kQK;       // bf16 elements per tile (36 KB)
constexpr int kMaxIdx = 1024;               // top-k entries staged in LDS per split

struct AttnArgs {
  const uint16_t* qt;
  const void* kv;
  const float* kv_scale;
  const uint16_t* pe;
  const int32_t* lens;
  const int32_t* topk_idx;
  float* part_o;
  float* part_ml;
  int H, Hp, T, topk, NS, CH, head_blocks;
  float scale_log2;
};

__device__ __forceinline__ int swz(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }
__device__ __forceinline__ int tile_off(int t, int ch) { return t * kQK + ((ch ^ swz(t)) << 3); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_void*)p;
}

// 16-byte global -> LDS copy for each lane: lane l's 16 bytes from `src` land
// at LDS byte address base + 16 l (base must be wave-uniform).  Written as
// inline asm so the compiler's wait-count tracking does not treat every later
// LDS read as possibly depending on it; completion is awaited explicitly with
// s_waitcnt vmcnt before the workgroup barrier that publishes the tile.
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(base)
               : "memory", "m0");
}

__device__ __forceinline__ u32x2 ds_read_tr16(const uint16_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Sequence length clamped to the buffer, and the number of selected entries
// the splits walk (top-k rows of a sequence with no valid row select nothing).
__device__ __forceinline__ int seq_len(const int32_t* lens, int b, int T) {
  const int len = lens[b];
  return len < 0 ? 0 : (len > T ? T : len);
}
__device__ __forceinline__ int selected_entries(int len, int topk) {
  return topk > 0 ? (len > 0 ? topk : 0) : len;
}

template <int S>
struct Stage {
  static constexpr int value = S;
};

template <bool FP8, bool TOPK>
__global__ __launch_bounds__(256, 1) void attn_split_kernel(AttnArgs a) {
  const int split = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int len = seq_len(a.lens, b, a.T);
  const int n_b = selected_entries(len, TOPK ? a.topk : 0);
  const int p0 = split * a.CH;
  if (p0 >= n_b) return;  // whole workgroup: nothing selected in this split
  const int p1 = min(p0 + a.CH, n_b);
  const int ntiles = (p1 - p0 + kTT - 1) / kTT;

  // One LDS array per ring slot (not one 2-D array): the slot a tile lives in
  // is a compile-time constant below, which lets the compiler see that the
  // LDS-DMA writes in flight target other slots than the one being read, so
  // it does not wait for them.
  __shared__ __attribute__((aligned(16))) uint16_t sT0[kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t sT1[kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t sT2[kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t sT3[kTileElems];
  static_assert(kStages == 4, "one LDS array per ring slot");
  auto slot = [&](auto S) -> uint16_t* {
    constexpr int st = decltype(S)::value;
    if constexpr (st == 0) return sT0;
    else if constexpr (st == 1) return sT1;
    else if constexpr (st == 2) return sT2;
    else return sT3;
  };
  __shared__ uint32_t sMask[kStages];
  __shared__ int sIdx[TOPK ? kMaxIdx : 1];

  const bool active = wave < a.head_blocks;
  const int n = lane & 31, g = lane >> 5;
  const int head = wave * 32 + n;
  const size_t seq_row0 = (size_t)b * a.T;

  if (TOPK) {  // stage this split's row indices; invalid entries become -1
    for (int i = tid; i < p1 - p0; i += 256) {
      const int r = a.topk_idx[(size_t)b * a.topk + p0 + i];
      sIdx[i] = (r >= 0 && r < len) ? r : -1;
    }
    __syncthreads();
  }
  // Row of tile position t (any valid row when the position selects nothing:
  // its score is masked, and it must only be finite).
  auto tile_row = [&](int pt, int t, bool& ok) -> int {
    const int pos = pt + t;
    if (TOPK) {
      const int r = pos < p1 ? sIdx[pos - p0] : -1;
      ok = r >= 0;
      return ok ? r : 0;
    }
    ok = pos < p1;
    return ok ? pos : p1 - 1;
  };
  auto publish_mask = [&](int pt, int stage) {
    if (wave == 0) {
      bool ok = false;
      if (lane < 32) (void)tile_row(pt, lane, ok);
      const uint32_t m = (uint32_t)__ballot(ok && lane < 32);
      if (lane == 0) sMask[stage] = m;
    }
  };

  // ---- bf16 tiles: direct global -> LDS.  Instruction i of the tile writes LDS
  // chunks 64i .. 64i+63 (lane order); wave w issues i = w, w+4, ..., w+32.
  auto issue_bf16 = [&](int j, auto S) {
    const int pt = p0 + j * kTT, stage = decltype(S)::value;
    uint16_t* dst = slot(S);
    // Lane position P = 64i + lane walks i = wave, wave+4, ...: P grows by 256
    // = 3 rows (of 72 chunks) + 40 chunks per instruction.  The position is
    // laundered so the nine (row, chunk) pairs are recomputed per tile rather
    // than kept live across the loop.
    int P = 64 * wave + lane;
    asm volatile("" : "+v"(P));
    int t = P / 72, phys = P - 72 * t;
#pragma unroll
    for (int k = 0; k < 9; ++k) {
      const int ch = phys ^ swz(t);
      bool ok;
      const size_t row = seq_row0 + tile_row(pt, t, ok);
      const uint16_t* src = ch < 64 ? (const uint16_t*)a.kv + row * kC + ch * 8
                                    : a.pe + row * kR + (ch - 64) * 8;
      lds_dma16(src, lds_addr(dst + 512 * (wave + 4 * k)));
      phys += 40;
      t += 3;
      if (phys >= 72) {
        phys -= 72;
        t += 1;
      }
    }
    publish_mask(pt, stage);
  };

  // ---- FP8 tiles through registers: 4 units of 16 codes + 1 rotary chunk per thread
  u32x4 c8[FP8 ? 4 : 1];
  float csc[FP8 ? 4 : 1];
  u32x4 pev;
  auto load_fp8 = [&](int j) {
    const int pt = p0 + j * kTT;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int u = tid + 256 * k, t = u >> 5, cc = u & 31;
      bool ok;
      const size_t row = seq_row0 + tile_row(pt, t, ok);
      c8[k] = *(const u32x4*)((const uint8_t*)a.kv + row * kC + cc * 16);
      csc[k] = a.kv_scale[row * 4 + (cc >> 3)];
    }
    bool ok;
    const size_t row = seq_row0 + tile_row(pt, tid >> 3, ok);
    pev = *(const u32x4*)(a.pe + row * kR + (tid & 7) * 8);
  };
  auto store_fp8 = [&](int j, auto S) {
    const int stage = decltype(S)::value;
    uint16_t* dst = slot(S);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int u = tid + 256 * k, t = u >> 5, cc = u & 31;
      uint32_t w[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t q = c8[k][d];
        w[2 * d] = pack_bf(e4m3fn_to_f32(q & 0xFFu) * csc[k], e4m3fn_to_f32((q >> 8) & 0xFFu) * csc[k]);
        w[2 * d + 1] = pack_bf(e4m3fn_to_f32((q >> 16) & 0xFFu) * csc[k], e4m3fn_to_f32(q >> 24) * csc[k]);
      }
      *(u32x4*)(dst + tile_off(t, 2 * cc)) = u32x4{w[0], w[1], w[2], w[3]};
      *(u32x4*)(dst + tile_off(t, 2 * cc + 1)) = u32x4{w[4], w[5], w[6], w[7]};
    }
    *(u32x4*)(dst + tile_off(tid >> 3, 64 + (tid & 7))) = pev;
    publish_mask(p0 + j * kTT, stage);
  };

  // O accumulators.  Every definition of o[] is an MFMA result (zero operands
  // for the initial value and in the rescale below): a VALU definition would
  // make the compiler keep the loop-carried accumulators in VGPRs and copy
  // all 256 of them every iteration.
  const u32x4 zq = {0u, 0u, 0u, 0u};
  f32x16 o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = mfma32(zq, zq, f32x16{});
  float m_run = -INFINITY, l_run = 0.f;

  // Per-lane LDS bases (element offsets inside a tile).
  //   score k-step st reads logical chunk 2st+g of row n:
  //     phys = 8(st>>2) + ((2(st&3)+g) ^ F(n))          -> 4 bases + immediates
  //   update (c-block cb, k-step u, half h): lane 4r+q of 16-lane group G reads
  //     row 16u + 8h + 4(G>>1) + r, columns 32cb + 16(G&1) + 4q .. +3  -> 2 bases
  const int fn = swz(n);
  int sc_base[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) sc_base[k] = n * kQK + (((2 * k + g) ^ fn) << 3);
  const int G = lane >> 4, i16 = lane & 15, rr = i16 >> 2, qq = i16 & 3;
  const int tr_t = 4 * (G >> 1) + rr;
  const int tr_x = 2 * (G & 1) + (qq >> 1);
  int tr_base[2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
    tr_base[par] = tr_t * kQK + (((4 * par + tr_x) ^ swz(tr_t)) << 3) + 4 * (qq & 1);

  // ---- pipeline prologue: the first tiles and the query are loaded together,
  // and everything is complete before the loop (the loop's own waits then only
  // concern tiles)
  if (FP8) {
    load_fp8(0);
  } else {
    issue_bf16(0, Stage<0>{});
    if (1 < ntiles) issue_bf16(1, Stage<1>{});
    if (2 < ntiles) issue_bf16(2, Stage<2>{});
  }
  // Absorbed query + q_pe of this lane's head: k-step s covers elements 16s..16s+15,
  // lane group g holds 8 of them.
  u32x4 qreg[36];
  if (active) {
    const u32x4* src = (const u32x4*)(a.qt + ((size_t)b * a.Hp + head) * kQK);
#pragma unroll
    for (int s = 0; s < 36; ++s) qreg[s] = src[2 * s + g];
  }
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));  // vmcnt(0)
  if (FP8) store_fp8(0, Stage<0>{});

  // Tile j lives in ring slot S = j % kStages (a compile-time constant here).
  auto body = [&](int j, auto S) {
    constexpr int st = decltype(S)::value;
    if (!FP8) {
      // tiles j+1 .. j+kStages-2 may stay in flight (9 loads each per thread)
      if (j + kStages - 2 < ntiles) __builtin_amdgcn_s_waitcnt((9 * (kStages - 2) & 15) | (0x7 << 4) | (0xF << 8) | (((9 * (kStages - 2)) >> 4) << 14));
      else __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));
    }
    // tile j visible to every wave; every wave is done with tile j-1.  The
    // bf16 path waited on its own LDS-DMA loads above, so a plain s_barrier
    // suffices (__syncthreads would also wait for the tiles still in flight).
    if (FP8) __syncthreads();
    else asm volatile("s_barrier" ::: "memory");
    if (!FP8) {
      if (j + kStages - 1 < ntiles) issue_bf16(j + kStages - 1, Stage<(st + kStages - 1) % kStages>{});
    } else if (j + 1 < ntiles) {
      load_fp8(j + 1);
    }
    const uint16_t* tile = slot(S);
    if (active) {
      // Scores.  The 36 MFMAs accumulate in VGPRs (inline asm: the compiler
      // would put this accumulator in AGPRs, where O already takes all 256).
      // Back-to-back MFMAs of one shape accumulating into the same registers
      // need no wait states; the s_nop after the chain covers the MFMA-write ->
      // VALU-read hazard (>= 18 wait states for this 8-pass instruction).
      // Operand reads run three k-steps ahead of the MFMAs.
      f32x16 s;
      u32x4 ka[4];
#pragma unroll
      for (int st = 0; st < 3; ++st) ka[st] = *(const u32x4*)(tile + sc_base[st & 3] + 64 * (st >> 2));
#pragma unroll
      for (int st = 0; st < 36; ++st) {
        if (st + 3 < 36)
          ka[(st + 3) & 3] = *(const u32x4*)(tile + sc_base[(st + 3) & 3] + 64 * ((st + 3) >> 2));
        if (st == 0)
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(ka[0]), "v"(qreg[0]));
        else
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(ka[st & 3]), "v"(qreg[st]));
      }
      asm volatile("s_nop 15\n\ts_nop 3" : "+v"(s));
      const uint32_t mask = sMask[st];
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int t = 8 * (e >> 2) + 4 * g + (e & 3);
        if (!((mask >> t) & 1u)) s[e] = -INFINITY;
        mx = fmaxf(mx, s[e]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // online softmax in log2 units; the running max only moves when the new
      // one exceeds it by more than 8 (probabilities stay <= 2^8), which skips
      // most rescales of O without changing the result
      const float mt = mx * a.scale_log2;
      const float m_use = (m_run == -INFINITY || mt > m_run + 8.0f) ? fmaxf(mt, m_run) : m_run;
      const float m_sub = (m_use == -INFINITY) ? 0.f : m_use;
      const float alpha = (m_use == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_use);
      float p[16];
      float lsum = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[e] = __builtin_amdgcn_exp2f(fmaf(s[e], a.scale_log2, -m_sub));
        lsum += p[e];
      }
      l_run = l_run * alpha + lsum;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          f32x16 t = o[i];
          asm volatile("" : "+v"(t));  // scale a copy; o[i] itself stays an MFMA value
          o[i] = mfma32(zq, zq, t * alpha);
        }
      }
      m_run = m_use;
      const u32x4 pb0 = {pack_bf_finite(p[0], p[1]), pack_bf_finite(p[2], p[3]),
                         pack_bf_finite(p[4], p[5]), pack_bf_finite(p[6], p[7])};
      const u32x4 pb1 = {pack_bf_finite(p[8], p[9]), pack_bf_finite(p[10], p[11]),
                         pack_bf_finite(p[12], p[13]), pack_bf_finite(p[14], p[15])};
      // Update: each c-block needs four transposing reads (rows 4g+r, 8+4g+r,
      // 16+4g+r, 24+4g+r); the next block's reads are issued before this
      // block's MFMAs.
      u32x2 vt[2][4];
      {
        const uint16_t* base = tile + tr_base[0];
#pragma unroll
        for (int q = 0; q < 4; ++q) vt[0][q] = ds_read_tr16(base + 8 * q * kQK);
      }
#pragma unroll
      for (int cb = 0; cb < 16; ++cb) {
        if (cb + 1 < 16) {
          const uint16_t* base = tile + tr_base[(cb + 1) & 1] + 64 * ((cb + 1) >> 1);
#pragma unroll
          for (int q = 0; q < 4; ++q) vt[(cb + 1) & 1][q] = ds_read_tr16(base + 8 * q * kQK);
        }
        const u32x2* v = vt[cb & 1];
        o[cb] = mfma32(u32x4{v[0][0], v[0][1], v[1][0], v[1][1]}, pb0, o[cb]);
        o[cb] = mfma32(u32x4{v[2][0], v[2][1], v[3][0], v[3][1]}, pb1, o[cb]);
      }
    }
    if (FP8 && j + 1 < ntiles) store_fp8(j + 1, Stage<(st + 1) % kStages>{});
  };
  for (int j0 = 0; j0 < ntiles; j0 += kStages) {
    body(j0, Stage<0>{});
    if (j0 + 1 < ntiles) body(j0 + 1, Stage<1>{});
    if (j0 + 2 < ntiles) body(j0 + 2, Stage<2>{});
    if (j0 + 3 < ntiles) body(j0 + 3, Stage<3>{});
  }

  // ---- partial result of this split: O normalised by its own l, plus (m, l)
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (active && head < a.H) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* po = a.part_o + (((size_t)b * a.NS + split) * a.H + head) * kC;
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = 32 * cb + 8 * q + 4 * g;
        *(f32x4*)(po + c) = f32x4{o[cb][4 * q] * inv, o[cb][4 * q + 1] * inv,
                                  o[cb][4 * q + 2] * inv, o[cb][4 * q + 3] * inv};
      }
    }
    if (g == 0) {
      float* pm = a.part_ml + (((size_t)b * a.NS + split) * a.H + head) * 2;
      pm[0] = l_tot > 0.f ? m_run : -INFINITY;
      pm[1] = l_tot;
    }
  }
}

// ---------------------------------------------------------------------------
// combine: grid (H, B), 64 threads; lane owns 8 consecutive latent columns.
//   M = max_s m_s,  w_s = l_s 2^(m_s - M),  o = sum_s w_s O_s / sum_s w_s
// The split loop is unrolled by 4 so each lane keeps eight 16-byte loads in
// flight.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void combine_kernel(const float* __restrict__ part_o,
                                                     const float* __restrict__ part_ml,
                                                     const int32_t* __restrict__ lens,
                                                     uint16_t* __restrict__ olat, int H, int T,
                                                     int topk, int NS, int CH) {
  const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int n_b = selected_entries(seq_len(lens, b, T), topk);
  const int ns = (n_b + CH - 1) / CH;
  const size_t split_stride = (size_t)H * kC;
  const float* pm = part_ml + ((size_t)b * NS * H + h) * 2;
  const float* po = part_o + ((size_t)b * NS * H + h) * kC + 8 * lane;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) {
    const float2 ml = *(const float2*)(pm + (size_t)s * H * 2);
    if (ml.y > 0.f) M = fmaxf(M, ml.x);
  }
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  int s = 0;
  for (; s + 4 <= ns; s += 4) {
    f32x4 v[4][2];
    float w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float2 ml = *(const float2*)(pm + (size_t)(s + k) * H * 2);
      w[k] = ml.y > 0.f ? ml.y * exp2f(ml.x - M) : 0.f;
      v[k][0] = *(const f32x4*)(po + (s + k) * split_stride);
      v[k][1] = *(const f32x4*)(po + (s + k) * split_stride + 4);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (w[k] > 0.f) {
        L += w[k];
        acc0 += w[k] * v[k][0];
        acc1 += w[k] * v[k][1];
      }
    }
  }
  for (; s < ns; ++s) {
    const float2 ml = *(const float2*)(pm + (size_t)s * H * 2);
    if (ml.y > 0.f) {
      const float w = ml.y * exp2f(ml.x - M);
      L += w;
      acc0 += w * *(const f32x4*)(po + s * split_stride);
      acc1 += w * *(const f32x4*)(po + s * split_stride + 4);
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* dst = olat + ((size_t)b * H + h) * kC + 8 * lane;
  *(u32x4*)dst = u32x4{pack_bf(acc0[0] * inv, acc0[1] * inv), pack_bf(acc0[2] * inv, acc0[3] * inv),
                       pack_bf(acc1[0] * inv, acc1[1] * inv), pack_bf(acc1[2] * inv, acc1[3] * inv)};
}

// ---------------------------------------------------------------------------
// uproj: out[b,h,d] = sum_c o[b,h,c] W_UV[h][d][c].  grid (H, 4 d-blocks of 32),
// one wave; MFMA 16x16x32 with the sequences as the M dimension (blocks of 16)
// and two 16-wide d blocks as N.  The wave's W_UV slice (32 rows x 512, 32 KB)
// is loaded into registers up front and reused for every block of sequences.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void uproj_kernel(const uint16_t* __restrict__ olat,
                                                   const uint16_t* __restrict__ wkv_b,
                                                   uint16_t* __restrict__ out, int B, int H) {
  const int h = blockIdx.x, d0 = 32 * blockIdx.y;
  const int lane = threadIdx.x, r = lane & 15, g = lane >> 4;
  const uint16_t* w0 = wkv_b + ((size_t)h * (kDN + kDV) + kDN + d0 + r) * kC + 8 * g;
  const uint16_t* w1 = w0 + (size_t)16 * kC;
  u32x4 bw0[16], bw1[16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    bw0[ks] = *(const u32x4*)(w0 + 32 * ks);
    bw1[ks] = *(const u32x4*)(w1 + 32 * ks);
  }
  for (int b0 = 0; b0 < B; b0 += 16) {
    const int bb = b0 + r;
    const bool bok = bb < B;
    const uint16_t* arow = olat + ((size_t)(bok ? bb : 0) * H + h) * kC + 8 * g;
    u32x4 av[16];
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) av[ks] = bok ? *(const u32x4*)(arow + 32 * ks) : u32x4{0, 0, 0, 0};
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      acc0 = mfma16(av[ks], bw0[ks], acc0);
      acc1 = mfma16(av[ks], bw1[ks], acc1);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ob = b0 + 4 * g + j;
      if (ob < B) {
        uint16_t* dst = out + ((size_t)ob * H + h) * kDV + d0 + r;
        dst[0] = (uint16_t)f2bf(acc0[j]);
        dst[16] = (uint16_t)f2bf(acc1[j]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_decode(const mla_params& p, const DecodeArgs& d, hipStream_t stream) {
  const DecodePlan plan = make_decode_plan(p);
  const int B = p.batch, H = p.num_heads;
  char* ws = (char*)d.workspace;
  uint16_t* qt = (uint16_t*)(ws + plan.off_qt);
  float* part_o = (float*)(ws + plan.off_part_o);
  float* part_ml = (float*)(ws + plan.off_part_ml);
  uint16_t* olat = (uint16_t*)(ws + plan.off_olat);
  hipEvent_t* ev = (hipEvent_t*)p.trace_events;
  hipError_t err;
#define MLA_TRACE(i)                                       \
  if (ev) {                                                \
    err = hipEventRecord(ev[i], stream);                   \
    if (err != hipSuccess) return err;                     \
  }

  MLA_TRACE(0);
  absorb_kernel<<<dim3(plan.heads_padded, 4), 256, 0, stream>>>(
      (const uint16_t*)d.q_nope, (const uint16_t*)d.q_pe, (const uint16_t*)d.wkv_b, qt, B, H,
      plan.heads_padded);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  MLA_TRACE(1);

  AttnArgs aa;
  aa.qt = qt;
  aa.kv = d.kv_cache;
  aa.kv_scale = d.kv_scale;
  aa.pe = (const uint16_t*)d.pe_cache;
  aa.lens = d.cache_lens;
  aa.topk_idx = d.topk_idx;
  aa.part_o = part_o;
  aa.part_ml = part_ml;
  aa.H = H;
  aa.Hp = plan.heads_padded;
  aa.T = p.max_seq_len;
  aa.topk = p.topk;
  aa.NS = plan.num_splits;
  aa.CH = plan.chunk_rows;
  aa.head_blocks = plan.head_blocks;
  aa.scale_log2 = p.softmax_scale * 1.4426950408889634f;
  const dim3 agrid(plan.num_splits, B);
  MLA_TRACE(2);
  const bool fp8 = p.kv_dtype == MLA_KV_FP8_E4M3_B128, topk = p.topk > 0;
  if (fp8 && topk) attn_split_kernel<true, true><<<agrid, 256, 0, stream>>>(aa);
  else if (fp8) attn_split_kernel<true, false><<<agrid, 256, 0, stream>>>(aa);
  else if (topk) attn_split_kernel<false, true><<<agrid, 256, 0, stream>>>(aa);
  else attn_split_kernel<false, false><<<agrid, 256, 0, stream>>>(aa);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  MLA_TRACE(3);

  MLA_TRACE(4);
  combine_kernel<<<dim3(H, B), 64, 0, stream>>>(part_o, part_ml, d.cache_lens, olat, H,
                                                  p.max_seq_len, p.topk, plan.num_splits,
                                                  plan.chunk_rows);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  MLA_TRACE(5);

  MLA_TRACE(6);
  uproj_kernel<<<dim3(H, 4), 64, 0, stream>>>(olat, (const uint16_t*)d.wkv_b,
                                                           (uint16_t*)d.out, B, H);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  MLA_TRACE(7);
#undef MLA_TRACE
  return hipSuccess;
}

}  // namespace mla
