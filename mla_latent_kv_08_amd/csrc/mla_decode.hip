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
// chunk of the selection in tiles of 32 cache rows.  Each tile is staged in
// LDS twice:
//   sK  row-major  [t][576]     A operand of the scores  S^T = K . Qa^T
//   sV  transposed [c][32]      A operand of the update  O^T += V^T . P^T
// Wave w owns heads 32w..32w+31: Qa for them lives in registers (B operand,
// 36 k-steps of 16), O^T (512 x 32 fp32) lives in 16 accumulator blocks.
// The S^T accumulator layout gives every lane one head (l%32) and 16 of the
// 32 rows; the other 16 sit in lane l^32, so the per-head softmax statistics
// need a single cross-lane exchange.  The probabilities are re-used as the
// B operand of the update without moving: the row order inside each k-step
// is permuted instead, by storing sV with rows t at position tau(t) (bits 2
// and 3 of t swapped).
//
// LDS swizzles (16-byte chunk index XOR a function of the row) keep the
// b128 reads and writes of both copies free of bank conflicts:
//   sK: chunk' = chunk ^ ((t >> 3) & 3)     sV: chunk' = chunk ^ ((c >> 1) & 3)
// ---------------------------------------------------------------------------
constexpr int kTT = kTileRows;          // rows per tile
constexpr int kSKStride = kQK;          // bf16 per sK row (swizzled, no padding)
constexpr int kSVStride = kTT;          // bf16 per sV row

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

__device__ __forceinline__ int sk_off(int t, int chunk) {
  return t * kSKStride + ((chunk ^ ((t >> 3) & 3)) << 3);
}
__device__ __forceinline__ int sv_off(int c, int chunk) {
  return c * kSVStride + ((chunk ^ ((c >> 1) & 3)) << 3);
}

template <bool FP8, bool TOPK>
__global__ __launch_bounds__(256, 1) void attn_split_kernel(AttnArgs a) {
  const int split = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int len = a.lens[b];
  len = len < 0 ? 0 : (len > a.T ? a.T : len);
  const int n_b = TOPK ? a.topk : len;
  const int p0 = split * a.CH;
  if (p0 >= n_b) return;  // whole workgroup: nothing selected in this split
  const int p1 = min(p0 + a.CH, n_b);

  __shared__ __attribute__((aligned(16))) uint16_t sK[kTT * kSKStride];
  __shared__ __attribute__((aligned(16))) uint16_t sV[kC * kSVStride];
  __shared__ uint32_t sMask;

  const bool active = wave < a.head_blocks;
  const int n = lane & 31, g = lane >> 5;
  const int head = wave * 32 + n;
  const uint16_t* sk_base[2] = {sK + sk_off(n, g), sK + sk_off(n, 2 + g)};
  const uint16_t* sv_base[2] = {sV + sv_off(n, g), sV + sv_off(n, 2 + g)};

  // Absorbed query + q_pe of this lane's head: k-step s covers elements 16s..16s+15,
  // lane group g holds 8 of them.
  u32x4 qreg[36];
  if (active) {
    const u32x4* src = (const u32x4*)(a.qt + ((size_t)b * a.Hp + head) * kQK);
#pragma unroll
    for (int s = 0; s < 36; ++s) qreg[s] = src[2 * s + g];
  }
  f32x16 o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // ---- tile loader: thread owns rows 4rq..4rq+3 and column octets co0, co0+32
  const int rq = tid & 7, co0 = tid >> 3;
  const int pe_t = tid >> 3, pe_ch = tid & 7;
  const size_t seq_row0 = (size_t)b * a.T;

  auto row_of = [&](int pt, int t, int& row) -> bool {
    const int pos = pt + t;
    if (pos >= p1) return false;
    if (TOPK) {
      const int r = a.topk_idx[(size_t)b * a.topk + pos];
      if (r < 0 || r >= len) return false;
      row = r;
    } else {
      row = pos;
    }
    return true;
  };

  // prefetch registers
  u32x4 lat[2][4];            // bf16 path: 8 latent values per (unit, row)
  u32x2 lat8[2][4];           // fp8 path: 8 codes per (unit, row)
  float lsc[2][4];            // fp8 path: block scale per (unit, row)
  u32x4 pev;
  uint32_t tile_mask = 0;

  auto load_tile = [&](int pt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int row = 0;
      const bool ok = row_of(pt, 4 * rq + i, row);
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int co = co0 + 32 * it;
        if (FP8) {
          const uint8_t* base = (const uint8_t*)a.kv + (seq_row0 + row) * kC;
          lat8[it][i] = ok ? *(const u32x2*)(base + co * 8) : u32x2{0, 0};
          lsc[it][i] = ok ? a.kv_scale[(seq_row0 + row) * 4 + (co >> 4)] : 0.f;
        } else {
          const uint16_t* base = (const uint16_t*)a.kv + (seq_row0 + row) * kC;
          lat[it][i] = ok ? *(const u32x4*)(base + co * 8) : u32x4{0, 0, 0, 0};
        }
      }
    }
    {
      int row = 0;
      const bool ok = row_of(pt, pe_t, row);
      pev = ok ? *(const u32x4*)(a.pe + (seq_row0 + row) * kR + pe_ch * 8) : u32x4{0, 0, 0, 0};
    }
    if (wave == 0) {
      int row = 0;
      const bool ok = lane < 32 && row_of(pt, lane, row);
      tile_mask = (uint32_t)__ballot(ok);
    }
  };

  auto store_tile = [&]() {
    u32x4 v[2][4];
#pragma unroll
    for (int it = 0; it < 2; ++it) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (FP8) {
          const float s = lsc[it][i];
          uint32_t w[4];
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const uint32_t c4 = lat8[it][i][j];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
              const float x0 = e4m3fn_to_f32((c4 >> (16 * k)) & 0xFFu) * s;
              const float x1 = e4m3fn_to_f32((c4 >> (16 * k + 8)) & 0xFFu) * s;
              w[2 * j + k] = pack_bf(x0, x1);
            }
          }
          v[it][i] = u32x4{w[0], w[1], w[2], w[3]};
        } else {
          v[it][i] = lat[it][i];
        }
      }
    }
    // row-major copy
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int i = 0; i < 4; ++i) *(u32x4*)(sK + sk_off(4 * rq + i, co0 + 32 * it)) = v[it][i];
    *(u32x4*)(sK + sk_off(pe_t, 64 + pe_ch)) = pev;
    // transposed copy: rows 4rq..4rq+3 land at tau0..tau0+3
    const int tau0 = 16 * (rq >> 2) + 8 * (rq & 1) + 4 * ((rq >> 1) & 1);
    const int tchunk = tau0 >> 3, thalf = (tau0 >> 2) & 1;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int co = co0 + 32 * it;
      const uint32_t odd = co & 1;
      // odd column octets write their elements in swapped pairs (k ^ 1) so that
      // lanes of both parities hit different banks
      const uint32_t sel_a = odd ? 0x07060302u : 0x05040100u;
      const uint32_t sel_b = odd ? 0x05040100u : 0x07060302u;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t r0 = v[it][0][d], r1 = v[it][1][d], r2 = v[it][2][d], r3 = v[it][3][d];
        const u32x2 wa = {__builtin_amdgcn_perm(r1, r0, sel_a), __builtin_amdgcn_perm(r3, r2, sel_a)};
        const u32x2 wb = {__builtin_amdgcn_perm(r1, r0, sel_b), __builtin_amdgcn_perm(r3, r2, sel_b)};
        const int ca = 8 * co + ((2 * d) ^ (int)odd);
        const int cb = 8 * co + ((2 * d + 1) ^ (int)odd);
        *(u32x2*)(sV + sv_off(ca, tchunk) + 4 * thalf) = wa;
        *(u32x2*)(sV + sv_off(cb, tchunk) + 4 * thalf) = wb;
      }
    }
    if (tid == 0) sMask = tile_mask;
  };

  load_tile(p0);
  for (int pt = p0; pt < p1; pt += kTT) {
    __syncthreads();  // previous tile fully consumed
    store_tile();
    __syncthreads();
    if (pt + kTT < p1) load_tile(pt + kTT);  // in flight during this tile's math
    if (active) {
      // scores S^T[t][head] for the 32 rows of the tile
      // k-step st = 2j + u reads chunk 2st + g = 4j + (2u + g); the swizzle only
      // touches the low two chunk bits, so each lane needs two base addresses
      // and the rest is an immediate offset
      f32x16 s = f32x16{};
#pragma unroll
      for (int st = 0; st < 36; ++st) {
        const u32x4 ka = *(const u32x4*)(sk_base[st & 1] + 32 * (st >> 1));
        s = mfma32(ka, qreg[st], s);
      }
      const uint32_t mask = sMask;
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
      const float alpha = (m_use == m_run) ? 1.f : exp2f(m_run - m_use);
      float p[16];
      float lsum = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[e] = exp2f(fmaf(s[e], a.scale_log2, -m_sub));
        lsum += p[e];
      }
      l_run = l_run * alpha + lsum;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) o[i] *= alpha;
      }
      m_run = m_use;
      const u32x4 pb0 = {pack_bf_finite(p[0], p[1]), pack_bf_finite(p[2], p[3]),
                         pack_bf_finite(p[4], p[5]), pack_bf_finite(p[6], p[7])};
      const u32x4 pb1 = {pack_bf_finite(p[8], p[9]), pack_bf_finite(p[10], p[11]),
                         pack_bf_finite(p[12], p[13]), pack_bf_finite(p[14], p[15])};
#pragma unroll
      for (int cb = 0; cb < 16; ++cb) {  // rows c = 32cb + n: swizzle depends on n only
        const u32x4 v0 = *(const u32x4*)(sv_base[0] + 32 * 32 * cb);
        const u32x4 v1 = *(const u32x4*)(sv_base[1] + 32 * 32 * cb);
        o[cb] = mfma32(v0, pb0, o[cb]);
        o[cb] = mfma32(v1, pb1, o[cb]);
      }
    }
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
// combine: grid (H, B), 128 threads; thread owns 4 consecutive latent columns.
//   M = max_s m_s,  w_s = l_s 2^(m_s - M),  o = sum_s w_s O_s / sum_s w_s
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128) void combine_kernel(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml,
                                                      const int32_t* __restrict__ lens,
                                                      uint16_t* __restrict__ olat, int H, int T,
                                                      int topk, int NS, int CH) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  int len = lens[b];
  len = len < 0 ? 0 : (len > T ? T : len);
  const int n_b = topk > 0 ? topk : len;
  const int ns = (n_b + CH - 1) / CH;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) {
    const float* pm = part_ml + (((size_t)b * NS + s) * H + h) * 2;
    if (pm[1] > 0.f) M = fmaxf(M, pm[0]);
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float* pm = part_ml + (((size_t)b * NS + s) * H + h) * 2;
    const float l = pm[1];
    if (l > 0.f) {
      const float w = l * exp2f(pm[0] - M);
      L += w;
      const f32x4 v = *(const f32x4*)(part_o + (((size_t)b * NS + s) * H + h) * kC + 4 * tid);
      acc += w * v;
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* dst = olat + ((size_t)b * H + h) * kC + 4 * tid;
  *(u32x2*)dst = u32x2{pack_bf(acc[0] * inv, acc[1] * inv), pack_bf(acc[2] * inv, acc[3] * inv)};
}

// ---------------------------------------------------------------------------
// uproj: out[b,h,d] = sum_c o[b,h,c] W_UV[h][d][c].  grid (H, ceil(B/16)),
// 256 threads; wave w owns d = 32w..32w+31 (two 16-wide blocks), MFMA 16x16x32
// with the sequences as the M dimension (padded to 16).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void uproj_kernel(const uint16_t* __restrict__ olat,
                                                    const uint16_t* __restrict__ wkv_b,
                                                    uint16_t* __restrict__ out, int B, int H) {
  const int h = blockIdx.x, b0 = blockIdx.y * 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int bb = b0 + r;
  const bool bok = bb < B;
  const uint16_t* arow = olat + ((size_t)(bok ? bb : 0) * H + h) * kC;
  const uint16_t* w0 = wkv_b + ((size_t)h * (kDN + kDV) + kDN + 32 * wave + r) * kC;
  const uint16_t* w1 = w0 + (size_t)16 * kC;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    const int c = 32 * ks + 8 * g;
    const u32x4 av = bok ? *(const u32x4*)(arow + c) : u32x4{0, 0, 0, 0};
    const u32x4 bv0 = *(const u32x4*)(w0 + c);
    const u32x4 bv1 = *(const u32x4*)(w1 + c);
    acc0 = mfma16(av, bv0, acc0);
    acc1 = mfma16(av, bv1, acc1);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ob = b0 + 4 * g + j;
    if (ob < B) {
      uint16_t* dst = out + ((size_t)ob * H + h) * kDV + 32 * wave + r;
      dst[0] = (uint16_t)f2bf(acc0[j]);
      dst[16] = (uint16_t)f2bf(acc1[j]);
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
  combine_kernel<<<dim3(H, B), 128, 0, stream>>>(part_o, part_ml, d.cache_lens, olat, H,
                                                  p.max_seq_len, p.topk, plan.num_splits,
                                                  plan.chunk_rows);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  MLA_TRACE(5);

  MLA_TRACE(6);
  uproj_kernel<<<dim3(H, (B + 15) / 16), 256, 0, stream>>>(olat, (const uint16_t*)d.wkv_b,
                                                           (uint16_t*)d.out, B, H);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  MLA_TRACE(7);
#undef MLA_TRACE
  return hipSuccess;
}

}  // namespace mla
