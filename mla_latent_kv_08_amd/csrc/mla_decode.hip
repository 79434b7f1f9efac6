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

#include <algorithm>

#include "mla_cache_store.hpp"
#include "mla_device.hpp"
#include "mla_launch.hpp"
#include "mla_plan.hpp"

namespace mla {

// Sequence length clamped to the buffer, and the number of entries of the
// selection (top-k rows of a sequence with no valid row select nothing).
__device__ __forceinline__ int seq_len(const int32_t* lens, int b, int T) {
  const int len = lens[b];
  return len < 0 ? 0 : (len > T ? T : len);
}
// Rows seen by query token v = b * s + i (the last s cached positions are the
// s query tokens; token i sees the rows up to its own).
__device__ __forceinline__ int query_len(const int32_t* lens, int v, int s, int T) {
  const int len = s == 1 ? seq_len(lens, v, T) : seq_len(lens, v / s, T) - (s - 1 - v % s);
  return len < 0 ? 0 : len;
}
__device__ __forceinline__ int selected_entries(int len, int topk) {
  return topk > 0 ? (len > 0 ? topk : 0) : len;
}

// Inclusive prefix sum over the 256 threads of a workgroup (wavefront
// shuffles, then the four wave totals through LDS); *total receives the sum
// of all 256 values.  sc: 4 ints of LDS.
__device__ int block_scan_256(int v, int* sc, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  if (lane == 63) sc[w] = v;
  __syncthreads();
  const int s0 = sc[0], s1 = sc[1], s2 = sc[2], s3 = sc[3];
  __syncthreads();  // sc free for the next call
  *total = s0 + s1 + s2 + s3;
  return v + (w > 0 ? s0 : 0) + (w > 1 ? s1 : 0) + (w > 2 ? s2 : 0);
}

// Sum, maximum and sum over the 256 threads of a workgroup, in one pass,
// returned to every thread.  red: 12 long longs of LDS.
__device__ void block_reduce3_256(long long& a, long long& m, long long& c, long long* red) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    a += __shfl_xor(a, o, 64);
    const long long y = __shfl_xor(m, o, 64);
    m = y > m ? y : m;
    c += __shfl_xor(c, o, 64);
  }
  if ((tid & 63) == 0) {
    red[3 * (tid >> 6)] = a;
    red[3 * (tid >> 6) + 1] = m;
    red[3 * (tid >> 6) + 2] = c;
  }
  __syncthreads();
  a = red[0] + red[3] + red[6] + red[9];
  m = red[1];
#pragma unroll
  for (int k = 1; k < 4; ++k) m = red[3 * k + 1] > m ? red[3 * k + 1] : m;
  c = red[2] + red[5] + red[8] + red[11];
  __syncthreads();
}

// Sum over the 256 threads of a workgroup, returned to every thread.
__device__ long long block_sum_256(long long v, long long* red) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  const long long r = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return r;
}

constexpr int kPlanCache = 2048;  // per-sequence values kept in LDS by the planner

constexpr int kXcds = 8;  // MI355X: accelerator complex dies, each with its own L2

// Attention workgroup i runs on XCD i % 8 (round-robin dispatch).  Of the n
// workgroups in use, XCD x (workgroups x, x + 8, ...) takes the plan slots
// [x q + min(x, r), ...) in order, q = n / 8, r = n % 8, so the workgroups of
// one sequence share an L2 and fetch its absorbed query there once.  This is
// the workgroup that runs plan slot s.
__device__ __forceinline__ int xcd_workgroup(int s, int n) {
  const int q = n / kXcds, r = n % kXcds, big = r * (q + 1);
  int x, k;
  if (s < big) {
    x = s / (q + 1);
    k = s - x * (q + 1);
  } else {
    x = r + (s - big) / q;
    k = (s - big) - (x - r) * q;
  }
  return x + kXcds * k;
}

// Work plan of one decode call, computed by one workgroup of 256 threads (the
// split is described with make_decode_plan) over the B work items (item v =
// b s + i seeing query_len rows of sequence v / s: the query tokens, s per
// sequence, or with packed tokens the sequences, s = 1): picks the tile
// budget S, then
// writes wcum[b] = k_0 + ... + k_{b-1} (wcum[B] = workgroups in use) and, for
// each of the G attention workgroups, the record {item, first tile, end
// tile, clamped length} (item -1: workgroup unused) and the plan slot its
// partial goes to, so that a workgroup starts from two independent loads
// (plan_groups, after two helpers).

// floor(a / b) and ceil(a / b) for 0 <= a < 2^52 and b >= 1.  Both are
// exact in double, and a non-integer quotient a/b lies at least 1/b from the
// nearest integer n, more than half an ulp of n (n * 2^-53 < 1/b because
// n * b <= a + b < 2^53), so rounding never lands on n: floor and ceil of the
// correctly rounded quotient are exact, and far cheaper than a 64-bit integer
// division.
__device__ __forceinline__ long long floor_div(long long a, long long b) {
  return (long long)floor((double)a / (double)b);
}
__device__ __forceinline__ long long ceil_div(long long a, long long b) {
  return (long long)ceil((double)a / (double)b);
}

// LDS of the planner (the caller's buffer, kPlanLdsBytes).
constexpr int kPlanLdsBytes = 12 * 8 + 4 * 4 + (3 * kPlanCache + 1) * 4 + 32 * 4;

__device__ void plan_groups(const int32_t* lens, int B, int s, int T, int topk, int min_tiles,
                            int G, int32_t* wcum, int4* rec, int32_t* slot_of, char* lds) {
  long long* red = (long long*)lds;           // [12]
  int* sc = (int*)(lds + 96);                 // [4]
  int* tl = sc + 4;                           // [kPlanCache] tiles of sequence b
  int* sl = tl + kPlanCache;                  // [kPlanCache] clamped length of sequence b
  int* sw = sl + kPlanCache;                  // [kPlanCache + 1] first workgroup of sequence b
  const int tid = threadIdx.x;
  auto tiles_of = [&](int bb) -> int {
    return (selected_entries(query_len(lens, bb, s, T), topk) + kTileRows - 1) / kTileRows;
  };
  auto tiles = [&](int bb) -> int { return bb < kPlanCache ? tl[bb] : tiles_of(bb); };
  long long tot = 0, mx = 0, nonempty = 0;
  for (int bb = tid; bb < B; bb += 256) {
    const int len = query_len(lens, bb, s, T);
    const int t = (selected_entries(len, topk) + kTileRows - 1) / kTileRows;
    if (bb < kPlanCache) {
      tl[bb] = t;
      sl[bb] = len;
    }
    tot += t;
    mx = t > mx ? t : mx;
    nonempty += t > 0;
  }
  block_reduce3_256(tot, mx, nonempty, red);  // (its barrier also publishes tl, sl)
  long long S = mx > 0 ? mx : 1;
  if (mx > 0 && nonempty < kTargetCUs) {
    // sum ceil(t_b / S) <= tot / S + nonempty, so S = ceil(tot / (256 - nonempty))
    // fits, and nothing below ceil(tot / 256) does: search between the two.
    // Every S searched is >= tot / 256 and <= mx < 2^26, so the counts stay
    // below 256 + B and 32-bit arithmetic suffices.
    long long lo = (tot + kTargetCUs - 1) / kTargetCUs;
    long long hi = ceil_div(tot, kTargetCUs - nonempty);
    if (lo < 1) lo = 1;
    if (hi > mx) hi = mx;  // S = mx gives one workgroup per sequence, which fits
    if (lo > hi) lo = hi;
    int* cnt = sc + 4 + 3 * kPlanCache + 1;  // [4][8] wave partial counts
    while (lo < hi) {
      // smallest S in [lo, hi] that fits (the count is non-increasing in S):
      // test 8 budgets spread over [lo, hi) in one pass
      const long long span = hi - lo;
      uint32_t cand[8];
      int c[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        cand[i] = (uint32_t)(lo + (span <= 8 ? (i < span ? i : span - 1) : span * i / 8));
        c[i] = 0;
      }
      for (int bb = tid; bb < B; bb += 256) {
        const uint32_t t = (uint32_t)tiles(bb);
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] += (int)ceil_div(t, cand[i]);
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] += __shfl_xor(c[i], o, 64);
      }
      if ((tid & 63) == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) cnt[8 * (tid >> 6) + i] = c[i];
      }
      __syncthreads();
      long long nlo = lo, nhi = hi;
      for (int i = 7; i >= 0; --i) {  // candidates ascend: bracket the first that fits
        const int tot_i = cnt[i] + cnt[8 + i] + cnt[16 + i] + cnt[24 + i];
        if (tot_i <= kTargetCUs) nhi = cand[i];
        else if ((long long)cand[i] + 1 > nlo) nlo = (long long)cand[i] + 1;
      }
      __syncthreads();
      lo = nlo;
      hi = nhi < lo ? lo : nhi;
    }
    S = lo;
  }
  if (S < min_tiles) S = min_tiles;
  if (topk > 0 && S > kMaxTopkGroupTiles) S = kMaxTopkGroupTiles;
  // workgroups in use (records are placed by xcd_workgroup over this count)
  long long cnt = 0;
  for (int bb = tid; bb < B; bb += 256) cnt += ceil_div(tiles(bb), S);
  const int used = (int)block_sum_256(cnt, red);
  auto put = [&](int slot, int4 r) {
    const int i = xcd_workgroup(slot, used);
    rec[i] = r;
    slot_of[i] = slot;
  };
  int run = 0, total;
  for (int base = 0; base < B; base += 256) {
    const int bb = base + tid;
    const int k = bb < B ? (int)ceil_div(tiles(bb), S) : 0;
    const int incl = block_scan_256(k, sc, &total);
    if (bb < B) {
      wcum[bb + 1] = run + incl;
      if (bb <= kPlanCache) sw[bb] = run + incl - k;
      if (bb >= kPlanCache) {  // long batches: these records come from the sequence's own thread
        const int t = tiles_of(bb), len = query_len(lens, bb, s, T);
        for (int p = 0; p < k; ++p)
          put(run + incl - k + p,
              make_int4(bb, (int)floor_div((long long)p * t, k), (int)floor_div((long long)(p + 1) * t, k), len));
      }
    }
    run += total;
  }
  const int nb_cached = B < kPlanCache ? B : kPlanCache;
  if (tid == 0) {
    wcum[0] = 0;
    if (B <= kPlanCache) sw[B] = run;
  }
  __syncthreads();
  // records of the workgroups of the first nb_cached sequences, one per
  // thread: workgroup i belongs to the last sequence b with sw[b] <= i
  // (sequences without tiles share their successor's sw, so they are never
  // the last one below a used workgroup)
  const int used_cached = sw[nb_cached];
  for (int i = tid; i < used_cached; i += 256) {
    int lo = 0, hi = nb_cached - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sw[mid] <= i) lo = mid;
      else hi = mid - 1;
    }
    const int t = tl[lo], k = sw[lo + 1] - sw[lo], p = i - sw[lo];
    put(i, make_int4(lo, (int)floor_div((long long)p * t, k), (int)floor_div((long long)(p + 1) * t, k), sl[lo]));
  }
  for (int i = used + tid; i < G; i += 256) rec[i] = make_int4(-1, 0, 0, 0);
}

enum RowWriteMode { kNoWrite = 0, kWriteBf16 = 1, kWriteFp8 = 2 };

struct RowWrite {
  const uint16_t* kv_new;  // [B][512]
  const uint16_t* pe_new;  // [B][64]
  void* kv;                // bf16 or E4M3 codes [B][T][512]
  float* kv_scale;         // [B][T][4] for the FP8 cache
  uint16_t* pe;            // [B][T][64]
};

// Writer workgroup w of nw: the new rows of the Bq = batch x s query tokens,
// token v = b s + i at cache row cache_lens[b] - s + i; bf16 rows as 72
// 16-byte chunks per thread item, FP8 rows as four 128-element blocks per
// wavefront item.
template <int WRITE>
__device__ __forceinline__ void write_new_rows(const RowWrite& rw, const int32_t* lens, int Bq, int s,
                                               int T, int w, int nw) {
  const int tid = threadIdx.x;
  if (WRITE == kWriteBf16) {
    for (long long g = (long long)w * 256 + tid; g < (long long)Bq * 72; g += (long long)nw * 256) {
      const int v = (int)(g / 72), ch = (int)(g % 72), b = v / s;
      const long long r = (long long)lens[b] - s + (v - b * s);
      if (r < 0 || r >= T) continue;
      store_row_chunk_bf16(rw.kv_new, rw.pe_new, (uint16_t*)rw.kv, rw.pe, (size_t)v,
                           (size_t)b * T + (size_t)r, ch);
    }
  } else if (WRITE == kWriteFp8) {
    const int lane = tid & 63;
    for (long long g = (long long)w * 4 + (tid >> 6); g < (long long)Bq * 4; g += (long long)nw * 4) {
      const int v = (int)(g >> 2), blk = (int)(g & 3), b = v / s;
      const long long r = (long long)lens[b] - s + (v - b * s);
      if (r < 0 || r >= T) continue;  // uniform per wave
      store_row_block_fp8(rw.kv_new, rw.pe_new, (uint8_t*)rw.kv, rw.kv_scale, rw.pe, (size_t)v,
                          (size_t)b * T + (size_t)r, blk, lane);
    }
  }
}

// ---------------------------------------------------------------------------
// absorb: grid (Hx + 1 + writer columns, 4 column blocks of 128, query-token
// ranges), 256 threads, Hx = H + the padding rows of a work item.  B counts
// query tokens (batch x s); work item it holds the ps tokens it ps .. + ps - 1
// (ps = 1, or s when a sequence's tokens share their attention work), whose
// query rows are packed as row i H + h for token i and head h.
// Workgroup (Hx, 0, 0) computes the attention work plan instead; in
// the fused step the workgroups of the writer columns (z = 0) store the new
// cache rows of every sequence at positions cache_lens[b] - s .. - 1 (before
// the attention kernel, which is launched after this one, reads the caches).
//
// Head h, columns 128y..128y+127: the W_UK slice (128 d x 128 c) is staged in
// LDS and held as MFMA B fragments, wave w taking 32 columns; each block of 32
// query tokens is one 32x32 tile per wave (8 MFMAs over d), staged through LDS
// and stored into qt in the attention kernel's fragment order:
//   qt[it][row block rb][k-step st][lane][8], lane = 32 g + (row % 32),
// holding the absorbed-query / q_pe elements 16 st + 8 g .. +7 of row
// 32 rb + (row % 32), so that each of the attention's query loads reads 1 KB
// contiguous per wave.  Workgroup H + j zeroes padding row ps H + j of every
// item.
// ---------------------------------------------------------------------------
template <int WRITE>
__global__ __launch_bounds__(256, 3) void absorb_kernel(const uint16_t* __restrict__ q_nope,
                                                     const uint16_t* __restrict__ q_pe,
                                                     const uint16_t* __restrict__ wkv_b,
                                                     uint16_t* __restrict__ qt, int B, int s, int ps,
                                                     int H, int Hx, int Hp, int bz,
                                                     const int32_t* __restrict__ lens,
                                                     int T, int topk, int min_group_tiles,
                                                     int G, int32_t* wcum, int4* rec,
                                                     int32_t* slot_of, RowWrite rw) {
  // one LDS buffer: the planner's arrays, or the W_UK tile, whose space the
  // output tile reuses once the fragments are in registers
  constexpr int kWRow = 128 + 8;  // padded tile rows (bf16)
  constexpr int kLds = 128 * kWRow * 2 > kPlanLdsBytes ? 128 * kWRow * 2 : kPlanLdsBytes;
  __shared__ __attribute__((aligned(16))) char smem[kLds];
  const int h = blockIdx.x, cblk = blockIdx.y, tid = threadIdx.x;
  const int NI = B / ps;  // work items
  if (h >= Hx) {
    if (blockIdx.z != 0) return;
    if (h == Hx) {  // the plan is over work items, each seeing its last token's rows
      if (cblk == 0) plan_groups(lens, NI, s / ps, T, topk, min_group_tiles, G, wcum, rec, slot_of, smem);
    } else if (WRITE != kNoWrite) {
      write_new_rows<WRITE>(rw, lens, B, s, T, (h - Hx - 1) * 4 + cblk, (gridDim.x - Hx - 1) * 4);
    }
    return;
  }
  const int b_lo = blockIdx.z * bz, b_hi = min(B, b_lo + bz);
  const int HB = Hp >> 5;
  // element offset of chunk (8 values from c, c % 8 == 0) of query row `row`
  // of work item it in qt
  auto frag_row = [&](int it, int row, int c) -> size_t {
    return (((size_t)it * HB + (row >> 5)) * 36 + (c >> 4)) * 512 + (((c >> 3) & 1) * 32 + (row & 31)) * 8;
  };
  // the same for head h of query token b
  auto frag = [&](int b, int c) -> size_t {
    const int it = ps == 1 ? b : b / ps;
    return frag_row(it, (b - it * ps) * H + h, c);
  };
  if (h >= H) {  // padding rows: zero (the attention waves read them); items are
                 // numbered below the tokens, so the z ranges cover them too
    const int row = ps * H + (h - H), it_hi = min(b_hi, NI);
    const int per_b = cblk == 0 ? 24 : 16;
    for (int i = tid; i < (it_hi - b_lo) * per_b; i += 256) {
      const int it = b_lo + i / per_b, ch = i % per_b;
      const int c = ch < 16 ? cblk * 128 + 8 * ch : kC + 8 * (ch - 16);
      *(u32x4*)(qt + frag_row(it, row, c)) = u32x4{0, 0, 0, 0};
    }
    return;
  }
  uint16_t(*sW)[kWRow] = (uint16_t(*)[kWRow])smem;  // W_UK[h][d][128y + c]
  uint16_t(*sD)[kWRow] = (uint16_t(*)[kWRow])smem;  // output tile [b][c], after the fragments
  const int lane = tid & 63, wave = tid >> 6;
  const int cc = 32 * wave + (lane & 31), kg = lane >> 5;
  // A operand of a block of 32 query tokens: lane holds q_nope[b0 + lane % 32]
  // [h][16 ks + 8 kg .. +7]; the first block is loaded with the weights
  u32x4 av[8];
  auto load_q = [&](int b0) {
    const int bb = b0 + (lane & 31);
    const bool ok = bb < b_hi;
    const uint16_t* qrow = q_nope + ((size_t)(ok ? bb : b_lo) * H + h) * kDN + 8 * kg;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) av[ks] = ok ? *(const u32x4*)(qrow + 16 * ks) : u32x4{0, 0, 0, 0};
  };
  load_q(b_lo);
  for (int i = tid; i < 128 * 16; i += 256) {
    const int r = i >> 4, ch = i & 15;
    *(u32x4*)&sW[r][8 * ch] = *(const u32x4*)(wkv_b + ((size_t)h * (kDN + kDV) + r) * kC + cblk * 128 + 8 * ch);
  }
  __syncthreads();
  u32x4 bw[8];  // B[k = d][n = c]: lane holds d = 16 ks + 8 kg + j of column cc
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bw[ks][j] = (uint32_t)sW[16 * ks + 8 * kg + 2 * j][cc] | ((uint32_t)sW[16 * ks + 8 * kg + 2 * j + 1][cc] << 16);
  }
  for (int b0 = b_lo; b0 < b_hi; b0 += 32) {
    if (b0 != b_lo) load_q(b0);
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) acc = mfma32(av[ks], bw[ks], acc);
    __syncthreads();  // fragments read (first block) / sD read (later blocks)
#pragma unroll
    for (int e = 0; e < 16; ++e) sD[8 * (e >> 2) + 4 * kg + (e & 3)][cc] = (uint16_t)f2bf(acc[e]);
    __syncthreads();
    for (int i = tid; i < 32 * 16; i += 256) {
      const int r = i >> 4, ch = i & 15;
      if (b0 + r < b_hi) *(u32x4*)(qt + frag(b0 + r, cblk * 128 + 8 * ch)) = *(const u32x4*)&sD[r][8 * ch];
    }
  }
  if (cblk == 0) {  // q_pe: elements 512..575
    for (int i = tid; i < 8 * (b_hi - b_lo); i += 256) {
      const int b = b_lo + (i >> 3), part = i & 7;
      *(u32x4*)(qt + frag(b, kC + 8 * part)) = *(const u32x4*)(q_pe + ((size_t)b * H + h) * kR + 8 * part);
    }
  }
}

// ---------------------------------------------------------------------------
// attention (split-T flash decoding over a balanced tile split)
//
// grid: the plan's workgroups (at most one per CU, one round in the usual
// case) times the head split HS (1, 2 or 4: a short plan's workgroups are
// split by head blocks so that more CUs share its fixed loads), 256 threads
// = 4 waves (one per SIMD).  Plan workgroup i handles a run of tiles of one
// query token (see make_decode_plan) and its HS workgroups write the
// unnormalised partial O with (m, l) into plan slot slot_of[i].  Its tiles
// (32 cache rows in LDS, row-major [t][576]: 512 latent then 64 rotary
// values) stream through a ring of kStages tiles.  Per tile:
//   1. scores: wave w owns the workgroup's head block w (heads
//      32 (hb0 + w) .. +31; waves past the workgroup's blocks only run the
//      update).  S^T[t][h] = K[t][:] . Qa[h][:] with 36 MFMA 32x32x16 (A:
//      16-byte row reads of the tile, B: the wave's Qa in 144 registers).
//      Lane l holds head l%32, rows 8(e/4)+4(l/32)+e%4.
//   2. online softmax of those heads (the other 16 rows of a head sit in lane
//      l^32); P (bf16) goes to sP[head][tau], tau = row with bits 2 and 3
//      swapped, which makes each lane's 8 consecutive P values contiguous.
//   3. update, split by latent columns: wave w owns O^T[c][h] for c in
//      128w..128w+127 and the workgroup's NHB head blocks (4 NHB accumulator
//      blocks; 256 AGPRs at NHB = 4).  O^T += V^T . P^T with A = V^T from
//      ds_read_tr16_b64 transposing reads of the tile (each read feeds NHB
//      head blocks) and B = P^T from sP.
// Splitting the update by columns keeps the LDS bytes per MFMA low: per tile
// and workgroup 144 KB of score-operand reads, 32 KB of transposing reads and
// 40 KB of P traffic.  At the end each lane's accumulators leave as bf16
// straight to the partial in fragment order (1 KB per store and wave).
//
// bf16 cache: tile j+1 is copied global -> LDS directly (no registers) while
// tile j is processed, its nine loads per thread spread over the score MFMAs.
// One tile in flight per workgroup keeps the loads from ever waiting for
// queue space (a second queued tile makes the issuing wave stall until the
// first lands).  FP8 cache: each wave stages its part of tile j+2 (codes,
// scales, rotary rows) in its own LDS region by direct loads (a dense tile's
// spread over the score chain), and converts its part of tile j+1 to
// bf16(float(code) * scale) in one pass before the score chain of tile j.
//
// LDS swizzle: logical 16-byte chunk ch of row t sits at chunk ch ^ F(t),
// F(t) = 4((t>>1)&1) + ((t>>2)&3), which only permutes chunks inside their
// aligned group of 8.  gfx950 LDS serves 256 bytes per cycle (64 banks): a
// b128 read is served 16 lanes at a time and a b64 transposing read 32 lanes
// at a time.  With the 1152-byte row stride this F puts the 16 rows of a score
// read, and the 4 rows x 4 chunks of a transposing read, on distinct banks.
// ---------------------------------------------------------------------------
constexpr int kTT = kTileRows;              // rows per tile
constexpr int kStages = 3;                  // tiles in the LDS ring
constexpr int kTileElems = kTT * kQK;       // bf16 elements per tile (36 KB)
constexpr int kMaxIdx = kMaxTopkGroupTiles * kTT;  // top-k entries staged per workgroup
constexpr int kAttnWaves = 4;
constexpr int kAttnThreads = 64 * kAttnWaves;
constexpr int kPStride = 40;                // bf16 per sP row (32 + 8 padding)
constexpr int kScoreAhead = 4;              // score operand reads issued ahead of their MFMA
constexpr int kOStride = 520;               // bf16 per staged output row (512 + 8 padding)
// FP8 staging region of one wave: latent block `wave` (128 codes) of the 32
// rows of a tile, the 32 rows' four scales, and rotary rows 8 wave .. +7.
constexpr int kFp8WaveCodes = kTT * kBlk;                   // 4096
constexpr int kFp8WaveScales = kTT * 4;                     // 128
constexpr int kFp8WaveRope = 8 * kR * 2;                    // 1024
constexpr int kFp8Wave = kFp8WaveCodes + kFp8WaveScales + kFp8WaveRope;
constexpr int kFp8Stage = 4 * kFp8Wave;
static_assert(32 * kOStride <= kTileElems, "a 32-head block of O fits one ring slot");

struct AttnArgs {
  const uint16_t* qt;
  const void* kv;
  const float* kv_scale;
  const uint16_t* pe;
  const int32_t* topk_idx;
  const int4* rec;        // [grid] {work item or -1, first tile, end tile, length}
  const int32_t* slot_of; // [grid] plan slot (partial index) of each workgroup
  uint16_t* part_o;       // [grid][Hp][512]
  float* part_ml;         // [grid][H][2]
  // H: query rows per work item (ps x heads), Hp: H padded to 32; s: work
  // items per sequence (item b reads sequence b / s); ps: query tokens per
  // item (1, or the sequence's s tokens, rows i hq .. for token i); hq: heads
  int s, H, Hp, T, topk, head_blocks, ps, hq;
  int head_split;  // workgroups per plan workgroup, each with head_blocks / head_split blocks
  float scale_log2;
};

__device__ __forceinline__ int swz(int t) { return (((t >> 1) & 1) << 2) | ((t >> 2) & 3); }
__device__ __forceinline__ int tile_off(int t, int ch) { return t * kQK + ((ch ^ swz(t)) << 3); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// 4-byte global -> LDS copy for each lane (lane l's dword at base + OFF + 4 l),
// issued after `dep` is available.
template <int OFF>
__device__ __forceinline__ void lds_dma4_after(const void* src, uint32_t base, uint32_t dep) {
  asm volatile("s_add_u32 m0, %1, %2\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(base), "i"(OFF), "v"(dep)
               : "memory", "m0", "scc");
}

// The same copies addressed as a 64-bit scalar base plus a 32-bit per-lane
// byte offset (no per-lane 64-bit address arithmetic).  The base must be
// the same in every lane; it is moved to scalar registers explicitly.
__device__ __forceinline__ uint64_t uniform64(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
template <int OFF>
__device__ __forceinline__ void lds_dma16_s(uint64_t sbase, uint32_t voff, uint32_t base, uint32_t dep) {
  asm volatile("s_add_u32 m0, %2, %3\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(base), "i"(OFF), "v"(dep)
               : "memory", "m0", "scc");
}
template <int OFF>
__device__ __forceinline__ void lds_dma4_s(uint64_t sbase, uint32_t voff, uint32_t base, uint32_t dep) {
  asm volatile("s_add_u32 m0, %2, %3\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(base), "i"(OFF), "v"(dep)
               : "memory", "m0", "scc");
}

// lds_dma16 issued after `dep` is available: when dep was read from the LDS
// bytes this load overwrites, that read has completed first.
template <int OFF>
__device__ __forceinline__ void lds_dma16_after(const void* src, uint32_t base, uint32_t dep) {
  asm volatile("s_add_u32 m0, %1, %2\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(base), "i"(OFF), "v"(dep)
               : "memory", "m0", "scc");
}

__device__ __forceinline__ u32x2 ds_read_tr16(const uint16_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Workgroup barrier that publishes this wave's LDS writes but, unlike
// __syncthreads, does not wait for its global loads still in flight.
#define MLA_LDS_BARRIER()                                           \
  do {                                                              \
    __builtin_amdgcn_s_waitcnt(0xC07F); /* lgkmcnt(0) only */      \
    asm volatile("s_barrier" ::: "memory");                         \
  } while (0)

// Lambdas of the attention kernel carry accumulators by reference: they must
// be inlined, or those live in scratch memory.
#define MLA_INLINE __attribute__((always_inline))

template <int S>
struct Stage {
  static constexpr int value = S;
};

// NHB: head blocks per workgroup the update keeps accumulators for (4; or the
// workgroup's exact count 1 or 2 when it has that few: no MFMAs on blocks
// whose probabilities would all be zero).  PACK: the work item is a sequence
// whose ps query tokens share the tiles; each query row is then masked at its
// own token's length (token i of ps sees len - (ps - 1 - i) rows).
template <bool FP8, bool TOPK, int NHB, bool PACK = false>
__global__ __launch_bounds__(kAttnThreads, 1) void attn_kernel(AttnArgs a) {
  // Workgroup x runs head group hq (of HS) of plan workgroup grp; the HS
  // workgroups of one plan workgroup sit on its XCD (x % 8 == grp % 8) and
  // share its tiles in that XCD's L2.
  const int HS = a.head_split, x = blockIdx.x;
  const int grp = (x / (8 * HS)) * 8 + (x & 7), hq = (x >> 3) % HS;
  const int nhb = a.head_blocks / HS, hb0 = hq * nhb;  // this workgroup's head blocks
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int4 rec = a.rec[grp];
  const int part_slot = a.slot_of[grp];
  if (rec.x < 0) return;  // whole workgroup: not used by the plan
  const int b = rec.x, t_lo = rec.y, t_hi = rec.z, len = rec.w;
  const int n_b = TOPK ? (len > 0 ? a.topk : 0) : len;
  const int p0 = t_lo * kTT, p1 = min(t_hi * kTT, n_b);
  const int ntiles = t_hi - t_lo;
  const size_t seq_row0 = (size_t)(a.s == 1 ? b : b / a.s) * a.T;  // b: work item
  const size_t slot_id = part_slot;

  // One LDS array per ring slot (not one 2-D array): the slot a tile lives in
  // is a compile-time constant in the loop body below.
  __shared__ __attribute__((aligned(16))) uint16_t sT0[kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t sT1[kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t sT2[kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t sP[2 * 128 * kPStride];  // by tile parity
  __shared__ float sAlpha[2 * 128];                                          // by tile parity
  __shared__ uint32_t sMask[kStages];
  __shared__ uint32_t sRescale[3];  // by tile mod 3: some head of the tile rescales
  __shared__ int sIdx[TOPK ? kMaxIdx : 1];
  // FP8 cache: raw tile (codes [32][512] B, scales [32][4] fp32, rotary
  // [32][64] bf16) staged by direct loads one tile ahead
  __shared__ __attribute__((aligned(16))) uint8_t sF[FP8 ? kFp8Stage : 16];
  static_assert(kStages == 3, "one LDS array per ring slot");
  auto slot = [&](auto S) MLA_INLINE -> uint16_t* {
    constexpr int st = decltype(S)::value;
    if constexpr (st == 0) return sT0;
    else if constexpr (st == 1) return sT1;
    else return sT2;
  };

  const bool active = wave < nhb;  // this wave has score heads
  const int n = lane & 31, g = lane >> 5;
  const int head = wave * 32 + n;           // in this workgroup (P rows, alpha)
  const int ghead = (hb0 + wave) * 32 + n;  // query row of the work item
  // Rows this lane's query token sees (padding rows: any value), recomputed
  // from the lane number at each use: a value held across the loop would take
  // a register the score chain needs.
  auto row_lim = [&]() MLA_INLINE -> int {
    int ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    const int row = (hb0 + wave) * 32 + (ln & 31);
    return len - (a.ps - 1 - min(row / a.hq, a.ps - 1));
  };

  // P rows and l of heads without a score wave stay zero; their alpha stays 1.
  for (int i = tid; i < 2 * 128 * kPStride / 2; i += kAttnThreads) ((uint32_t*)sP)[i] = 0u;
  if (tid < 128) {
    sAlpha[tid] = 1.f;
    sAlpha[128 + tid] = 1.f;
  }

  // Per-lane LDS bases (element offsets inside a tile).
  //   score k-step st reads logical chunk 2st+g of row n:
  //     phys = 8(st>>2) + ((2(st&3)+g) ^ F(n))                 -> 4 bases
  //   update (column block m, k-step u, half h): lane 4r+q of 16-lane group
  //     Q reads row 16u + 8h + 4(Q>>1) + r, columns
  //     128w + 32m + 16(Q&1) + 4q .. +3                         -> 4 bases
  const int fn = swz(n);
  int sc_base[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) sc_base[k] = n * kQK + (((2 * k + g) ^ fn) << 3);
  const int lq = lane >> 4, rr = (lane & 15) >> 2, qq = lane & 3;
  const int tr_x = 2 * (lq & 1) + (qq >> 1);
  int tr_base[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int tr_t = 8 * h + 4 * (lq >> 1) + rr;
#pragma unroll
    for (int par = 0; par < 2; ++par)
      tr_base[h][par] = tr_t * kQK + 128 * wave + (((4 * par + tr_x) ^ swz(tr_t)) << 3) + 4 * (qq & 1);
  }

  if (TOPK) {  // stage this workgroup's row indices; invalid entries become -1
    for (int i = tid; i < p1 - p0; i += kAttnThreads) {
      const int r = a.topk_idx[(size_t)b * a.topk + p0 + i];
      sIdx[i] = (r >= 0 && r < len) ? r : -1;
    }
  }
  if (tid < 3) sRescale[tid] = 0u;
  __syncthreads();

  // Row of tile position t (any valid row when the position selects
  // nothing: its score is masked, and it must only be finite).
  auto tile_row = [&](int pt, int t) MLA_INLINE -> int {
    const int pos = pt + t;
    if (TOPK) {
      const int r = pos < p1 ? sIdx[pos - p0] : -1;
      return r >= 0 ? r : 0;
    }
    return pos < p1 ? pos : p1 - 1;
  };
  // Bit t of a tile's mask: tile row t selects a position.
  auto publish_mask = [&](int pt, int stage) MLA_INLINE {
    if (TOPK) {
      if (wave == 0) {
        const int pos = pt + lane;
        const bool ok = lane < 32 && pos < p1 && sIdx[pos - p0] >= 0;
        const uint32_t m = (uint32_t)__ballot(ok);
        if (lane == 0) sMask[stage] = m;
      }
    } else if (tid == 0) {
      const int rows = p1 - pt;
      sMask[stage] = rows >= 32 ? 0xFFFFFFFFu : ((1u << rows) - 1u);
    }
  };

  // ---- bf16 tiles: direct global -> LDS.  Instruction i (0..35) of a tile
  // writes LDS chunks 64i .. 64i+63 in lane order; wave w issues i = w + 4k.
  // Lane position P = 64i + lane grows by 256 = 3 rows (of 72 chunks) + 40
  // chunks per instruction.
  struct DmaCursor {
    int t, phys;
  };
  auto dma_start = [&]() MLA_INLINE -> DmaCursor {
    int P = 64 * wave + lane;
    asm volatile("" : "+v"(P));  // recomputed per tile, not kept live
    const int t = P / 72;
    return DmaCursor{t, P - 72 * t};
  };
  // base: LDS byte address of the tile slot plus 1024 * wave, laundered so
  // the compiler keeps one value per tile instead of nine per slot.
  auto dma_base = [&](uint16_t* dst) MLA_INLINE -> uint32_t {
    uint32_t base = lds_addr(dst) + 1024u * wave;
    asm volatile("" : "+s"(base));
    return base;
  };
  auto dma_step = [&](DmaCursor& c, int pt, uint32_t base, auto K) MLA_INLINE {
    constexpr int k = decltype(K)::value;
    const int ch = c.phys ^ swz(c.t);
    const size_t row = seq_row0 + tile_row(pt, c.t);
    const uint16_t* src = ch < 64 ? (const uint16_t*)a.kv + row * kC + ch * 8
                                  : a.pe + row * kR + (ch - 64) * 8;
    lds_dma16<4096 * k>(src, base);
    c.phys += 40;
    c.t += 3;
    if (c.phys >= 72) {
      c.phys -= 72;
      c.t += 1;
    }
  };
  auto dma_all = [&](DmaCursor& c, int pt, uint32_t base) MLA_INLINE {
    dma_step(c, pt, base, Stage<0>{});
    dma_step(c, pt, base, Stage<1>{});
    dma_step(c, pt, base, Stage<2>{});
    dma_step(c, pt, base, Stage<3>{});
    dma_step(c, pt, base, Stage<4>{});
    dma_step(c, pt, base, Stage<5>{});
    dma_step(c, pt, base, Stage<6>{});
    dma_step(c, pt, base, Stage<7>{});
    dma_step(c, pt, base, Stage<8>{});
  };
  auto issue_bf16 = [&](int j, auto S) MLA_INLINE {
    const int pt = p0 + j * kTT;
    DmaCursor c = dma_start();
    const uint32_t base = dma_base(slot(S));
    dma_all(c, pt, base);
    publish_mask(pt, decltype(S)::value);
  };
  // Fast path for a dense tile of 32 selected rows: the rows are consecutive,
  // so each of a lane's nine loads sits at a fixed byte offset from the tile's
  // first latent or rotary row.  Offsets are 16-bit (latent t*1024 + ch*16 <
  // 32768, rotary t*128 + (ch-64)*16 with bit 15 set), two per register,
  // computed once; a load then costs a select and a 64-bit add instead of
  // the row / chunk / swizzle arithmetic.
  uint32_t doff[5] = {0u, 0u, 0u, 0u, 0u};
  if (!FP8 && !TOPK) {
    DmaCursor c = dma_start();
    auto put = [&](auto K) MLA_INLINE {  // explicit steps: doff is only indexed by constants
      constexpr int k = decltype(K)::value;
      const int ch = c.phys ^ swz(c.t);
      const uint32_t off = ch < 64 ? (uint32_t)(c.t * 1024 + ch * 16) : (uint32_t)(c.t * 128 + (ch - 64) * 16) | 0x8000u;
      doff[k >> 1] |= off << (16 * (k & 1));
      c.phys += 40;
      c.t += 3;
      if (c.phys >= 72) {
        c.phys -= 72;
        c.t += 1;
      }
    };
    put(Stage<0>{});
    put(Stage<1>{});
    put(Stage<2>{});
    put(Stage<3>{});
    put(Stage<4>{});
    put(Stage<5>{});
    put(Stage<6>{});
    put(Stage<7>{});
    put(Stage<8>{});
  }
  struct FullTile {
    const char* kv;
    const char* pe;
    uint32_t base;
  };
  auto full_tile = [&](int j, auto S) MLA_INLINE -> FullTile {
    const int pt = p0 + j * kTT;
    return FullTile{(const char*)a.kv + (seq_row0 + pt) * (size_t)(kC * 2),
                    (const char*)a.pe + (seq_row0 + pt) * (size_t)(kR * 2), dma_base(slot(S))};
  };
  auto full_load = [&](const FullTile& ft, auto K) MLA_INLINE {
    constexpr int k = decltype(K)::value;
    uint32_t d = doff[k >> 1];
    asm volatile("" : "+v"(d));  // unpacked here, not kept as nine 64-bit offsets
    const uint32_t o = (d >> (16 * (k & 1))) & 0xFFFFu;
    const char* pe_row = ft.pe;  // select values, not struct members (keeps ft in registers)
    const char* kv_row = ft.kv;
    const char* src = ((o & 0x8000u) ? pe_row : kv_row) + (o & 0x7FFFu);
    lds_dma16<4096 * k>(src, ft.base);
  };
  auto full_all = [&](const FullTile& ft) MLA_INLINE {
    full_load(ft, Stage<0>{});
    full_load(ft, Stage<1>{});
    full_load(ft, Stage<2>{});
    full_load(ft, Stage<3>{});
    full_load(ft, Stage<4>{});
    full_load(ft, Stage<5>{});
    full_load(ft, Stage<6>{});
    full_load(ft, Stage<7>{});
    full_load(ft, Stage<8>{});
  };

  // ---- FP8 tiles: every wave stages and converts its own part of a tile, so
  // no barrier separates the staging from the conversion.  Wave w's region of
  // sF receives, by direct loads one tile ahead of the conversion:
  //   units u = 0..3 (1 KB each, rows 8u .. 8u+7): lane l's 16 bytes are codes
  //     16 (l % 8) .. +15 of latent block w of row 8u + l / 8
  //   scales: 4 bytes per lane l < 32, the block-w scale of row 8 (l % 4) + l / 4
  //     (so lane l reads the scales of its four rows 8u + l / 8 as one 16 bytes)
  //   rotary: 16 bytes, chunk l % 8 of rotary row 8 w + l / 8
  // The conversion writes bf16(float(code) * scale) of lane l's 16 codes per
  // unit, and the rotary rows, into the tile's ring slot.
  uint8_t* const fregion = sF + (FP8 ? kFp8Wave * wave : 0);
  // lane index recomputed at each use: hoisted per-slot addresses would not
  // fit in the registers the loop leaves
  auto fresh_lane = [&]() MLA_INLINE -> int {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    return ln;
  };
  // Per-lane byte offsets of a dense tile of 32 selected rows, from its first
  // row, packed two 16-bit values per register (computed once):
  //   fo_a: codes of unit 0 (kv bytes) | bf16 rotary store (tile elements)
  //   fo_b: scale (kv_scale bytes)     | rotary load (pe bytes)
  //   fo_st[p]: bf16 stores of units p, p + 2 (tile elements), halves 0 | 1
  uint32_t fo_a = 0u, fo_b = 0u, fo_st0 = 0u, fo_st1 = 0u;
  // unpacked at each use (hoisted per-slot addresses would not fit)
  auto fresh = [](uint32_t v) MLA_INLINE -> uint32_t {
    asm volatile("" : "+v"(v));
    return v;
  };
  if (FP8) {  // (with top-k only the rotary store offset is used)
    const int x = lane >> 3, c = lane & 7;
    fo_a = (uint32_t)(x * kC + kBlk * wave + 16 * c) | ((uint32_t)tile_off(8 * wave + x, 64 + c) << 16);
    if (!TOPK)
      fo_b = (uint32_t)(16 * (8 * (lane & 3) + (lane >> 2)) + 4 * wave) | ((uint32_t)((8 * wave + x) * kR * 2 + 16 * c) << 16);
    fo_st0 = (uint32_t)tile_off(x, 16 * wave + 2 * c) | ((uint32_t)tile_off(x, 16 * wave + 2 * c + 1) << 16);
    fo_st1 = (uint32_t)tile_off(8 + x, 16 * wave + 2 * c) | ((uint32_t)tile_off(8 + x, 16 * wave + 2 * c + 1) << 16);
  }
  // Load n of a raw tile: 0 scales, 1..4 code units 0..3, 5 rotary rows (the
  // staging bytes they replace have been read: the caller waits for that).
  // A dense tile of 32 selected rows takes the fixed offsets above from its
  // first row (scalar base): this form is also issued inside the score chain,
  // which has no registers to spare for the general form's per-lane rows.
  auto fp8_load_full = [&](int j, auto N) MLA_INLINE {
    constexpr uint32_t dep = 0u;
    constexpr int n = decltype(N)::value;
    const size_t r0 = seq_row0 + p0 + j * kTT;
    uint32_t base = lds_addr(fregion);
    asm volatile("" : "+s"(base));
    if constexpr (n >= 1 && n <= 4) {
      constexpr int u = n - 1;
      lds_dma16_s<1024 * u>(uniform64((const uint8_t*)a.kv + r0 * kC + 4096 * u), fresh(fo_a) & 0xFFFFu, base, dep);
    } else if constexpr (n == 0) {
      if (lane < 32) lds_dma4_s<kFp8WaveCodes>(uniform64(a.kv_scale + r0 * 4), fresh(fo_b) & 0xFFFFu, base, dep);
    } else {
      lds_dma16_s<kFp8WaveCodes + kFp8WaveScales>(uniform64(a.pe + r0 * kR), fresh(fo_b) >> 16, base, dep);
    }
  };
  // Any tile (a dense one goes to the form above; any other computes each
  // lane's row).
  auto fp8_load = [&](int j, auto N) MLA_INLINE {
    constexpr uint32_t dep = 0u;  // no read to order after
    constexpr int n = decltype(N)::value;
    const int pt = p0 + j * kTT;
    if (!TOPK && pt + kTT <= p1) {
      fp8_load_full(j, N);
      return;
    }
    uint32_t base = lds_addr(fregion);
    asm volatile("" : "+s"(base));
    const int ln = fresh_lane();
    if constexpr (n >= 1 && n <= 4) {
      constexpr int u = n - 1;
      const int r = 8 * u + (ln >> 3);
      const size_t row = seq_row0 + tile_row(pt, r);
      lds_dma16_after<1024 * u>((const uint8_t*)a.kv + row * kC + kBlk * wave + 16 * (ln & 7), base, dep);
    } else if constexpr (n == 0) {
      if (ln < 32) {
        const int r = 8 * (ln & 3) + (ln >> 2);
        const size_t row = seq_row0 + tile_row(pt, r);
        lds_dma4_after<kFp8WaveCodes>(a.kv_scale + row * 4 + wave, base, dep);
      }
    } else {
      const int r = 8 * wave + (ln >> 3);
      const size_t row = seq_row0 + tile_row(pt, r);
      lds_dma16_after<kFp8WaveCodes + kFp8WaveScales>(a.pe + row * kR + 8 * (ln & 7), base, dep);
    }
  };
  auto fp8_load_all = [&](int j) MLA_INLINE {
    fp8_load(j, Stage<0>{});
    fp8_load(j, Stage<1>{});
    fp8_load(j, Stage<2>{});
    fp8_load(j, Stage<3>{});
    fp8_load(j, Stage<4>{});
    fp8_load(j, Stage<5>{});
  };
  auto fp8_read = [&](auto U) MLA_INLINE -> u32x4 {
    return *(const u32x4*)(fregion + 1024 * decltype(U)::value + 16 * fresh_lane());
  };
  auto fp8_scales = [&]() MLA_INLINE -> f32x4 {  // scales of rows 8u + l / 8, u = 0..3
    return *(const f32x4*)(fregion + kFp8WaveCodes + 16 * (fresh_lane() >> 3));
  };
  // four codes -> two packed bf16 pairs, bf16(float(code) * scale)
  auto fp8_cvt4 = [&](uint32_t q, float sc) MLA_INLINE -> u32x2 {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)q, false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)q, true);
    return u32x2{cvt_pk_bf16(lo[0] * sc, lo[1] * sc), cvt_pk_bf16(hi[0] * sc, hi[1] * sc)};
  };
  // store half `c` (8 values) of unit u of this lane into the tile: units u
  // and u + 2 share the swizzle (rows 8u + l/8 and 8u + 16 + l/8)
  auto fp8_store = [&](uint16_t* dst, auto U, int c, const u32x4& w) MLA_INLINE {
    constexpr int u = decltype(U)::value;
    const uint32_t pk = fresh((u & 1) ? fo_st1 : fo_st0);
    const uint32_t off = c ? (pk >> 16) : (pk & 0xFFFFu);
    *(u32x4*)(dst + off + (u >> 1) * 16 * kQK) = w;
  };
  auto fp8_write = [&](uint16_t* dst, auto U, const u32x4& q, float sc) MLA_INLINE {
    const u32x2 a = fp8_cvt4(q[0], sc), b = fp8_cvt4(q[1], sc);
    const u32x2 c = fp8_cvt4(q[2], sc), d = fp8_cvt4(q[3], sc);
    fp8_store(dst, U, 0, u32x4{a[0], a[1], b[0], b[1]});
    fp8_store(dst, U, 1, u32x4{c[0], c[1], d[0], d[1]});
  };
  auto fp8_rope_read = [&]() MLA_INLINE -> u32x4 {
    return *(const u32x4*)(fregion + kFp8WaveCodes + kFp8WaveScales + 16 * fresh_lane());
  };
  auto fp8_rope_write = [&](uint16_t* dst, const u32x4& v) MLA_INLINE {
    *(u32x4*)(dst + (fresh(fo_a) >> 16)) = v;
  };
  auto fp8_rope = [&](uint16_t* dst) MLA_INLINE { fp8_rope_write(dst, fp8_rope_read()); };
  // the whole conversion of tile j into slot S in one go (prologue, and waves
  // without score heads)
  auto fp8_convert_all = [&](int j, auto S) MLA_INLINE {
    uint16_t* dst = slot(S);
    const f32x4 sc = fp8_scales();
    const u32x4 q0 = fp8_read(Stage<0>{}), q1 = fp8_read(Stage<1>{});
    const u32x4 q2 = fp8_read(Stage<2>{}), q3 = fp8_read(Stage<3>{});
    fp8_write(dst, Stage<0>{}, q0, sc[0]);
    fp8_write(dst, Stage<1>{}, q1, sc[1]);
    fp8_write(dst, Stage<2>{}, q2, sc[2]);
    fp8_write(dst, Stage<3>{}, q3, sc[3]);
    fp8_rope(dst);
    publish_mask(p0 + j * kTT, decltype(S)::value);
  };

  // O accumulators o[NHB m + nb]: columns 128w + 32m + ..., heads 32nb + ...
  // Every definition of o[] is an MFMA result (zero operands for the initial
  // value and in the rescale below): a VALU definition would make the
  // compiler keep the loop-carried accumulators in VGPRs and copy them every
  // iteration.
  const u32x4 zq = {0u, 0u, 0u, 0u};
  f32x16 o[4 * NHB];
#pragma unroll
  for (int i = 0; i < 4 * NHB; ++i) o[i] = mfma32(zq, zq, f32x16{});
  float m_run = -INFINITY, l_run = 0.f;

  // ---- pipeline prologue: the first tiles and the query are loaded
  // together, and everything is complete before the loop
  if (!FP8) issue_bf16(0, Stage<0>{});
  else fp8_load_all(0);
  // Absorbed query + q_pe of this lane's head: k-step s covers elements
  // 16s..16s+15, lane group g holds 8 of them (stored in this order by the
  // absorb kernel: one 1 KB row per wave and k-step).
  u32x4 qreg[36];
  if (active) {
    const u32x4* src = (const u32x4*)(a.qt + ((size_t)b * a.head_blocks + hb0 + wave) * (36 * 512)) + lane;
#pragma unroll
    for (int st = 0; st < 36; ++st) qreg[st] = src[64 * st];
  }
  MLA_WAIT_VMCNT(0);
  if (FP8) {  // this wave's part of tile 0 into slot 0, then the raw tile 1 on its way
    fp8_convert_all(0, Stage<0>{});
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): staging reads done before the reload
    if (1 < ntiles) fp8_load_all(1);
  }

  // ---- software pipeline over the tiles, one workgroup barrier per tile.
  // Body j: barrier; loads of tile j+1 (slot of tile j-2); scores of tile j;
  // then the update with tile j-1 (its P, the rescale by its alpha) with the
  // softmax of tile j interleaved, so the VALU work of the softmax runs while
  // the matrix cores work on the update.  P and alpha are double-buffered by
  // tile parity and the rescale flags cycle over three tiles: each is written
  // in body j, read in body j+1 and cleared in body j+2, with a barrier
  // between every two of these.
  auto pbuf = [&](int jj) MLA_INLINE -> uint16_t* { return sP + (jj & 1) * (128 * kPStride); };
  auto rescale = [&](int jj) MLA_INLINE {
    if (sRescale[(jj + 3) % 3]) {  // rare: some head's running max moved
      const float* al_src = sAlpha + (jj & 1) * 128;
      float al[NHB];
#pragma unroll
      for (int nb = 0; nb < NHB; ++nb) al[nb] = al_src[32 * nb + n];
#pragma unroll
      for (int i = 0; i < 4 * NHB; ++i) {
        f32x16 tcopy = o[i];
        asm volatile("" : "+v"(tcopy));  // scale a copy; o[i] itself stays an MFMA value
        o[i] = mfma32(zq, zq, tcopy * al[i % NHB]);
      }
    }
  };
  // Update step (u, m): A = 2 transposing reads of tile pt (rows 16u + 4g + r
  // and 16u + 8 + 4g + r), B = P^T of head block nb (pb, 16 bytes per lane).
  auto tr_read_any = [&](const uint16_t* pt, int u, int m) MLA_INLINE -> u32x4 {
    const uint16_t* base = pt + 16 * u * kQK + 64 * (m >> 1);
    const u32x2 v0 = ds_read_tr16(base + tr_base[0][m & 1]);
    const u32x2 v1 = ds_read_tr16(base + tr_base[1][m & 1]);
    return u32x4{v0[0], v0[1], v1[0], v1[1]};
  };
  auto pv_mfma_any = [&](const u32x4& va, const u32x4 (&pb)[NHB], int m) MLA_INLINE {
#pragma unroll
    for (int nb = 0; nb < NHB; ++nb) o[NHB * m + nb] = mfma32(va, pb[nb], o[NHB * m + nb]);
  };
  auto pb_read_any = [&](const uint16_t* pp, u32x4 (&pb)[NHB], int u) MLA_INLINE {
#pragma unroll
    for (int nb = 0; nb < NHB; ++nb) pb[nb] = *(const u32x4*)(pp + (32 * nb + n) * kPStride + 16 * u + 8 * g);
  };
  // Update with tile jp interleaved with the softmax of tile j held in s:
  // eight scheduling regions, each with the four MFMAs of one update step
  // (whose A operand was read one region earlier) and a slice of the softmax.
  auto update_softmax = [&](auto PV, const uint16_t* ptile, int jp, f32x16& s, int j,
                            uint32_t mask) MLA_INLINE {
    constexpr bool pv = decltype(PV)::value;  // false: softmax only (the first tile)
    // In-order issue: VALU work only runs under an MFMA if it sits between
    // MFMAs in program order, so each region is laid out as its LDS reads,
    // then MFMA, VALU x5, MFMA, VALU x5, ... (masks: 0x100 LDS read, 0x8
    // MFMA, 0x2 VALU, 0x200 LDS write).
    auto interleave = [&]() MLA_INLINE {
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int r = 0; r < NHB; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x002, 64, 0);
      __builtin_amdgcn_sched_group_barrier(0x200, 8, 0);
    };
    const uint16_t* pp = pbuf(jp);
    u32x4 pb[NHB], va[4];
    float mx, m_use, m_sub, alpha;
    auto tr_read = [&](const uint16_t* pt, int u, int m) MLA_INLINE -> u32x4 {
      if constexpr (pv) return tr_read_any(pt, u, m);
      else return u32x4{0u, 0u, 0u, 0u};
    };
    auto pv_mfma = [&](const u32x4& va, const u32x4(&pb)[NHB], int m) MLA_INLINE {
      if constexpr (pv) pv_mfma_any(va, pb, m);
    };
    auto pb_read = [&](const uint16_t* pp, u32x4(&pb)[NHB], int u) MLA_INLINE {
      if constexpr (pv) pb_read_any(pp, pb, u);
    };
    pb_read(pp, pb, 0);
    va[0] = tr_read(ptile, 0, 0);
    va[1] = tr_read(ptile, 0, 1);
    va[2] = tr_read(ptile, 0, 2);
    // region 0 (A operands are read three steps ahead of their MFMAs)
    va[3] = tr_read(ptile, 0, 3);
    pv_mfma(va[0], pb, 0);
    if (mask != 0xFFFFFFFFu) {  // partial tile (wave-uniform branch)
      const uint32_t ml = (mask >> (4 * g)) & 0x0F0F0F0Fu;  // rows 8a + 4g + b -> bit 8a + b
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (!((ml >> (8 * (e >> 2) + (e & 3))) & 1u)) s[e] = -INFINITY;
    }
    mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    // region 1: the other 16 rows of this lane's head sit in lane l ^ 32
    va[0] = tr_read(ptile, 1, 0);
    pv_mfma(va[1], pb, 1);
    mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(s[8], s[9]), fmaxf(s[10], s[11])),
                         fmaxf(fmaxf(s[12], s[13]), fmaxf(s[14], s[15]))));
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    // region 2: online softmax in log2 units; the running max only moves when
    // the new one exceeds it by more than 8 (probabilities stay <= 2^8), which
    // skips most rescales of O without changing the result
    va[1] = tr_read(ptile, 1, 1);
    pv_mfma(va[2], pb, 2);
    {
      const float mt = mx * a.scale_log2;
      m_use = (m_run == -INFINITY || mt > m_run + 8.0f) ? fmaxf(mt, m_run) : m_run;
      m_sub = (m_use == -INFINITY) ? 0.f : m_use;
      alpha = (m_use == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_use);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] = __builtin_amdgcn_exp2f(fmaf(s[e], a.scale_log2, -m_sub));
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    // region 3
    va[2] = tr_read(ptile, 1, 2);
    pv_mfma(va[3], pb, 3);
    pb_read(pp, pb, 1);  // B operand of the second k-step
#pragma unroll
    for (int e = 4; e < 8; ++e) s[e] = __builtin_amdgcn_exp2f(fmaf(s[e], a.scale_log2, -m_sub));
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    // region 4
    va[3] = tr_read(ptile, 1, 3);
    pv_mfma(va[0], pb, 0);
#pragma unroll
    for (int e = 8; e < 12; ++e) s[e] = __builtin_amdgcn_exp2f(fmaf(s[e], a.scale_log2, -m_sub));
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    // region 5
    pv_mfma(va[1], pb, 1);
#pragma unroll
    for (int e = 12; e < 16; ++e) s[e] = __builtin_amdgcn_exp2f(fmaf(s[e], a.scale_log2, -m_sub));
    const float lsum = (((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]))) +
                       (((s[8] + s[9]) + (s[10] + s[11])) + ((s[12] + s[13]) + (s[14] + s[15])));
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    // region 6: P rows 8a + 4g + b land at tau = 16(a>>1) + 8g + 4(a&1) + b:
    // two contiguous 16-byte pieces per lane
    pv_mfma(va[2], pb, 2);
    l_run = l_run * alpha + lsum;
    m_run = m_use;
    if (active) {  // waves without score heads leave their (zero) P rows alone
      uint16_t* prow = pbuf(j) + head * kPStride + 8 * g;
      *(u32x4*)(prow) = u32x4{cvt_pk_bf16(s[0], s[1]), cvt_pk_bf16(s[2], s[3]),
                              cvt_pk_bf16(s[4], s[5]), cvt_pk_bf16(s[6], s[7])};
      *(u32x4*)(prow + 16) = u32x4{cvt_pk_bf16(s[8], s[9]), cvt_pk_bf16(s[10], s[11]),
                                   cvt_pk_bf16(s[12], s[13]), cvt_pk_bf16(s[14], s[15])};
    }
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    // region 7
    pv_mfma(va[3], pb, 3);
    if (active) {
      if (g == 0) sAlpha[(j & 1) * 128 + head] = alpha;
      if (alpha != 1.f) sRescale[j % 3] = 1u;  // benign race: every writer stores 1
    }
    interleave();
    __builtin_amdgcn_sched_barrier(0);
  };
  // The update alone (after the last tile).
  auto update_only = [&](const uint16_t* ptile, int jp) MLA_INLINE {
    const uint16_t* pp = pbuf(jp);
    u32x4 pb[NHB];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      pb_read_any(pp, pb, u);
#pragma unroll
      for (int m = 0; m < 4; ++m) pv_mfma_any(tr_read_any(ptile, u, m), pb, m);
    }
  };

  // Tile j lives in ring slot S = j % kStages (a compile-time constant here).
  auto body = [&](int j, auto S, auto PV) MLA_INLINE {
    constexpr int st = decltype(S)::value;
    constexpr int s1 = (st + 1) % kStages;  // slot of tile j + 1 (held tile j - 2)
    constexpr int sp = (st + 2) % kStages;  // slot of tile j - 1
    // Barrier: tile j visible to every wave (the bf16 path first waits for its
    // own loads of it); P, alpha and flag of tile j-1 visible; every wave is
    // done with tile j-2 and with the P buffer and flag the softmax of tile j
    // is about to write.
    if (!FP8) MLA_WAIT_VMCNT(0);
    MLA_LDS_BARRIER();
    // tile j+1: a full dense tile is loaded by the fast path, its nine loads
    // per thread spread over the score MFMAs; any other tile in one burst here
    // (the FP8 cache is staged and converted below).
    const bool fast = !FP8 && !TOPK && j + 1 < ntiles && p0 + (j + 2) * kTT <= p1;
    // top-k: the gathered tile j+1 is loaded one load per group of score
    // MFMAs too (each load looks its row up in the staged indices)
    const bool gather = !FP8 && TOPK && j + 1 < ntiles;
    const bool fp8_cv = FP8 && j + 1 < ntiles, fp8_ld = FP8 && j + 2 < ntiles;
    // a full dense tile j+2 is reloaded inside the score chain, any other in one burst
    const bool fp8_in_chain = FP8 && !TOPK && active && fp8_ld && p0 + (j + 3) * kTT <= p1;
    const FullTile ft = full_tile(j + 1, Stage<s1>{});
    if (!FP8 && j + 1 < ntiles) {
      if (fast || gather) publish_mask(p0 + (j + 1) * kTT, s1);
      else issue_bf16(j + 1, Stage<s1>{});
    }
    DmaCursor gc{0, 0};
    uint32_t gbase = 0u;
    if constexpr (TOPK && !FP8) {
      if (gather) {
        gc = dma_start();
        gbase = dma_base(slot(Stage<s1>{}));
      }
    }
    if (tid == 0) sRescale[(j + 1) % 3] = 0u;  // flag of tile j-2: read in body j-1
    const uint16_t* tile = slot(S);
    f32x16 s = {};  // waves without score heads run the softmax on zeros
    // FP8: this wave's part of tile j+1 (staged during tile j-1) is converted
    // into its slot in one pass, then the raw tile j+2 is loaded into the
    // staging region (its own reads of it done): a full dense tile by six
    // loads spread over the score chain (issued back to back they stall the
    // wave), any other here.  In one pass the score MFMAs that follow run
    // without waiting on the conversion's LDS traffic.
    if constexpr (FP8) {
      if (fp8_cv) {
        MLA_WAIT_VMCNT(0);
        fp8_convert_all(j + 1, Stage<s1>{});
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): staging reads done before the reload
      if (fp8_ld && !fp8_in_chain) fp8_load_all(j + 2);
    }
    if (active) {
      // Scores.  The 36 MFMAs accumulate in VGPRs (inline asm: the compiler
      // would put this accumulator in AGPRs, where O already takes all 256).
      // Back-to-back MFMAs of one shape accumulating into the same registers
      // need no wait states; the s_nop after the chain covers the MFMA-write
      // -> VALU-read hazard (>= 18 wait states for this 8-pass instruction).
      // Operand reads run kScoreAhead k-steps ahead of the MFMAs (enough LDS
      // requests in flight to cover its latency with one wave per SIMD).
      u32x4 ka[kScoreAhead + 1];
#pragma unroll
      for (int k = 0; k < kScoreAhead; ++k) ka[k] = *(const u32x4*)(tile + sc_base[k & 3] + 64 * (k >> 2));
      // nine explicitly instantiated groups of four k-steps (keeps the chain
      // fully unrolled, so qreg is indexed by constants)
      auto step = [&](auto Q, auto KK) MLA_INLINE {
        constexpr int kk = decltype(KK)::value;
        constexpr int k = 4 * decltype(Q)::value + kk;
        if constexpr (k + kScoreAhead < 36)
          ka[(k + kScoreAhead) % (kScoreAhead + 1)] =
              *(const u32x4*)(tile + sc_base[(k + kScoreAhead) & 3] + 64 * ((k + kScoreAhead) >> 2));
        if constexpr (k == 0)
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(ka[0]), "v"(qreg[0]));
        else
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(ka[k % (kScoreAhead + 1)]), "v"(qreg[k]));
        if constexpr (kk == 1) {
          if (fast) full_load(ft, Q);
          if constexpr (TOPK && !FP8) {
            if (gather) dma_step(gc, p0 + (j + 1) * kTT, gbase, Q);
          }
          if constexpr (FP8 && !TOPK && decltype(Q)::value < 6) {
            if (fp8_in_chain) fp8_load_full(j + 2, Q);
          }
        }
        if constexpr (k == 35) asm volatile("s_nop 15\n\ts_nop 3" : "+v"(s));
      };
      auto group = [&](auto Q) MLA_INLINE {
        step(Q, Stage<0>{});
        step(Q, Stage<1>{});
        step(Q, Stage<2>{});
        step(Q, Stage<3>{});
      };
      group(Stage<0>{});
      group(Stage<1>{});
      group(Stage<2>{});
      group(Stage<3>{});
      group(Stage<4>{});
      group(Stage<5>{});
      group(Stage<6>{});
      group(Stage<7>{});
      group(Stage<8>{});
    } else if (fast) {
      full_all(ft);
    } else if (gather) {
      dma_all(gc, p0 + (j + 1) * kTT, gbase);
    }
    uint32_t mask = sMask[st];
    if constexpr (PACK) {  // and the rows this lane's token sees (per lane)
      const int r = row_lim() - (p0 + j * kTT);
      mask = r >= kTT ? mask : (r <= 0 ? 0u : mask & ((1u << r) - 1u));
    }
    // one code path for every wave inside the loop (branches around the
    // update would merge 256 accumulator registers); the first tile, which
    // has no update before it, is peeled off the loop
    if constexpr (decltype(PV)::value) rescale(j - 1);
    update_softmax(PV, slot(Stage<sp>{}), j - 1, s, j, mask);
  };
  body(0, Stage<0>{}, Stage<0>{});
  for (int j0 = 1; j0 < ntiles; j0 += kStages) {
    body(j0, Stage<1>{}, Stage<1>{});
    if (j0 + 1 < ntiles) body(j0 + 1, Stage<2>{}, Stage<1>{});
    if (j0 + 2 < ntiles) body(j0 + 2, Stage<0>{}, Stage<1>{});
  }
  // drain: the update with the last tile
  {
    MLA_LDS_BARRIER();
    const int jl = ntiles - 1;
    rescale(jl);
    const int sl = jl % kStages;
    const uint16_t* lt = sl == 0 ? slot(Stage<0>{}) : (sl == 1 ? slot(Stage<1>{}) : slot(Stage<2>{}));
    update_only(lt, jl);
  }

  // ---- partial result: (m, l) in fp32 and the unnormalised O in bf16, each
  // lane's accumulators stored in fragment order:
  //   part_o[slot][head block nb][wave][m][q2][lane][8]
  // holds O[head 32 nb + lane % 32][128 wave + 32 m + 16 q2 + 8 (j / 4)
  // + 4 (lane / 32) + j % 4] at position j, one 1 KB row per store.
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (active && g == 0 && ghead < a.H) {
    float* pm = a.part_ml + (slot_id * a.H + ghead) * 2;
    pm[0] = l_tot > 0.f ? m_run : -INFINITY;
    pm[1] = l_tot;
  }
  uint16_t* dst = a.part_o + slot_id * (size_t)a.Hp * kC + (size_t)hb0 * (32 * 512) + (size_t)wave * (8 * 512) + 8 * lane;
  auto store_block = [&](auto NB) MLA_INLINE {
    constexpr int nb = decltype(NB)::value;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const f32x16& ob = o[NHB * m + nb];
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2)
        *(u32x4*)(dst + (size_t)nb * (32 * 512) + (2 * m + q2) * 512) =
            u32x4{cvt_pk_bf16(ob[8 * q2], ob[8 * q2 + 1]), cvt_pk_bf16(ob[8 * q2 + 2], ob[8 * q2 + 3]),
                  cvt_pk_bf16(ob[8 * q2 + 4], ob[8 * q2 + 5]), cvt_pk_bf16(ob[8 * q2 + 6], ob[8 * q2 + 7])};
    }
  };
  store_block(Stage<0>{});
  if constexpr (NHB > 1) {
    if (nhb > 1) store_block(Stage<1>{});
  }
  if constexpr (NHB > 3) {
    if (nhb > 2) store_block(Stage<2>{});
    if (nhb > 3) store_block(Stage<3>{});
  }
}

// ---------------------------------------------------------------------------
// combine: grid (work items, head_blocks * 32 partial rows), 64 x NG threads
// (NG = 1, 2, 4 or 8 groups, about one per four partials an item has on
// average).  H here counts an item's query rows.  Row r of a partial is (row
// block r / 32, wave, m, q2) in the attention kernel's fragment order: 64
// lanes x 8 values, lane l holding query row 32 (r / 32) + l % 32.  Thread
// (lane, group sg) merges that chunk over every NG-th partial of item b
// (slots wcum[b] .. wcum[b+1] - 1) with a running maximum, the groups are
// merged through LDS, and
//   o = sum_j 2^(m_j - M) O_j / sum_j 2^(m_j - M) l_j,  M = max_j m_j
// (over the partials with l_j > 0; none: zeros) goes to olat[b][h][c].
// ---------------------------------------------------------------------------
constexpr int kCombineGroups = 8;

struct Merge {
  float M = -INFINITY, L = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // add weight 2^m times the partial (values v[e] * scale, sum l)
  __device__ __forceinline__ void add(float m, float l, const float* v) {
    if (!(l > 0.f)) return;  // nothing selected in that split
    if (m > M) {
      const float sc = exp2f(M - m);  // M = -inf: 0
      L *= sc;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= sc;
      M = m;
    }
    const float w = exp2f(m - M);
    L = fmaf(w, l, L);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, v[e], acc[e]);
  }
};

__global__ __launch_bounds__(64 * kCombineGroups) void combine_kernel(
    const uint16_t* __restrict__ part_o, const float* __restrict__ part_ml,
    const int32_t* __restrict__ wcum, uint16_t* __restrict__ olat, int H, int Hp) {
  const int NG = blockDim.x >> 6;
  const int b = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, sg = tid >> 6;
  const int h = 32 * (r >> 5) + (lane & 31);
  const bool hv = h < H;
  const size_t s0 = (size_t)wcum[b];
  const int ns = wcum[b + 1] - wcum[b];
  const float* pm = part_ml + (s0 * H + (hv ? h : 0)) * 2;
  const uint16_t* po = part_o + s0 * Hp * kC + (size_t)r * 512 + 8 * lane;
  const size_t ml_stride = (size_t)H * 2, o_stride = (size_t)Hp * kC;
  extern __shared__ float sRed[];  // [NG - 1][64][10]: sized per launch
  Merge mg;
  auto unpack = [](const u32x4& v, float* f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[2 * j] = bf_lo(v[j]);
      f[2 * j + 1] = bf_hi(v[j]);
    }
  };
  if (hv) {
    int s = sg;
    for (; s + 3 * NG < ns; s += 4 * NG) {  // four partials of this group in flight
      u32x4 v[4];
      float2 ml[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        ml[k] = *(const float2*)(pm + (s + NG * k) * ml_stride);
        v[k] = *(const u32x4*)(po + (size_t)(s + NG * k) * o_stride);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float f[8];
        unpack(v[k], f);
        mg.add(ml[k].x, ml[k].y, f);
      }
    }
    for (; s < ns; s += NG) {
      const float2 ml = *(const float2*)(pm + s * ml_stride);
      const u32x4 v = *(const u32x4*)(po + (size_t)s * o_stride);
      float f[8];
      unpack(v, f);
      mg.add(ml.x, ml.y, f);
    }
  }
  if (sg > 0) {
    float* d = sRed + ((sg - 1) * 64 + lane) * 10;
#pragma unroll
    for (int e = 0; e < 8; ++e) d[e] = mg.acc[e];
    d[8] = mg.M;
    d[9] = mg.L;
  }
  __syncthreads();
  if (sg == 0 && hv) {
    for (int k = 0; k < NG - 1; ++k) {
      const float* d = sRed + (k * 64 + lane) * 10;
      // a group's (acc, L) is already relative to 2^M_k: merge as a partial
      // with m = M_k, l = L_k and values acc_k / 1
      mg.add(d[8], d[9], d);
    }
    const float inv = mg.L > 0.f ? 1.f / mg.L : 0.f;
    // row r = (head block, wave, m, q2): columns 128 wave + 32 m + 16 q2 + 4 (lane / 32)
    const int c0 = 128 * ((r >> 3) & 3) + 32 * ((r >> 1) & 3) + 16 * (r & 1) + 4 * (lane >> 5);
    uint16_t* dst = olat + ((size_t)b * H + h) * kC + c0;
    const float* a = mg.acc;
    *(u32x2*)dst = u32x2{pack_bf(a[0] * inv, a[1] * inv), pack_bf(a[2] * inv, a[3] * inv)};
    *(u32x2*)(dst + 8) = u32x2{pack_bf(a[4] * inv, a[5] * inv), pack_bf(a[6] * inv, a[7] * inv)};
  }
}

// ---------------------------------------------------------------------------
// uproj: out[b,h,d] = sum_c o[b,h,c] W_UV[h][d][c].  grid (H, 4 d-blocks of 32,
// shares of the query tokens), one wave; MFMA 16x16x32 with the tokens as the
// M dimension (blocks of 16) and two 16-wide d blocks as N.  The wave's W_UV
// slice (32 rows x 512, 32 KB) is loaded into registers up front and reused
// for every block of tokens of its share.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void uproj_kernel(const uint16_t* __restrict__ olat,
                                                   const uint16_t* __restrict__ wkv_b,
                                                   uint16_t* __restrict__ out, int B, int H) {
  const int h = blockIdx.x, d0 = 32 * blockIdx.y;
  const int lane = threadIdx.x, r = lane & 15, g = lane >> 4;
  // A operand of the block of sequences b0 .. b0 + 15: lane holds o[b0 + r][h][32 ks + 8 g .. +7]
  auto load_a = [&](int b0, u32x4 (&av)[16]) {
    const int bb = b0 + r;
    const bool bok = bb < B;
    const uint16_t* arow = olat + ((size_t)(bok ? bb : 0) * H + h) * kC + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) av[ks] = bok ? *(const u32x4*)(arow + 32 * ks) : u32x4{0, 0, 0, 0};
  };
  // the first block's rows go out with the weights, and each next block's
  // before the current block's MFMAs, so only one load latency is exposed
  u32x4 av[16], an[16];
  // this workgroup's token blocks: a contiguous share of the ceil(B / 16)
  const int nblk = (B + 15) >> 4, per = (nblk + gridDim.z - 1) / gridDim.z;
  const int b_begin = blockIdx.z * per * 16, b_end = min(B, (blockIdx.z + 1) * per * 16);
  if (b_begin >= b_end) return;
  load_a(b_begin, av);
  const uint16_t* w0 = wkv_b + ((size_t)h * (kDN + kDV) + kDN + d0 + r) * kC + 8 * g;
  const uint16_t* w1 = w0 + (size_t)16 * kC;
  u32x4 bw0[16], bw1[16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    bw0[ks] = *(const u32x4*)(w0 + 32 * ks);
    bw1[ks] = *(const u32x4*)(w1 + 32 * ks);
  }
  for (int b0 = b_begin; b0 < b_end; b0 += 16) {
    if (b0 + 16 < b_end) load_a(b0 + 16, an);
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
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) av[ks] = an[ks];
  }
}

// The attention instance for a workgroup's head-block count (1, 2, or up to 4).
template <bool FP8, bool TOPK, bool PACK>
static void (*attn_instance(int nhb))(AttnArgs) {
  return nhb == 1 ? attn_kernel<FP8, TOPK, 1, PACK> : nhb == 2 ? attn_kernel<FP8, TOPK, 2, PACK> : attn_kernel<FP8, TOPK, 4, PACK>;
}

// ---------------------------------------------------------------------------
hipError_t launch_decode(const mla_params& p, const DecodeArgs& d, const CacheWriteArgs* write,
                         hipStream_t stream, void* latent_out) {
  const DecodePlan plan = make_decode_plan(p);
  const int s = p.seqlen_q, B = p.batch * s, H = p.num_heads;  // B: query tokens
  const int ps = plan.pack_s, NI = (int)plan.items, rows = plan.rows;  // work items of ps tokens
  char* ws = (char*)d.workspace;
  uint16_t* qt = (uint16_t*)(ws + plan.off_qt);
  uint16_t* part_o = (uint16_t*)(ws + plan.off_part_o);
  float* part_ml = (float*)(ws + plan.off_part_ml);
  uint16_t* olat = latent_out ? (uint16_t*)latent_out : (uint16_t*)(ws + plan.off_olat);
  hipEvent_t* ev = (hipEvent_t*)p.trace_events;
  auto evk = [&](int k) -> hipEvent_t const* { return ev ? ev + 2 * k : nullptr; };
  hipError_t err;
  int32_t* wcum = (int32_t*)(ws + plan.off_wcum);
  int4* rec = (int4*)(ws + plan.off_rec);
  int32_t* slot_of = (int32_t*)(ws + plan.off_slot);

  const bool fp8 = p.kv_dtype == MLA_KV_FP8_E4M3_B128, topk = p.topk > 0;
  RowWrite rw{};
  int write_cols = 0;
  auto absorb = absorb_kernel<kNoWrite>;
  if (write) {
    rw = RowWrite{(const uint16_t*)write->kv_new, (const uint16_t*)write->pe_new, write->kv_cache,
                  write->kv_scale, (uint16_t*)write->pe_cache};
    // about one item per thread (bf16) or per wavefront (FP8), at most 64 columns
    const long long items_per_col = fp8 ? 16 : 1024, items = (long long)B * (fp8 ? 4 : 72);
    write_cols = (int)std::min<long long>((items + items_per_col - 1) / items_per_col, 64);
    absorb = fp8 ? absorb_kernel<kWriteFp8> : absorb_kernel<kWriteBf16>;
  }
  // sequences per absorb workgroup: blocks of 32, over at most 8 ranges
  const int chunks = (B + 31) / 32, zs = std::min(chunks, 8);
  const int bz = 32 * ((chunks + zs - 1) / zs);
  // columns: H heads, the padding rows of an item, the planner, the writers
  const int hx = H + (plan.heads_padded - rows);
  err = launch_kernel(absorb, dim3(hx + 1 + write_cols, 4, (B + bz - 1) / bz),
                      dim3(256), stream, evk(0), (const uint16_t*)d.q_nope, (const uint16_t*)d.q_pe,
                      (const uint16_t*)d.wkv_b, qt, B, s, ps, H, hx, plan.heads_padded, bz, d.cache_lens,
                      p.max_seq_len, p.topk, plan.min_group_tiles, (int)plan.max_groups, wcum, rec,
                      slot_of, rw);
  if (err != hipSuccess) return err;

  AttnArgs aa;
  aa.qt = qt;
  aa.kv = d.kv_cache;
  aa.kv_scale = d.kv_scale;
  aa.pe = (const uint16_t*)d.pe_cache;
  aa.topk_idx = d.topk_idx;
  aa.rec = rec;
  aa.slot_of = slot_of;
  aa.part_o = part_o;
  aa.part_ml = part_ml;
  aa.s = s / ps;
  aa.H = rows;
  aa.Hp = plan.heads_padded;
  aa.ps = ps;
  aa.hq = H;
  aa.T = p.max_seq_len;
  aa.topk = p.topk;
  aa.head_blocks = plan.head_blocks;
  aa.head_split = plan.head_split;
  aa.scale_log2 = p.softmax_scale * 1.4426950408889634f;
  const dim3 agrid((unsigned)(plan.max_groups * plan.head_split));
  // workgroups with one or two head blocks get their own accumulator count
  const int nhb = plan.head_blocks / plan.head_split;
  // (packed tokens: dense selections only)
  auto attn = fp8 ? (topk ? attn_instance<true, true, false>(nhb)
                          : ps > 1 ? attn_instance<true, false, true>(nhb) : attn_instance<true, false, false>(nhb))
                  : (topk ? attn_instance<false, true, false>(nhb)
                          : ps > 1 ? attn_instance<false, false, true>(nhb) : attn_instance<false, false, false>(nhb));
  err = launch_kernel(attn, agrid, dim3(kAttnThreads), stream, evk(1), aa);
  if (err != hipSuccess) return err;

  // partial groups per combine thread block: about one per 4 partials of the
  // average sequence (at most 256 partials are in use when B <= 256)
  // (work items: olat [item][ps H rows][512] is olat [token][H][512])
  const long long avg_parts = std::max<long long>(1, std::min<long long>(plan.max_groups, 256) / NI);
  const int ng = avg_parts >= 32 ? 8 : (avg_parts >= 16 ? 4 : (avg_parts >= 8 ? 2 : 1));
  err = launch_kernel_lds(combine_kernel, dim3(NI, plan.head_blocks * 32), dim3(64 * ng),
                          (size_t)(ng - 1) * 64 * 10 * sizeof(float), stream, evk(2),
                      (const uint16_t*)part_o, (const float*)part_ml, (const int32_t*)wcum, olat, rows,
                      plan.heads_padded);
  if (err != hipSuccess) return err;
  if (latent_out) return hipSuccess;  // the caller takes the latent output

  // few heads leave CUs idle: then the token blocks are split too (each share
  // of them loads the head's W_UV slice again, from L2)
  const int uz = std::min((B + 15) / 16, std::max(1, kTargetCUs / (4 * H)));
  err = launch_kernel(uproj_kernel, dim3(H, 4, uz), dim3(64), stream, evk(3), (const uint16_t*)olat,
                      (const uint16_t*)d.wkv_b, (uint16_t*)d.out, B, H);
  if (err != hipSuccess) return err;
  return hipSuccess;
}

}  // namespace mla
