/*
 * mla_oracle.c -- plain, slow CPU oracle for weight-absorbed MLA decode over a
 * latent KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library; the two are independent
 * implementations of the same definitions.
 *
 * Sources (the pages this follows):
 *  - "DeepSeek-V3.2-Exp . KV cache" (decode view, position 1000): the cache
 *    write excerpt (FP8 round trip of the latent, then slice write of the
 *    latent and rotary rows) and the "MQA decode" excerpt (absorb q_nope
 *    through the key half of wkv_b, score against both caches times
 *    softmax_scale, add the top-k index mask, softmax, reduce against the
 *    latent cache, up-project through the value half of wkv_b).
 *  - "DeepSeek MLA Architecture: ... cuts KV cache by 93%", section 3
 *    (score = content term + rotary term, k_R shared by all heads) and
 *    section 4 (absorbed query; values aggregated in latent space, then W_UV).
 *  - The same article, sections 4-5: the output projection W_O applied to
 *    the heads' up-projected outputs concatenated (feature 128 h + d), and
 *    its offline fusion with the value half, W_OV = W_O W_UV per head,
 *    applied to the latent output (feature 512 h + c).
 *  - OCP 8-bit floating point specification, E4M3 ("FN": no infinities,
 *    S.1111.111 is NaN, largest finite 448).
 *
 * Precision: every decode step is carried out in IEEE double.  The FP8 block
 * quantiser works in fp32, because there the floating-point result decides
 * an integer code and the page's quantiser works in fp32 (the dequantised
 * value is code.float() * scale, cast back to bf16).
 *
 * Readings where the pages leave a step open (all listed in the design notes):
 *  - FP8 format: E4M3FN, one fp32 scale per 128 contiguous latent elements,
 *    scale = blockmax / 448 (fp32 division), code = RNE-saturating
 *    E4M3FN(x / scale) (fp32 division); a block whose scale is 0 gets all
 *    codes 0.
 *  - The decode sees the latent the page's cache holds: bf16(code * scale).
 *  - Per-sequence end: end_b = min(max(cache_lens[b], 0), max_seq_len).
 *  - s > 1 query tokens: they are the last s cached positions of the
 *    sequence, and token i (0-based) sees the rows up to its own,
 *    t < end_b - (s - 1 - i) (the MQA decode excerpt carries the s dimension
 *    in its einsums but prints its mask for one token only).  With top-k,
 *    token i has its own index row topk_idx[b][i].
 *  - Top-k: the selected positions are the SET of entries i of topk_idx[b]
 *    with 0 <= i < end_b (the page's scatter of 0 into a -inf mask is
 *    idempotent, so duplicates count once; order is irrelevant).
 *  - No selected position: the output row is 0.
 *  - Cache write: rows r = start_pos[b] + i outside [0, max_seq_len) are
 *    dropped (out-of-range slice positions store nothing).
 *
 * Parity of the end-to-end float values against an external worked example is
 * unpinned (the pages print none); the tests pin the oracle against the naive
 * expanded-MHA form, closed forms, invariants and torch's E4M3FN cast.
 */
#include "mla_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_C 512   /* kv_lora_rank: width of the latent c_KV */
#define ORC_R 64    /* qk_rope_head_dim: width of the shared rotary key k_R */
#define ORC_DN 128  /* qk_nope_head_dim */
#define ORC_DV 128  /* v_head_dim */
#define ORC_BLK 128 /* FP8 quantisation block (latent elements per scale) */

/* ------------------------------------------------------------------ */
/* Scalar formats                                                      */
/* ------------------------------------------------------------------ */

/* bf16 is the top half of an IEEE binary32. */
double oracle_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Round a binary32 to bf16, to nearest, ties to even (NaN kept NaN). */
uint16_t oracle_bf16_round(float x) {
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
    return (uint16_t)((u >> 16) | 0x0040u); /* quiet NaN */
  uint32_t lower = u & 0xFFFFu;
  uint32_t upper = u >> 16;
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
  return (uint16_t)upper;
}

/* OCP E4M3FN: value of a code.  Exponent bias 7; exponent field 0 holds the
 * subnormals m/8 * 2^-6; S.1111.111 is NaN; there are no infinities. */
double oracle_e4m3fn_value(uint8_t code) {
  int s = (code >> 7) & 1;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  if (e == 0xF && m == 0x7) return NAN;
  double mag = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  return s ? -mag : mag;
}

/* OCP E4M3FN encoder, round to nearest with ties to the even code, saturating
 * to the largest finite magnitude 448.  Done by exhaustive search over the
 * 127 non-negative finite codes: the nearest one wins; on a tie the code
 * with a zero last mantissa bit wins.  NaN maps to 0x7F. */
uint8_t oracle_e4m3fn_encode(float v) {
  if (isnan(v)) return 0x7F;
  double a = fabs((double)v);
  int best = 0;
  double bestd = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {
    double d = fabs(oracle_e4m3fn_value((uint8_t)c) - a);
    if (d < bestd || (d == bestd && (c & 1) == 0)) {
      bestd = d;
      best = c;
    }
  }
  return (uint8_t)(best | (signbit(v) ? 0x80 : 0x00));
}

/* Array form of the encoder (used by the tests to sweep many values). */
void oracle_e4m3fn_encode_array(const float* v, uint8_t* codes, size_t n) {
  for (size_t i = 0; i < n; ++i) codes[i] = oracle_e4m3fn_encode(v[i]);
}

/* ------------------------------------------------------------------ */
/* Footprint (page "MLA KV Cache Memory Footprint for 128K Context",   */
/* memory table and calculator; page "KV cache": 576 values/position)  */
/* ------------------------------------------------------------------ */

int oracle_values_per_position(void) { return ORC_C + ORC_R; }

/* Latent-only bytes for seq_len positions at bytes_per_elem bytes each
 * (the pages' table counts the 512-wide latent only). */
double oracle_latent_bytes(double seq_len, int bytes_per_elem) {
  return seq_len * ORC_C * (double)bytes_per_elem;
}

/* ------------------------------------------------------------------ */
/* Cache write (page "KV cache", cache write excerpt)                  */
/* ------------------------------------------------------------------ */

/* One 128-element block: scale = amax / 448 in fp32; code = E4M3FN(x/scale). */
static void quantise_block(const uint16_t* x, uint8_t* codes, float* scale_out) {
  float amax = 0.0f;
  for (int i = 0; i < ORC_BLK; ++i) {
    float v = (float)oracle_bf16_value(x[i]);
    float av = fabsf(v);
    if (av > amax) amax = av;
  }
  float scale = amax / 448.0f;
  *scale_out = scale;
  for (int i = 0; i < ORC_BLK; ++i) {
    if (scale == 0.0f) {
      codes[i] = 0x00;
    } else {
      float v = (float)oracle_bf16_value(x[i]);
      float q = v / scale;
      codes[i] = oracle_e4m3fn_encode(q);
    }
  }
}

int oracle_cache_write(int B, int s, int max_seq_len, int fp8, const uint16_t* kv_new,
                       const uint16_t* pe_new, const int32_t* start_pos, void* kv_cache,
                       float* kv_scale, uint16_t* pe_cache) {
  if (B < 0 || s < 0 || max_seq_len <= 0) return 1;
  /* rows are independent: one (b, i) per iteration */
#pragma omp parallel for schedule(static)
  for (long long bi = 0; bi < (long long)B * s; ++bi) {
    {
      const int b = (int)(bi / s), i = (int)(bi % s);
      long long r = (long long)start_pos[b] + i;
      if (r < 0 || r >= max_seq_len) continue; /* dropped */
      const uint16_t* src = kv_new + ((size_t)b * s + i) * ORC_C;
      const uint16_t* srcp = pe_new + ((size_t)b * s + i) * ORC_R;
      size_t row = (size_t)b * max_seq_len + (size_t)r;
      if (fp8) {
        uint8_t* dst = (uint8_t*)kv_cache + row * ORC_C;
        for (int j = 0; j < ORC_C / ORC_BLK; ++j)
          quantise_block(src + j * ORC_BLK, dst + j * ORC_BLK,
                         &kv_scale[row * (ORC_C / ORC_BLK) + j]);
      } else {
        uint16_t* dst = (uint16_t*)kv_cache + row * ORC_C;
        memcpy(dst, src, ORC_C * sizeof(uint16_t));
      }
      memcpy(pe_cache + row * ORC_R, srcp, ORC_R * sizeof(uint16_t));
    }
  }
  return 0;
}

/* Latent element c of cached row `row` as the decode sees it: the bf16 value,
 * or for the FP8 cache bf16(float(code) * scale) as on the page. */
static double latent_at(int fp8, const void* kv_cache, const float* kv_scale, size_t row, int c) {
  if (!fp8) return oracle_bf16_value(((const uint16_t*)kv_cache)[row * ORC_C + c]);
  uint8_t code = ((const uint8_t*)kv_cache)[row * ORC_C + c];
  float prod = (float)oracle_e4m3fn_value(code) * kv_scale[row * (ORC_C / ORC_BLK) + c / ORC_BLK];
  return oracle_bf16_value(oracle_bf16_round(prod));
}

/* ------------------------------------------------------------------ */
/* Decode (page "KV cache", MQA decode excerpt; MLA article, s.3-4)    */
/* ------------------------------------------------------------------ */

/* One (query token q = b * s + i, head h) output row out[128]; optionally
 * the softmax probabilities over positions 0..max_seq_len-1 (0 where not
 * selected) and the latent output o[512] of step 4 (before the
 * up-projection).  out may be NULL when only the latent output is wanted. */
static void decode_one(const oracle_decode_args* a, int q, int h, double* out, double* probs,
                       double* latent) {
  const int T = a->max_seq_len;
  const int b = q / a->s, i_tok = q % a->s;
  int end = a->cache_lens[b];
  if (end < 0) end = 0;
  if (end > T) end = T;
  end -= a->s - 1 - i_tok; /* rows up to this token's own */
  if (end < 0) end = 0;

  /* Selected positions. */
  unsigned char* sel = (unsigned char*)calloc((size_t)T, 1);
  if (a->topk > 0) {
    for (int i = 0; i < a->topk; ++i) {
      int32_t t = a->topk_idx[(size_t)q * a->topk + i];
      if (t >= 0 && t < end) sel[t] = 1;
    }
  } else {
    for (int t = 0; t < end; ++t) sel[t] = 1;
  }

  /* Step 1, absorb: qa[c] = sum_d q_nope[b,h,d] * wkv_b[h, d, c], d < 128. */
  double qa[ORC_C];
  for (int c = 0; c < ORC_C; ++c) {
    double acc = 0.0;
    for (int d = 0; d < ORC_DN; ++d) {
      double qn = oracle_bf16_value(a->q_nope[((size_t)q * a->H + h) * ORC_DN + d]);
      double w = oracle_bf16_value(a->wkv_b[((size_t)h * (ORC_DN + ORC_DV) + d) * ORC_C + c]);
      acc += qn * w;
    }
    qa[c] = acc;
  }

  /* Step 2, scores: (qa . c_KV[t] + q_pe . k_R[t]) * softmax_scale. */
  double* score = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
  for (int t = 0; t < T; ++t) {
    score[t] = -INFINITY;
    if (!sel[t]) continue;
    size_t row = (size_t)b * T + (size_t)t;
    double content = 0.0;
    for (int c = 0; c < ORC_C; ++c) content += qa[c] * latent_at(a->fp8, a->kv_cache, a->kv_scale, row, c);
    double rope = 0.0;
    for (int r = 0; r < ORC_R; ++r) {
      double qp = oracle_bf16_value(a->q_pe[((size_t)q * a->H + h) * ORC_R + r]);
      double kr = oracle_bf16_value(a->pe_cache[row * ORC_R + r]);
      rope += qp * kr;
    }
    score[t] = (content + rope) * a->softmax_scale;
  }

  /* Step 3, softmax over the selected positions: max, exp, normalise. */
  double m = -INFINITY;
  for (int t = 0; t < T; ++t)
    if (sel[t] && score[t] > m) m = score[t];
  double sum = 0.0;
  for (int t = 0; t < T; ++t) {
    double p = sel[t] ? exp(score[t] - m) : 0.0;
    score[t] = p;
    sum += p;
  }
  for (int t = 0; t < T; ++t) score[t] = (sum > 0.0) ? score[t] / sum : 0.0;
  if (probs) memcpy(probs, score, sizeof(double) * (size_t)T);

  /* Step 4, reduce against the latent cache: o[c] = sum_t p[t] * c_KV[t, c]. */
  double o[ORC_C];
  for (int c = 0; c < ORC_C; ++c) o[c] = 0.0;
  for (int t = 0; t < T; ++t) {
    if (!sel[t]) continue;
    size_t row = (size_t)b * T + (size_t)t;
    for (int c = 0; c < ORC_C; ++c) o[c] += score[t] * latent_at(a->fp8, a->kv_cache, a->kv_scale, row, c);
  }

  if (latent) memcpy(latent, o, sizeof o);

  /* Step 5, up-project: out[d] = sum_c o[c] * wkv_b[h, 128 + d, c]. */
  for (int d = 0; out && d < ORC_DV; ++d) {
    double acc = 0.0;
    for (int c = 0; c < ORC_C; ++c) {
      double w = oracle_bf16_value(a->wkv_b[((size_t)h * (ORC_DN + ORC_DV) + ORC_DN + d) * ORC_C + c]);
      acc += o[c] * w;
    }
    out[d] = acc;
  }
  free(score);
  free(sel);
}

int oracle_decode(const oracle_decode_args* a, int n_pairs, const int32_t* pairs, double* out,
                  double* probs) {
  if (!a || a->B < 0 || a->H <= 0 || a->max_seq_len <= 0 || a->topk < 0 || a->s < 1) return 1;
  if (a->topk > 0 && !a->topk_idx) return 1;
  if (a->fp8 && !a->kv_scale) return 1;
  int n = pairs ? n_pairs : a->B * a->s * a->H;
#pragma omp parallel for schedule(dynamic, 1)
  for (int i = 0; i < n; ++i) {
    int q = pairs ? pairs[2 * i] : i / a->H;
    int h = pairs ? pairs[2 * i + 1] : i % a->H;
    decode_one(a, q, h, out + (size_t)i * ORC_DV, probs ? probs + (size_t)i * a->max_seq_len : NULL,
               NULL);
  }
  return 0;
}

/* The latent attention output of steps 1-4 for the same (q, h) pairs:
 * olat: double [n][C], o[c] = sum_t p[t] c_KV[t, c] (MLA article, section 4:
 * the weights multiply the cached 512-wide latents directly; the value
 * up-projection comes after). */
int oracle_decode_latent(const oracle_decode_args* a, int n_pairs, const int32_t* pairs,
                         double* olat) {
  if (!a || a->B < 0 || a->H <= 0 || a->max_seq_len <= 0 || a->topk < 0 || a->s < 1) return 1;
  if (a->topk > 0 && !a->topk_idx) return 1;
  if (a->fp8 && !a->kv_scale) return 1;
  if (!olat) return 1;
  int n = pairs ? n_pairs : a->B * a->s * a->H;
#pragma omp parallel for schedule(dynamic, 1)
  for (int i = 0; i < n; ++i) {
    int q = pairs ? pairs[2 * i] : i / a->H;
    int h = pairs ? pairs[2 * i + 1] : i % a->H;
    decode_one(a, q, h, NULL, NULL, olat + (size_t)i * ORC_C);
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* Output projection (MLA article, section 5: W_O after the value      */
/* up-projection; section 4: W_OV = W_O W_UV fused offline)            */
/* ------------------------------------------------------------------ */

/* y[m][n] = sum_k x[m][k] * w[n][k]: the linear layer's weight is stored
 * [out features][in features].  With x = the up-projected output
 * [tokens][H * 128] (feature 128 h + d) and w = W_O it is the layer output;
 * with x = the latent output [tokens][H * 512] (feature 512 h + c) and
 * w = W_OV it is the same output through the fused weight. */
int oracle_output_projection(int M, int K, int N, const double* x, const double* w, double* y) {
  if (M < 0 || K < 1 || N < 1 || !x || !w || !y) return 1;
#pragma omp parallel for schedule(static)
  for (long long mn = 0; mn < (long long)M * N; ++mn) {
    const int m = (int)(mn / N), n = (int)(mn % N);
    double acc = 0.0;
    for (int k = 0; k < K; ++k) acc += x[(size_t)m * K + k] * w[(size_t)n * K + k];
    y[mn] = acc;
  }
  return 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
