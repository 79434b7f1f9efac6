/*
 * mla_oracle.h -- plain CPU oracle for weight-absorbed MLA decode.
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU-baseline leg; never by the GPU library.
 *
 * All tensors are host arrays, row-major, bf16 passed as raw uint16 bits.
 * Shapes (C = 512 latent, R = 64 rotary, Dn = Dv = 128; s query tokens per
 * sequence):
 *   q_nope [B][s][H][Dn], q_pe [B][s][H][R], wkv_b [H][Dn+Dv][C]
 *   kv_cache  bf16 [B][max_seq_len][C]  or  E4M3FN codes uint8 [B][max_seq_len][C]
 *   kv_scale  fp32 [B][max_seq_len][C/128] (FP8 cache only)
 *   pe_cache  bf16 [B][max_seq_len][R]
 *   cache_lens int32 [B], topk_idx int32 [B][s][topk] (topk > 0 only)
 */
#ifndef MLA_ORACLE_H
#define MLA_ORACLE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct oracle_decode_args {
  int B, H, max_seq_len;
  int s;     /* query tokens per sequence (>= 1): the last s cached positions */
  int fp8;   /* 0: bf16 latent cache; 1: E4M3FN codes + per-128 fp32 scales */
  int topk;  /* 0: dense over [0, end_b); >0: entries per row of topk_idx */
  double softmax_scale;
  const uint16_t* q_nope;
  const uint16_t* q_pe;
  const uint16_t* wkv_b;
  const void* kv_cache;
  const float* kv_scale;
  const uint16_t* pe_cache;
  const int32_t* cache_lens;
  const int32_t* topk_idx;
} oracle_decode_args;

double oracle_bf16_value(uint16_t bits);
uint16_t oracle_bf16_round(float x);
double oracle_e4m3fn_value(uint8_t code);
uint8_t oracle_e4m3fn_encode(float v);
void oracle_e4m3fn_encode_array(const float* v, uint8_t* codes, size_t n);
int oracle_values_per_position(void);
double oracle_latent_bytes(double seq_len, int bytes_per_elem);

/* Writes rows start_pos[b] + i (i < s) of kv_new [B][s][C] / pe_new [B][s][R];
 * rows outside [0, max_seq_len) are dropped.  Returns 0 on success. */
int oracle_cache_write(int B, int s, int max_seq_len, int fp8, const uint16_t* kv_new,
                       const uint16_t* pe_new, const int32_t* start_pos, void* kv_cache,
                       float* kv_scale, uint16_t* pe_cache);

/* Decode for n_pairs (q, h) pairs, q = b * s + i the query token i of
 * sequence b (pairs = int32 [n_pairs][2]), or for every (q, h) in q-major
 * order when pairs is NULL.  out: double [n][Dv]; probs (optional): double
 * [n][max_seq_len].  Returns 0 on success. */
int oracle_decode(const oracle_decode_args* a, int n_pairs, const int32_t* pairs, double* out,
                  double* probs);

/* Latent output of the same steps before the up-projection, for the same
 * pairs: olat double [n][C].  Returns 0 on success. */
int oracle_decode_latent(const oracle_decode_args* a, int n_pairs, const int32_t* pairs,
                         double* olat);

/* y[m][n] = sum_k x[m][k] * w[n][k] in double (x [M][K], w [N][K], y [M][N]).
 * Returns 0 on success. */
int oracle_output_projection(int M, int K, int N, const double* x, const double* w, double* y);

int oracle_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
