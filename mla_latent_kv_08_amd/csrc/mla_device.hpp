// mla_device.hpp -- gfx950 device helpers shared by the decode and cache-write
// kernels: bf16/E4M3FN conversions, MFMA wrappers, wavefront reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kC = 512;    // latent width
constexpr int kR = 64;     // rotary key width
constexpr int kQK = 576;   // latent + rotary: values per cached position
constexpr int kDN = 128;   // q_nope / key-half rows per head
constexpr int kDV = 128;   // value-half rows per head
constexpr int kBlk = 128;  // FP8 block: latent elements per scale

typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef float f32x16 __attribute__((__vector_size__(64)));
typedef float f32x4 __attribute__((__vector_size__(16)));
typedef uint32_t u32x4 __attribute__((__vector_size__(16)));
typedef uint32_t u32x2 __attribute__((__vector_size__(8)));

// bf16 halves of a packed dword as fp32 (exact).
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even, NaN kept quiet NaN.
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
// Same rounding for values known to be finite (softmax probabilities).
__device__ __forceinline__ uint32_t f2bf_finite(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf(float lo, float hi) {
  return f2bf(lo) | (f2bf(hi) << 16);
}
__device__ __forceinline__ uint32_t pack_bf_finite(float lo, float hi) {
  return f2bf_finite(lo) | (f2bf_finite(hi) << 16);
}
// Two fp32 -> packed bf16 with gfx950's v_cvt_pk_bf16_f32 (round to nearest
// even, NaN stays NaN); used for the softmax probabilities and the normalised
// partial outputs of the attention kernel.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// OCP E4M3FN -> fp32 (exact: every E4M3FN value is an fp32 value).
// Exponent bias 7; exponent field 0 holds subnormals m * 2^-9.
__device__ __forceinline__ float e4m3fn_to_f32(uint32_t code) {
  uint32_t e = (code >> 3) & 0xFu, m = code & 0x7u;
  float mag;
  if (e == 0xFu && m == 0x7u) mag = __uint_as_float(0x7FC00000u);
  else if (e == 0) mag = (float)m * 0.001953125f;               // m * 2^-9
  else mag = __uint_as_float(((e + 120u) << 23) | (m << 20));   // (1 + m/8) * 2^(e-7)
  return (code & 0x80u) ? -mag : mag;
}

// fp32 -> OCP E4M3FN, round to nearest even, saturating to +-448 (0x7E),
// sign of zero kept, NaN -> 0x7F.  Written from the format definition: the
// magnitude is scaled by a power of two so that one E4M3FN step becomes one
// integer step, rounded with rint (ties to even), then re-assembled.
__device__ __forceinline__ uint32_t f32_to_e4m3fn(float v) {
  const uint32_t bits = __float_as_uint(v);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = fabsf(v);
  if (a != a) return 0x7Fu;
  if (a >= 464.0f) return sign | 0x7Eu;  // 464 is the tie between 448 and 480 -> 448
  const int e = (int)((bits >> 23) & 0xFFu) - 127;
  uint32_t code;
  if (e < -6) {
    code = (uint32_t)rintf(a * 512.0f);  // subnormal grid 2^-9; 8 -> smallest normal
  } else {
    uint32_t q = (uint32_t)rintf(ldexpf(a, 3 - e));  // in [8, 16]
    int ee = e;
    if (q == 16u) { q = 8u; ee += 1; }
    code = ((uint32_t)(ee + 7) << 3) | (q - 8u);
  }
  if (code > 0x7Eu) code = 0x7Eu;
  return sign | code;
}

// D(32x32) += A(32x16) * B(16x32), bf16 inputs, fp32 accumulate.
// Lane l holds A[l%32][8*(l/32) + j] and B[8*(l/32) + j][l%32], j = 0..7;
// D element e of lane l is D[8*(e/4) + 4*(l/32) + e%4][l%32].
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// D(16x16) += A(16x32) * B(32x16).  Lane l holds A[l%16][8*(l/16) + j] and
// B[8*(l/16) + j][l%16]; D element j of lane l is D[4*(l/16) + j][l%16].
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

typedef __attribute__((address_space(3))) void lds_void;

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_void*)p;
}

// 16-byte global -> LDS copy for each lane: lane l's 16 bytes from `src` land
// at LDS byte address base + OFF + 16 l (base must be wave-uniform).  Written as
// inline asm so the compiler's wait-count tracking does not treat every later
// LDS read as possibly depending on it; completion is awaited explicitly with
// s_waitcnt vmcnt (before a barrier when other waves read the data).
template <int OFF>
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t base) {
  asm volatile("s_add_u32 m0, %1, %2\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(base), "i"(OFF)
               : "memory", "m0", "scc");
}

// s_waitcnt vmcnt(n) leaving the other counters unconstrained.
#define MLA_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (0x7 << 4) | (0xF << 8) | (((n) >> 4) << 14))

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace mla
