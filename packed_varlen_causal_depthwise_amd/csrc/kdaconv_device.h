// Device helpers for the packed causal conv kernels (gfx950, wave64).
//
// The stored word of an output is bf16(act(acc)) where acc is the FP32
// accumulator, act is SiLU or the identity, SiLU(a) = a / (1 + exp(-a)) with exp
// correctly rounded to binary32 and the add and divide rounded to binary32, and
// bf16() rounds to nearest even (page "vllm.models.kimi_k3.nvidia.ops.kda_conv",
// module docstring: FP32 arithmetic, SiLU, FP32 -> bf16 round to nearest even).
//
// Only the final bf16 word is observable, so SiLU takes a fast path built on the
// hardware exp2 and reciprocal (a few FP32 ulps off the binary32 SiLU) and the
// word it rounds to is kept whenever the fast value is farther than that error
// bound from a bf16 rounding boundary: then the binary32 SiLU lies on the same
// side and rounds to the same word. The rare rest (and NaN, and a < kFastSiluMin
// where the fast exp argument loses accuracy) goes through an exact evaluation in
// double precision. The map from every FP32 input to its word is checked against
// the CPU reference on all 2^32 inputs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kdaconv {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Smallest accumulator the fast SiLU serves; below it, and for NaN, the exact path runs.
constexpr float kFastSiluMin = -8.0f;
// Bound, in FP32 ulps (distance between bit patterns), on |fast SiLU - binary32 SiLU|
// for kFastSiluMin <= a. Fast values within this many ulps of a bf16 rounding
// boundary are recomputed exactly.
constexpr uint32_t kSiluUlpBound = 16;

// bf16 -> FP32 is exact: the bf16 pattern is the upper half of the FP32 word.
__device__ __forceinline__ float widen_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float widen_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two FP32 values -> two bf16 words (round to nearest even), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// SiLU from the hardware exp2 and reciprocal; a few ulps from the binary32 value
// for a >= kFastSiluMin.
__device__ __forceinline__ float silu_fast(float a) {
  const float e = __builtin_amdgcn_exp2f(a * -1.44269504088896341f);
  return a * __builtin_amdgcn_rcpf(1.0f + e);
}

// True when y lies within kSiluUlpBound ulps of a point halfway between two bf16
// numbers (its low half-word within the bound of 0x8000).
__device__ __forceinline__ bool near_bf16_boundary(float y) {
  const uint32_t u = __float_as_uint(y);
  return ((u + (0x8000u + kSiluUlpBound)) << 16) <= ((2u * kSiluUlpBound) << 16);
}

// FP32 -> bf16 word, round to nearest even, NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t bf16_word_exact(float y) {
  if (y != y) return 0x7FC0u;
  const uint32_t u = __float_as_uint(y);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// The exact path is out of line (a call), so its double-precision temporaries do
// not count against the register budget of the streaming loop that rarely needs
// it (0 = inline).
#ifndef KDACONV_EXACT_OUTLINED
#define KDACONV_EXACT_OUTLINED 1
#endif
#if KDACONV_EXACT_OUTLINED
#define KDACONV_EXACT_INLINE __noinline__
#else
#define KDACONV_EXACT_INLINE __forceinline__
#endif

// The stored word by the defining steps. exp runs in double precision and is
// rounded once to binary32; the quotient is formed in double from the two binary32
// operands and rounded once to binary32, which equals the binary32 quotient (53 >=
// 2 * 24 + 2 bits, so the double rounding is innocuous).
__device__ KDACONV_EXACT_INLINE uint32_t act_word_exact(float a, bool silu) {
  float y = a;
  if (silu) {
    const float e = (float)exp(-(double)a);
    const float d = 1.0f + e;
    y = (float)((double)a / (double)d);
  }
  return bf16_word_exact(y);
}

// Does the fast path's word for accumulator a (fast SiLU value y) need the exact path?
template <bool kSilu>
__device__ __forceinline__ bool needs_exact(float a, float y) {
  if (kSilu) return !(a >= kFastSiluMin) | near_bf16_boundary(y);
  return a != a;
}

// R rows of N accumulators -> R rows of N stored words, two per 32-bit word
// (element k of a row in half-word k & 1 of word k / 2). One branch covers the
// rare exact path of all R * N elements, so the rows' fast paths can overlap.
template <bool kSilu, int N, int R>
__device__ __forceinline__ void activate_rows(const float (&acc)[R][N], uint32_t (&w)[R][N / 2]) {
  float y[R][N];
  bool redo = false;
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int k = 0; k < N; ++k) {
      y[r][k] = kSilu ? silu_fast(acc[r][k]) : acc[r][k];
      redo |= needs_exact<kSilu>(acc[r][k], y[r][k]);
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) w[r][i] = pack_bf16x2(y[r][2 * i], y[r][2 * i + 1]);
  }
  if (__builtin_expect(redo, 0)) {
    // Rare: collect this lane's elements that need the exact path, then run one
    // copy of it per element (selects instead of register-array indexing).
    uint32_t todo = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int k = 0; k < N; ++k) todo |= (uint32_t)needs_exact<kSilu>(acc[r][k], y[r][k]) << (r * N + k);
    }
    while (todo) {
      const int e = __builtin_ctz(todo);
      todo &= todo - 1;
      float a = acc[0][0];
#pragma unroll
      for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int k = 0; k < N; ++k) a = (e == r * N + k) ? acc[r][k] : a;
      }
      const uint32_t word = act_word_exact(a, kSilu);
      const int k = e % N;
      const uint32_t shift = (k & 1) * 16;
      const uint32_t keep = ~(0xFFFFu << shift);
      const uint32_t put = word << shift;
#pragma unroll
      for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int i = 0; i < N / 2; ++i)
          w[r][i] = (e == r * N + 2 * i + (k & 1)) ? ((w[r][i] & keep) | put) : w[r][i];
      }
    }
  }
}

// N accumulators -> N stored words (one row of activate_rows).
template <bool kSilu, int N>
__device__ __forceinline__ void activate_words(const float (&acc)[N], uint32_t (&w)[N / 2]) {
  const float (&a1)[1][N] = *reinterpret_cast<const float (*)[1][N]>(&acc);
  uint32_t (&w1)[1][N / 2] = *reinterpret_cast<uint32_t (*)[1][N / 2]>(&w);
  activate_rows<kSilu, N, 1>(a1, w1);
}

}  // namespace kdaconv
