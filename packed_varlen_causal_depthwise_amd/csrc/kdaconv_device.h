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
// side and rounds to the same word. The rare rest (and NaN, and large negative
// accumulators, where the rounded exp2 argument loses accuracy) goes through an
// exact evaluation in double precision. The map from every FP32 input to its word
// is checked against the CPU reference on all 2^32 inputs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kdaconv {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Bound, in FP32 ulps (distance between bit patterns), on |fast SiLU - binary32 SiLU|
// wherever the fast path is trusted. Fast values within this many ulps of a bf16
// rounding boundary are recomputed exactly.
constexpr uint32_t kSiluUlpBound = 16;
// The fast path is trusted while its exp2 result stays below 2048, which holds for
// every a above about -7.6 (the product a * -log2(e) is rounded before the exp2, an
// error that grows with |a|). Larger results, and NaN (either sign), are taken by
// the exact path. Compared as bit patterns: exp2 never returns a negative number,
// and every NaN pattern lies above the threshold.
constexpr uint32_t kFastExpLimitBits = 0x45000000u;  // 2048.0f

// bf16 -> FP32 is exact: the bf16 pattern is the upper half of the FP32 word.
__device__ __forceinline__ float widen_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float widen_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two FP32 values -> two bf16 words (round to nearest even), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// SiLU from the hardware exp2 and reciprocal; e receives the exp2 result, which
// decides whether the value can be trusted (kFastExpLimitBits).
__device__ __forceinline__ float silu_fast(float a, float& e) {
  e = __builtin_amdgcn_exp2f(a * -1.44269504088896341f);
  return a * __builtin_amdgcn_rcpf(1.0f + e);
}

// Key of a fast value: its low half-word moved to the top plus an offset, so that
// the key is at least kNearKey exactly when the half-word lies within
// kSiluUlpBound of 0x8000, the point halfway between two bf16 numbers.
constexpr uint32_t kNearKey = (0x10000u - 2u * kSiluUlpBound - 1u) << 16;
constexpr uint32_t kNearOffset = 0u - ((0x8000u + kSiluUlpBound + 1u) << 16);
__device__ __forceinline__ uint32_t near_key(float y) {
  return (__float_as_uint(y) << 16) + kNearOffset;
}
// The same key in one instruction (the compiler emits a shift and an add, since the
// fused form takes no literal operand): offset must hold kNearOffset.
__device__ __forceinline__ uint32_t near_key_fused(float y, uint32_t offset) {
  uint32_t key;
  asm("v_lshl_add_u32 %0, %1, 16, %2" : "=v"(key) : "v"(y), "s"(offset));
  return key;
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

// Accumulators at or below this bound take the exact path. Every a with exp2 result
// at least 2048 (kFastExpLimitBits) lies below about -7.62, so the per-element test
// below flags a superset of what the reduction in activate_rows detects.
constexpr float kExactBelow = -7.5f;

// Does the fast word of accumulator a (fast value y) need the exact path? SiLU:
// y near a bf16 rounding boundary, or a below kExactBelow, or NaN; identity: NaN.
template <bool kSilu>
__device__ __forceinline__ bool needs_exact(float a, float y) {
  if (kSilu) return near_key(y) >= kNearKey || !(a >= kExactBelow);
  return a != a;
}

// R rows of N accumulators -> R rows of N fast words, two per 32-bit word (element k
// of a row in half-word k & 1 of word k / 2); y receives the fast values. Returns
// whether any element may need the exact path. The test is a reduction over all
// R * N elements (unsigned maxima of the keys and of the exp2 bit patterns; for the
// identity, a sum that is NaN if any term is) followed by one compare, so it costs
// about one instruction per element; a true result is followed by needs_exact on
// each element.
template <bool kSilu, int N, int R>
__device__ __forceinline__ bool activate_rows(const float (&acc)[R][N], float (&y)[R][N],
                                              uint32_t (&w)[R][N / 2]) {
  const uint32_t offset = kNearOffset;
  uint32_t key_max = 0, exp_max = 0;
  float sum = 0.0f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int k = 0; k < N; ++k) {
      if (kSilu) {
        float e;
        y[r][k] = silu_fast(acc[r][k], e);
        key_max = max(key_max, near_key_fused(y[r][k], offset));
        exp_max = max(exp_max, __float_as_uint(e));
      } else {
        y[r][k] = acc[r][k];
        sum += acc[r][k];
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) w[r][i] = pack_bf16x2(y[r][2 * i], y[r][2 * i + 1]);
  }
  return kSilu ? (key_max >= kNearKey || exp_max >= kFastExpLimitBits) : sum != sum;
}

// Elements whose fast word must be replaced, collected per wave in LDS and
// rewritten with their exact words in passes of 64 (one per lane). Deferring
// them lets a wave run the exact path once for the elements of many rows instead
// of once per row group in which any of its 64 lanes needs it. A flush first waits
// for the wave's earlier stores, so each exact word lands after the fast word it
// replaces. count is uniform across the wave.
template <int kCapacity>
struct FixupList {
  uint2* slots;  // kCapacity entries {accumulator bits, output offset} in LDS
  uint32_t count;

  // Appends {acc, offset} for every lane where flag holds.
  __device__ __forceinline__ void append(bool flag, float acc, uint32_t offset) {
    const uint64_t mask = __ballot(flag);
    if (mask == 0) return;
    if (flag) {
      const uint32_t below = __builtin_amdgcn_mbcnt_hi(
          (uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
      slots[count + below] = make_uint2(__float_as_uint(acc), offset);
    }
    count += (uint32_t)__popcll(mask);
  }

  // Whether appends of up to `incoming` more entries still fit.
  __device__ __forceinline__ bool fits(uint32_t incoming) const {
    return count + incoming <= (uint32_t)kCapacity;
  }

  // Writes the exact word of every entry through store(word, offset) and empties
  // the list.
  template <bool kSilu, class Store>
  __device__ __forceinline__ void flush(int lane, Store store) {
    if (count == 0) return;
    __builtin_amdgcn_s_waitcnt(0);  // earlier stores of this wave have completed
    for (uint32_t base = 0; base < count; base += 64) {
      const uint32_t i = base + (uint32_t)lane;
      if (i < count) {
        const uint2 e = slots[i];
        store(act_word_exact(__uint_as_float(e.x), kSilu), e.y);
      }
    }
    count = 0;
  }
};

}  // namespace kdaconv
