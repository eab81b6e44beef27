// Device helpers for the packed causal conv kernels (gfx950, wave64).
//
// The stored word of an output is word(act(acc)) where acc is the FP32
// accumulator, act is SiLU or the identity, SiLU(a) = a / (1 + exp(-a)) with exp
// correctly rounded to binary32 and the add and divide rounded to binary32, and
// word() is the output format's rounding: bf16 or fp16 to nearest even, or the
// FP32 value itself; NaN results are stored as the format's canonical quiet NaN
// (page "vllm.models.kimi_k3.nvidia.ops.kda_conv", module docstring: FP32
// arithmetic, SiLU, rounding to nearest even; packed_causal_conv1d_fn: output in
// x's dtype; packed_causal_conv1d_supported: bf16, fp16 or FP32 x).
//
// For the 16-bit formats only the rounded word is observable, so SiLU takes a fast
// path built on the hardware exp2 and reciprocal (a few FP32 ulps off the binary32
// SiLU) and the word it rounds to is kept whenever the fast value is farther than
// that error bound from a rounding boundary of the format: then the binary32 SiLU
// lies on the same side and rounds to the same word. The rare rest (and NaN, large
// negative accumulators, where the rounded exp2 argument loses accuracy, and for
// fp16 the accumulators whose SiLU is an fp16 subnormal) goes through an exact
// evaluation. The FP32 format stores the binary32 SiLU itself, so every element
// takes the exact evaluation's main step (exp in double precision, rounded once),
// and only arguments whose double exp lies near a binary32 rounding boundary go on
// to a double-double exp. The map from every FP32 input to its word is checked
// against the CPU reference on all 2^32 inputs, for every format.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kdaconv {

// Element formats of x and out (the output takes x's format); the numbers are the
// kdaconv_dtype codes of the C interface.
enum : int { kBF16 = 0, kF16 = 1, kF32 = 2 };

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Bytes of one element of a format.
template <int kF>
constexpr int element_bytes() {
  return kF == kF32 ? 4 : 2;
}

// --------------------------------------------------------------------------------------
// Widening and packing.

// bf16 -> FP32 is exact: the bf16 pattern is the upper half of the FP32 word.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp16 -> FP32 with the hardware conversion (exact for numbers; a signalling NaN
// comes out quiet with its payload).
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Element 0 or 1 of a 32-bit word of a 16-bit format, widened.
template <int kF>
__device__ __forceinline__ float widen_half(uint32_t w, int hi) {
  if (kF == kF16) return hi ? f16_hi(w) : f16_lo(w);
  return hi ? bf16_hi(w) : bf16_lo(w);
}

// Two FP32 values -> two words of a 16-bit format, round to nearest even (one
// v_cvt_pk_bf16_f32 or v_cvt_pk_f16_f32).
template <int kF>
__device__ __forceinline__ uint32_t pack_pair(float lo, float hi) {
  const f32x2 v = {lo, hi};
  if (kF == kF16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// The stored word of a binary32 result, by the format's rule (canonical NaN).
template <int kF>
__device__ __forceinline__ uint32_t word_exact(float y) {
  if (kF == kF32) return y != y ? 0x7FC00000u : __float_as_uint(y);
  if (kF == kF16) {
    if (y != y) return 0x7E00u;
    return __builtin_bit_cast(uint16_t, (_Float16)y);
  }
  if (y != y) return 0x7FC0u;
  const uint32_t u = __float_as_uint(y);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// --------------------------------------------------------------------------------------
// Fast SiLU for the 16-bit formats.

// Where the fast path is trusted, and how far from the binary32 SiLU it may be. The
// error, in FP32 ulps (distance between bit patterns), comes from the rounded exp2
// argument (about |a| * 2^-24 relative, so it grows with -a), the exp2 and
// reciprocal approximations and two roundings. Measured on gfx950 over all 2^32
// inputs: at most 3 ulps for a >= 0, 5 for -4 <= a < 0, 9 for -7.5 <= a < -4. The
// bounds below keep one ulp to spare, and the exhaustive activation-map tests check
// the resulting words on every input.
//
// Each format trades the width of the nearness window against how many accumulators
// skip the fast path. bf16 drops 16 bits, so even a 10-ulp window is rare (0.03 % of
// values) and the fast path is trusted down to a = -7.5. fp16 drops 13 bits, where a
// 10-ulp window would send 0.26 % of values to the exact path; it trusts the fast
// path only down to a = -4 and uses the 6-ulp bound that holds there.
//
//   silu_bound<kF>()      bound on the error where the fast path is trusted
//   exact_below<kF>()     accumulators below it take the exact path
//   fast_exp_limit<kF>()  row test for them: every a below exact_below has an exp2
//                         result at or above this bit pattern (1800.0f, under the
//                         1808.04 that a = -7.5 gives; 54.5f, under the 54.598 of
//                         a = -4; both far beyond the exp2 error), so a row whose
//                         largest exp2 result is smaller holds none. NaN of either
//                         sign also lies above it: exp2 never returns a negative
//                         number and every NaN pattern is larger.
template <int kF>
constexpr uint32_t silu_bound() {
  return kF == kF16 ? 6u : 10u;
}
template <int kF>
constexpr float exact_below() {
  return kF == kF16 ? -4.0f : -7.5f;
}
template <int kF>
constexpr uint32_t fast_exp_limit() {
  return kF == kF16 ? 0x425A0000u : 0x44E10000u;
}

// SiLU from the hardware exp2 and reciprocal; e receives the exp2 result, which
// decides whether the value can be trusted (fast_exp_limit).
__device__ __forceinline__ float silu_fast(float a, float& e) {
  e = __builtin_amdgcn_exp2f(a * -1.44269504088896341f);
  return a * __builtin_amdgcn_rcpf(1.0f + e);
}

// Dropped bits of each 16-bit format (fp16: normal range; subnormal results are
// sent to the exact path separately).
template <int kF>
constexpr int dropped_bits() {
  return kF == kF16 ? 13 : 16;
}

// Nearness keys. A format keeps the upper bits of the FP32 word and drops the low
// dropped_bits<kF>() bits; the value is halfway between two neighbours of the format
// when they equal half their range. The key moves the dropped bits to the top of a word
// and adds an offset, so that it is at least near_limit<kF>() exactly when the
// dropped bits lie within silu_bound<kF>() of the halfway point.
template <int kF>
constexpr uint32_t near_limit() {
  return ((1u << dropped_bits<kF>()) - 2u * silu_bound<kF>() - 1u) << (32 - dropped_bits<kF>());
}
template <int kF>
constexpr uint32_t near_offset() {
  return 0u - (((1u << (dropped_bits<kF>() - 1)) + silu_bound<kF>() + 1u) << (32 - dropped_bits<kF>()));
}
template <int kF>
__device__ __forceinline__ uint32_t near_key(float y) {
  return (__float_as_uint(y) << (32 - dropped_bits<kF>())) + near_offset<kF>();
}
// The same key in one instruction (the compiler emits a shift and an add, since the
// fused form takes no literal operand): offset must hold near_offset<kF>().
template <int kF>
__device__ __forceinline__ uint32_t near_key_fused(float y, uint32_t offset) {
  uint32_t key;
  asm("v_lshl_add_u32 %0, %1, %2, %3" : "=v"(key) : "v"(y), "n"(32 - dropped_bits<kF>()), "s"(offset));
  return key;
}

// fp16: a SiLU below 2^-14 in magnitude is an fp16 subnormal, whose rounding
// boundaries the key does not see. For a above exact_below that needs |a| < 2^-12.6
// (SiLU(a) = a * sigmoid(a) with sigmoid(a) > 0.4 there), so |a| < 2^-12 goes exact.
constexpr float kTinyF16 = 0x1p-12f;

// --------------------------------------------------------------------------------------
// Exact evaluation.

// exp in double precision, rounded once to binary32, and the key of the dropped bits
// of the double value: the binary32 rounding keeps the top 23 of its 52 fraction bits,
// so the low 29 bits of the low word decide it, halfway at 2^28. The key is at least
// kDoubleNearLimit when they lie within 2^12 of halfway (about 2^-40 relative), far
// wider than the error of the double exp; only those arguments need more precision.
// The key does not apply where the binary32 result is subnormal (a > 87.3), where
// 1 + exp(-a) rounds to 1 whatever the last bit of exp(-a), nor does any result there
// need it.
constexpr uint32_t kDoubleWindow = 1u << 12;
constexpr uint32_t kDoubleNearLimit = ((1u << 29) - 2u * kDoubleWindow - 1u) << 3;
constexpr uint32_t kDoubleNearOffset = 0u - (((1u << 28) + kDoubleWindow + 1u) << 3);

__device__ __forceinline__ float exp_neg_double(float a, uint32_t& key) {
  const double ed = exp(-(double)a);
  key = ((uint32_t)__double_as_longlong(ed) << 3) + kDoubleNearOffset;
  return (float)ed;
}

// Double-double helpers (Knuth's two-sum and the FMA two-product).
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
  s = a + b;
  const double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}
__device__ __forceinline__ void quick_two_sum(double a, double b, double& s, double& e) {
  s = a + b;
  e = b - (s - a);
}

// exp(x) as hi + lo with a relative error far below 2^-90, for binary32 x with
// |x| <= 104 (beyond, the binary32 result is 0, a subnormal that cannot matter, or
// infinity). Argument reduction x = k ln2 + r with ln 2 as a double-double, then
// exp(r) = 1 + r/1 (1 + r/2 (1 + ... (1 + r/22))) in double-double arithmetic
// (|r| <= 0.35, so the dropped terms are below 2^-103), scaled by 2^k.
__device__ __forceinline__ void exp_double_double(float x, double& hi, double& lo) {
  const double kLn2Hi = 0x1.62e42fefa39efp-1;
  const double kLn2Lo = 0x1.abc9e3b39803fp-56;
  const double xd = (double)x;
  const double k = __builtin_rint(xd * 0x1.71547652b82fep+0);
  // k * kLn2Hi exactly as ph + pl; x - ph is exact (Sterbenz: x and ph within a
  // factor of two whenever k != 0).
  const double ph = k * kLn2Hi;
  const double pl = __builtin_fma(k, kLn2Hi, -ph);
  double rh, rl;
  two_sum(xd - ph, -pl, rh, rl);
  rl -= k * kLn2Lo;
  quick_two_sum(rh, rl, rh, rl);
  double sh = 1.0, sl = 0.0;
#pragma unroll 1
  for (int n = 22; n >= 1; --n) {
    // (sh, sl) * (rh, rl)
    double th = sh * rh;
    double tl = __builtin_fma(sh, rh, -th) + (sh * rl + sl * rh);
    quick_two_sum(th, tl, th, tl);
    // / n: q = th / n, remainder th - q n exact by FMA
    const double dn = (double)n;
    const double qh = th / dn;
    const double rem = __builtin_fma(-qh, dn, th);
    const double ql = (rem + tl) / dn;
    // 1 + q
    double uh, ul;
    two_sum(1.0, qh, uh, ul);
    ul += ql;
    quick_two_sum(uh, ul, sh, sl);
  }
  const int ki = (int)k;
  hi = __builtin_ldexp(sh, ki);
  lo = __builtin_ldexp(sl, ki);
}

// exp(x) correctly rounded to binary32 (normal results; subnormal results may be one
// unit off at an exact double midpoint, which no use here can observe).
__device__ __forceinline__ float exp_binary32_escalated(float x) {
  if (!(x >= -104.0f)) return x != x ? x : 0.0f;
  if (x > 104.0f) return __builtin_inff();
  double hi, lo;
  exp_double_double(x, hi, lo);
  // hi is the double nearest to hi + lo, so rounding hi to binary32 is right unless
  // hi is itself halfway between two binary32 numbers; then lo's sign decides.
  const uint64_t bits = (uint64_t)__double_as_longlong(hi);
  if ((bits & 0x1FFFFFFFull) == 0x10000000ull && lo != 0.0)
    hi = lo > 0.0 ? __longlong_as_double((long long)(bits + 1)) : __longlong_as_double((long long)(bits - 1));
  return (float)hi;
}

// exp(-a) correctly rounded to binary32 (within the normal range, see above).
__device__ __forceinline__ float exp_neg_binary32(float a) {
  uint32_t key;
  const float e = exp_neg_double(a, key);
  if (key >= kDoubleNearLimit) return exp_binary32_escalated(-a);
  return e;
}

// The binary32 SiLU by the defining steps.
__device__ __forceinline__ float silu_binary32(float a) {
  const float e = exp_neg_binary32(a);
  const float d = 1.0f + e;
  return a / d;
}

// The exact path is out of line (a call), so its double-precision temporaries do
// not count against the register budget of the streaming code that rarely needs it.
template <int kF>
__device__ __noinline__ uint32_t act_word_exact(float a, bool silu) {
  return word_exact<kF>(silu ? silu_binary32(a) : a);
}

// --------------------------------------------------------------------------------------
// Activation of rows of accumulators.

// Does the word of accumulator a (value y, aux from activate_rows) need the exact
// path? SiLU, bf16: y near a rounding boundary (its key recomputed here), a below
// exact_below, or NaN; SiLU, fp16: the same with the key from aux, or a subnormal
// result; SiLU, FP32: the double exp near a binary32 rounding boundary (key in aux),
// or a NaN value; identity: NaN.
template <int kF, bool kSilu>
__device__ __forceinline__ bool needs_exact(float a, float y, uint32_t aux) {
  if (!kSilu) return a != a;
  if (kF == kF32) return aux >= kDoubleNearLimit || y != y;
  const uint32_t key = kF == kF16 ? aux : near_key<kF>(y);
  const bool near = key >= near_limit<kF>() || !(a >= exact_below<kF>());
  if (kF == kF16) return near || __builtin_fabsf(a) < kTinyF16;
  return near;
}

// Words per row of N elements.
template <int kF, int N>
constexpr int row_words() {
  return kF == kF32 ? N : N / 2;
}

// R rows of N accumulators -> R rows of words (16-bit formats: element k of a row in
// half-word k & 1 of word k / 2; FP32: one word per element); y receives the values
// whose words were formed, aux what needs_exact takes besides. Returns whether any
// element may need the exact path. The test is a reduction over all R * N elements
// (unsigned maxima of keys and of exp2 bit patterns, a minimum of magnitudes, or a
// sum that is NaN if any term is) followed by one compare, so it costs about one
// instruction per element; a true result is followed by needs_exact on each element.
template <int kF, bool kSilu, int N, int R>
__device__ __forceinline__ bool activate_rows(const float (&acc)[R][N], float (&y)[R][N],
                                              uint32_t (&aux)[R][N],
                                              uint32_t (&w)[R][row_words<kF, N>()]) {
  const uint32_t offset = near_offset<kF>();
  uint32_t key_max = 0, exp_max = 0;
  float sum = 0.0f;
  float amin = __builtin_inff();
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int k = 0; k < N; ++k) {
      aux[r][k] = 0;
      if (kSilu && kF == kF32) {
        const float e = exp_neg_double(acc[r][k], aux[r][k]);
        y[r][k] = acc[r][k] / (1.0f + e);
        key_max = max(key_max, aux[r][k]);
        sum += y[r][k];
      } else if (kSilu) {
        float e;
        y[r][k] = silu_fast(acc[r][k], e);
        const uint32_t key = near_key_fused<kF>(y[r][k], offset);
        if (kF == kF16) aux[r][k] = key;
        key_max = max(key_max, key);
        exp_max = max(exp_max, __float_as_uint(e));
        if (kF == kF16) amin = __builtin_fminf(amin, __builtin_fabsf(acc[r][k]));
      } else {
        y[r][k] = acc[r][k];
        sum += acc[r][k];
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (kF == kF32) {
#pragma unroll
      for (int k = 0; k < N; ++k) w[r][k] = __float_as_uint(y[r][k]);
    } else {
#pragma unroll
      for (int i = 0; i < N / 2; ++i) w[r][i] = pack_pair<kF>(y[r][2 * i], y[r][2 * i + 1]);
    }
  }
  if (!kSilu) return sum != sum;
  if (kF == kF32) return key_max >= kDoubleNearLimit || sum != sum;
  const bool flag = key_max >= near_limit<kF>() || exp_max >= fast_exp_limit<kF>();
  if (kF == kF16) return flag || amin < kTinyF16;
  return flag;
}

// Elements whose word must be replaced, collected per wave in LDS and rewritten
// with their exact words in passes of 64 (one per lane). Deferring them lets a
// wave run the exact path once for the elements of many rows instead of once per
// row group in which any of its 64 lanes needs it. A flush first waits for the
// wave's earlier stores, so each exact word lands after the word it replaces.
// count is uniform across the wave.
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

  // Writes the exact word (format kF) of every entry through store(word, offset)
  // and empties the list.
  template <int kF, bool kSilu, class Store>
  __device__ __forceinline__ void flush(int lane, Store store) {
    if (count == 0) return;
    __builtin_amdgcn_s_waitcnt(0);  // earlier stores of this wave have completed
    for (uint32_t base = 0; base < count; base += 64) {
      const uint32_t i = base + (uint32_t)lane;
      if (i < count) {
        const uint2 e = slots[i];
        store(act_word_exact<kF>(__uint_as_float(e.x), kSilu), e.y);
      }
    }
    count = 0;
  }
};

}  // namespace kdaconv
