/*
 * CPU oracle for the packed varlen causal depthwise width-4 convolution.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the bench's CPU
 * baseline load this file's library. It is plain, single-threaded and slow on
 * purpose, shares no code with the HIP path and is the definition the HIP path
 * is held to, bit for bit.
 *
 * What it computes comes from the page "vllm.models.kimi_k3.nvidia.ops.kda_conv":
 *   - module docstring, second paragraph: bf16 input widened to FP32 exactly,
 *     the stock conv arithmetic in FP32 with FP32 weights and FP32 conv state,
 *     SiLU, FP32 -> bf16 rounding to nearest even, output as dense
 *     (tokens, part_dim) planes;
 *   - module docstring, third paragraph: a sequence's conv state is read at its
 *     first token and the updated state written back once;
 *   - packed_causal_conv1d_fn docstring: semantics of causal_conv1d_fn on x.T,
 *     conv_states of shape (cache lines, dim, 3) updated in place, width-4
 *     taps, plane i holds channels [i*part_dim, (i+1)*part_dim);
 *   - packed_causal_conv1d_fn source: activation "silu"/"swish"/True selects
 *     SiLU; a null block id disables the state of the sequences mapped to it;
 *   - packed_causal_conv1d_supported: x may be bf16, fp16 or FP32, the state and
 *     the weights are FP32, and the output has x's dtype (the function's
 *     docstring); the arithmetic is FP32 for every input dtype (the note after
 *     the module docstring: the stock kernel computes in the state dtype).
 * and, for the decode step with a bf16 state, from the page
 * "vllm.models.kimi_k3.amd.ops.kda_decode": is_fused_kda_decode_supported (bf16
 * input, bf16 conv state) and make_decode_conv1d_weight_loader (the FP32 weight
 * mirrored width-major); its readings are stated at the function.
 *
 * Readings taken where the page is silent (each is listed in the design doc):
 *   - tap 3 multiplies the current token, tap 0 the token three back (causal
 *     conv as a left-padded cross-correlation);
 *   - state index 0 is the oldest of the three history values;
 *   - accumulation: start from the bias (or +0.0f), then one fused
 *     multiply-add per tap, oldest tap first;
 *   - SiLU is a / (1 + exp(-a)) with exp correctly rounded to binary32 and the
 *     add and the divide rounded to binary32 (round to nearest even);
 *   - the output rounds the FP32 result to x's dtype, to nearest even (bf16
 *     and fp16; an FP32 output is the result itself); fp16 keeps subnormal
 *     results and overflows to infinity;
 *   - a NaN result becomes the canonical quiet NaN of the output format:
 *     0x7FC0 (bf16), 0x7E00 (fp16), 0x7FC00000 (FP32);
 *   - fp16 -> FP32 widening is the IEEE 754 conversion: exact for every number;
 *     a NaN keeps its sign and payload and becomes quiet. bf16 -> FP32 and the
 *     FP32 input keep every bit (the state stores these widened values);
 *   - a sequence whose cache line is the null block runs from zero history and
 *     neither reads nor writes the state; has_initial_state false runs from
 *     zero history and still writes the state;
 *   - a cache line outside [0, num_cache_lines) names no line, and the sequence
 *     is treated like a null-block sequence (zero history, no state access);
 *   - a zero-length sequence does nothing.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math (see oracle/__init__.py).
 */
#include <math.h>
#include <quadmath.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL 1

static uint32_t bits_of(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return u;
}

static float float_of(uint32_t u) {
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* bf16 -> FP32. A bf16 number is the upper half of the FP32 word with the
 * same value, so the widening is exact. */
float oracle_bf16_to_f32(uint16_t h) { return float_of((uint32_t)h << 16); }

/* FP32 -> bf16, round to nearest, ties to even. bf16 keeps the upper 16 bits
 * of the FP32 word; the lower 16 bits decide the rounding. Values past the
 * largest bf16 round to infinity by the same rule (the carry runs into the
 * exponent). NaN becomes the quiet NaN 0x7FC0. */
uint16_t oracle_f32_to_bf16(float y) {
  if (isnan(y)) return 0x7FC0;
  uint32_t u = bits_of(y);
  uint32_t kept = u >> 16;       /* truncation toward zero */
  uint32_t dropped = u & 0xFFFFu; /* fraction of one bf16 ulp, in 1/65536 */
  if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1;
  return (uint16_t)kept;
}

/* Element formats of x and of the output (the output takes x's format). */
#define ORACLE_BF16 0
#define ORACLE_F16 1
#define ORACLE_F32 2

/* binary16 -> FP32 (IEEE 754 binary16: sign, 5 exponent bits biased by 15, 10
 * fraction bits). Numbers widen exactly: a subnormal is fraction * 2^-24, a
 * normal (1 + fraction / 1024) * 2^(exponent - 15). NaN keeps sign and payload
 * (fraction moved to the top of the FP32 fraction) and gets the quiet bit. */
float oracle_f16_to_f32(uint16_t h) {
  uint32_t sign = (uint32_t)(h >> 15) << 31;
  uint32_t expo = (h >> 10) & 0x1Fu;
  uint32_t frac = h & 0x3FFu;
  if (expo == 0x1Fu) {
    if (frac == 0) return float_of(sign | 0x7F800000u);
    return float_of(sign | 0x7FC00000u | (frac << 13));
  }
  float mag = expo == 0 ? ldexpf((float)frac, -24) : ldexpf((float)(1024u + frac), (int)expo - 25);
  return sign ? -mag : mag;
}

/* oracle_f16_to_f32 as a bit pattern (a float return value passed through a
 * double would lose a signalling NaN). */
uint32_t oracle_f16_to_f32_bits(uint16_t h) { return bits_of(oracle_f16_to_f32(h)); }

/* FP32 -> binary16, round to nearest, ties to even. The magnitude is divided by
 * the binary16 quantum of its binade (2^-24 below 2^-14, where binary16 numbers
 * are subnormal; 2^(e - 10) in [2^e, 2^(e+1))), an exact scaling by a power of
 * two, rounded to an integer with rintf (ties to even under the default mode)
 * and encoded. Magnitudes at or above 65520, the midpoint between the largest
 * binary16 number 65504 (odd last bit) and 2^16, round to infinity. NaN becomes
 * the quiet NaN 0x7E00. */
uint16_t oracle_f32_to_f16(float y) {
  if (isnan(y)) return 0x7E00;
  uint16_t sign = signbit(y) ? 0x8000 : 0;
  float a = fabsf(y);
  if (a >= 65520.0f) return sign | 0x7C00;
  if (a < 0x1p-14f) {
    /* m <= 1024; m == 1024 is 2^-14, the smallest normal, code 0x0400 */
    uint32_t m = (uint32_t)rintf(a * 0x1p24f);
    return (uint16_t)(sign | m);
  }
  int e;
  frexpf(a, &e);
  e -= 1; /* a in [2^e, 2^(e+1)), -14 <= e <= 15 */
  uint32_t m = (uint32_t)rintf(ldexpf(a, 10 - e)); /* in [1024, 2048] */
  if (m == 2048) {
    m = 1024;
    e += 1;
  }
  return (uint16_t)(sign | (uint32_t)((e + 15) << 10) | (m - 1024));
}

/* The stored FP32 word of an FP32 result: its bits, NaN -> 0x7FC00000. */
uint32_t oracle_f32_word(float y) { return isnan(y) ? 0x7FC00000u : bits_of(y); }

/* Element of x (format fmt) at index i, widened to FP32. */
static float load_x(const void* x, int fmt, int64_t i) {
  if (fmt == ORACLE_F32) return ((const float*)x)[i];
  uint16_t h = ((const uint16_t*)x)[i];
  return fmt == ORACLE_F16 ? oracle_f16_to_f32(h) : oracle_bf16_to_f32(h);
}

/* FP32 result -> stored word of format fmt. */
static uint32_t store_word(float y, int fmt) {
  if (fmt == ORACLE_F32) return oracle_f32_word(y);
  return fmt == ORACLE_F16 ? oracle_f32_to_f16(y) : oracle_f32_to_bf16(y);
}

/* Midpoint test for the correctly rounded exp below: nonzero when the double
 * value e lies within 2^-40 * e of a point halfway between two adjacent binary32
 * numbers (2^128 counts as the number above FLT_MAX). */
static int near_binary32_midpoint(double e) {
  if (!(e > 0.0) || isinf(e) || e >= 0x1p129) return 0;
  float r = (float)e;
  float below;
  if (isinf(r)) {
    below = 0x1.fffffep127f;
  } else if ((double)r > e) {
    below = nextafterf(r, 0.0f);
  } else {
    below = r;
  }
  float up = nextafterf(below, INFINITY);
  double above = isinf(up) ? 0x1p128 : (double)up;
  double mid = 0.5 * ((double)below + above); /* exact in double */
  return fabs(e - mid) <= 0x1p-40 * e;
}

/* exp(x) correctly rounded to binary32, round to nearest even.
 *
 * Method (the two-step scheme of the CORE-MATH project, Sibidanov, Zimmermann
 * and Glondu, ARITH 2022, written here from its description): evaluate exp in
 * double precision, whose relative error (libm, well under 2^-50) is far below
 * the half-ulp of binary32, and round that to binary32. The rounding can only go
 * wrong when the double value sits within its error of a binary32 midpoint; for
 * those inputs the value is recomputed in 113-bit quad precision (libquadmath)
 * and rounded from there. oracle/certify_expf.py checks the result against
 * mpmath at 160 bits on every input the midpoint test catches and on a random
 * sample of the rest. */
float oracle_crexpf(float x) {
  if (isnan(x)) return x + x;
  double e = exp((double)x);
  if (near_binary32_midpoint(e)) {
    __float128 q = expq((__float128)x);
    return (float)q;
  }
  return (float)e;
}

/* Nonzero when oracle_crexpf(x) took the quad-precision branch. */
int oracle_crexpf_escalates(float x) {
  if (isnan(x)) return 0;
  return near_binary32_midpoint(exp((double)x));
}

/* SiLU y = a / (1 + exp(-a)) with each operation rounded to binary32. */
static float silu32(float a) {
  float e = oracle_crexpf(-a);
  float d = 1.0f + e;
  return a / d;
}

/* The map from an FP32 accumulator to the stored word of format fmt: SiLU (or
 * y = a when silu == 0), then rounding to the format. */
uint32_t oracle_act_word(float a, int silu, int fmt) {
  return store_word(silu ? silu32(a) : a, fmt);
}

/* The same map for the bf16 output. */
uint16_t oracle_act_bf16(float a, int silu) { return (uint16_t)oracle_act_word(a, silu, ORACLE_BF16); }

/* oracle_act_word over count consecutive FP32 bit patterns starting at first;
 * out holds uint16 words (bf16, fp16) or uint32 words (FP32). */
void oracle_act_word_range(uint32_t first, uint64_t count, int silu, int fmt, void* out) {
  for (uint64_t i = 0; i < count; ++i) {
    uint32_t w = oracle_act_word(float_of((uint32_t)(first + i)), silu, fmt);
    if (fmt == ORACLE_F32)
      ((uint32_t*)out)[i] = w;
    else
      ((uint16_t*)out)[i] = (uint16_t)w;
  }
}

/* oracle_act_word over n FP32 bit patterns given in an array. */
void oracle_act_word_list(const uint32_t* in, uint64_t n, int silu, int fmt, void* out) {
  for (uint64_t i = 0; i < n; ++i) {
    uint32_t w = oracle_act_word(float_of(in[i]), silu, fmt);
    if (fmt == ORACLE_F32)
      ((uint32_t*)out)[i] = w;
    else
      ((uint16_t*)out)[i] = (uint16_t)w;
  }
}

/* bf16 forms of the two above. */
void oracle_act_bf16_range(uint32_t first, uint64_t count, int silu, uint16_t* out) {
  oracle_act_word_range(first, count, silu, ORACLE_BF16, out);
}

void oracle_act_bf16_list(const uint32_t* in, uint64_t n, int silu, uint16_t* out) {
  oracle_act_word_list(in, n, silu, ORACLE_BF16, out);
}

/* The FP32 accumulator of one output: bias (or +0.0f), then one fused
 * multiply-add per tap, oldest tap first. w points at the channel's four taps
 * (stride ws1 between taps); hist holds e[t-3], e[t-2], e[t-1], cur is e[t]. */
static float conv_acc(const float* w, int64_t ws1, const float* bias_c,
                      const float hist[3], float cur) {
  float acc = bias_c ? *bias_c : 0.0f;
  acc = fmaf(w[0 * ws1], hist[0], acc);
  acc = fmaf(w[1 * ws1], hist[1], acc);
  acc = fmaf(w[2 * ws1], hist[2], acc);
  acc = fmaf(w[3 * ws1], cur, acc);
  return acc;
}

/* The whole operation on host arrays.
 *
 * x:           elements of format fmt (ORACLE_BF16 / ORACLE_F16: uint16 bit
 *              patterns; ORACLE_F32: float), row t / channel c at
 *              x[t * x_row_stride + c], t < num_tokens.
 * weight:      FP32, tap k of channel c at weight[c * w_stride0 + k * w_stride1].
 * bias:        FP32 (dim,) or NULL.
 * conv_states: FP32, history k of channel c of line l at
 *              conv_states[l * cs_stride0 + c * cs_stride1 + k * cs_stride2];
 *              updated in place.
 * query_start_loc: int32 (num_seqs + 1), sequence s owns rows [qsl[s], qsl[s+1]).
 * cache_indices:   int32, the line of sequence s at cache_indices[s * ci_stride];
 *                  a value outside [0, num_cache_lines) acts as the null block.
 * has_initial_state: one byte per sequence, nonzero = start from the stored state;
 *                    NULL = no sequence has one.
 * out:         words of format fmt (uint16 for bf16 and fp16, uint32 for FP32),
 *              dense (dim / part_dim, num_tokens, part_dim); rows no sequence
 *              owns are left as they are.
 * Returns ORACLE_EINVAL (and writes nothing) for shapes or metadata it cannot
 * give a meaning to; ORACLE_OK otherwise. */
int oracle_packed_causal_conv1d(
    const void* x, int fmt, int64_t num_tokens, int64_t dim, int64_t x_row_stride,
    const float* weight, int64_t w_stride0, int64_t w_stride1, const float* bias,
    float* conv_states, int64_t num_cache_lines, int64_t cs_stride0, int64_t cs_stride1,
    int64_t cs_stride2, const int32_t* query_start_loc, int64_t num_seqs,
    const int32_t* cache_indices, int64_t ci_stride, const uint8_t* has_initial_state,
    int64_t part_dim, int silu, int has_null_block, int64_t null_block_id, void* out) {
  if (fmt != ORACLE_BF16 && fmt != ORACLE_F16 && fmt != ORACLE_F32) return ORACLE_EINVAL;
  if (num_tokens < 0 || dim < 0 || num_seqs < 0 || part_dim <= 0 || dim % part_dim != 0)
    return ORACLE_EINVAL;
  if (x_row_stride < dim) return ORACLE_EINVAL;
  /* Metadata check first, so that a rejected call leaves every output alone. */
  for (int64_t s = 0; s < num_seqs; ++s) {
    int64_t start = query_start_loc[s], end = query_start_loc[s + 1];
    if (start < 0 || end < start || end > num_tokens) return ORACLE_EINVAL;
  }

  for (int64_t s = 0; s < num_seqs; ++s) {
    int64_t start = query_start_loc[s], end = query_start_loc[s + 1];
    int64_t len = end - start;
    if (len == 0) continue; /* nothing to convolve, state untouched */
    int64_t line = cache_indices[s * ci_stride];
    int live = !(has_null_block && line == null_block_id) && line >= 0 && line < num_cache_lines;
    int init = live && has_initial_state && has_initial_state[s];
    for (int64_t c = 0; c < dim; ++c) {
      float hist[3] = {0.0f, 0.0f, 0.0f}; /* e[t-3], e[t-2], e[t-1] */
      if (init)
        for (int k = 0; k < 3; ++k)
          hist[k] = conv_states[line * cs_stride0 + c * cs_stride1 + k * cs_stride2];
      const float* w = weight + c * w_stride0;
      const float* b = bias ? bias + c : NULL;
      int64_t plane = c / part_dim, col = c % part_dim;
      for (int64_t i = 0; i < len; ++i) {
        int64_t t = start + i;
        float cur = load_x(x, fmt, t * x_row_stride + c);
        float acc = conv_acc(w, w_stride1, b, hist, cur);
        uint32_t word = oracle_act_word(acc, silu, fmt);
        int64_t o = (plane * num_tokens + t) * part_dim + col;
        if (fmt == ORACLE_F32)
          ((uint32_t*)out)[o] = word;
        else
          ((uint16_t*)out)[o] = (uint16_t)word;
        hist[0] = hist[1];
        hist[1] = hist[2];
        hist[2] = cur;
      }
      /* The window now holds the last three values of (history ++ x). */
      if (live)
        for (int k = 0; k < 3; ++k)
          conv_states[line * cs_stride0 + c * cs_stride1 + k * cs_stride2] = hist[k];
    }
  }
  return ORACLE_OK;
}

/* The decode step with the operands of the fused decode kernel on page
 * "vllm.models.kimi_k3.amd.ops.kda_decode": bf16 x with a bf16 conv state (the
 * dtypes is_fused_kda_decode_supported admits) and the FP32 weight mirrored
 * width-major, [part][width][channel within the part] (the docstring of
 * make_decode_conv1d_weight_loader). Row b of x is the one token of sequence b;
 * its history is the sequence's stored line.
 *
 * weight:      FP32, tap k of channel c at weight[(c / part_dim) * w_part_stride +
 *              (c % part_dim) * w_stride0 + k * w_stride1] (width-major:
 *              w_part_stride = 4 * part_dim, w_stride0 = 1, w_stride1 = part_dim).
 * conv_states: bf16 words, history k of channel c of line l at
 *              conv_states[l * cs_stride0 + c * cs_stride1 + k * cs_stride2].
 * Everything else as in oracle_packed_causal_conv1d, with one token per sequence
 * and every initial-state flag set.
 *
 * Readings (the page prints the dtypes and the weight layout, not the arithmetic):
 *   - the arithmetic is the FP32 chain of the prefill page: the weight is FP32 and
 *     bf16 values widen exactly, so the history and the token enter the chain as
 *     FP32 values and the output is rounded as for the FP32 state;
 *   - the line then holds entries 1 and 2 and the token. These are bf16 values
 *     already, so the words are kept as they are (a NaN keeps its payload); no
 *     rounding takes place. */
int oracle_packed_causal_conv1d_update_bf16_state(
    const uint16_t* x, int64_t batch, int64_t dim, int64_t x_row_stride,
    const float* weight, int64_t w_part_stride, int64_t w_stride0, int64_t w_stride1,
    const float* bias, uint16_t* conv_states, int64_t num_cache_lines, int64_t cs_stride0,
    int64_t cs_stride1, int64_t cs_stride2, const int32_t* cache_indices, int64_t ci_stride,
    int64_t part_dim, int silu, int has_null_block, int64_t null_block_id, uint16_t* out) {
  if (batch < 0 || dim < 0 || part_dim <= 0 || dim % part_dim != 0 || x_row_stride < dim)
    return ORACLE_EINVAL;
  for (int64_t b = 0; b < batch; ++b) {
    int64_t line = cache_indices[b * ci_stride];
    int live = line >= 0 && line < num_cache_lines && !(has_null_block && line == null_block_id);
    for (int64_t c = 0; c < dim; ++c) {
      uint16_t words[3] = {0, 0, 0}; /* +0.0 history when there is no line */
      if (live)
        for (int k = 0; k < 3; ++k)
          words[k] = conv_states[line * cs_stride0 + c * cs_stride1 + k * cs_stride2];
      float hist[3];
      for (int k = 0; k < 3; ++k) hist[k] = oracle_bf16_to_f32(words[k]);
      uint16_t xw = x[b * x_row_stride + c];
      int64_t plane = c / part_dim, col = c % part_dim;
      const float* w = weight + plane * w_part_stride + col * w_stride0;
      float acc = conv_acc(w, w_stride1, bias ? bias + c : NULL, hist, oracle_bf16_to_f32(xw));
      out[(plane * batch + b) * part_dim + col] = (uint16_t)oracle_act_word(acc, silu, ORACLE_BF16);
      if (live) {
        conv_states[line * cs_stride0 + c * cs_stride1 + 0 * cs_stride2] = words[1];
        conv_states[line * cs_stride0 + c * cs_stride1 + 1 * cs_stride2] = words[2];
        conv_states[line * cs_stride0 + c * cs_stride1 + 2 * cs_stride2] = xw;
      }
    }
  }
  return ORACLE_OK;
}

/* Certificate scan for oracle_crexpf over the FP32 bit patterns [first, first+count):
 * counts the inputs that take the quad branch and, among them, returns the
 * smallest distance (relative to the value) between the quad result and the
 * nearest binary32 midpoint, as a power-of-two exponent in *min_log2_gap.
 * Inputs with an escalation are written to cand (up to cand_cap of them). */
uint64_t oracle_crexpf_scan(uint32_t first, uint64_t count, uint32_t* cand, uint64_t cand_cap,
                            double* min_log2_gap) {
  uint64_t n = 0;
  double worst = 0.0;
  for (uint64_t i = 0; i < count; ++i) {
    uint32_t u = (uint32_t)(first + i);
    float x = float_of(u);
    if (!oracle_crexpf_escalates(x)) continue;
    if (n < cand_cap) cand[n] = u;
    ++n;
    __float128 q = expq((__float128)x);
    double e = (double)q;
    float r = (float)q;
    float below = ((double)r > e) ? nextafterf(r, 0.0f) : r;
    if (isinf(r)) below = 0x1.fffffep127f;
    float up = nextafterf(below, INFINITY);
    __float128 above = isinf(up) ? (__float128)0x1p128 : (__float128)up;
    __float128 mid = ((__float128)below + above) / 2;
    __float128 gap = (q - mid) / q;
    if (gap < 0) gap = -gap;
    double g = log2((double)gap);
    if (n == 1 || g < worst) worst = g;
  }
  *min_log2_gap = worst;
  return n;
}
