/*
 * libkdaconv: the packed varlen causal depthwise width-4 convolution of the
 * KDA prefill (the short convolution over the packed Q|K|V columns of the
 * in_proj output), for AMD Instinct MI355X (gfx950).
 *
 * Operation (page "vllm.models.kimi_k3.nvidia.ops.kda_conv": module docstring,
 * the packed_causal_conv1d_fn docstring and source, and
 * packed_causal_conv1d_supported for the admitted dtypes):
 *   For every sequence s, owning rows [qsl[s], qsl[s+1]) of x, and every channel c
 *   of dim = parts * part_dim channels, with e = (3 history values) ++ (the
 *   sequence's inputs widened to FP32):
 *     acc  = bias[c] (or +0.0f); then acc = fma(w[c][k], e[t-3+k], acc) for k = 0..3
 *     y    = SiLU(acc) = acc / (1 + exp(-acc)), each step in binary32 (or y = acc)
 *     out[c / part_dim][t][c % part_dim] = y in x's format: rounded to bf16 or
 *            fp16 to nearest even (fp16 keeps subnormals and overflows to
 *            infinity), or y itself for FP32
 *   The history is conv_states[cache_indices[s]][c][0..2] (index 0 oldest) when
 *   has_initial_state[s] is set, zeros otherwise. After the call that line holds
 *   the last three values of e. A sequence whose line equals null_block_id (when
 *   has_null_block is set) runs from zeros and leaves the states alone. A
 *   zero-length sequence does nothing. The result is bit-identical to a plain
 *   FP32 evaluation of these steps with a correctly rounded exp. NaN results are
 *   stored as the format's canonical quiet NaN (0x7FC0, 0x7E00, 0x7FC00000).
 *   bf16 and FP32 inputs widen bit for bit; fp16 inputs widen by the IEEE 754
 *   conversion (exact for numbers, a signalling NaN becomes quiet). The state
 *   receives the widened values.
 *
 * Conventions for every entry point:
 *   - Sizes and strides count ELEMENTS, not bytes. Pointers are DEVICE pointers
 *     unless stated otherwise, owned by the caller; the library allocates no
 *     memory, keeps no state between calls, never synchronises and never reads
 *     device data on the host. Work is queued on `stream` (NULL = the default
 *     stream) and the call returns before it finishes.
 *   - The launch geometry depends only on num_tokens, num_seqs and dim, so a
 *     call can be captured in a HIP graph and replayed with new device data of
 *     the same shapes.
 *   - Return values are the kdaconv_status codes below. Nothing is launched when
 *     a check fails; the output and the states are then left as they were.
 *   - Thread-safe: calls on different streams may run concurrently as long as
 *     they do not write the same memory.
 */
#ifndef KDACONV_H_
#define KDACONV_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t. */
struct ihipStream_t;
typedef struct ihipStream_t* kdaconv_stream_t;

typedef enum kdaconv_status {
  KDACONV_OK = 0,
  KDACONV_EINVAL = 1,       /* an argument is outside its documented range */
  KDACONV_EUNSUPPORTED = 2, /* meaningful, but a layout or size this library does not handle */
  KDACONV_ELAUNCH = 3       /* the HIP runtime refused the launch */
} kdaconv_status;

typedef enum kdaconv_activation {
  KDACONV_ACT_NONE = 0,
  KDACONV_ACT_SILU = 1
} kdaconv_activation;

/* Element format of x and of the output (the output takes x's format). */
typedef enum kdaconv_dtype {
  KDACONV_BF16 = 0,
  KDACONV_F16 = 1,
  KDACONV_F32 = 2
} kdaconv_dtype;

/*
 * The convolution (packed_causal_conv1d_fn on the page named above).
 *
 * x                  elements of format dtype; element (t, c) at
 *                    x[t * x_row_stride + c], rows t < num_tokens, channels c < dim.
 *                    Only columns [0, dim) are read. x_row_stride >= dim, any
 *                    value (page: unit column stride, any row stride). x must be
 *                    aligned to its element size (else EUNSUPPORTED). 4 channels
 *                    move as one vector whatever the alignment, so a Q|K|V slice
 *                    may start at any column; vectors at addresses that are not
 *                    multiples of 8 bytes (bf16, fp16) or 16 bytes (FP32) cost
 *                    some speed.
 * dtype              KDACONV_BF16, KDACONV_F16 or KDACONV_F32 (else EINVAL): the
 *                    format of x and of out.
 * weight             FP32; tap k of channel c at weight[c * weight_stride0 +
 *                    k * weight_stride1] (page layout [channel, width], width 4).
 * bias               FP32 (dim,) contiguous, or NULL for none.
 * conv_states        FP32, logical shape (num_cache_lines, dim, 3): history k of
 *                    channel c of line l at conv_states[l * cs_stride0 +
 *                    c * cs_stride1 + k * cs_stride2]. Read and written in place.
 *                    Any layout the strides describe: (lines, dim, 3) contiguous and
 *                    "dim first" (lines, 3, dim) take vector paths; a state wider
 *                    than 3 (lines, dim, W) passes its strides, entries 0..2 are the
 *                    history and the rest are not touched (the page's launch passes
 *                    the three strides and not the width).
 * query_start_loc    int32 (num_seqs + 1): sequence s owns rows [qsl[s], qsl[s+1]).
 *                    Must be non-decreasing with qsl[num_seqs] <= num_tokens; rows
 *                    outside every sequence are neither read nor written.
 * cache_indices      int32, the line of sequence s at cache_indices[s *
 *                    cache_indices_stride]. Live lines (not the null block) must be
 *                    distinct within a call. A line outside [0, num_cache_lines) is
 *                    treated like the null block (no state read or write).
 * has_initial_state  one byte per sequence (nonzero = start from the stored line),
 *                    or NULL: every sequence starts from zeros.
 * part_dim           channels per output plane; dim % part_dim == 0 (else EINVAL)
 *                    and part_dim % 8 == 0 (else EUNSUPPORTED).
 * activation         KDACONV_ACT_NONE or KDACONV_ACT_SILU (else EINVAL).
 * has_null_block,
 * null_block_id      when has_null_block != 0, sequences whose line equals
 *                    null_block_id skip the state (page: HAS_NULL_BLOCK).
 * out                elements of format dtype, dense (dim / part_dim, num_tokens,
 *                    part_dim), aligned to the element size (see x). Rows no
 *                    sequence owns are left unwritten.
 *
 * Device-data preconditions (not checked; violating them gives unspecified
 * values but no access outside the buffers described above): query_start_loc
 * non-decreasing and within [0, num_tokens]; distinct live lines.
 * num_tokens == 0, num_seqs == 0 or dim == 0 returns KDACONV_OK with no launch.
 */
int kdaconv_packed_causal_conv1d(
    const void* x, int dtype, int64_t num_tokens, int64_t dim, int64_t x_row_stride,
    const float* weight, int64_t weight_stride0, int64_t weight_stride1,
    const float* bias,
    float* conv_states, int64_t num_cache_lines,
    int64_t cs_stride0, int64_t cs_stride1, int64_t cs_stride2,
    const int32_t* query_start_loc, int64_t num_seqs,
    const int32_t* cache_indices, int64_t cache_indices_stride,
    const uint8_t* has_initial_state,
    int64_t part_dim, int activation, int has_null_block, int64_t null_block_id,
    void* out, kdaconv_stream_t stream);

/*
 * The decode step: the packed causal conv1d update of one token per sequence
 * (page "vllm.models.kimi_k3.amd.ops.kda_decode": the first of the three steps its
 * fused decode kernel replaces), with the FP32 state of the prefill op. Sequence b
 * of the batch owns row b of x. Its result is that of kdaconv_packed_causal_conv1d
 * on the same x with query_start_loc = {0, 1, ..., batch} and every
 * has_initial_state set: the history is the stored line (zeros for the null block,
 * whose line is neither read nor written), out[c / part_dim][b][c % part_dim] is the
 * activated, rounded tap sum, and the line becomes entries 1, 2 and the new token.
 * With an FP32 state the arithmetic is FP32 for every x dtype (page
 * "vllm.models.kimi_k3.nvidia.ops.kda_conv", packed_causal_conv1d_supported's note).
 * The bf16 state of the decode page's kernel is taken by
 * kdaconv_packed_causal_conv1d_update_bf16_state below.
 *
 * x                  elements of format dtype, (batch, dim) at row stride
 *                    x_row_stride (alignment as for the prefill op).
 * weight, bias,
 * conv_states,
 * cache_indices,
 * part_dim,
 * activation,
 * has_null_block,
 * null_block_id      as for kdaconv_packed_causal_conv1d; cache_indices has one
 *                    entry per sequence of the batch.
 * out                elements of format dtype, dense (dim / part_dim, batch, part_dim),
 *                    aligned to the element size.
 *
 * Precondition (not checked): live lines distinct within the batch.
 * batch == 0 or dim == 0 returns KDACONV_OK with no launch. Status codes and
 * their checks are those of kdaconv_packed_causal_conv1d, with batch in place of
 * num_tokens and num_seqs.
 */
int kdaconv_packed_causal_conv1d_update(
    const void* x, int dtype, int64_t batch, int64_t dim, int64_t x_row_stride,
    const float* weight, int64_t weight_stride0, int64_t weight_stride1,
    const float* bias,
    float* conv_states, int64_t num_cache_lines,
    int64_t cs_stride0, int64_t cs_stride1, int64_t cs_stride2,
    const int32_t* cache_indices, int64_t cache_indices_stride,
    int64_t part_dim, int activation, int has_null_block, int64_t null_block_id,
    void* out, kdaconv_stream_t stream);

/*
 * The decode step with the operands of the fused decode kernel on page
 * "vllm.models.kimi_k3.amd.ops.kda_decode": a bf16 conv state and the FP32 weight
 * mirrored width-major (is_fused_kda_decode_supported admits a bf16 input with a bf16
 * conv state, not dim-first; make_decode_conv1d_weight_loader's docstring gives the
 * weight as [qkv, width, channel]). The page prints no arithmetic. The reading taken:
 * the state's bf16 values and the token widen exactly to FP32 and go through the same
 * FP32 chain, activation and rounding as kdaconv_packed_causal_conv1d_update, so the
 * output equals that call on the widened state; the line then holds entries 1 and 2
 * and the token, whose words are kept unchanged (they are bf16 values already; a NaN
 * keeps its payload).
 *
 * x                  bf16 (batch, dim) at row stride x_row_stride (alignment as for
 *                    the prefill op). dtype must be KDACONV_BF16 (the page's gate);
 *                    fp16 and FP32 give EUNSUPPORTED, unknown codes EINVAL.
 * weight             FP32; tap k of channel c at weight[(c / part_dim) *
 *                    weight_part_stride + (c % part_dim) * weight_stride0 + k *
 *                    weight_stride1]. The page's width-major (dim / part_dim, 4,
 *                    part_dim) array is part stride 4 * part_dim, stride0 1, stride1
 *                    part_dim, and the prefill op's (dim, 4) array is 4 * part_dim,
 *                    4, 1; both take vector paths when 16-byte aligned, any other
 *                    strides a scalar one.
 * conv_states        bf16 words, logical shape (num_cache_lines, dim, 3): history k
 *                    of channel c of line l at conv_states[l * cs_stride0 + c *
 *                    cs_stride1 + k * cs_stride2]; (lines, dim, 3) contiguous and
 *                    8-byte aligned takes a vector path, any other strides a scalar
 *                    one. Read and written in place.
 * bias, cache_indices,
 * part_dim, activation,
 * has_null_block,
 * null_block_id, out as for kdaconv_packed_causal_conv1d_update (out is bf16).
 *
 * Precondition (not checked): live lines distinct within the batch.
 * batch == 0 or dim == 0 returns KDACONV_OK with no launch. Status codes and their
 * checks are those of kdaconv_packed_causal_conv1d_update, and a negative
 * weight_part_stride gives EUNSUPPORTED.
 */
int kdaconv_packed_causal_conv1d_update_bf16_state(
    const void* x, int dtype, int64_t batch, int64_t dim, int64_t x_row_stride,
    const float* weight, int64_t weight_part_stride, int64_t weight_stride0,
    int64_t weight_stride1, const float* bias,
    uint16_t* conv_states, int64_t num_cache_lines,
    int64_t cs_stride0, int64_t cs_stride1, int64_t cs_stride2,
    const int32_t* cache_indices, int64_t cache_indices_stride,
    int64_t part_dim, int activation, int has_null_block, int64_t null_block_id,
    void* out, kdaconv_stream_t stream);

/*
 * Host-only check of the same arguments (page: packed_causal_conv1d_supported):
 * returns the status kdaconv_packed_causal_conv1d would return before launching.
 * Pointers are only compared with NULL and tested for alignment, never
 * dereferenced, so host addresses may stand in for device ones. Makes no HIP call.
 */
int kdaconv_validate(
    const void* x, int dtype, int64_t num_tokens, int64_t dim, int64_t x_row_stride,
    const float* weight, int64_t weight_stride0, int64_t weight_stride1,
    const float* bias,
    const float* conv_states, int64_t num_cache_lines,
    int64_t cs_stride0, int64_t cs_stride1, int64_t cs_stride2,
    const int32_t* query_start_loc, int64_t num_seqs,
    const int32_t* cache_indices, int64_t cache_indices_stride,
    const uint8_t* has_initial_state,
    int64_t part_dim, int activation, int has_null_block, int64_t null_block_id,
    const void* out);

/*
 * The device map from an FP32 accumulator to the stored word of format dtype,
 * exactly as the convolution kernel applies it (SiLU or none, then the format's
 * rounding; module docstring of the page named above), evaluated for the `count`
 * FP32 bit patterns first, first + 1, ... (wrapping at 2^32). out: device array of
 * `count` words (uint16 for bf16 and fp16, uint32 for FP32), 16-byte aligned.
 * count must be a multiple of 8 (else EINVAL). Used to check the kernel's
 * activation against a reference on every input.
 */
int kdaconv_activation_map(uint32_t first, int64_t count, int activation, int dtype, void* out,
                           kdaconv_stream_t stream);

/* Static English text for a status code. Never NULL. */
const char* kdaconv_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int kdaconv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDACONV_H_ */
