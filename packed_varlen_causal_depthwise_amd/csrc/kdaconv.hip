// libkdaconv: packed varlen causal depthwise width-4 convolution for MI355X (gfx950).
//
// Page "vllm.models.kimi_k3.nvidia.ops.kda_conv" (module docstring; the
// packed_causal_conv1d_fn docstring and source; packed_causal_conv1d_supported)
// defines the operation; include/kdaconv.h states it in full.
//
// Work decomposition. A program is one wave64 handling a tile of R consecutive
// tokens of one sequence over 64 * kLaneChannels channels: each lane owns
// kLaneChannels consecutive channels, so every x row and every output row of the
// tile moves as one vector per lane (8 bytes for bf16 and fp16, 16 for FP32; R is
// 16 for the 16-bit formats and 8 for FP32, so a wave's loads in flight stay the
// same). Tile j of sequence s covers rows [start + j*R, start + (j+1)*R) of the
// sequence. Programs 0 .. num_seqs-1 are the sequences' first tiles, which need no
// search; the later programs go to row blocks q, each owning the later tile (if
// any) that starts in rows [(q+1) R, (q+2) R), whose sequence the wave finds with a
// radix-64 search over query_start_loc (one ballot per level). The last row blocks
// are split into halves and quarters (describe_tile), so that the waves that run at
// the end of the launch are short. The grid depends only on host sizes, so the
// launch can be captured in a graph; programs without a tile exit at once. The
// launch is one-dimensional; workgroups dispatched together cover whole rows, in
// chunks ordered so that each column group stays on one XCD (wave_slot). Waves are
// short, and the dispatcher keeps every SIMD supplied with new ones until the end
// (long-lived waves started together finish unevenly, since a SIMD issues from its
// oldest wave first).
//
// Memory. A wave issues the loads of its 3 history rows and of all its tile rows
// before any arithmetic. Tile rows are streamed (nontemporal), except the last
// three, which the next tile of the column block reads again as its history and
// which therefore stay cacheable (in the L2 of the XCD that runs both tiles), like
// the history loads themselves. Outputs are
// streamed. x and out are addressed through buffer descriptors based at the
// tile's first row: the lane's channel offset is a fixed vector register and each
// row's offset a scalar. Lanes past the launch's last channel (only in a partial
// last column block) redo the last active lane's channels: same rows, same
// weights, and the same state read by the same instruction of the same wave, so
// they store the same bytes to the same place and the stores need no branch.
//
// State. Only the first tile of a sequence reads the sequence's conv-state line,
// and the same program writes the updated line after its reads (page, module
// docstring).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "kdaconv.h"
#include "kdaconv_device.h"

namespace kdaconv {
namespace {

constexpr int kWave = 64;
constexpr int kLaneChannels = 4;  // channels per lane
// Tiles of at most this many rows (short sequences, a sequence's last rows) take a
// path that loads only kShort rows. On 4096 sequences of 1-4 tokens it measured 15 %
// faster than loading all R rows; 8 rows gained half as much; longer workloads are
// unchanged.
constexpr int kShort = 4;
// The launch's last row blocks are split so that about this many waves compute
// half tiles and, after them, this many quarter tiles (for 18 column blocks: the
// 1024 rows before the last 256 in 8-row parts, and those 256 in 4-row parts).
constexpr int kHalfTileWaves = 2304;
constexpr int kQuarterTileWaves = 1152;
constexpr int kMinWaves = 4;  // occupancy target (waves per SIMD)
// Small calls (at most this many tokens, one sequence or sequences averaging at least
// kSmallCallTokensPerSeq tokens) take 8-row tiles: twice the waves for a launch that
// would not fill the GPU. Interleaved, outputs identical, 4608 channels: one sequence of
// 1024 tokens 8.56 -> 7.92 us (fp16 10.36 -> 8.88 us), of 2048 tokens 11.73 -> 11.26 us;
// 64 tokens at 384 channels 6.46 -> 5.86 us. Slower: one sequence of 2560 tokens
// (12.90 -> 13.09 us) or 3072 tokens (14.39 -> 15.04 us), and 8 sequences of 988 tokens
// in all (7.92 -> 8.03 us).
constexpr int64_t kSmallCallTokens = 2048;
constexpr int64_t kSmallCallTokensPerSeq = 256;
// Fixup list entries per wave (8 bytes each in LDS): room for one row group of
// every lane beyond the entries that trigger a flush.
constexpr int kFixCapacity = 640;
// Cache-policy bits of buffer loads and stores (gfx950: 1 = sc0, 2 = nt, 16 = sc1).
constexpr int kStream = 2;  // nontemporal
constexpr int kKeep = 0;  // default caching
constexpr uint32_t kDescWord3 = 0x00020000u;  // gfx9 raw buffer: 32-bit data format
constexpr int32_t kRange = 0x7FFFFFFF;
// Conv-state element formats: the FP32 state of the prefill op, and the bf16 state
// of the decode step with the fused decode kernel's operands.
constexpr int kStateF32 = 0;
constexpr int kStateBF16 = 1;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Tokens per program for each format.
template <int kF>
constexpr int rows_per_tile() {
  return kF == kF32 ? 8 : 16;
}

int rows_per_tile(int dtype) { return dtype == kF32 ? rows_per_tile<kF32>() : rows_per_tile<kBF16>(); }

// Buffer loads and stores of kBytes per lane. A lane's vector may start at any element
// of x or out (a Q|K|V slice at any column, rows any number of elements apart): queues of
// the HSA runtime on gfx9-family GPUs run with unaligned vector memory access enabled,
// which the compiler's own code for the amdhsa target also relies on (it moves
// unaligned copies with 8-byte loads and stores). Vectors that are not naturally aligned
// cost some speed, not correctness.
template <int kBytes>
struct Lane;

template <>
struct Lane<8> {
  typedef u32x2 vec;
  template <int kPolicy>
  static __device__ __forceinline__ vec load(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, vo, so, kPolicy);
  }
  template <int kPolicy>
  static __device__ __forceinline__ void store(vec v, __amdgpu_buffer_rsrc_t r, uint32_t vo,
                                               uint32_t so) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, vo, so, kPolicy);
  }
};

template <>
struct Lane<16> {
  typedef u32x4 vec;
  template <int kPolicy>
  static __device__ __forceinline__ vec load(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, vo, so, kPolicy);
  }
  template <int kPolicy>
  static __device__ __forceinline__ void store(vec v, __amdgpu_buffer_rsrc_t r, uint32_t vo,
                                               uint32_t so) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, vo, so, kPolicy);
  }
};

struct ConvParams {
  const char* x;
  const float* weight;
  const float* bias;
  float* states;
  const int32_t* __restrict__ qsl;
  const int32_t* __restrict__ cache_indices;
  const uint8_t* __restrict__ has_init;
  char* out;  // first plane of this launch
  int64_t x_row_stride;
  int64_t w_stride0, w_stride1;
  int64_t w_part_stride;  // tap k of channel c at (c / part_dim) * w_part_stride +
                          // (c % part_dim) * w_stride0 + k * w_stride1
  int64_t cs_stride0, cs_stride1, cs_stride2;
  int64_t ci_stride;
  int64_t num_cache_lines;
  int64_t plane_stride;  // num_tokens * part_dim
  int64_t null_block_id;
  int32_t num_tokens;
  int32_t num_seqs;
  int32_t col_begin;  // first channel of this launch
  int32_t col_end;  // one past its last channel
  int32_t col_blocks;  // column blocks of 64 * kLaneChannels channels in this launch
  int32_t programs;  // programs per column block
  int32_t split_half;  // first row block whose later tile is taken by 2 programs
  int32_t split_quarter;  // first row block whose later tile is taken by 4 programs
  // Division of the workgroup index by the workgroups per program (set by the
  // launcher): n / groups = (umulhi(n, group_magic) + n) >> group_shift for n < 2^31.
  uint32_t group_magic;
  int32_t group_shift;
  // The same for 8 * groups (prefill: workgroups per chunk of 8 programs), and the
  // number of whole chunks; 0 selects the plain order.
  uint32_t chunk_magic;
  int32_t chunk_shift;
  int32_t full_chunks;
  int32_t part_dim;
  int32_t search_levels;  // radix-64 levels: smallest L with 64^L >= num_seqs
  int32_t search_top;  // 64^(search_levels - 1)
  int32_t has_null_block;
  int32_t weight_vec;  // weight is (dim, 4) contiguous and 16-byte aligned
  int32_t weight_wm;  // bf16-state decode: weight is width-major with 4-aligned strides,
                      // 16-byte aligned (a lane's 4 channels of one tap are one vector)
  int32_t bias_vec;  // bias is 16-byte aligned
  int32_t state_vec;  // each state line is (dim, 3) contiguous and 16-byte aligned
                      // (bf16 state: 8-byte aligned)
  int32_t state_rows;  // each state line is 3 rows of dim contiguous channels ("dim first"),
                       // 16-byte aligned, row and line strides multiples of 4
};

// Program and column block of this wave. Divisions by run-time values go through
// a multiplier and shift set by the launcher (the hardware has no integer divide,
// and a division would put a dependent chain of about thirty instructions in front
// of every wave's first load).
//
// Plain order: workgroup n is program n / groups, column group n % groups.
//
// Prefill order: the hardware hands workgroup n to XCD n % 8, and each XCD has its
// own L2. A tile's 3 history rows are the last rows of the tile above it in the
// same column group, so the workgroups are ordered in chunks of 8 programs x
// `groups` column groups such that the 8 programs of a column group run on one XCD:
// in a chunk, XCD x takes column groups x, 8 + x, ... for all 8 programs (in program
// order), then `groups % 8` of the remaining (program, group) pairs, taken in runs
// of consecutive programs. With 9 column groups, 8 of every 9 tiles find their
// history rows in their own XCD's L2 instead of in the memory-side cache (16384 x
// 4608: 57.4 -> 56.6 us; 64 sequences of 16384 tokens: 60.2 -> 59.3 us). The
// programs of a chunk still run together, so the launch keeps moving through the
// rows in order; a last partial chunk takes the plain order. Launches with fewer
// than 8 column groups keep the plain order: no XCD gets a whole column group, and
// on 4096 sequences of 1-4 tokens at 576 channels (first tiles only) the chunked
// order measured 22.6 -> 25.2 us.
struct WaveSlot {
  int p;
  int cb;
};
template <int kG>
__device__ __forceinline__ WaveSlot wave_slot(const ConvParams& P, int wave) {
  const uint32_t n = blockIdx.x;
  const uint32_t groups = ((uint32_t)P.col_blocks + kG - 1) / kG;
  const uint32_t c = (__umulhi(n, P.chunk_magic) + n) >> P.chunk_shift;
  if (c < (uint32_t)P.full_chunks) {
    const uint32_t k = n - c * 8u * groups;  // index within the chunk
    const uint32_t x = k & 7u;  // its XCD
    const uint32_t i = k >> 3;  // its place in the XCD's share of the chunk
    const uint32_t whole = groups >> 3;  // column groups per XCD for all 8 programs
    uint32_t g, pi;
    if (i < 8u * whole) {
      g = 8u * (i >> 3) + x;
      pi = i & 7u;
    } else {
      // Remaining pairs (column group whole*8 + j, program pi) in order L = 8 j + pi;
      // XCD x takes L in [x r, x r + r) with r = groups % 8.
      const uint32_t L = x * (groups & 7u) + (i - 8u * whole);
      g = 8u * whole + (L >> 3);
      pi = L & 7u;
    }
    return WaveSlot{(int)(8u * c + pi), (int)g * kG + wave};
  }
  const uint32_t b = n - (uint32_t)P.full_chunks * 8u * groups;
  const uint32_t p = (__umulhi(b, P.group_magic) + b) >> P.group_shift;
  return WaveSlot{(int)(8u * (uint32_t)P.full_chunks + p), (int)(b - p * groups) * kG + wave};
}

// A multiplier and shift that divide every n < 2^31 by d >= 1:
// n / d = (umulhi(n, m) + n) >> l with l = ceil(log2 d), m = floor(2^32 (2^l - d) / d)
// + 1 (the round-up method of Granlund and Montgomery).
void division_by(uint64_t d, uint32_t& magic, int32_t& shift) {
  int l = 0;
  while ((1ull << l) < d) ++l;
  magic = (uint32_t)(((1ull << 32) * ((1ull << l) - d)) / d + 1);
  shift = l;
}

// wave_slot's parameters: the plain order (xcd_chunks false) or the prefill order.
void set_wave_order(ConvParams& P, uint64_t groups, bool xcd_chunks) {
  division_by(groups, P.group_magic, P.group_shift);
  division_by(8 * groups, P.chunk_magic, P.chunk_shift);
  P.full_chunks = xcd_chunks ? P.programs / 8 : 0;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, kRange, kDescWord3);
}

// The lane's V elements of one row, widened to FP32. The widened values pass
// through an empty asm statement: the compiler cannot recompute them later from the
// packed word (rematerialization), which would keep the row's registers alive.
template <int kF, int V>
__device__ __forceinline__ void unpack(typename Lane<V * element_bytes<kF>()>::vec v, float (&f)[V]) {
  if (kF == kF32) {
#pragma unroll
    for (int i = 0; i < V; ++i) f[i] = __uint_as_float(v[i]);
  } else {
#pragma unroll
    for (int i = 0; i < V / 2; ++i) {
      f[2 * i] = widen_half<kF>(v[i], 0);
      f[2 * i + 1] = widen_half<kF>(v[i], 1);
      asm volatile("" : "+v"(f[2 * i]), "+v"(f[2 * i + 1]));
    }
  }
}

// Sequence s and its raw bounds qsl[s], qsl[s + 1]; s = -1 if none.
struct SeqBounds {
  int s;
  int q0;
  int q1;
};

// The sequence containing row r: the largest s in [0, num_seqs) with qsl[s] <= r,
// with qsl[s] and qsl[s + 1], by a radix-64 search (one ballot per level; for a
// non-decreasing qsl the lanes whose entry passes form a prefix of the wave). The
// last level reads consecutive entries, so the bounds come from its lanes: a wave
// waits on one round trip to qsl per level.
__device__ __forceinline__ SeqBounds find_sequence(const ConvParams& P, int r, int lane) {
  if (P.search_levels == 0) {
    // One sequence: both bounds in one round trip.
    const int q0 = P.qsl[0];
    const int q1 = P.qsl[1];
    if (q0 > r) return SeqBounds{-1, 0, 0};
    return SeqBounds{0, q0, q1};
  }
  int base = 0;
  int stride = P.search_top;
  int q = 0;
  int cnt = 0;
  for (int level = 0; level < P.search_levels; ++level) {
    const int idx = base + lane * stride;
    q = idx <= P.num_seqs ? P.qsl[idx] : 0;  // qsl has num_seqs + 1 entries
    const bool ok = idx < P.num_seqs && q <= r;
    const uint64_t m = __ballot(ok);
    cnt = __popcll(m);
    if (cnt == 0) return SeqBounds{-1, 0, 0};
    base += (cnt - 1) * stride;
    stride /= kWave;
  }
  // The last level had stride 1: lane cnt - 1 read qsl[base], lane cnt qsl[base + 1].
  const int q0 = __builtin_amdgcn_readlane(q, cnt - 1);
  const int q1 = cnt < kWave ? __builtin_amdgcn_readlane(q, cnt) : P.qsl[base + 1];
  return SeqBounds{base, q0, q1};
}

// One tile: program p of the launch's column block, resolved to its sequence.
struct Tile {
  int valid;  // program p covers rows of a sequence
  int s;  // sequence
  int j;  // tile index within the sequence
  int t0;  // first row
  int n;  // rows (1 .. R)
  int halo;  // 3 history rows precede t0 in x (j > 0), else 0
  int end;  // one past the sequence's last row
};

// Program map. Programs [0, num_seqs) are the first tiles of the sequences, in
// order: no search, and the sequence's line and state can be requested at once.
// The later programs go to row blocks q = 0, 1, ...: block q owns the later tile
// (j >= 1) whose first row lies in [(q + 1) R, (q + 2) R), if there is one. Every
// later tile is preceded by R rows of its own sequence, so later tiles start at
// least R rows apart and each block holds at most one; its sequence is the one
// containing row (q + 1) R. A later tile starts before row T, so blocks
// q < cdiv(T, R) - 1 suffice. Blocks below split_half take one program each;
// blocks from split_half to split_quarter take two, each computing one half of the
// tile's rows, and the blocks from split_quarter on take four, one quarter each.
// The last blocks are dispatched last, so the waves that run when no more are
// waiting to start carry a half or a quarter of a tile: at the end of the launch
// the SIMDs compute the last rows as they arrive instead of each holding the rows
// of a few full tiles (measured: 16384 tokens x 4608 channels, 58.8 -> 56.9 us).
// The grid depends only on host sizes.
template <int R>
__device__ __forceinline__ Tile describe_tile(const ConvParams& P, int p, int lane) {
  Tile d{0, 0, 0, 0, 1, 0, 0};
  const int T = P.num_tokens;
  if (p < P.num_seqs) {
    const int start = min(max(P.qsl[p], 0), T);
    const int end = min(max(P.qsl[p + 1], start), T);
    if (end <= start) return d;  // empty sequence
    d.valid = 1;
    d.s = p;
    d.t0 = start;
    d.n = min(R, end - start);
    d.end = end;
    return d;
  }
  // Row block q, and the part h of its tile (of `parts`) this program computes.
  const int pl = p - P.num_seqs;
  int q, parts, h;
  if (pl < P.split_half) {
    q = pl;
    parts = 1;
    h = 0;
  } else {
    const int ph = pl - P.split_half;
    const int nh = 2 * (P.split_quarter - P.split_half);
    if (ph < nh) {
      q = P.split_half + ph / 2;
      parts = 2;
      h = ph % 2;
    } else {
      q = P.split_quarter + (ph - nh) / 4;
      parts = 4;
      h = (ph - nh) % 4;
    }
  }
  const int r0 = (q + 1) * R;
  if (r0 >= T) return d;
  const SeqBounds b = find_sequence(P, r0, lane);
  if (b.s < 0) return d;
  const int start = min(max(b.q0, 0), T);
  const int end = min(max(b.q1, start), T);
  if (r0 < start || r0 >= end) return d;
  const int j = (r0 - start + R - 1) / R;  // the first tile starting at or after r0
  const int t0 = start + j * R;
  if (j < 1 || t0 >= end) return d;
  // Rows [ts, ts + n) of the tile [t0, min(t0 + R, end)); the 3 rows before ts
  // belong to the same sequence, since t0 >= start + R.
  const int ts = t0 + h * (R / parts);
  const int n = min(R / parts, min(t0 + R, end) - ts);
  if (n <= 0) return d;
  d.valid = 1;
  d.s = b.s;
  d.j = j;
  d.t0 = ts;
  d.n = n;
  d.halo = 3;
  d.end = end;
  return d;
}

// The per-wave part of the convolution shared by the prefill and decode kernels:
// the lane's channels, its weights and bias, the state line's I/O, prefill tiles
// and decode steps.
template <int kF, int V, int R, bool kBias, bool kSilu, int kS = kStateF32>
struct ConvWorker {
  static constexpr int kBytes = element_bytes<kF>();
  // A lane's V elements of a row of x or out move as one load or store.
  typedef Lane<V * kBytes> L;
  typedef typename L::vec vec;

  const ConvParams& P;
  int lane;
  int cl;  // first channel of the lane (inactive lanes redo the last active lane)
  bool active;
  uint32_t xvo, ovo, xrow_bytes, orow_bytes;
  __amdgpu_buffer_rsrc_t orsrc;  // the launch's output, row 0 of its first plane
  float w0[V], w1[V], w2[V], w3[V], bs[V];
  FixupList<kFixCapacity> fix;

  float* stage;  // the wave's LDS slice of 3 V kWave floats for state lines
  int cfirst;  // first channel of the wave

  __device__ __forceinline__ ConvWorker(const ConvParams& params, int lane_, int cb, uint2* slots,
                                        float* stage_)
      : P(params), lane(lane_), fix{slots, 0u}, stage(stage_) {
    cfirst = P.col_begin + cb * kWave * V;
    const int c0 = P.col_begin + (cb * kWave + lane) * V;
    active = c0 < P.col_end;
    cl = active ? c0 : P.col_end - V;
    xvo = (uint32_t)(cl * kBytes);
    xrow_bytes = (uint32_t)(P.x_row_stride * kBytes);
    orow_bytes = (uint32_t)(P.part_dim * kBytes);
    const int plane = (cl - P.col_begin) / P.part_dim;
    const int col = (cl - P.col_begin) - plane * P.part_dim;
    ovo = (uint32_t)((plane * P.plane_stride + col) * kBytes);
    orsrc = make_rsrc(P.out);
  }

  // Weights and bias: 16-byte vectors when the layout allows. Issued before any x
  // rows: vector memory operations complete in issue order, so loads issued after
  // the rows could only be used once all the rows had arrived.
  __device__ __forceinline__ void load_weights() {
    if (kS == kStateBF16 && P.weight_wm) {
      // Width-major: tap k of the lane's V channels (one plane, consecutive columns)
      // is V consecutive floats.
      const __amdgpu_buffer_rsrc_t wr = make_rsrc(P.weight);
      const int plane = cl / P.part_dim;
      const uint32_t base = (uint32_t)(plane * P.w_part_stride + (cl - plane * P.part_dim));
#pragma unroll
      for (int i = 0; i < V / 4; ++i) {
        const uint32_t o = (base + 4u * i) * 4u;
        const u32x4 t0 = __builtin_amdgcn_raw_buffer_load_b128(wr, o, 0, kKeep);
        const u32x4 t1 = __builtin_amdgcn_raw_buffer_load_b128(wr, o + (uint32_t)P.w_stride1 * 4u, 0, kKeep);
        const u32x4 t2 = __builtin_amdgcn_raw_buffer_load_b128(wr, o + (uint32_t)P.w_stride1 * 8u, 0, kKeep);
        const u32x4 t3 = __builtin_amdgcn_raw_buffer_load_b128(wr, o + (uint32_t)P.w_stride1 * 12u, 0, kKeep);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          w0[4 * i + k] = __uint_as_float(t0[k]);
          w1[4 * i + k] = __uint_as_float(t1[k]);
          w2[4 * i + k] = __uint_as_float(t2[k]);
          w3[4 * i + k] = __uint_as_float(t3[k]);
        }
      }
    } else if (kS == kStateBF16 && !P.weight_vec) {
      // Any strides, with the part stride; the lane's channels lie in one plane.
      const int plane = cl / P.part_dim;
      const float* base = P.weight + plane * P.w_part_stride;
#pragma unroll
      for (int k = 0; k < V; ++k) {
        const float* wp = base + (int64_t)(cl + k - plane * P.part_dim) * P.w_stride0;
        w0[k] = wp[0];
        w1[k] = wp[P.w_stride1];
        w2[k] = wp[2 * P.w_stride1];
        w3[k] = wp[3 * P.w_stride1];
      }
    } else if (P.weight_vec) {
      const __amdgpu_buffer_rsrc_t wr = make_rsrc(P.weight);
#pragma unroll
      for (int k = 0; k < V; ++k) {
        const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(wr, (uint32_t)(cl + k) * 16u, 0, kKeep);
        w0[k] = __uint_as_float(t[0]);
        w1[k] = __uint_as_float(t[1]);
        w2[k] = __uint_as_float(t[2]);
        w3[k] = __uint_as_float(t[3]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < V; ++k) {
        const float* wp = P.weight + (int64_t)(cl + k) * P.w_stride0;
        w0[k] = wp[0];
        w1[k] = wp[P.w_stride1];
        w2[k] = wp[2 * P.w_stride1];
        w3[k] = wp[3 * P.w_stride1];
      }
    }
    if (kBias && P.bias_vec) {
      const __amdgpu_buffer_rsrc_t br = make_rsrc(P.bias);
#pragma unroll
      for (int k = 0; k < V; k += 4) {
        const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(br, (uint32_t)(cl + k) * 4u, 0, kKeep);
        bs[k] = __uint_as_float(t[0]);
        bs[k + 1] = __uint_as_float(t[1]);
        bs[k + 2] = __uint_as_float(t[2]);
        bs[k + 3] = __uint_as_float(t[3]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < V; ++k) bs[k] = kBias ? P.bias[cl + k] : 0.0f;
    }
  }

  // The lane's V channels of state line `line`: h0, h1, h2 = entries 0, 1, 2.
  __device__ __forceinline__ void load_state(int64_t line, float (&h0)[V], float (&h1)[V],
                                             float (&h2)[V]) const {
    const float* sp = P.states + line * P.cs_stride0;
    if (P.state_vec) {
      // The lane's V channels x 3 values are 3V consecutive floats.
      const __amdgpu_buffer_rsrc_t sr = make_rsrc(sp);
      float f[3 * V];
#pragma unroll
      for (int i = 0; i < 3 * V / 4; ++i) {
        const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(sr, (uint32_t)cl * 12u + 16u * i, 0, kKeep);
        f[4 * i] = __uint_as_float(t[0]);
        f[4 * i + 1] = __uint_as_float(t[1]);
        f[4 * i + 2] = __uint_as_float(t[2]);
        f[4 * i + 3] = __uint_as_float(t[3]);
      }
#pragma unroll
      for (int k = 0; k < V; ++k) {
        h0[k] = f[3 * k];
        h1[k] = f[3 * k + 1];
        h2[k] = f[3 * k + 2];
      }
    } else if (P.state_rows) {
      // History k of the lane's V channels: V consecutive floats of row k.
      const __amdgpu_buffer_rsrc_t sr = make_rsrc(sp);
      const uint32_t row = (uint32_t)P.cs_stride2 * 4u;
#pragma unroll
      for (int i = 0; i < V / 4; ++i) {
        const uint32_t o = (uint32_t)(cl + 4 * i) * 4u;
        const u32x4 t0 = __builtin_amdgcn_raw_buffer_load_b128(sr, o, 0, kKeep);
        const u32x4 t1 = __builtin_amdgcn_raw_buffer_load_b128(sr, o + row, 0, kKeep);
        const u32x4 t2 = __builtin_amdgcn_raw_buffer_load_b128(sr, o + 2 * row, 0, kKeep);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          h0[4 * i + k] = __uint_as_float(t0[k]);
          h1[4 * i + k] = __uint_as_float(t1[k]);
          h2[4 * i + k] = __uint_as_float(t2[k]);
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < V; ++k) {
        const float* cp = sp + (int64_t)(cl + k) * P.cs_stride1;
        h0[k] = cp[0];
        h1[k] = cp[P.cs_stride2];
        h2[k] = cp[2 * P.cs_stride2];
      }
    }
  }

  // Writes entries 0, 1, 2 of the lane's V channels of line `line`.
  __device__ __forceinline__ void store_state(int64_t line, const float (&h0)[V],
                                              const float (&h1)[V], const float (&h2)[V]) const {
    float* sp = P.states + line * P.cs_stride0;
    if (P.state_vec) {
      float f[3 * V];
#pragma unroll
      for (int k = 0; k < V; ++k) {
        f[3 * k] = h0[k];
        f[3 * k + 1] = h1[k];
        f[3 * k + 2] = h2[k];
      }
      float4* sv = reinterpret_cast<float4*>(sp + (int64_t)cl * 3);
#pragma unroll
      for (int i = 0; i < 3 * V / 4; ++i)
        sv[i] = make_float4(f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3]);
    } else if (P.state_rows) {
#pragma unroll
      for (int i = 0; i < V / 4; ++i) {
        float* cp = sp + cl + 4 * i;
        *reinterpret_cast<float4*>(cp) = make_float4(h0[4 * i], h0[4 * i + 1], h0[4 * i + 2], h0[4 * i + 3]);
        *reinterpret_cast<float4*>(cp + P.cs_stride2) =
            make_float4(h1[4 * i], h1[4 * i + 1], h1[4 * i + 2], h1[4 * i + 3]);
        *reinterpret_cast<float4*>(cp + 2 * P.cs_stride2) =
            make_float4(h2[4 * i], h2[4 * i + 1], h2[4 * i + 2], h2[4 * i + 3]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < V; ++k) {
        float* cp = sp + (int64_t)(cl + k) * P.cs_stride1;
        cp[0] = h0[k];
        cp[P.cs_stride2] = h1[k];
        cp[2 * P.cs_stride2] = h2[k];
      }
    }
  }

  // Staged write of entries 0, 1, 2 of the wave's channels of a contiguous (dim, 3)
  // line. The wave's channels [cfirst, cfirst + n) are 12 n consecutive bytes of the
  // line, and lane l's V channels are bytes [12 V l, 12 V (l + 1)) of that part.
  // Written directly, each store instruction would cover every third 16-byte piece of
  // the part, a third of each cache line it touches. Instead every lane writes its
  // 3 V floats to the wave's own LDS slice at the same place, and each store
  // instruction then takes 64 consecutive 16-byte pieces (1 KB) from the slice to the
  // line (4096 decode steps at dim 4608: 121.6 -> 107.9 us). The buffer descriptor's
  // range is the part's length, so pieces at or past its end, read by lanes past the
  // launch's last channel, are dropped by the hardware; those lanes write the last
  // active lane's slot, with its values. Only this wave uses its slice, and the LDS
  // performs a wave's operations in order; the waits keep the compiler from moving
  // slice accesses across each other and make each phase's writes complete before
  // the next phase reads.
  __device__ __forceinline__ static void slice_fence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only (vmcnt and expcnt at their maxima)
    asm volatile("" ::: "memory");
  }
  __device__ __forceinline__ void store_state_staged(int64_t line, const float (&h0)[V],
                                                     const float (&h1)[V], const float (&h2)[V]) const {
    constexpr int kPieces = 3 * V / 4;  // 16-byte pieces per lane
    u32x4* s4 = reinterpret_cast<u32x4*>(stage);
    const int slot = (cl - cfirst) / V;
    float f[3 * V];
#pragma unroll
    for (int k = 0; k < V; ++k) {
      f[3 * k] = h0[k];
      f[3 * k + 1] = h1[k];
      f[3 * k + 2] = h2[k];
    }
    slice_fence();  // earlier reads of the slice are done
#pragma unroll
    for (int q = 0; q < kPieces; ++q) {
      u32x4 t;
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = __float_as_uint(f[4 * q + e]);
      s4[kPieces * slot + q] = t;
    }
    slice_fence();
    const int n = min(kWave * V, P.col_end - cfirst);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        P.states + line * P.cs_stride0 + (int64_t)cfirst * 3, (short)0, n * 12, kDescWord3);
#pragma unroll
    for (int q = 0; q < kPieces; ++q)
      __builtin_amdgcn_raw_buffer_store_b128(s4[lane + kWave * q], r, (uint32_t)(lane + kWave * q) * 16u, 0, kKeep);
  }

  // bf16 state lines. Values widen exactly (the word in the upper half of the FP32
  // word) and go back by taking that half again, so entries and tokens are stored
  // with their words unchanged.
  __device__ __forceinline__ static float widen_bf16(uint32_t word16) {
    return __uint_as_float(word16 << 16);
  }
  __device__ __forceinline__ static uint32_t bf16_word(float v) { return __float_as_uint(v) >> 16; }

  // The lane's V channels of bf16 state line `line`: h0, h1, h2 = entries 0, 1, 2.
  __device__ __forceinline__ void load_state16(int64_t line, float (&h0)[V], float (&h1)[V],
                                               float (&h2)[V]) const {
    const uint16_t* sp = reinterpret_cast<const uint16_t*>(P.states) + line * P.cs_stride0;
    if (P.state_vec) {
      // The lane's V channels x 3 entries are 3V consecutive words, 8-byte aligned.
      const __amdgpu_buffer_rsrc_t sr = make_rsrc(sp);
      uint32_t d[3 * V / 2];
#pragma unroll
      for (int i = 0; i < 3 * V / 4; ++i) {
        const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(sr, (uint32_t)cl * 6u + 8u * i, 0, kKeep);
        d[2 * i] = t[0];
        d[2 * i + 1] = t[1];
      }
#pragma unroll
      for (int k = 0; k < V; ++k) {
        uint32_t e[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          const int idx = 3 * k + j;
          e[j] = (d[idx / 2] >> (16 * (idx % 2))) & 0xFFFFu;
        }
        h0[k] = widen_bf16(e[0]);
        h1[k] = widen_bf16(e[1]);
        h2[k] = widen_bf16(e[2]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < V; ++k) {
        const uint16_t* cp = sp + (int64_t)(cl + k) * P.cs_stride1;
        h0[k] = widen_bf16(cp[0]);
        h1[k] = widen_bf16(cp[P.cs_stride2]);
        h2[k] = widen_bf16(cp[2 * P.cs_stride2]);
      }
    }
  }

  // Writes entries 0, 1, 2 of the lane's V channels of bf16 line `line`, any strides
  // (active lanes only).
  __device__ __forceinline__ void store_state16(int64_t line, const float (&h0)[V],
                                                const float (&h1)[V], const float (&h2)[V]) const {
    uint16_t* sp = reinterpret_cast<uint16_t*>(P.states) + line * P.cs_stride0;
#pragma unroll
    for (int k = 0; k < V; ++k) {
      uint16_t* cp = sp + (int64_t)(cl + k) * P.cs_stride1;
      cp[0] = (uint16_t)bf16_word(h0[k]);
      cp[P.cs_stride2] = (uint16_t)bf16_word(h1[k]);
      cp[2 * P.cs_stride2] = (uint16_t)bf16_word(h2[k]);
    }
  }

  // Staged write of a contiguous (dim, 3) bf16 line, as store_state_staged does for
  // FP32 lines: the wave's channels [cfirst, cfirst + n) are 6 n consecutive bytes and
  // lane l's V channels bytes [6 V l, 6 V (l + 1)). Lanes write their 6 V bytes to the
  // slice at their slot; then each of 3 V / 4 store instructions takes 64 consecutive
  // 8-byte pieces (512 bytes). 6 n is a multiple of 8 (n is a multiple of 4), so no
  // piece straddles the end of the part, and pieces at or past it (read from bytes of
  // the slice no lane wrote) are dropped by the descriptor's range.
  __device__ __forceinline__ void store_state16_staged(int64_t line, const float (&h0)[V],
                                                       const float (&h1)[V],
                                                       const float (&h2)[V]) const {
    constexpr int kPieces = 3 * V / 4;  // 8-byte pieces per lane
    u32x2* s2 = reinterpret_cast<u32x2*>(stage);
    const int slot = (cl - cfirst) / V;
    uint32_t e[3 * V];
#pragma unroll
    for (int k = 0; k < V; ++k) {
      e[3 * k] = bf16_word(h0[k]);
      e[3 * k + 1] = bf16_word(h1[k]);
      e[3 * k + 2] = bf16_word(h2[k]);
    }
    slice_fence();  // earlier reads of the slice are done
#pragma unroll
    for (int q = 0; q < kPieces; ++q) {
      u32x2 t;
      t[0] = e[4 * q] | (e[4 * q + 1] << 16);
      t[1] = e[4 * q + 2] | (e[4 * q + 3] << 16);
      s2[kPieces * slot + q] = t;
    }
    slice_fence();
    const int n = min(kWave * V, P.col_end - cfirst);
    uint16_t* sp = reinterpret_cast<uint16_t*>(P.states) + line * P.cs_stride0 + (int64_t)cfirst * 3;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(sp, (short)0, n * 6, kDescWord3);
#pragma unroll
    for (int q = 0; q < kPieces; ++q)
      __builtin_amdgcn_raw_buffer_store_b64(s2[lane + kWave * q], r, (uint32_t)(lane + kWave * q) * 8u, 0, kKeep);
  }

  // Decode steps of sequences s0 .. s0 + kSeq - 1 (those below num_seqs): all their
  // loads (cache lines, x rows, state lines) are issued before any arithmetic, then
  // each sequence is computed and stored in turn.
  template <int kSeq, bool kStaged>
  __device__ __forceinline__ void decode_many(int s0) {
    int64_t line[kSeq];
    bool live[kSeq];
    vec xw[kSeq];
    float h0[kSeq][V], h1[kSeq][V], h2[kSeq][V];
#pragma unroll
    for (int i = 0; i < kSeq; ++i) {
      const int s = s0 + i;
      line[i] = s < P.num_seqs ? P.cache_indices[(int64_t)s * P.ci_stride] : -1;
      live[i] = s < P.num_seqs && !(P.has_null_block && line[i] == P.null_block_id) &&
                line[i] >= 0 && line[i] < P.num_cache_lines;
    }
#pragma unroll
    for (int i = 0; i < kSeq; ++i) {
      const int s = min(s0 + i, P.num_seqs - 1);
      const __amdgpu_buffer_rsrc_t xr = make_rsrc(P.x + (int64_t)s * P.x_row_stride * kBytes);
      xw[i] = L::template load<kStream>(xr, xvo, 0);
    }
#pragma unroll
    for (int i = 0; i < kSeq; ++i) {
      if (live[i]) {
        if (kS == kStateBF16)
          load_state16(line[i], h0[i], h1[i], h2[i]);
        else
          load_state(line[i], h0[i], h1[i], h2[i]);
      } else {
#pragma unroll
        for (int k = 0; k < V; ++k) h0[i][k] = h1[i][k] = h2[i][k] = 0.0f;
      }
    }
#pragma unroll
    for (int i = 0; i < kSeq; ++i) {
      const int s = s0 + i;
      if (s >= P.num_seqs) break;
      float xv[V];
      unpack<kF, V>(xw[i], xv);
      float acc[1][V];
#pragma unroll
      for (int k = 0; k < V; ++k) {
        float a = bs[k];
        a = __builtin_fmaf(w0[k], h0[i][k], a);
        a = __builtin_fmaf(w1[k], h1[i][k], a);
        a = __builtin_fmaf(w2[k], h2[i][k], a);
        a = __builtin_fmaf(w3[k], xv[k], a);
        acc[0][k] = a;
      }
      constexpr int kWords = row_words<kF, V>();
      uint32_t words[1][kWords];
      float y[1][V];
      uint32_t aux[1][V];
      const bool check = activate_rows<kF, kSilu, V, 1>(acc, y, aux, words);
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(check) != 0, 0)) {
#pragma unroll
        for (int k = 0; k < V; ++k) {
          if (needs_exact<kF, kSilu>(acc[0][k], y[0][k], aux[0][k])) {
            const uint32_t wd = act_word_exact<kF>(acc[0][k], kSilu);
            if (kBytes == 4)
              words[0][k] = wd;
            else if (k & 1)
              words[0][k / 2] = (words[0][k / 2] & 0xFFFFu) | (wd << 16);
            else
              words[0][k / 2] = (words[0][k / 2] & 0xFFFF0000u) | wd;
          }
        }
      }
      vec o;
#pragma unroll
      for (int w = 0; w < kWords; ++w) o[w] = words[0][w];
      L::template store<kStream>(o, orsrc, ovo, (uint32_t)s * orow_bytes);
      if (kS == kStateBF16) {
        if (kStaged && live[i])
          store_state16_staged(line[i], h1[i], h2[i], xv);
        else if (live[i] && active)
          store_state16(line[i], h1[i], h2[i], xv);
      } else if (kStaged && live[i]) {
        store_state_staged(line[i], h1[i], h2[i], xv);
      } else if (live[i] && active) {
        store_state(line[i], h1[i], h2[i], xv);
      }
    }
  }

  // Makes the compiler treat the values as used here, so that the wait for the loads
  // that produce them is placed here and not deferred to a later point.
  __device__ __forceinline__ static void pin(float (&f)[V]) {
#pragma unroll
    for (int k = 0; k < V; ++k) asm volatile("" : "+v"(f[k]));
  }

  // One valid tile of at most RR rows: loads, history, taps, activation, stores, and
  // (first tile of a sequence, kFirst) the state update.
  //
  // Loads. Vector memory operations complete in issue order and the compiler waits
  // for each row just before its arithmetic, so every row is computed as soon as it
  // has arrived while the later rows are still on their way. A later tile therefore
  // issues its 3 history rows first, then its RR rows, and takes its history as soon
  // as those three have arrived. A first tile issues its rows first, then reads the
  // sequence's line and state (a dependent chain that should not delay the rows) and
  // waits for everything before its first row. The two orders are separate copies of
  // the code (kFirst): joined, the compiler would have to assume the slower one and
  // wait for all rows before the first row of every tile. All RR row loads are always
  // issued (rows past the tile's end repeat its last row), so their count does not
  // depend on the tile. Tile rows are streamed, except the last three, which the next
  // tile of the column block reads again as its history.
  //
  // Nothing is called inside the row loop: a call there would keep every live value
  // (weights, history, rows in flight) in registers the callee preserves, raising
  // the register count and with it cutting the waves per SIMD, or would put them on
  // the stack. Elements that need the exact path are appended to the list; if a tile
  // has more of them than the list holds, the tile is rewritten after its rows
  // (redo_tile).
  template <int RR, bool kFirst>
  __device__ __forceinline__ void tile(const Tile& d) {
    vec rows[RR];
    float h0[V], h1[V], h2[V];
    bool live = false;
    int64_t line = 0;
    const __amdgpu_buffer_rsrc_t xr =
        make_rsrc(P.x + (int64_t)(d.t0 - d.halo) * P.x_row_stride * kBytes);
    auto issue_rows = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < RR; ++r) {
        const uint32_t off = (uint32_t)(min(r, d.n - 1) + d.halo) * xrow_bytes;
        rows[r] = r < RR - 3 ? L::template load<kStream>(xr, xvo, off)
                             : L::template load<kKeep>(xr, xvo, off);
      }
    };
    if (!kFirst) {
      // History e[t0-3], e[t0-2], e[t0-1]: the 3 rows before the tile.
      vec hv[3];
#pragma unroll
      for (int r = 0; r < 3; ++r) hv[r] = L::template load<kKeep>(xr, xvo, (uint32_t)r * xrow_bytes);
      issue_rows();
      __builtin_amdgcn_sched_barrier(0);  // the history is unpacked after all issues
      unpack<kF, V>(hv[0], h0);
      unpack<kF, V>(hv[1], h1);
      unpack<kF, V>(hv[2], h2);
      pin(h0);
      pin(h1);
      pin(h2);
    } else {
      // History: the stored state if the sequence is live and has an initial state,
      // else zeros. The line and the flag are requested before the rows, so that
      // waiting for them does not wait for the rows as well (vector loads complete in
      // order); the state, which depends on them, is requested while the rows are on
      // their way. They are loaded at a lane offset the compiler cannot see is zero,
      // so it keeps them as per-lane values and waits for them only where they are
      // made wave-uniform, after the rows have been issued.
      int vzero;
      asm volatile("v_mov_b32 %0, 0" : "=v"(vzero));
      const int32_t line_v = __builtin_amdgcn_raw_buffer_load_b32(
          make_rsrc(P.cache_indices + (int64_t)d.s * P.ci_stride), (uint32_t)vzero, 0, kKeep);
      const uint32_t init_v = P.has_init != nullptr
          ? __builtin_amdgcn_raw_buffer_load_b8(make_rsrc(P.has_init + d.s), (uint32_t)vzero, 0, kKeep)
          : 0u;
      issue_rows();
      line = __builtin_amdgcn_readfirstlane(line_v);
      live = !(P.has_null_block && line == P.null_block_id) && line >= 0 &&
             line < P.num_cache_lines;
      const bool init = live && __builtin_amdgcn_readfirstlane(init_v) != 0;
      if (init) {
        load_state(line, h0, h1, h2);
        pin(h0);
        pin(h1);
        pin(h2);
      } else {
#pragma unroll
        for (int k = 0; k < V; ++k) h0[k] = h1[k] = h2[k] = 0.0f;
      }
    }

    bool overflow = false;  // wave-uniform
    // Row r of the tile: taps, activation, store, history shift, and the elements
    // whose fast word may be wrong recorded in the list.
    auto row = [&](int r) __attribute__((always_inline)) {
      float xv[V], acc[1][V];
      unpack<kF, V>(rows[r], xv);
#pragma unroll
      for (int k = 0; k < V; ++k) {
        float a = bs[k];
        a = __builtin_fmaf(w0[k], h0[k], a);
        a = __builtin_fmaf(w1[k], h1[k], a);
        a = __builtin_fmaf(w2[k], h2[k], a);
        a = __builtin_fmaf(w3[k], xv[k], a);
        acc[0][k] = a;
        h0[k] = h1[k];
        h1[k] = h2[k];
        h2[k] = xv[k];
      }
      constexpr int kWords = row_words<kF, V>();
      uint32_t words[1][kWords];
      float y[1][V];
      uint32_t aux[1][V];
      const bool check = activate_rows<kF, kSilu, V, 1>(acc, y, aux, words);
      vec o;
#pragma unroll
      for (int i = 0; i < kWords; ++i) o[i] = words[0][i];
      const uint32_t ro = (uint32_t)(d.t0 + r) * orow_bytes;
      L::template store<kStream>(o, orsrc, ovo, ro);
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(check) != 0, 0)) {
        if (!fix.fits(V * kWave)) {
          overflow = true;
        } else {
#pragma unroll
          for (int k = 0; k < V; ++k)
            fix.append(needs_exact<kF, kSilu>(acc[0][k], y[0][k], aux[0][k]), acc[0][k],
                       ovo + (uint32_t)(kBytes * k) + ro);
        }
      }
    };
    if (d.n == RR) {
      // Full tile: straight-line code, no conditions.
#pragma unroll
      for (int r = 0; r < RR; ++r) row(r);
    } else {
#pragma unroll
      for (int r = 0; r < RR; ++r)
        if (r < d.n) row(r);
    }
    if (__builtin_expect(overflow, 0)) redo_tile(d, line, live);

    // Updated state: the last three values of (history ++ x) for this sequence,
    // written by the sequence's first tile after its reads.
    if (kFirst && live && (active || P.state_vec)) {
      if (d.t0 + d.n < d.end) {
        // The sequence continues past this tile: its last rows are end-3 .. end-1.
        const __amdgpu_buffer_rsrc_t tr = make_rsrc(P.x + (int64_t)(d.end - 3) * P.x_row_stride * kBytes);
        unpack<kF, V>(L::template load<kKeep>(tr, xvo, 0), h0);
        unpack<kF, V>(L::template load<kKeep>(tr, xvo, xrow_bytes), h1);
        unpack<kF, V>(L::template load<kKeep>(tr, xvo, 2 * xrow_bytes), h2);
      }
      if (P.state_vec)
        store_state_staged(line, h0, h1, h2);
      else
        store_state(line, h0, h1, h2);
    }
  }

  // Element c of row t of x, widened.
  __device__ __forceinline__ float x_at(int64_t t, int c) const {
    const char* rowp = P.x + t * P.x_row_stride * kBytes;
    if (kF == kF32) return reinterpret_cast<const float*>(rowp)[c];
    return widen_half<kF>(reinterpret_cast<const uint16_t*>(rowp)[c], 0);
  }

  // Rare: more elements of the tile needed the exact path than the list holds (only
  // tiles full of values next to rounding boundaries, or of NaN or infinity). The
  // list is flushed, then every element of the tile is rewritten with its exact
  // word, one at a time and with every operand loaded again just before its use, so
  // that only the loop's indices are live across the call of the exact evaluation.
  // It runs before the first tile's state update, so the state line it reads is the
  // one the tile started from.
  __device__ __forceinline__ void redo_tile(const Tile& d, int64_t line, bool live) {
    auto fix_store = [&](uint32_t word, uint32_t offset) __attribute__((always_inline)) {
      store_word(word, offset);
    };
    fix.template flush<kF, kSilu>(lane, fix_store);  // also waits for the tile's stores
    const bool init = !d.halo && live && P.has_init != nullptr && P.has_init[d.s] != 0;
#pragma unroll 1
    for (int r = 0; r < d.n; ++r) {
#pragma unroll 1
      for (int k = 0; k < V; ++k) {
        const int c = cl + k;
        const float* wp = P.weight + (int64_t)c * P.w_stride0;
        float a = kBias ? P.bias[c] : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = r - 3 + i;  // row of e relative to the tile's first row
          float e;
          if (rr >= 0 || d.halo)
            e = x_at((int64_t)d.t0 + rr, c);
          else
            e = init ? P.states[line * P.cs_stride0 + (int64_t)c * P.cs_stride1 + (3 + rr) * P.cs_stride2]
                     : 0.0f;
          a = __builtin_fmaf(wp[i * P.w_stride1], e, a);
        }
        store_word(act_word_exact<kF>(a, kSilu), ovo + (uint32_t)(kBytes * k) + (uint32_t)(d.t0 + r) * orow_bytes);
      }
    }
  }

  // One exact word at a byte offset of the launch's output.
  __device__ __forceinline__ void store_word(uint32_t word, uint32_t offset) {
    if (kBytes == 4)
      __builtin_amdgcn_raw_buffer_store_b32(word, orsrc, offset, 0, kStream);
    else
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)word, orsrc, offset, 0, kStream);
  }

  // Rewrites the recorded elements with their exact words.
  __device__ __forceinline__ void finish() {
    auto fix_store = [&](uint32_t word, uint32_t offset) __attribute__((always_inline)) {
      store_word(word, offset);
    };
    fix.template flush<kF, kSilu>(lane, fix_store);
  }
};

// One wave per tile (or part of one); a workgroup holds kG waves, the same rows in
// kG adjacent column blocks (a column group). wave_slot maps the one-dimensional
// launch to programs and column groups so that workgroups dispatched together cover
// whole rows.
template <int kF, int V, int R, int kG, bool kBias, bool kSilu>
__global__ __launch_bounds__(kWave * kG) __attribute__((amdgpu_waves_per_eu(kMinWaves))) void packed_conv_kernel(const ConvParams P) {
  static_assert(V % 4 == 0, "the vector weight, bias and state paths take 4 channels at a time");
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const WaveSlot slot = wave_slot<kG>(P, wave);
  const int p = slot.p;
  const int cb = slot.cb;
  if (cb >= P.col_blocks) return;
  // Weights first: their loads overlap the search for the tile's sequence.
  __shared__ uint2 fix_slots[kG][kFixCapacity];
  __shared__ float stage[kG][3 * V * kWave];
  ConvWorker<kF, V, R, kBias, kSilu, kStateF32> w(P, lane, cb, fix_slots[wave], stage[wave]);
  w.load_weights();
  const Tile d = describe_tile<R>(P, p, lane);
  if (!d.valid) return;
  // One copy of the tile code per size class: rows of short sequences and of a
  // sequence's end, the half and quarter tiles at the end of the launch, whole
  // tiles; each loads only the rows of its class.
  constexpr int kQ = R / 4 > kShort ? R / 4 : kShort;
  constexpr int kH = R / 2 > kQ ? R / 2 : kQ;
  if (d.halo) {
    if (d.n <= kShort)
      w.template tile<kShort, false>(d);
    else if (kQ > kShort && d.n <= kQ)
      w.template tile<kQ, false>(d);
    else if (kH > kQ && d.n <= kH)
      w.template tile<kH, false>(d);
    else
      w.template tile<R, false>(d);
  } else {
    if (d.n <= kShort)
      w.template tile<kShort, true>(d);
    else if (kH > kShort && d.n <= kH)
      w.template tile<kH, true>(d);
    else
      w.template tile<R, true>(d);
  }
  w.finish();
}

// Decode update: program p is sequences kSeq p .. kSeq p + kSeq - 1 (rows of x), one
// wave per column block, kG column blocks per workgroup. No search: every sequence
// has exactly one token.
template <int kF, int V, int kSeq, int kG, bool kBias, bool kSilu, int kS>
__global__ __launch_bounds__(kWave * kG) void packed_conv_update_kernel(const ConvParams P) {
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const WaveSlot slot = wave_slot<kG>(P, wave);
  const int p = slot.p;
  const int cb = slot.cb;
  if (cb >= P.col_blocks) return;
  __shared__ float stage[kG][3 * V * kWave];
  ConvWorker<kF, V, 1, kBias, kSilu, kS> w(P, lane, cb, nullptr, stage[wave]);
  w.load_weights();
  if (P.state_vec)
    w.template decode_many<kSeq, true>(p * kSeq);
  else
    w.template decode_many<kSeq, false>(p * kSeq);
}

// The activation map on consecutive FP32 bit patterns, 8 per lane as two rows of 4,
// through the same activate_rows, needs_exact and FixupList code the convolution
// uses (one wave per block, so each block owns its list).
template <int kF, bool kSilu>
__global__ __launch_bounds__(kWave) void activation_map_kernel(uint32_t first, uint64_t count,
                                                               void* __restrict__ out) {
  const int lane = threadIdx.x;
  const uint64_t block_first = (uint64_t)blockIdx.x * kWave * 8;
  const uint64_t i = block_first + (uint64_t)lane * 8;
  if (i >= count) return;
  float acc[2][4], y[2][4];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[r][k] = __uint_as_float(first + (uint32_t)(i + 4 * r + k));
  }
  uint32_t w[2][row_words<kF, 4>()];
  uint32_t aux[2][4];
  const bool check = activate_rows<kF, kSilu, 4, 2>(acc, y, aux, w);
  if (kF == kF32) {
    uint4* o = reinterpret_cast<uint4*>(static_cast<uint32_t*>(out) + i);
    o[0] = make_uint4(w[0][0], w[0][1], w[0][2], w[0][3]);
    o[1] = make_uint4(w[1][0], w[1][1], w[1][2], w[1][3]);
  } else {
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + i) = make_uint4(w[0][0], w[0][1], w[1][0], w[1][1]);
  }
  __shared__ uint2 fix_slots[kFixCapacity];
  FixupList<kFixCapacity> fix{fix_slots, 0u};
  auto fix_store = [&](uint32_t word, uint32_t offset) __attribute__((always_inline)) {
    if (kF == kF32)
      static_cast<uint32_t*>(out)[block_first + offset] = word;
    else
      static_cast<uint16_t*>(out)[block_first + offset] = (uint16_t)word;
  };
  if (__builtin_amdgcn_ballot_w64(check) != 0) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        fix.append(needs_exact<kF, kSilu>(acc[r][k], y[r][k], aux[r][k]), acc[r][k],
                   (uint32_t)lane * 8 + 4 * r + k);
    }
  }
  fix.template flush<kF, kSilu>(lane, fix_store);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }
bool element_aligned(const void* p, int64_t eb) {
  return (reinterpret_cast<uintptr_t>(p) & (uintptr_t)(eb - 1)) == 0;
}
bool known_dtype(int dtype) { return dtype == kBF16 || dtype == kF16 || dtype == kF32; }

int64_t dtype_bytes(int dtype) { return dtype == kF32 ? 4 : 2; }

int validate(const void* x, int dtype, int64_t num_tokens, int64_t dim, int64_t x_row_stride,
             const float* weight, int64_t ws0, int64_t ws1, const float* conv_states,
             int64_t num_cache_lines, int64_t cs0, int64_t cs1, int64_t cs2, const int32_t* qsl,
             int64_t num_seqs, const int32_t* ci, int64_t ci_stride, int64_t part_dim,
             int activation, const void* out) {
  if (num_tokens < 0 || dim < 0 || num_seqs < 0 || num_cache_lines < 0) return KDACONV_EINVAL;
  if (!known_dtype(dtype)) return KDACONV_EINVAL;
  if (part_dim <= 0 || dim % part_dim != 0) return KDACONV_EINVAL;
  if (x_row_stride < dim) return KDACONV_EINVAL;
  if (activation != KDACONV_ACT_NONE && activation != KDACONV_ACT_SILU) return KDACONV_EINVAL;
  const int64_t eb = dtype_bytes(dtype);
  // Plane rows are whole 16-byte pieces (x, out and x's rows need only be aligned to the
  // element size).
  if (part_dim % 8 != 0) return KDACONV_EUNSUPPORTED;
  if (ws0 < 0 || ws1 < 0 || cs0 < 0 || cs1 < 0 || cs2 < 0 || ci_stride < 0)
    return KDACONV_EUNSUPPORTED;
  // int32 token and sequence indices; 32-bit offsets within a program's rows
  // and within one output plane.
  if (num_tokens > INT32_MAX - 1 || num_seqs > INT32_MAX / 2 || dim > INT32_MAX / 2)
    return KDACONV_EUNSUPPORTED;
  const int64_t rows = rows_per_tile(dtype);
  if ((4 * ((num_tokens + rows - 1) / rows) + num_seqs) * ((dim + kWave * kLaneChannels - 1) / (kWave * kLaneChannels)) > INT32_MAX)
    return KDACONV_EUNSUPPORTED;
  if (x_row_stride * eb * (rows + 3) > INT32_MAX) return KDACONV_EUNSUPPORTED;
  if (num_tokens * part_dim * eb > INT32_MAX / 2) return KDACONV_EUNSUPPORTED;
  if (dim * cs1 * 4 > INT32_MAX) return KDACONV_EUNSUPPORTED;
  if (num_tokens == 0 || num_seqs == 0 || dim == 0) return KDACONV_OK;
  if (!x || !weight || !conv_states || !qsl || !ci || !out) return KDACONV_EINVAL;
  if (!element_aligned(x, eb) || !element_aligned(out, eb)) return KDACONV_EUNSUPPORTED;
  return KDACONV_OK;
}

// Host checks of the decode step's arguments, for either state format (state_bytes
// per state element); the weight part stride is checked by the bf16-state entry.
int validate_update(const void* x, int dtype, int64_t batch, int64_t dim, int64_t x_row_stride,
                    const float* weight, int64_t ws0, int64_t ws1, int64_t wps,
                    const void* conv_states, int64_t state_bytes, int64_t num_cache_lines,
                    int64_t cs0, int64_t cs1, int64_t cs2, const int32_t* cache_indices,
                    int64_t ci_stride, int64_t part_dim, int activation, const void* out) {
  if (batch < 0 || dim < 0 || num_cache_lines < 0) return KDACONV_EINVAL;
  if (!known_dtype(dtype)) return KDACONV_EINVAL;
  if (part_dim <= 0 || dim % part_dim != 0) return KDACONV_EINVAL;
  if (x_row_stride < dim) return KDACONV_EINVAL;
  if (activation != KDACONV_ACT_NONE && activation != KDACONV_ACT_SILU) return KDACONV_EINVAL;
  const int64_t eb = dtype_bytes(dtype);
  if (part_dim % 8 != 0) return KDACONV_EUNSUPPORTED;
  if (ws0 < 0 || ws1 < 0 || wps < 0 || cs0 < 0 || cs1 < 0 || cs2 < 0 || ci_stride < 0)
    return KDACONV_EUNSUPPORTED;
  if (batch > INT32_MAX - 1 || dim > INT32_MAX / 2) return KDACONV_EUNSUPPORTED;
  if (batch * ((dim + kWave * kLaneChannels - 1) / (kWave * kLaneChannels)) > INT32_MAX)
    return KDACONV_EUNSUPPORTED;
  if (batch * part_dim * eb > INT32_MAX / 2) return KDACONV_EUNSUPPORTED;
  if (dim * cs1 * state_bytes > INT32_MAX) return KDACONV_EUNSUPPORTED;
  if (batch == 0 || dim == 0) return KDACONV_OK;
  if (!x || !weight || !conv_states || !cache_indices || !out) return KDACONV_EINVAL;
  if (!element_aligned(x, eb) || !element_aligned(out, eb)) return KDACONV_EUNSUPPORTED;
  return KDACONV_OK;
}

template <int kF, int V, int R, int kG>
void launch_group(ConvParams P, bool bias, bool silu, hipStream_t st) {
  const uint64_t groups = ((uint64_t)P.col_blocks + kG - 1) / kG;
  set_wave_order(P, groups, groups >= 8);
  const dim3 grid((unsigned)((uint64_t)P.programs * groups));
  const dim3 block(kWave * kG);
  if (bias) {
    if (silu)
      hipLaunchKernelGGL((packed_conv_kernel<kF, V, R, kG, true, true>), grid, block, 0, st, P);
    else
      hipLaunchKernelGGL((packed_conv_kernel<kF, V, R, kG, true, false>), grid, block, 0, st, P);
  } else {
    if (silu)
      hipLaunchKernelGGL((packed_conv_kernel<kF, V, R, kG, false, true>), grid, block, 0, st, P);
    else
      hipLaunchKernelGGL((packed_conv_kernel<kF, V, R, kG, false, false>), grid, block, 0, st, P);
  }
}

template <int kF, int V, int R>
void launch_rows(ConvParams P, int64_t cols, bool bias, bool silu, hipStream_t st) {
  P.col_blocks = (int32_t)((cols / V + kWave - 1) / kWave);
  // Row blocks that can hold a later tile, and how many of the last ones are split.
  // When the sequences average under two tiles, few blocks hold a later tile and
  // splitting would mostly add programs that find nothing; no block is split then.
  const int64_t blocks = std::max<int64_t>(0, (P.num_tokens + R - 1) / R - 1);
  const bool split = P.num_tokens >= 2 * (int64_t)R * P.num_seqs;
  const int64_t quarter = split ? std::min<int64_t>(blocks, (kQuarterTileWaves + 4 * P.col_blocks - 1) / (4 * P.col_blocks)) : 0;
  const int64_t half = split ? std::min<int64_t>(blocks - quarter, (kHalfTileWaves + 2 * P.col_blocks - 1) / (2 * P.col_blocks)) : 0;
  P.split_quarter = (int32_t)(blocks - quarter);
  P.split_half = (int32_t)(blocks - quarter - half);
  P.programs = (int32_t)(P.num_seqs + P.split_half + 2 * half + 4 * quarter);
  // Two waves per workgroup measured 3-4 % faster on the 16384 x 4608 bf16
  // workload; with an odd number of column blocks the second wave of every last
  // workgroup would idle, and one wave per workgroup is kept.
  if (P.col_blocks % 2 == 0)
    launch_group<kF, V, R, 2>(P, bias, silu, st);
  else
    launch_group<kF, V, R, 1>(P, bias, silu, st);
}

template <int kF, int V>
void launch(ConvParams P, int64_t cols, bool bias, bool silu, hipStream_t st) {
  constexpr int R = rows_per_tile<kF>();
  if constexpr (R > 8) {
    if (P.num_tokens <= kSmallCallTokens &&
        (P.num_seqs == 1 || P.num_tokens >= kSmallCallTokensPerSeq * P.num_seqs)) {
      launch_rows<kF, V, 8>(P, cols, bias, silu, st);
      return;
    }
  }
  launch_rows<kF, V, R>(P, cols, bias, silu, st);
}

template <int kF, int V, int kSeq, int kG, int kS>
void launch_update_group(ConvParams P, bool bias, bool silu, hipStream_t st) {
  const uint64_t groups = ((uint64_t)P.col_blocks + kG - 1) / kG;
  set_wave_order(P, groups, false);
  const dim3 grid((unsigned)((uint64_t)P.programs * groups));
  const dim3 block(kWave * kG);
  if (bias) {
    if (silu)
      hipLaunchKernelGGL((packed_conv_update_kernel<kF, V, kSeq, kG, true, true, kS>), grid, block, 0, st, P);
    else
      hipLaunchKernelGGL((packed_conv_update_kernel<kF, V, kSeq, kG, true, false, kS>), grid, block, 0, st, P);
  } else {
    if (silu)
      hipLaunchKernelGGL((packed_conv_update_kernel<kF, V, kSeq, kG, false, true, kS>), grid, block, 0, st, P);
    else
      hipLaunchKernelGGL((packed_conv_update_kernel<kF, V, kSeq, kG, false, false, kS>), grid, block, 0, st, P);
  }
}

template <int kF, int V, int kSeq, int kS>
void launch_update_seq(ConvParams P, bool bias, bool silu, hipStream_t st) {
  P.programs = (P.num_seqs + kSeq - 1) / kSeq;
  if (P.col_blocks % 2 == 0)
    launch_update_group<kF, V, kSeq, 2, kS>(P, bias, silu, st);
  else
    launch_update_group<kF, V, kSeq, 1, kS>(P, bias, silu, st);
}

// Sequences per decode wave: as many as keep at least 2048 waves in the launch (two per
// SIMD), at most 4. Interleaved timing at dim 4608: 1024 sequences 35.5 -> 31.4 us with
// several sequences per wave instead of one; 256 sequences 12.0 -> 11.8 us with 2; 64
// sequences unchanged with 1. Eight sequences per wave need about 180 VGPRs, two waves
// per SIMD: 4096 sequences took 113.6 us with eight and 107.9 us with four.
template <int kF, int V, int kS = kStateF32>
void launch_update(ConvParams P, int64_t cols, bool bias, bool silu, hipStream_t st) {
  P.col_blocks = (int32_t)((cols / V + kWave - 1) / kWave);
  const int64_t waves1 = (int64_t)P.num_seqs * P.col_blocks;
  if (waves1 >= 4 * 2048)
    launch_update_seq<kF, V, 4, kS>(P, bias, silu, st);
  else if (waves1 >= 2 * 2048)
    launch_update_seq<kF, V, 2, kS>(P, bias, silu, st);
  else
    launch_update_seq<kF, V, 1, kS>(P, bias, silu, st);
}

// Fields of ConvParams shared by both operations.
void fill_common(ConvParams& P, const void* x, int64_t num_tokens, int64_t x_row_stride,
                 const float* weight, int64_t ws0, int64_t ws1, const float* bias,
                 float* conv_states, int64_t num_cache_lines, int64_t cs0, int64_t cs1, int64_t cs2,
                 const int32_t* cache_indices, int64_t ci_stride, int64_t dim, int64_t part_dim,
                 int has_null_block, int64_t null_block_id) {
  P.x = static_cast<const char*>(x);
  P.weight = weight;
  P.bias = bias;
  P.states = conv_states;
  P.qsl = nullptr;
  P.cache_indices = cache_indices;
  P.has_init = nullptr;
  P.x_row_stride = x_row_stride;
  P.w_stride0 = ws0;
  P.w_stride1 = ws1;
  P.cs_stride0 = cs0;
  P.cs_stride1 = cs1;
  P.cs_stride2 = cs2;
  P.ci_stride = ci_stride;
  P.num_cache_lines = num_cache_lines;
  P.plane_stride = num_tokens * part_dim;
  P.null_block_id = null_block_id;
  P.num_tokens = (int32_t)num_tokens;
  P.part_dim = (int32_t)part_dim;
  P.search_levels = 0;
  P.search_top = 1;
  P.split_half = 0;
  P.split_quarter = 0;
  P.group_magic = 1;
  P.group_shift = 0;
  P.chunk_magic = 1;
  P.chunk_shift = 0;
  P.full_chunks = 0;
  P.has_null_block = has_null_block != 0;
  P.w_part_stride = part_dim * ws0;
  P.weight_vec = ws0 == 4 && ws1 == 1 && aligned16(weight);
  P.weight_wm = 0;
  P.bias_vec = bias != nullptr && aligned16(bias);
  P.state_vec = cs1 == 3 && cs2 == 1 && cs0 % 4 == 0 && aligned16(conv_states);
  P.state_rows = cs1 == 1 && cs2 >= dim && cs2 % 4 == 0 && cs0 % 4 == 0 &&
                 aligned16(conv_states) && (2 * cs2 + dim) * 4 < INT32_MAX;
}

// Launches op(P, cols) over groups of whole planes small enough that a lane's offset
// into the group's output (planes * num_tokens * part_dim * element bytes) stays
// below 2^31. One launch in every realistic case.
template <class Op>
void for_plane_groups(ConvParams& P, int64_t num_tokens, int64_t dim, int64_t part_dim,
                      int64_t eb, void* out, Op op) {
  const int64_t plane_bytes = num_tokens * part_dim * eb;
  const int64_t planes = dim / part_dim;
  const int64_t per_launch = plane_bytes > 0 ? std::max<int64_t>(1, INT32_MAX / plane_bytes) : planes;
  for (int64_t pl = 0; pl < planes; pl += per_launch) {
    const int64_t pe = std::min(planes, pl + per_launch);
    P.col_begin = (int32_t)(pl * part_dim);
    P.col_end = (int32_t)(pe * part_dim);
    P.out = static_cast<char*>(out) + pl * P.plane_stride * eb;
    op(P, (pe - pl) * part_dim);
  }
}

}  // namespace
}  // namespace kdaconv

using namespace kdaconv;

static_assert(KDACONV_BF16 == kBF16 && KDACONV_F16 == kF16 && KDACONV_F32 == kF32,
              "format codes of the interface and the kernels agree");

extern "C" int kdaconv_validate(const void* x, int dtype, int64_t num_tokens, int64_t dim,
                                int64_t x_row_stride, const float* weight, int64_t weight_stride0,
                                int64_t weight_stride1, const float* bias,
                                const float* conv_states, int64_t num_cache_lines,
                                int64_t cs_stride0, int64_t cs_stride1, int64_t cs_stride2,
                                const int32_t* query_start_loc, int64_t num_seqs,
                                const int32_t* cache_indices, int64_t cache_indices_stride,
                                const uint8_t* has_initial_state, int64_t part_dim, int activation,
                                int has_null_block, int64_t null_block_id, const void* out) {
  (void)bias;
  (void)has_initial_state;
  (void)has_null_block;
  (void)null_block_id;
  return validate(x, dtype, num_tokens, dim, x_row_stride, weight, weight_stride0, weight_stride1,
                  conv_states, num_cache_lines, cs_stride0, cs_stride1, cs_stride2,
                  query_start_loc, num_seqs, cache_indices, cache_indices_stride, part_dim,
                  activation, out);
}

extern "C" int kdaconv_packed_causal_conv1d(
    const void* x, int dtype, int64_t num_tokens, int64_t dim, int64_t x_row_stride,
    const float* weight, int64_t weight_stride0, int64_t weight_stride1, const float* bias,
    float* conv_states, int64_t num_cache_lines, int64_t cs_stride0, int64_t cs_stride1,
    int64_t cs_stride2, const int32_t* query_start_loc, int64_t num_seqs,
    const int32_t* cache_indices, int64_t cache_indices_stride, const uint8_t* has_initial_state,
    int64_t part_dim, int activation, int has_null_block, int64_t null_block_id, void* out,
    kdaconv_stream_t stream) {
  const int rc = validate(x, dtype, num_tokens, dim, x_row_stride, weight, weight_stride0,
                          weight_stride1, conv_states, num_cache_lines, cs_stride0, cs_stride1,
                          cs_stride2, query_start_loc, num_seqs, cache_indices,
                          cache_indices_stride, part_dim, activation, out);
  if (rc != KDACONV_OK || num_tokens == 0 || num_seqs == 0 || dim == 0) return rc;

  const int64_t eb = dtype_bytes(dtype);
  ConvParams P;
  fill_common(P, x, num_tokens, x_row_stride, weight, weight_stride0, weight_stride1, bias,
              conv_states, num_cache_lines, cs_stride0, cs_stride1, cs_stride2, cache_indices,
              cache_indices_stride, dim, part_dim, has_null_block, null_block_id);
  P.qsl = query_start_loc;
  P.has_init = has_initial_state;
  P.num_seqs = (int32_t)num_seqs;
  int levels = 0;
  int64_t reach = 1;
  while (reach < num_seqs) {
    reach *= kWave;
    ++levels;
  }
  P.search_levels = levels;
  P.search_top = (int32_t)(levels > 0 ? reach / kWave : 1);

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool silu = activation == KDACONV_ACT_SILU;
  const bool has_bias = bias != nullptr;
  for_plane_groups(P, num_tokens, dim, part_dim, eb, out, [&](ConvParams& Q, int64_t cols) {
    if (dtype == kF32)
      launch<kF32, kLaneChannels>(Q, cols, has_bias, silu, st);
    else if (dtype == kF16)
      launch<kF16, kLaneChannels>(Q, cols, has_bias, silu, st);
    else
      launch<kBF16, kLaneChannels>(Q, cols, has_bias, silu, st);
  });
  return hipGetLastError() == hipSuccess ? KDACONV_OK : KDACONV_ELAUNCH;
}

extern "C" int kdaconv_packed_causal_conv1d_update(
    const void* x, int dtype, int64_t batch, int64_t dim, int64_t x_row_stride,
    const float* weight, int64_t weight_stride0, int64_t weight_stride1, const float* bias,
    float* conv_states, int64_t num_cache_lines, int64_t cs_stride0, int64_t cs_stride1,
    int64_t cs_stride2, const int32_t* cache_indices, int64_t cache_indices_stride,
    int64_t part_dim, int activation, int has_null_block, int64_t null_block_id, void* out,
    kdaconv_stream_t stream) {
  const int rc = validate_update(x, dtype, batch, dim, x_row_stride, weight, weight_stride0,
                                 weight_stride1, 0, conv_states, 4, num_cache_lines, cs_stride0,
                                 cs_stride1, cs_stride2, cache_indices, cache_indices_stride,
                                 part_dim, activation, out);
  if (rc != KDACONV_OK || batch == 0 || dim == 0) return rc;
  const int64_t eb = dtype_bytes(dtype);

  ConvParams P;
  fill_common(P, x, batch, x_row_stride, weight, weight_stride0, weight_stride1, bias,
              conv_states, num_cache_lines, cs_stride0, cs_stride1, cs_stride2, cache_indices,
              cache_indices_stride, dim, part_dim, has_null_block, null_block_id);
  P.num_seqs = (int32_t)batch;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool silu = activation == KDACONV_ACT_SILU;
  const bool has_bias = bias != nullptr;
  for_plane_groups(P, batch, dim, part_dim, eb, out, [&](ConvParams& Q, int64_t cols) {
    if (dtype == kF32)
      launch_update<kF32, kLaneChannels>(Q, cols, has_bias, silu, st);
    else if (dtype == kF16)
      launch_update<kF16, kLaneChannels>(Q, cols, has_bias, silu, st);
    else
      launch_update<kBF16, kLaneChannels>(Q, cols, has_bias, silu, st);
  });
  return hipGetLastError() == hipSuccess ? KDACONV_OK : KDACONV_ELAUNCH;
}

extern "C" int kdaconv_packed_causal_conv1d_update_bf16_state(
    const void* x, int dtype, int64_t batch, int64_t dim, int64_t x_row_stride,
    const float* weight, int64_t weight_part_stride, int64_t weight_stride0,
    int64_t weight_stride1, const float* bias, uint16_t* conv_states, int64_t num_cache_lines,
    int64_t cs_stride0, int64_t cs_stride1, int64_t cs_stride2, const int32_t* cache_indices,
    int64_t cache_indices_stride, int64_t part_dim, int activation, int has_null_block,
    int64_t null_block_id, void* out, kdaconv_stream_t stream) {
  const int rc = validate_update(x, dtype, batch, dim, x_row_stride, weight, weight_stride0,
                                 weight_stride1, weight_part_stride, conv_states, 2,
                                 num_cache_lines, cs_stride0, cs_stride1, cs_stride2,
                                 cache_indices, cache_indices_stride, part_dim, activation, out);
  if (rc != KDACONV_OK) return rc;
  if (dtype != KDACONV_BF16) return KDACONV_EUNSUPPORTED;
  if (batch == 0 || dim == 0) return KDACONV_OK;

  ConvParams P;
  fill_common(P, x, batch, x_row_stride, weight, weight_stride0, weight_stride1, bias,
              reinterpret_cast<float*>(conv_states), num_cache_lines, cs_stride0, cs_stride1,
              cs_stride2, cache_indices, cache_indices_stride, dim, part_dim, has_null_block,
              null_block_id);
  P.num_seqs = (int32_t)batch;
  P.w_part_stride = weight_part_stride;
  const int64_t parts = dim / part_dim;
  const int64_t w_extent = (parts - 1) * weight_part_stride + part_dim + 3 * weight_stride1;
  P.weight_vec = weight_stride0 == 4 && weight_stride1 == 1 && weight_part_stride == 4 * part_dim &&
                 aligned16(weight);
  P.weight_wm = weight_stride0 == 1 && weight_stride1 % 4 == 0 && weight_part_stride % 4 == 0 &&
                aligned16(weight) && w_extent * 4 < INT32_MAX;
  P.state_vec = cs_stride1 == 3 && cs_stride2 == 1 && cs_stride0 % 4 == 0 && aligned8(conv_states);
  P.state_rows = 0;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool silu = activation == KDACONV_ACT_SILU;
  const bool has_bias = bias != nullptr;
  for_plane_groups(P, batch, dim, part_dim, 2, out, [&](ConvParams& Q, int64_t cols) {
    launch_update<kBF16, kLaneChannels, kStateBF16>(Q, cols, has_bias, silu, st);
  });
  return hipGetLastError() == hipSuccess ? KDACONV_OK : KDACONV_ELAUNCH;
}

extern "C" int kdaconv_activation_map(uint32_t first, int64_t count, int activation, int dtype,
                                      void* out, kdaconv_stream_t stream) {
  if (count < 0 || count % 8 != 0 || count > ((int64_t)1 << 32)) return KDACONV_EINVAL;
  if (activation != KDACONV_ACT_NONE && activation != KDACONV_ACT_SILU) return KDACONV_EINVAL;
  if (!known_dtype(dtype)) return KDACONV_EINVAL;
  if (count == 0) return KDACONV_OK;
  if (!out) return KDACONV_EINVAL;
  if (!aligned16(out)) return KDACONV_EUNSUPPORTED;
  const uint64_t threads = (uint64_t)count / 8;
  const dim3 grid((unsigned)((threads + kWave - 1) / kWave));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool silu = activation == KDACONV_ACT_SILU;
#define KDACONV_MAP(F, S) \
  hipLaunchKernelGGL((activation_map_kernel<F, S>), grid, dim3(kWave), 0, st, first, (uint64_t)count, out)
  if (dtype == kF32) {
    if (silu) KDACONV_MAP(kF32, true); else KDACONV_MAP(kF32, false);
  } else if (dtype == kF16) {
    if (silu) KDACONV_MAP(kF16, true); else KDACONV_MAP(kF16, false);
  } else {
    if (silu) KDACONV_MAP(kBF16, true); else KDACONV_MAP(kBF16, false);
  }
#undef KDACONV_MAP
  return hipGetLastError() == hipSuccess ? KDACONV_OK : KDACONV_ELAUNCH;
}

extern "C" const char* kdaconv_status_string(int status) {
  switch (status) {
    case KDACONV_OK:
      return "ok";
    case KDACONV_EINVAL:
      return "invalid argument";
    case KDACONV_EUNSUPPORTED:
      return "unsupported layout or size";
    case KDACONV_ELAUNCH:
      return "kernel launch failed";
    default:
      return "unknown status";
  }
}

extern "C" int kdaconv_version(void) { return 300; }
