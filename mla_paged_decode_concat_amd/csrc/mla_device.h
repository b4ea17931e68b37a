// Internal device helpers for libmla_amd: element formats, wave reductions,
// and the split partition shared by decode stage 1 and stage 2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

enum : int { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2 };

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Element formats
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// E4M3 ("e4m3fn") code -> float, exact.  Exponent bias 7; exponent field 0 is
// subnormal (m * 2^-9); S.1111.111 is NaN.  Normal codes map to binary32 by
// re-biasing the exponent (7 -> 127) and left-aligning the 3 mantissa bits.
__device__ __forceinline__ float fp8_to_f32(uint32_t c) {
  const uint32_t s = (c & 0x80u) << 24;
  const uint32_t e = (c >> 3) & 0xfu;
  const uint32_t m = c & 0x7u;
  if (e == 0) return __uint_as_float(s | __float_as_uint((float)m * 0.001953125f));
  if (e == 0xfu && m == 0x7u) return __uint_as_float(s | 0x7fc00000u);
  return __uint_as_float(s | ((e + 120u) << 23) | (m << 20));
}

// float -> E4M3 code: round to nearest, ties to even; finite magnitudes
// >= 448 and infinities saturate to +-448 (0x7E); NaN -> 0x7F; sign kept.
// Below 2^-6 the codes are the integers round(|v| * 2^9) (subnormals, plus
// the carry into the smallest normal, whose code 0x08 follows 0x07).  From
// 2^-6 up the code is the binary32 exponent/top-3-mantissa field rounded at
// bit 20 and re-biased from 127 to 7 (120 << 3 = 960).
__device__ __forceinline__ uint32_t f32_to_fp8(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t s = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return s | 0x7fu;            // NaN
  if (a >= 0x43e00000u) return s | 0x7eu;           // >= 448 (and inf)
  if (a < 0x3c800000u) {                            // < 2^-6
    const float t = __uint_as_float(a) * 512.0f;    // exact scaling by 2^9
    return s | (uint32_t)__builtin_rintf(t);        // rint: ties to even
  }
  const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
  return s | ((r >> 20) - 960u);
}

// ---------------------------------------------------------------------------
// Wave-wide reductions (64 lanes, butterfly: every lane gets the result)
// ---------------------------------------------------------------------------

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ long long wave_sum_i64(long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int wave_max_i32(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
  return v;
}

// inclusive prefix sum across the wave
__device__ __forceinline__ long long wave_scan_i64(long long v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    long long t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

// ---------------------------------------------------------------------------
// Split partition.
//
// LITERAL: the pages' rule.  Request b with n tokens is cut into splits of
//   kps = ceil(n / S) tokens; split s covers [s*kps, min((s+1)*kps, n)) and
//   empty splits are skipped, so the non-empty ones are s = 0..ceil(n/kps)-1.
//
// BALANCED: the requests, each padded to a multiple of 32 tokens, are laid
//   end to end; that line is cut into G chunks of Q = pad32(ceil(total / G))
//   tokens, and chunk c is handled by stage-1 workgroup c.  The part of
//   request b inside chunk c is one partial.
//
// Partial slots.  The workspace holds B * S partial rows per head, used as
// one pool.  LITERAL: split s of request b is slot b * S + s.  BALANCED: the
// piece (chunk c, request b) is slot c + b.  Walking the line, each next
// piece has a larger chunk index, a larger request index, or both, so slots
// are distinct, and a request's pieces occupy consecutive slots
// [c_first + b, c_last + b].  With G <= B * (S - 1) (the host caps it) every
// slot is below B * S.  A long request may so take more than S partials when
// shorter ones leave slots free: the chunk count is bounded by the batch's
// slot total, not by its longest request.
// ---------------------------------------------------------------------------

enum : int { PART_LITERAL = 1, PART_BALANCED = 2 };

constexpr int kChunkAlign = 32;

__device__ __forceinline__ long long pad32(long long n) { return (n + 31) & ~31LL; }

struct BatchTotals {
  long long total;   // sum of padded lengths
  int n32_max;       // longest padded length
};

// Every lane of the calling wave gets the totals.
__device__ __forceinline__ BatchTotals batch_totals(const int32_t* __restrict__ seq_lens, int B, int lane) {
  long long tot = 0;
  int mx = 0;
  for (int b = lane; b < B; b += kWave) {
    const int n = max(seq_lens[b], 0);
    const long long p = pad32(n);
    tot += p;
    mx = max(mx, (int)p);
  }
  BatchTotals t;
  t.total = wave_sum_i64(tot);
  t.n32_max = wave_max_i32(mx);
  return t;
}

// a / d for a >= 0, d > 0.  When both fit in 32 bits (any batch below 4G
// tokens) this is the 32-bit division, a few dozen instructions instead of
// the 64-bit sequence's hundred-odd; the result is the same.
__device__ __forceinline__ long long div_nonneg(long long a, long long d) {
  if ((((unsigned long long)a | (unsigned long long)d) >> 32) == 0) return (long long)((uint32_t)a / (uint32_t)d);
  return a / d;
}

__device__ __forceinline__ long long balanced_chunk(const BatchTotals& t, int G) {
  const long long q = pad32(div_nonneg(t.total + G - 1, G));
  return q > 0 ? q : kChunkAlign;
}

// Number of partials stage 1 wrote for a request of n tokens whose padded
// start on the balanced line is `start`; its first slot is start / Q + b.
__device__ __forceinline__ int balanced_num_partials(long long start, int n, long long Q) {
  if (n <= 0) return 0;
  return (int)(div_nonneg(start + n - 1, Q) - div_nonneg(start, Q) + 1);
}

// Literal partition: tokens per piece of a request of n tokens, either the
// pages' ceil(n / S) or a fixed piece length (piece_len > 0, the same for
// every request whatever the batch), and the number of non-empty pieces.
__device__ __forceinline__ int literal_piece_tokens(int n, int S, int piece_len) {
  return piece_len > 0 ? piece_len : (n + S - 1) / S;
}
__device__ __forceinline__ int literal_num_partials(int n, int S, int piece_len) {
  if (n <= 0) return 0;
  const long long kps = literal_piece_tokens(n, S, piece_len);
  return (int)(((long long)n + kps - 1) / kps);
}
// Token range [a, e) of piece s (empty when it starts past the request),
// in 64-bit so that no piece index or length overflows.
__device__ __forceinline__ void literal_piece_range(int n, int S, int piece_len, int s, int& a, int& e) {
  const long long kps = literal_piece_tokens(n, S, piece_len);
  const long long a64 = (long long)s * kps;
  a = a64 < n ? (int)a64 : n;
  e = (int)(a64 + kps < (long long)n ? a64 + kps : (long long)n);
  if (e < a) e = a;
}

// The batch totals and request b's padded start from one pass over
// seq_lens (one load per lane for up to 64 requests); every lane gets them.
__device__ __forceinline__ BatchTotals batch_totals_and_start(const int32_t* __restrict__ seq_lens, int B, int b,
                                                              int lane, long long& start) {
  long long tot = 0, pre = 0;
  int mx = 0;
  for (int i = lane; i < B; i += kWave) {
    const long long p = pad32(max(seq_lens[i], 0));
    tot += p;
    mx = max(mx, (int)p);
    if (i < b) pre += p;
  }
  BatchTotals t;
  t.total = wave_sum_i64(tot);
  t.n32_max = wave_max_i32(mx);
  start = wave_sum_i64(pre);
  return t;
}

// ---------------------------------------------------------------------------
// Parameters shared by the decode kernels (passed by value).
// ---------------------------------------------------------------------------

struct DecodeParams {
  const void* q;
  long long q_sb, q_sh;            // elements
  const void* cache;
  long long block_stride;          // elements
  const int32_t* block_table;
  long long bt_stride;
  const int32_t* seq_lens;
  const float* kv_scale;           // device scalar (fp8 cache) or null
  float* ws;                       // partial rows [H, B*S, R], then LSEs [H, B*S]
  void* o;                         // [B, H, R]
  float* lse;                      // [B, H]
  float sm_scale;
  int B, H, S;
  int block_size;
  int bs_log2;                     // log2(block_size) when it is a power of two, else -1
  int partition;                   // PART_LITERAL | PART_BALANCED
  int G;                           // balanced: chunk count
  int heads_per_group;             // stage 1: heads per workgroup
  int token_split;                 // stage 1, 16- or 32-head groups: four waves split the tokens
  int kv_nt;                       // stage-1 tile loads carry the non-temporal hint (<= 2 head groups)
  int direct;                      // one partial per request (num_kv_splits == 1): stage 1 writes o
                                   // (q's dtype) and lse itself and stage 2 is not launched
  int len_min, len_max;            // literal partition: this stage-1 launch takes the requests
                                   // with len_min <= seq_len < len_max
  int piece_len;                   // literal partition: tokens per piece (0 = ceil(n / S))
};

// Page of token tok (tok >= 0) and its row in that page: a shift and a mask
// for the usual power-of-two block sizes (the branch is uniform), else the
// integer division, which costs a few dozen vector instructions per use.
__device__ __forceinline__ void page_split(const DecodeParams& p, int tok, int& pg, int& row) {
  if (p.bs_log2 >= 0) {
    pg = tok >> p.bs_log2;
    row = tok & (p.block_size - 1);
  } else {
    pg = tok / p.block_size;
    row = tok - pg * p.block_size;
  }
}
// Workspace layout (fp32, B*H*S*(R+1) values as the split workspace of the
// pages): the normalised partial outputs as rows [H, B*S, R] -- each row a
// multiple of 1 KB, so rows start on cache lines, and the slots of one head
// are consecutive rows -- followed by their LSEs [H, B*S].
__device__ __forceinline__ float* ws_row(const DecodeParams& p, int slot, int h, int R) {
  return p.ws + ((long long)h * p.B * p.S + slot) * R;
}
__device__ __forceinline__ float* ws_lse(const DecodeParams& p, int slot, int h, int R) {
  return p.ws + (long long)p.B * p.H * p.S * R + (long long)h * p.B * p.S + slot;
}

// Store four consecutive values of a head's partial output, columns
// c .. c+3.  With one partial per request the partial is the result: the
// merge would weight it by exp(0) = 1 and divide by 1, so it goes straight
// to o (bf16, rounded to nearest even as the merge rounds it) instead of the
// workspace.  DIRECT is p.direct, resolved by the caller once per row.
template <bool DIRECT>
__device__ __forceinline__ void store_partial4(const DecodeParams& p, int b, int slot, int h, int R, int c,
                                               float x0, float x1, float x2, float x3) {
  if constexpr (DIRECT) {
    uint16_t* o = reinterpret_cast<uint16_t*>(p.o) + ((long long)b * p.H + h) * R + c;
    *reinterpret_cast<uint2*>(o) =
        make_uint2(f32_to_bf16_rne(x0) | (f32_to_bf16_rne(x1) << 16), f32_to_bf16_rne(x2) | (f32_to_bf16_rne(x3) << 16));
  } else {
    float* w = ws_row(p, slot, h, R) + c;
    *reinterpret_cast<float4*>(w) = make_float4(x0, x1, x2, x3);
  }
}
__device__ __forceinline__ void store_partial_lse(const DecodeParams& p, int b, int slot, int h, int R, float lse) {
  if (p.direct) p.lse[(long long)b * p.H + h] = lse;
  else *ws_lse(p, slot, h, R) = lse;
}

}  // namespace mla
