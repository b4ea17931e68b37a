// Paged latent-KV cache write ("concat and cache"): scatter each token's
// kv_c[R] and k_pe[P] into one cache row [R + P] at slot_mapping[t], skipping
// padded tokens (slot < 0), optionally encoding to fp8 E4M3 with a per-tensor
// scale.  Behaviour follows the concat_and_cache_mla kernel of the "fix TP"
// vLLM diff (csrc/cache_kernels.cu); the layout here is MI355X-first: one
// 64-lane wave owns a whole row and moves it with 16-byte loads.
#include "mla_device.h"
#include "mla_launch.h"

namespace mla {

template <int IT> struct InElem;
template <> struct InElem<DT_F32> { using T = float; static constexpr int kVec = 4; };
template <> struct InElem<DT_BF16> { using T = uint16_t; static constexpr int kVec = 8; };

template <int IT>
__device__ __forceinline__ float in_to_f32(typename InElem<IT>::T x) {
  if constexpr (IT == DT_F32) return x; else return bf16_to_f32(x);
}


constexpr int kWriteWaves = 4;          // tokens in flight per workgroup

// Rotary embedding of one interleaved pair (x, y) by the angle with cosine c
// and sine s: (x c - y s, y c + x s).  Every product and sum is rounded to
// fp32 on its own (contraction into fused multiply-adds is switched off), so
// the value that is then encoded for the cache is fixed by fp32 arithmetic.
__device__ __forceinline__ float2 rope_pair(float x, float y, float c, float s) {
#pragma clang fp contract(off)
  const float xc = x * c, ys = y * s, yc = y * c, xs = x * s;
  return make_float2(xc - ys, yc + xs);
}

// Row of the rotary table for a token position; positions outside the table
// (a precondition violation) read the nearest row instead of faulting.
__device__ __forceinline__ const float* rope_row(const float* rope, long long max_position, long long pos, int P) {
  pos = pos < 0 ? 0 : (pos >= max_position ? max_position - 1 : pos);
  return rope + pos * P;
}

template <int CT>
__device__ __forceinline__ uint32_t encode_one(float v, float scale) {
  if constexpr (CT == DT_BF16) return f32_to_bf16_rne(v);
  else if constexpr (CT == DT_FP8) return f32_to_fp8(v / scale);
  else return __float_as_uint(v);
}

// Tokens per wave: a large batch (the bulk write of a prompt) gives each wave
// four tokens; a decode step's handful of tokens gets one token per wave so
// that every token's loads are in flight at once.
int write_tokens_per_wave(long long num_tokens) { return num_tokens <= 65536 ? 1 : 4; }

// The rows are streamed: each input row is read once and each cache row
// written once per call, so the 16-byte loads and stores carry the
// non-temporal hint and do not push reusable data out of L2 and the
// last-level cache (bulk write of 524288 bf16 rows: 244.8 -> 231.5 us).
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));

// Load `len` input elements of a row into the lanes' vectors; lane j takes
// elements [V (j + 64 i), V (j + 64 i) + V).
template <int IT, int N>
__device__ __forceinline__ void load_vecs(const typename InElem<IT>::T* __restrict__ src, int len, int lane,
                                          uint4 (&v)[N]) {
  constexpr int V = InElem<IT>::kVec;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const int i = (lane + kWave * k) * V;
    if (i < len) {
      const u32x4_nt t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(src + i));
      v[k] = make_uint4(t[0], t[1], t[2], t[3]);
    }
  }
}

// Store (or encode and store) the vectors loaded by load_vecs at dst_off.
template <int IT, int CT, int N>
__device__ __forceinline__ void store_vecs(void* __restrict__ dst_base, long long dst_off, int len, int lane,
                                           float scale, const uint4 (&v)[N]) {
  using T = typename InElem<IT>::T;
  constexpr int V = InElem<IT>::kVec;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const int i = (lane + kWave * k) * V;
    if (i >= len) continue;
    if constexpr (CT == IT) {
      T* dst = reinterpret_cast<T*>(dst_base) + dst_off + i;
      __builtin_nontemporal_store(u32x4_nt{v[k].x, v[k].y, v[k].z, v[k].w}, reinterpret_cast<u32x4_nt*>(dst));
    } else {
      // fp8 output: V codes from V inputs
      const T* e = reinterpret_cast<const T*>(&v[k]);
      uint32_t packed[V / 4];
#pragma unroll
      for (int q = 0; q < V / 4; ++q) {
        uint32_t w = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) w |= f32_to_fp8(in_to_f32<IT>(e[4 * q + j]) / scale) << (8 * j);
        packed[q] = w;
      }
      uint8_t* dst = reinterpret_cast<uint8_t*>(dst_base) + dst_off + i;
      if constexpr (V == 8) *reinterpret_cast<uint2*>(dst) = make_uint2(packed[0], packed[1]);
      else *reinterpret_cast<uint32_t*>(dst) = packed[0];
    }
  }
}

// Vector path: 16-byte loads and stores; alignment of kv_c / k_pe rows and
// of the cache rows to the vector size is checked by the host.  A token's
// input rows are loaded before its slot is known (they are in bounds for
// every token), so the slot lookup and the data loads overlap.
// Rotate the k_pe vector a lane loaded (V elements = V/2 pairs starting at
// element i) and store it encoded at dst_off + i.
template <int IT, int CT>
__device__ __forceinline__ void store_rope_vec(void* __restrict__ dst_base, long long dst_off, int P, int lane,
                                               float scale, const uint4& v, const float* __restrict__ trow) {
  using T = typename InElem<IT>::T;
  constexpr int V = InElem<IT>::kVec;
  const int i = lane * V;
  if (i >= P) return;
  const T* e = reinterpret_cast<const T*>(&v);
  float c[V / 2], s[V / 2];
  if constexpr (V == 8) {
    const float4 c4 = *reinterpret_cast<const float4*>(trow + i / 2);
    const float4 s4 = *reinterpret_cast<const float4*>(trow + P / 2 + i / 2);
    c[0] = c4.x; c[1] = c4.y; c[2] = c4.z; c[3] = c4.w;
    s[0] = s4.x; s[1] = s4.y; s[2] = s4.z; s[3] = s4.w;
  } else {
    const float2 c2 = *reinterpret_cast<const float2*>(trow + i / 2);
    const float2 s2 = *reinterpret_cast<const float2*>(trow + P / 2 + i / 2);
    c[0] = c2.x; c[1] = c2.y;
    s[0] = s2.x; s[1] = s2.y;
  }
  uint32_t code[V];
#pragma unroll
  for (int j = 0; j < V / 2; ++j) {
    const float2 r = rope_pair(in_to_f32<IT>(e[2 * j]), in_to_f32<IT>(e[2 * j + 1]), c[j], s[j]);
    code[2 * j] = encode_one<CT>(r.x, scale);
    code[2 * j + 1] = encode_one<CT>(r.y, scale);
  }
  if constexpr (CT == DT_F32) {
    float* dst = reinterpret_cast<float*>(dst_base) + dst_off + i;
    *reinterpret_cast<uint4*>(dst) = make_uint4(code[0], code[1], code[2], code[3]);
  } else if constexpr (CT == DT_BF16) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(dst_base) + dst_off + i;
    *reinterpret_cast<uint4*>(dst) = make_uint4(code[0] | (code[1] << 16), code[2] | (code[3] << 16),
                                                code[4] | (code[5] << 16), code[6] | (code[7] << 16));
  } else {
    uint8_t* dst = reinterpret_cast<uint8_t*>(dst_base) + dst_off + i;
    const uint32_t w0 = code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
    if constexpr (V == 8) {
      const uint32_t w1 = code[4] | (code[5] << 8) | (code[6] << 16) | (code[7] << 24);
      *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
    } else {
      *reinterpret_cast<uint32_t*>(dst) = w0;
    }
  }
}

template <int IT, int CT, bool ROPE>
__global__ __launch_bounds__(kWave * kWriteWaves) void cache_write_vec_kernel(WriteParams p) {
  using T = typename InElem<IT>::T;
  constexpr int V = InElem<IT>::kVec;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const float scale = (CT == DT_FP8) ? *p.scale : 1.0f;
  const long long first = ((long long)blockIdx.x * kWriteWaves + wave) * p.tokens_per_wave;
  const int D = p.R + p.P;
  static_assert(2 * kWave * V * (int)sizeof(T) >= 2048, "two vectors per lane cover a 512-wide row");
#pragma unroll 1
  for (int k = 0; k < p.tokens_per_wave; ++k) {
    const long long t = first + k;
    if (t >= p.num_tokens) return;
    uint4 c[2], e[1];
    load_vecs<IT>(reinterpret_cast<const T*>(p.kv_c) + t * p.kv_c_stride, p.R, lane, c);
    load_vecs<IT>(reinterpret_cast<const T*>(p.k_pe) + t * p.k_pe_stride, p.P, lane, e);
    const long long slot = p.slots[t];
    if (slot < 0) continue;                 // padded token
    const long long blk = slot / p.block_size;
    const long long off = slot - blk * p.block_size;
    const long long row = blk * p.block_stride + off * D;
    store_vecs<IT, CT>(p.cache, row, p.R, lane, scale, c);
    if constexpr (ROPE) {
      const float* trow = rope_row(p.rope, p.max_position, p.positions[t], p.P);
      store_rope_vec<IT, CT>(p.cache, row + p.R, p.P, lane, scale, e[0], trow);
    } else {
      store_vecs<IT, CT>(p.cache, row + p.R, p.P, lane, scale, e);
    }
  }
}

// Element-wise fallback for views whose rows are not 16-byte aligned.
template <int IT, int CT, bool ROPE>
__global__ __launch_bounds__(kWave * kWriteWaves) void cache_write_scalar_kernel(WriteParams p) {
  using T = typename InElem<IT>::T;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const float scale = (CT == DT_FP8) ? *p.scale : 1.0f;
  const long long first = ((long long)blockIdx.x * kWriteWaves + wave) * p.tokens_per_wave;
  const int D = p.R + p.P;
#pragma unroll 1
  for (int k = 0; k < p.tokens_per_wave; ++k) {
    const long long t = first + k;
    if (t >= p.num_tokens) return;
    const long long slot = p.slots[t];
    if (slot < 0) continue;
    const long long blk = slot / p.block_size;
    const long long off = slot - blk * p.block_size;
    const long long row = blk * p.block_stride + off * D;
    const int end = ROPE ? p.R : D;
    for (int i = lane; i < end; i += kWave) {
      const T x = i < p.R ? reinterpret_cast<const T*>(p.kv_c)[t * p.kv_c_stride + i]
                          : reinterpret_cast<const T*>(p.k_pe)[t * p.k_pe_stride + (i - p.R)];
      if constexpr (CT == IT) reinterpret_cast<T*>(p.cache)[row + i] = x;
      else reinterpret_cast<uint8_t*>(p.cache)[row + i] = (uint8_t)f32_to_fp8(in_to_f32<IT>(x) / scale);
    }
    if constexpr (ROPE) {
      const float* trow = rope_row(p.rope, p.max_position, p.positions[t], p.P);
      const T* kp = reinterpret_cast<const T*>(p.k_pe) + t * p.k_pe_stride;
      for (int j = lane; j < p.P / 2; j += kWave) {
        const float2 r = rope_pair(in_to_f32<IT>(kp[2 * j]), in_to_f32<IT>(kp[2 * j + 1]), trow[j], trow[p.P / 2 + j]);
        const uint32_t a = encode_one<CT>(r.x, scale), b = encode_one<CT>(r.y, scale);
        const long long d = row + p.R + 2 * j;
        if constexpr (CT == DT_F32) {
          reinterpret_cast<float*>(p.cache)[d] = r.x;
          reinterpret_cast<float*>(p.cache)[d + 1] = r.y;
        } else if constexpr (CT == DT_BF16) {
          reinterpret_cast<uint16_t*>(p.cache)[d] = (uint16_t)a;
          reinterpret_cast<uint16_t*>(p.cache)[d + 1] = (uint16_t)b;
        } else {
          reinterpret_cast<uint8_t*>(p.cache)[d] = (uint8_t)a;
          reinterpret_cast<uint8_t*>(p.cache)[d + 1] = (uint8_t)b;
        }
      }
    }
  }
}

// Rotary embedding of the rope part of q [N, H, R + P] in place: one lane
// per pair, 32 lanes per (token, head) row, two rows per wave.
template <int QT>
__global__ __launch_bounds__(kWave * kWriteWaves) void rope_q_kernel(RopeQParams p) {
  using T = typename InElem<QT>::T;
  const long long rowid = ((long long)blockIdx.x * kWriteWaves + threadIdx.x / kWave) * 2 + ((threadIdx.x >> 5) & 1);
  const int j = threadIdx.x & 31;
  if (rowid >= p.N * p.H || 2 * j >= p.P) return;
  const long long n = rowid / p.H;
  const int h = (int)(rowid - n * p.H);
  T* x = reinterpret_cast<T*>(p.q) + n * p.q_sn + h * p.q_sh + p.R + 2 * j;
  const float* trow = rope_row(p.rope, p.max_position, p.positions[n], p.P);
  const float2 r = rope_pair(in_to_f32<QT>(x[0]), in_to_f32<QT>(x[1]), trow[j], trow[p.P / 2 + j]);
  if constexpr (QT == DT_F32) {
    x[0] = r.x;
    x[1] = r.y;
  } else {
    x[0] = (T)f32_to_bf16_rne(r.x);
    x[1] = (T)f32_to_bf16_rne(r.y);
  }
}

template <int IT, int CT>
static hipError_t launch_write_t(const WriteParams& p, bool vec, hipStream_t stream) {
  const long long per_block = (long long)kWriteWaves * p.tokens_per_wave;
  const long long blocks = (p.num_tokens + per_block - 1) / per_block;
  dim3 grid((unsigned)blocks), block(kWave * kWriteWaves);
  if (p.rope) {
    if (vec) hipLaunchKernelGGL((cache_write_vec_kernel<IT, CT, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((cache_write_scalar_kernel<IT, CT, true>), grid, block, 0, stream, p);
  } else {
    if (vec) hipLaunchKernelGGL((cache_write_vec_kernel<IT, CT, false>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((cache_write_scalar_kernel<IT, CT, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_rope_q(int q_dtype, const RopeQParams& p, hipStream_t stream) {
  const long long rows = p.N * p.H;
  const long long per_block = 2LL * kWriteWaves;
  dim3 grid((unsigned)((rows + per_block - 1) / per_block)), block(kWave * kWriteWaves);
  if (q_dtype == DT_F32) hipLaunchKernelGGL((rope_q_kernel<DT_F32>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((rope_q_kernel<DT_BF16>), grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_cache_write(int in_dtype, int cache_dtype, const WriteParams& p, bool vec, hipStream_t stream) {
  if (in_dtype == DT_F32 && cache_dtype == DT_F32) return launch_write_t<DT_F32, DT_F32>(p, vec, stream);
  if (in_dtype == DT_F32 && cache_dtype == DT_FP8) return launch_write_t<DT_F32, DT_FP8>(p, vec, stream);
  if (in_dtype == DT_BF16 && cache_dtype == DT_BF16) return launch_write_t<DT_BF16, DT_BF16>(p, vec, stream);
  if (in_dtype == DT_BF16 && cache_dtype == DT_FP8) return launch_write_t<DT_BF16, DT_FP8>(p, vec, stream);
  return hipErrorInvalidValue;
}

}  // namespace mla
