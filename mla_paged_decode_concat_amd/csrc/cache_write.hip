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

// Tokens per wave: a large batch (the bulk write of a prompt) gives each wave
// four tokens; a decode step's handful of tokens gets one token per wave so
// that every token's loads are in flight at once.
int write_tokens_per_wave(long long num_tokens) { return num_tokens <= 65536 ? 1 : 4; }

// Load `len` input elements of a row into the lanes' vectors; lane j takes
// elements [V (j + 64 i), V (j + 64 i) + V).
template <int IT, int N>
__device__ __forceinline__ void load_vecs(const typename InElem<IT>::T* __restrict__ src, int len, int lane,
                                          uint4 (&v)[N]) {
  constexpr int V = InElem<IT>::kVec;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const int i = (lane + kWave * k) * V;
    if (i < len) v[k] = *reinterpret_cast<const uint4*>(src + i);
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
      *reinterpret_cast<uint4*>(dst) = v[k];
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
template <int IT, int CT>
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
    store_vecs<IT, CT>(p.cache, row + p.R, p.P, lane, scale, e);
  }
}

// Element-wise fallback for views whose rows are not 16-byte aligned.
template <int IT, int CT>
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
    for (int i = lane; i < D; i += kWave) {
      const T x = i < p.R ? reinterpret_cast<const T*>(p.kv_c)[t * p.kv_c_stride + i]
                          : reinterpret_cast<const T*>(p.k_pe)[t * p.k_pe_stride + (i - p.R)];
      if constexpr (CT == IT) reinterpret_cast<T*>(p.cache)[row + i] = x;
      else reinterpret_cast<uint8_t*>(p.cache)[row + i] = (uint8_t)f32_to_fp8(in_to_f32<IT>(x) / scale);
    }
  }
}

template <int IT, int CT>
static hipError_t launch_write_t(const WriteParams& p, bool vec, hipStream_t stream) {
  const long long per_block = (long long)kWriteWaves * p.tokens_per_wave;
  const long long blocks = (p.num_tokens + per_block - 1) / per_block;
  dim3 grid((unsigned)blocks), block(kWave * kWriteWaves);
  if (vec) hipLaunchKernelGGL((cache_write_vec_kernel<IT, CT>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((cache_write_scalar_kernel<IT, CT>), grid, block, 0, stream, p);
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
