// Skinny bf16 linear layer C = A W^T for the projections around the decode
// (the absorbed q_c -> q_nope and decode-output -> hidden projections of the
// "fix TP" vLLM diff, MLACommonImpl): A [M, K] is a decode batch (M small),
// W [N, K] a weight in linear-layer layout, streamed once from HBM.
//
// MI355X mapping
//   * The matrix cores compute C^T tiles: v_mfma_f32_16x16x32_bf16 with the
//     weight as the 16 x 32 operand (16 output features, read straight from
//     global memory into registers) and the activations as the 32 x 16
//     operand (16 batch rows, read from LDS).  A lane's accumulator then holds
//     4 consecutive output features of one batch row: 8- or 16-byte stores.
//   * Reduction order is permuted inside each 64-wide k step: lane group g
//     takes k in [16 g, 16 g + 16) split over the two MFMAs, so every lane
//     reads 32 contiguous bytes of a weight row and four lanes cover a whole
//     128-byte line -- each line the CU keeps in flight is fully used.  Both
//     operands use the same permutation, so the sum is unchanged.
//   * Workgroup = 4 waves x 64 output features; the batch rows (up to 64 per
//     launch) are staged through LDS in 256-wide k chunks, double-buffered
//     through registers.  When the feature blocks alone cannot fill the GPU,
//     K is split over workgroups and the fp32 partials are summed in a fixed
//     order by a second kernel (deterministic).
#include "mla_device.h"
#include "mla_launch.h"

namespace mla {

namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kNT = 256;        // output features per workgroup
constexpr int kKC = 256;        // k per LDS chunk of the batch rows
constexpr int kRowsMax = 64;    // batch rows per launch
constexpr int kChunkPieces = kRowsMax * kKC / 8 / 256;   // 16-byte pieces per thread per chunk (8)

// LDS offset (in bf16 elements) of row m, 16-byte piece q of a chunk; the
// piece index is XOR-swizzled by the row so that 16 rows read at the same k
// land in different banks.
__device__ __forceinline__ int a_off(int m, int q) { return m * kKC + ((q ^ (m & 7)) << 3); }

}  // namespace

template <int MB, bool SPLIT, int CT>
__global__ __launch_bounds__(256, 2) void linear_bf16_kernel(LinearParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kRowsMax * kKC];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int r = lane & 15;
  const int n0 = blockIdx.x * kNT + wave * 64;
  const int ks = blockIdx.y;
  const int k_begin = ks * p.k_per_split;
  const int k_end = min(p.K, k_begin + p.k_per_split);
  const int rows = 16 * MB;

  const uint16_t* __restrict__ A = reinterpret_cast<const uint16_t*>(p.A);
  const uint16_t* __restrict__ W = reinterpret_cast<const uint16_t*>(p.W);

  // weight rows of this wave's 4 feature blocks (clamped: rows >= N are
  // loaded from row N-1 and never stored)
  const uint16_t* wrow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) wrow[j] = W + (long long)min(n0 + 16 * j + r, p.N - 1) * p.ldw + 16 * g;

  // batch-row chunk loader: thread t moves pieces t + 256 i (row = piece / 32,
  // 16-byte piece q = piece % 32); rows >= M are zero
  u32x4_t pre[kChunkPieces];
  auto load_chunk = [&](int kc) {
    const int klen = min(kKC, k_end - kc);
#pragma unroll
    for (int i = 0; i < kChunkPieces; ++i) {
      const int piece = threadIdx.x + 256 * i;
      const int m = piece >> 5, q = piece & 31;
      pre[i] = u32x4_t{0u, 0u, 0u, 0u};
      if (m < rows && m < p.M && 8 * q < klen)
        pre[i] = *reinterpret_cast<const u32x4_t*>(A + (long long)m * p.lda + kc + 8 * q);
    }
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kChunkPieces; ++i) {
      const int piece = threadIdx.x + 256 * i;
      const int m = piece >> 5, q = piece & 31;
      if (m < rows) *reinterpret_cast<u32x4_t*>(&sA[buf][a_off(m, q)]) = pre[i];
    }
  };

  f32x4_t acc[4][MB];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < MB; ++i) acc[j][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  load_chunk(k_begin);
  store_chunk(0);
  __syncthreads();

  int buf = 0;
#pragma unroll 1
  for (int kc = k_begin; kc < k_end; kc += kKC) {
    const bool more = kc + kKC < k_end;
    if (more) load_chunk(kc + kKC);          // lands while this chunk is computed
    const int klen = min(kKC, k_end - kc);
    // weight fragments one 64-wide step ahead
    bf16x8_t wf[2][4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wf[0][j][0] = *reinterpret_cast<const bf16x8_t*>(wrow[j] + kc);
      wf[0][j][1] = *reinterpret_cast<const bf16x8_t*>(wrow[j] + kc + 8);
    }
#pragma unroll 1
    for (int kk = 0; kk < klen; kk += 128) {
      // two 64-wide steps per iteration so the ring index stays static
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int k = kk + 64 * h2;
        if (k >= klen) break;
        const int cur = h2, nxt = h2 ^ 1;
        if (k + 64 < klen) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            wf[nxt][j][0] = *reinterpret_cast<const bf16x8_t*>(wrow[j] + kc + k + 64);
            wf[nxt][j][1] = *reinterpret_cast<const bf16x8_t*>(wrow[j] + kc + k + 72);
          }
        }
        bf16x8_t af[MB][2];
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          const int m = 16 * i + r;
          const int q = (k >> 3) + 2 * g;
          af[i][0] = *reinterpret_cast<const bf16x8_t*>(&sA[buf][a_off(m, q)]);
          af[i][1] = *reinterpret_cast<const bf16x8_t*>(&sA[buf][a_off(m, q + 1)]);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < MB; ++i)
              acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[cur][j][h], af[i][h], acc[j][i], 0, 0, 0);
      }
    }
    if (more) {
      store_chunk(buf ^ 1);                  // the other buffer was last read two chunks ago
      __syncthreads();
      buf ^= 1;
    }
  }

  // lane holds C[16 i + r][n0 + 16 j + 4 g + (0..3)]
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + 16 * j + 4 * g;
    if (n >= p.N) continue;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int m = 16 * i + r;
      if (m >= p.M) continue;
      if constexpr (SPLIT) {
        float* dst = p.ws + ((long long)ks * p.M + m) * p.N + n;
        *reinterpret_cast<f32x4_t*>(dst) = acc[j][i];
      } else if constexpr (CT == DT_F32) {
        float* dst = reinterpret_cast<float*>(p.C) + (long long)m * p.ldc + n;
        *reinterpret_cast<f32x4_t*>(dst) = acc[j][i];
      } else {
        uint16_t* dst = reinterpret_cast<uint16_t*>(p.C) + (long long)m * p.ldc + n;
        const uint32_t lo = f32_to_bf16_rne(acc[j][i][0]) | (f32_to_bf16_rne(acc[j][i][1]) << 16);
        const uint32_t hi = f32_to_bf16_rne(acc[j][i][2]) | (f32_to_bf16_rne(acc[j][i][3]) << 16);
        *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
      }
    }
  }
}

// Sum of the split-K partials in split order, then the output dtype.
template <int CT>
__global__ __launch_bounds__(256) void linear_reduce_kernel(LinearParams p) {
  const long long e4 = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;   // first of 4 elements
  const long long total = (long long)p.M * p.N;
  if (e4 >= total) return;
  f32x4_t s = *reinterpret_cast<const f32x4_t*>(p.ws + e4);
  for (int k = 1; k < p.splits; ++k) s += *reinterpret_cast<const f32x4_t*>(p.ws + k * total + e4);
  const long long m = e4 / p.N, n = e4 - m * p.N;
  if constexpr (CT == DT_F32) {
    *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.C) + m * p.ldc + n) = s;
  } else {
    const uint32_t lo = f32_to_bf16_rne(s[0]) | (f32_to_bf16_rne(s[1]) << 16);
    const uint32_t hi = f32_to_bf16_rne(s[2]) | (f32_to_bf16_rne(s[3]) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.C) + m * p.ldc + n) = make_uint2(lo, hi);
  }
}

// Split count: the workgroups (feature blocks x splits) fill the two
// resident slots of every CU once, rounding down so that no second, mostly
// idle round of workgroups is left.
int linear_splits(int M, int N, int K, int cus) {
  (void)M;
  const int nblocks = (N + kNT - 1) / kNT;
  if (nblocks >= cus) return 1;
  int s = 2 * cus / nblocks;
  const int ksteps = K / 64;
  if (s > ksteps) s = ksteps;
  return s < 1 ? 1 : s;
}

template <int MB>
static hipError_t launch_mb(int c_dtype, const LinearParams& p, hipStream_t stream) {
  dim3 grid((unsigned)((p.N + kNT - 1) / kNT), (unsigned)p.splits), block(256);
  if (p.splits > 1) hipLaunchKernelGGL((linear_bf16_kernel<MB, true, DT_F32>), grid, block, 0, stream, p);
  else if (c_dtype == DT_F32) hipLaunchKernelGGL((linear_bf16_kernel<MB, false, DT_F32>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((linear_bf16_kernel<MB, false, DT_BF16>), grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_linear(int c_dtype, const LinearParams& p, hipStream_t stream) {
  hipError_t e;
  switch ((p.M + 15) / 16) {
    case 1: e = launch_mb<1>(c_dtype, p, stream); break;
    case 2: e = launch_mb<2>(c_dtype, p, stream); break;
    case 3: e = launch_mb<3>(c_dtype, p, stream); break;
    case 4: e = launch_mb<4>(c_dtype, p, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || p.splits == 1) return e;
  const long long total4 = (long long)p.M * p.N / 4;
  dim3 grid((unsigned)((total4 + 255) / 256)), block(256);
  if (c_dtype == DT_F32) hipLaunchKernelGGL((linear_reduce_kernel<DT_F32>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((linear_reduce_kernel<DT_BF16>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
