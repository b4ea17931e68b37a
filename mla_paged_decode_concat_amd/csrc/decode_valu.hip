// Split-KV MLA decode, stage 1, vector-ALU version: the generic path for any
// head count and the fp32 path.  Per (partial, group of 4 heads) it computes
// the softmax-normalised partial output and the partial LSE of the heads
// against the partial's token rows, as stage 1 of the split-KV decode does in
// the "fix TP" vLLM diff (vllm/attention/ops/triton_decode_attention.py,
// _fwd_grouped_kernel_stage1): scores over the full R + P row, values = the
// first R columns of the same row, online softmax, store acc / l and m + ln l.
//
// Layout: 8 waves per workgroup; wave w takes every 8th token of the partial
// (a token's dot products, online-softmax step and output update form a
// dependent chain, so more waves per partial shorten it: the tiny fp32
// workload's stage 1 took 21 us with 8, 32 us with 4 and 20-31 us with 16).
// A lane holds columns lane + 64 j of the current row, so each row read is
// coalesced; per-token dot products are finished with a wave butterfly.  The
// waves' (max, sum, acc) are merged through LDS at the end.
#include "mla_device.h"
#include "mla_launch.h"

namespace mla {

constexpr int kValuWaves = 8;
constexpr int kValuHeads = 4;   // heads per workgroup

template <int CT>
__device__ __forceinline__ float load_cache_elem(const void* base, long long idx) {
  if constexpr (CT == DT_F32) return reinterpret_cast<const float*>(base)[idx];
  else if constexpr (CT == DT_BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
  else return fp8_to_f32(reinterpret_cast<const uint8_t*>(base)[idx]);
}

template <int QT>
__device__ __forceinline__ float load_q_elem(const void* base, long long idx) {
  if constexpr (QT == DT_F32) return reinterpret_cast<const float*>(base)[idx];
  else return bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
}

template <int QT, int CT, int R, int P>
__device__ void valu_piece(const DecodeParams& p, int b, int h0, int a, int e, int part,
                           float (*sm_acc)[kValuHeads][R], float (*sm_ml)[kValuHeads][2]) {
  constexpr int D = R + P;
  constexpr int DJ = D / kWave;
  constexpr int RJ = R / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;

  // fp8: scores use code values; fold the per-tensor scale into the score
  // scale and the output (k_scale == v_scale).
  const float kvs = (CT == DT_FP8) ? *p.kv_scale : 1.0f;
  const float sscale = p.sm_scale * kvs;

  float qr[kValuHeads][DJ];
#pragma unroll
  for (int hh = 0; hh < kValuHeads; ++hh) {
    const int h = h0 + hh;
#pragma unroll
    for (int j = 0; j < DJ; ++j)
      qr[hh][j] = h < p.H ? load_q_elem<QT>(p.q, b * p.q_sb + h * p.q_sh + lane + kWave * j) : 0.0f;
  }
  float m[kValuHeads], l[kValuHeads], acc[kValuHeads][RJ];
#pragma unroll
  for (int hh = 0; hh < kValuHeads; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.0f;
#pragma unroll
    for (int j = 0; j < RJ; ++j) acc[hh][j] = 0.0f;
  }

  const int32_t* bt = p.block_table + b * p.bt_stride;
#pragma unroll 1
  for (int n = a + wave; n < e; n += kValuWaves) {
    const long long blk = bt[n / p.block_size];
    const long long row = blk * p.block_stride + (long long)(n % p.block_size) * D;
    float kv[DJ];
#pragma unroll
    for (int j = 0; j < DJ; ++j) kv[j] = load_cache_elem<CT>(p.cache, row + lane + kWave * j);
#pragma unroll
    for (int hh = 0; hh < kValuHeads; ++hh) {
      float d = 0.0f;
#pragma unroll
      for (int j = 0; j < DJ; ++j) d = fmaf(qr[hh][j], kv[j], d);
      const float s = wave_sum(d) * sscale;
      const float mn = fmaxf(m[hh], s);
      const float alpha = expf(m[hh] - mn);
      const float pe = expf(s - mn);
      l[hh] = l[hh] * alpha + pe;
#pragma unroll
      for (int j = 0; j < RJ; ++j) acc[hh][j] = acc[hh][j] * alpha + pe * kv[j];
      m[hh] = mn;
    }
  }

  // merge the waves through LDS
#pragma unroll
  for (int hh = 0; hh < kValuHeads; ++hh) {
#pragma unroll
    for (int j = 0; j < RJ; ++j) sm_acc[wave][hh][lane + kWave * j] = acc[hh][j];
    if (lane == 0) {
      sm_ml[wave][hh][0] = m[hh];
      sm_ml[wave][hh][1] = l[hh];
    }
  }
  __syncthreads();
  const int S = p.S;
  for (int idx = threadIdx.x; idx < kValuHeads * R; idx += kWave * kValuWaves) {
    const int hh = idx / R;
    const int d = idx - hh * R;
    const int h = h0 + hh;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kValuWaves; ++w) M = fmaxf(M, sm_ml[w][hh][0]);
    float L = 0.0f, o = 0.0f;
#pragma unroll
    for (int w = 0; w < kValuWaves; ++w) {
      const float mw = sm_ml[w][hh][0];
      if (mw == -INFINITY) continue;       // this wave saw no token
      const float c = expf(mw - M);
      L += sm_ml[w][hh][1] * c;
      o += sm_acc[w][hh][d] * c;
    }
    if (h < p.H) {
      const float v = o / L * kvs;
      if (p.direct) {
        // one partial per request: o and lse themselves, the same bits as
        // the merge of the single partial (weight exp(0) = 1, sum 1; its
        // fused 1 * v + 0 turns a -0 into +0, as the + 0.0f here does)
        const long long bh = (long long)b * p.H + h;
        if constexpr (QT == DT_F32) reinterpret_cast<float*>(p.o)[bh * R + d] = v + 0.0f;
        else reinterpret_cast<uint16_t*>(p.o)[bh * R + d] = (uint16_t)f32_to_bf16_rne(v + 0.0f);
        if (d == 0) p.lse[bh] = M + logf(L);
      } else {
        ws_row(p, part, h, R)[d] = v;
        if (d == 0) *ws_lse(p, part, h, R) = M + logf(L);
      }
    }
  }
  __syncthreads();   // LDS is reused by the next piece
}

template <int QT, int CT, int R, int P>
__global__ __launch_bounds__(kWave * kValuWaves) void stage1_valu_kernel(DecodeParams p) {
  __shared__ float sm_acc[kValuWaves][kValuHeads][R];
  __shared__ float sm_ml[kValuWaves][kValuHeads][2];
  const int lane = threadIdx.x & (kWave - 1);
  const int h0 = blockIdx.y * kValuHeads;

  if (p.partition == PART_LITERAL) {
    const int b = blockIdx.x / p.S;
    const int s = blockIdx.x - b * p.S;
    const int n = p.seq_lens[b];
    if (n <= 0) {
      if (p.direct) {   // an empty request: o = 0, lse = -inf, as the merge would write
        for (int i = threadIdx.x; i < kValuHeads * R; i += kWave * kValuWaves) {
          const int h = h0 + i / R;
          if (h >= p.H) continue;
          const long long idx = ((long long)b * p.H + h) * R + i % R;
          if constexpr (QT == DT_F32) reinterpret_cast<float*>(p.o)[idx] = 0.0f;
          else reinterpret_cast<uint16_t*>(p.o)[idx] = 0;
          if (i % R == 0) p.lse[(long long)b * p.H + h] = -INFINITY;
        }
      }
      return;
    }
    int a, e;
    literal_piece_range(n, p.S, p.piece_len, s, a, e);
    if (e <= a) return;
    valu_piece<QT, CT, R, P>(p, b, h0, a, e, b * p.S + s, sm_acc, sm_ml);
    return;
  }

  // balanced: workgroup blockIdx.x owns chunk [g*Q, (g+1)*Q) of the padded line
  const int g = blockIdx.x;
  const BatchTotals t = batch_totals(p.seq_lens, p.B, lane);
  const long long Q = balanced_chunk(t, p.G);
  const long long lo = (long long)g * Q;
  const long long hi = min(lo + Q, t.total);
  if (lo >= hi) return;
  long long carry = 0;
  for (int base = 0; base < p.B; base += kWave) {
    const int b = base + lane;
    const int n = b < p.B ? max(p.seq_lens[b], 0) : 0;
    const long long n32 = pad32(n);
    const long long incl = wave_scan_i64(n32, lane);
    const long long start = carry + incl - n32;
    const bool ov = n > 0 && start < hi && start + n > lo;
    unsigned long long mask = __ballot(ov);
    while (mask) {
      const int j = __ffsll((long long)mask) - 1;
      mask &= mask - 1;
      const long long st = __shfl(start, j, kWave);
      const int nn = __shfl(n, j, kWave);
      const int a = (int)(lo > st ? lo - st : 0);
      const int e = (int)min(hi - st, (long long)nn);
      valu_piece<QT, CT, R, P>(p, base + j, h0, a, e, g + base + j, sm_acc, sm_ml);   // slot c + b
    }
    carry += __shfl(incl, kWave - 1, kWave);
    if (carry >= hi) break;
  }
}

template <int QT, int CT>
static hipError_t launch_valu_t(const DecodeParams& p, int R, hipStream_t stream) {
  dim3 block(kWave * kValuWaves);
  const unsigned gx = p.partition == PART_LITERAL ? (unsigned)(p.B * p.S) : (unsigned)p.G;
  dim3 grid(gx, (unsigned)((p.H + kValuHeads - 1) / kValuHeads));
  if (R == 512) hipLaunchKernelGGL((stage1_valu_kernel<QT, CT, 512, 64>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((stage1_valu_kernel<QT, CT, 256, 64>), grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_stage1_valu(int q_dtype, int cache_dtype, int R, const DecodeParams& p, hipStream_t stream) {
  if (q_dtype == DT_F32 && cache_dtype == DT_F32) return launch_valu_t<DT_F32, DT_F32>(p, R, stream);
  if (q_dtype == DT_BF16 && cache_dtype == DT_BF16) return launch_valu_t<DT_BF16, DT_BF16>(p, R, stream);
  if (q_dtype == DT_BF16 && cache_dtype == DT_FP8) return launch_valu_t<DT_BF16, DT_FP8>(p, R, stream);
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Stage 2: merge each (request, head)'s partials by their LSEs
// ("fix TP" diff, _fwd_kernel_stage2; the merged LSE is returned as well, as
// forward_mqa in the Triton-MLA essay returns (o, lse)).
// One wave per (request, head); 4 heads per workgroup.  KC partial rows are
// loaded at a time: 8 as a rule, 4 at R = 512 when requests hold about 4
// partials or fewer (the smaller row buffer lets 8 waves share a SIMD
// instead of 5, so every wave's dependent loads of seq_lens and of its rows
// are in flight together; measured 19.8 -> 17.7 us on the V3 shape).
// ---------------------------------------------------------------------------

constexpr int kMergeWaves = 4;

template <int QT, int R, int KC>
__global__ __launch_bounds__(kWave * kMergeWaves) void stage2_merge_kernel(DecodeParams p) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  constexpr int V4 = R / (4 * kWave);   // 16-byte vectors per lane per partial row
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int hblocks = (p.H + kMergeWaves - 1) / kMergeWaves;
  const int b = blockIdx.x / hblocks;
  const int h = (blockIdx.x - b * hblocks) * kMergeWaves + wave;
  int k, first;
  if (p.partition == PART_LITERAL) {
    k = literal_num_partials(p.seq_lens[b], p.S, p.piece_len);
    first = b * p.S;
  } else {
    // The workgroup's waves are heads of one request: wave 0 works out the
    // request's partials for all of them.  (With eight waves per SIMD this
    // vector work, done by every wave, cost about as much as loading the
    // partial rows.)
    __shared__ int s_part[2];
    if (wave == 0) {
      long long start;
      const BatchTotals t = batch_totals_and_start(p.seq_lens, p.B, b, lane, start);
      const long long Q = balanced_chunk(t, p.G);
      if (lane == 0) {
        s_part[0] = balanced_num_partials(start, p.seq_lens[b], Q);
        s_part[1] = (int)div_nonneg(start, Q) + b;
      }
    }
    __syncthreads();
    k = s_part[0];
    first = s_part[1];
  }
  if (h >= p.H) return;
  k = __builtin_amdgcn_readfirstlane(k);
  first = __builtin_amdgcn_readfirstlane(first);
  // the request's partials are consecutive slots: partial s at rows + s R / 4
  const f32x4* rows = reinterpret_cast<const f32x4*>(ws_row(p, first, h, R));
  const float* lses = ws_lse(p, first, h, R);
  f32x4 acc[V4];
#pragma unroll
  for (int q = 0; q < V4; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  float M = -INFINITY, L = 0.0f;
  if (k > 0) {
    f32x4 v[KC][V4];
    auto load_rows = [&](int s0) {
#pragma unroll
      for (int j = 0; j < KC; ++j)
        if (s0 + j < k)
#pragma unroll
          for (int q = 0; q < V4; ++q) v[j][q] = rows[(long long)(s0 + j) * (R / 4) + lane + kWave * q];
    };
    load_rows(0);   // in flight while the LSEs are reduced
    for (int s = lane; s < k; s += kWave) M = fmaxf(M, lses[s]);
    M = wave_max(M);
    float Ls = 0.0f;
    for (int s = lane; s < k; s += kWave) Ls += expf(lses[s] - M);
    L = wave_sum(Ls);
    // weights of partials c0 .. c0+63 live one per lane; a partial's weight
    // is read from its lane
    for (int c0 = 0; c0 < k; c0 += kWave) {
      const float wl = c0 + lane < k ? expf(lses[c0 + lane] - M) : 0.0f;
      const int ce = min(k, c0 + kWave);
      for (int s0 = c0; s0 < ce; s0 += KC) {
        if (s0 > 0) load_rows(s0);
#pragma unroll
        for (int j = 0; j < KC; ++j) {
          if (s0 + j < ce) {
            const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), s0 + j - c0));
#pragma unroll
            for (int q = 0; q < V4; ++q) acc[q] += w * v[j][q];
          }
        }
      }
    }
    const float inv = 1.0f / L;
#pragma unroll
    for (int q = 0; q < V4; ++q) acc[q] *= inv;
  }
  const long long bh = (long long)b * p.H + h;
#pragma unroll
  for (int q = 0; q < V4; ++q) {
    const long long idx = bh * R + 4 * (lane + kWave * q);
    if constexpr (QT == DT_F32) {
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.o) + idx) = acc[q];
    } else {
      const uint32_t lo = f32_to_bf16_rne(acc[q][0]) | (f32_to_bf16_rne(acc[q][1]) << 16);
      const uint32_t hi = f32_to_bf16_rne(acc[q][2]) | (f32_to_bf16_rne(acc[q][3]) << 16);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.o) + idx) = make_uint2(lo, hi);
    }
  }
  if (lane == 0) p.lse[bh] = k > 0 ? M + logf(L) : -INFINITY;
}

// ---------------------------------------------------------------------------
// Merge of G shard results (o_g, lse_g) of the same queries: one wave per
// (request, head), 4 per workgroup; the weights are those of stage 2.
// ---------------------------------------------------------------------------
template <int DT, int R>
__global__ __launch_bounds__(kWave * kMergeWaves) void shard_merge_kernel(const void* __restrict__ o_parts,
                                                                          const float* __restrict__ lse_parts,
                                                                          int G, long long BH, void* o,
                                                                          float* lse) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  constexpr int V4 = R / (4 * kWave);   // 4-element groups per lane per row
  const int lane = threadIdx.x & (kWave - 1);
  const long long bh = (long long)blockIdx.x * kMergeWaves + threadIdx.x / kWave;
  if (bh >= BH) return;
  float M = -INFINITY;
  for (int g = lane; g < G; g += kWave) M = fmaxf(M, lse_parts[g * BH + bh]);
  M = wave_max(M);
  f32x4 acc[V4];
#pragma unroll
  for (int q = 0; q < V4; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  float L = 0.0f;
  if (M != -INFINITY) {
    float Ls = 0.0f;
    for (int g = lane; g < G; g += kWave) Ls += expf(lse_parts[g * BH + bh] - M);
    L = wave_sum(Ls);
#pragma unroll 4
    for (int g = 0; g < G; ++g) {
      const float w = expf(lse_parts[g * BH + bh] - M);   // 0 for an empty shard
      const long long row = (g * BH + bh) * R;
#pragma unroll
      for (int q = 0; q < V4; ++q) {
        const long long idx = row + 4 * (lane + kWave * q);
        // each shard row is read once: non-temporal loads (8 bf16 shards of
        // the V3 shape: 14.3 -> 13.6 us)
        f32x4 v;
        if constexpr (DT == DT_F32) {
          v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(o_parts) + idx));
        } else {
          typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
          const u32x2 u =
              __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(o_parts) + idx));
          v = f32x4{bf16_to_f32(u[0] & 0xffffu), bf16_to_f32(u[0] >> 16), bf16_to_f32(u[1] & 0xffffu),
                    bf16_to_f32(u[1] >> 16)};
        }
        acc[q] += w * v;
      }
    }
    const float inv = 1.0f / L;
#pragma unroll
    for (int q = 0; q < V4; ++q) acc[q] *= inv;
  }
#pragma unroll
  for (int q = 0; q < V4; ++q) {
    const long long idx = bh * R + 4 * (lane + kWave * q);
    if constexpr (DT == DT_F32) {
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(o) + idx) = acc[q];
    } else {
      const uint32_t lo = f32_to_bf16_rne(acc[q][0]) | (f32_to_bf16_rne(acc[q][1]) << 16);
      const uint32_t hi = f32_to_bf16_rne(acc[q][2]) | (f32_to_bf16_rne(acc[q][3]) << 16);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(o) + idx) = make_uint2(lo, hi);
    }
  }
  if (lane == 0) lse[bh] = M != -INFINITY ? M + logf(L) : -INFINITY;
}

hipError_t launch_shard_merge(int dtype, int R, const void* o_parts, const float* lse_parts, int G, long long BH,
                              void* o, float* lse, hipStream_t stream) {
  dim3 grid((unsigned)((BH + kMergeWaves - 1) / kMergeWaves)), block(kWave * kMergeWaves);
  if (dtype == DT_F32) {
    if (R == 512) hipLaunchKernelGGL((shard_merge_kernel<DT_F32, 512>), grid, block, 0, stream, o_parts, lse_parts, G, BH, o, lse);
    else hipLaunchKernelGGL((shard_merge_kernel<DT_F32, 256>), grid, block, 0, stream, o_parts, lse_parts, G, BH, o, lse);
  } else {
    if (R == 512) hipLaunchKernelGGL((shard_merge_kernel<DT_BF16, 512>), grid, block, 0, stream, o_parts, lse_parts, G, BH, o, lse);
    else hipLaunchKernelGGL((shard_merge_kernel<DT_BF16, 256>), grid, block, 0, stream, o_parts, lse_parts, G, BH, o, lse);
  }
  return hipGetLastError();
}

hipError_t launch_stage2(int q_dtype, int R, const DecodeParams& p, hipStream_t stream) {
  const int hblocks = (p.H + kMergeWaves - 1) / kMergeWaves;
  dim3 grid((unsigned)(p.B * hblocks)), block(kWave * kMergeWaves);
  // partials per request: at most S (literal), about G / B (balanced)
  const long long per_req = p.partition == PART_LITERAL ? p.S : ((long long)p.G + p.B - 1) / p.B;
  const bool kc4 = R == 512 && per_req <= 4;
  if (q_dtype == DT_F32) {
    if (R == 512) {
      if (kc4) hipLaunchKernelGGL((stage2_merge_kernel<DT_F32, 512, 4>), grid, block, 0, stream, p);
      else hipLaunchKernelGGL((stage2_merge_kernel<DT_F32, 512, 8>), grid, block, 0, stream, p);
    } else {
      hipLaunchKernelGGL((stage2_merge_kernel<DT_F32, 256, 8>), grid, block, 0, stream, p);
    }
  } else {
    if (R == 512) {
      if (kc4) hipLaunchKernelGGL((stage2_merge_kernel<DT_BF16, 512, 4>), grid, block, 0, stream, p);
      else hipLaunchKernelGGL((stage2_merge_kernel<DT_BF16, 512, 8>), grid, block, 0, stream, p);
    } else {
      hipLaunchKernelGGL((stage2_merge_kernel<DT_BF16, 256, 8>), grid, block, 0, stream, p);
    }
  }
  return hipGetLastError();
}

}  // namespace mla
