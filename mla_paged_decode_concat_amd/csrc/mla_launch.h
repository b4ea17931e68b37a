// Host-side launchers shared between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_device.h"

namespace mla {

struct WriteParams {
  const void* kv_c;
  const void* k_pe;
  long long kv_c_stride, k_pe_stride;   // elements
  const int64_t* slots;
  long long num_tokens;
  void* cache;
  long long block_stride;               // elements
  int block_size;
  int R, P;
  const float* scale;
  int tokens_per_wave;                  // write_tokens_per_wave(num_tokens)
  // rotary embedding of k_pe (rope == nullptr: none): per-token positions
  // and a [max_position, P] fp32 table of P/2 cosines then P/2 sines
  const int64_t* positions;
  const float* rope;
  long long max_position;
};

struct RopeQParams {
  void* q;
  long long q_sn, q_sh;                 // elements
  long long N;
  int H, R, P;
  const int64_t* positions;
  const float* rope;
  long long max_position;
};

int write_tokens_per_wave(long long num_tokens);

hipError_t launch_cache_write(int in_dtype, int cache_dtype, const WriteParams& p, bool vec, hipStream_t stream);
hipError_t launch_rope_q(int q_dtype, const RopeQParams& p, hipStream_t stream);

struct LinearParams {
  const void* A;                        // bf16 [M, K], row stride lda
  const void* W;                        // bf16 [N, K], row stride ldw
  void* C;                              // [M, N], row stride ldc
  float* ws;                            // split-K partials [splits, M, N] (splits > 1)
  long long lda, ldw, ldc;
  int M, N, K;                          // M <= 64 per launch
  int splits, k_per_split;              // k_per_split a multiple of 64
};

int linear_splits(int M, int N, int K, int cus);
hipError_t launch_linear(int c_dtype, const LinearParams& p, hipStream_t stream);

hipError_t launch_stage1_valu(int q_dtype, int cache_dtype, int R, const DecodeParams& p, hipStream_t stream);
hipError_t launch_stage1_mfma(int cache_dtype, int R, const DecodeParams& p, hipStream_t stream);
hipError_t launch_stage2(int q_dtype, int R, const DecodeParams& p, hipStream_t stream);
hipError_t launch_shard_merge(int dtype, int R, const void* o_parts, const float* lse_parts, int G, long long BH,
                              void* o, float* lse, hipStream_t stream);

// Stage-1 MFMA kernel geometry, needed by the host planner.
int mfma_heads_per_group(int H, int R, int cache_dtype, long long literal_items, int cus, int lds_per_cu);
bool mfma_group_ok(int heads_per_group);
bool mfma_supported(int H, int R, int cache_dtype);
int mfma_wgs_per_cu(int heads_per_group, int R, int cache_dtype, int lds_per_cu);

}  // namespace mla
