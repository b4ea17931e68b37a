// C ABI of libmla_amd (declared in include/mla.h): argument validation,
// split planning and kernel launches.  Nothing here reads device memory,
// allocates, or synchronises, so every call can be captured into a HIP graph.
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "mla.h"
#include "mla_launch.h"

using namespace mla;

namespace {

constexpr int kMaxDevices = 64;
int g_num_cus[kMaxDevices];   // 0 = not queried yet

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = __atomic_load_n(&g_num_cus[dev], __ATOMIC_RELAXED);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
  __atomic_store_n(&g_num_cus[dev], n, __ATOMIC_RELAXED);
  return n;
}

bool shape_supported(int R, int P) { return (R == 512 && P == 64) || (R == 256 && P == 64); }

int g_lds_per_cu[kMaxDevices];   // 0 = not queried yet

int device_lds_per_cu() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 160 * 1024;
  int n = __atomic_load_n(&g_lds_per_cu[dev], __ATOMIC_RELAXED);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess || n < 1)
    n = 160 * 1024;
  __atomic_store_n(&g_lds_per_cu[dev], n, __ATOMIC_RELAXED);
  return n;
}

int elem_bytes(int dt) { return dt == MLA_F32 ? 4 : dt == MLA_BF16 ? 2 : 1; }

// Scratch for mla_decode_noalloc: the split partials of one decode.  A
// __device__ variable exists once per GPU the module is loaded on.  In host
// code `scratch` only names the variable; its device address on the current
// GPU comes from hipGetSymbolAddress and is kept per device.
static __device__ __align__(256) float scratch[MLA_NOALLOC_SCRATCH_BYTES / sizeof(float)];
float* g_scratch[kMaxDevices];   // device address of `scratch` per device; null = not looked up yet

float* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  float* ptr = __atomic_load_n(&g_scratch[dev], __ATOMIC_ACQUIRE);
  if (ptr) return ptr;
  void* a = nullptr;
  if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || a == nullptr) return nullptr;
  ptr = static_cast<float*>(a);
  __atomic_store_n(&g_scratch[dev], ptr, __ATOMIC_RELEASE);
  return ptr;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported shape or dtype combination";
    case MLA_ERR_WORKSPACE: return "workspace too small";
    case MLA_ERR_HIP: return "HIP runtime or launch failure";
    default: return "unknown status";
  }
}

int mla_num_kv_splits(int64_t max_seq_len, int num_cus, int batch_invariant) {
  if (max_seq_len < 0 || num_cus < 1) return MLA_ERR_ARG;
  if (batch_invariant) return 1;
  int64_t s = (max_seq_len + 511) / 512;
  const int64_t cap = 2 * (int64_t)num_cus;
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  return (int)s;
}

size_t mla_decode_workspace_bytes(int B, int H, int num_kv_splits, int kv_lora_rank) {
  if (B < 1 || H < 1 || num_kv_splits < 1 || kv_lora_rank < 1) return 0;
  return (size_t)B * (size_t)H * (size_t)num_kv_splits * ((size_t)kv_lora_rank + 1) * sizeof(float);
}

}  // extern "C"

namespace {

int cache_write_impl(const void* kv_c, int64_t kv_c_row_stride, const void* k_pe, int64_t k_pe_row_stride,
                     int in_dtype, const int64_t* slot_mapping, int64_t num_tokens, void* cache, int cache_dtype,
                     int64_t num_blocks, int block_size, int64_t block_stride, int kv_lora_rank, int rope_dim,
                     const float* scale, const int64_t* positions, const float* rope, int64_t max_position,
                     void* stream) {
  if (in_dtype != MLA_F32 && in_dtype != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  if (cache_dtype != in_dtype && cache_dtype != MLA_FP8_E4M3) return MLA_ERR_UNSUPPORTED;
  if (!shape_supported(kv_lora_rank, rope_dim)) return MLA_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_blocks < 1 || block_size < 1) return MLA_ERR_ARG;
  const int D = kv_lora_rank + rope_dim;
  if (block_stride < (int64_t)block_size * D) return MLA_ERR_ARG;
  if (kv_c_row_stride < kv_lora_rank || k_pe_row_stride < rope_dim) return MLA_ERR_ARG;
  if ((cache_dtype == MLA_FP8_E4M3) != (scale != nullptr)) return MLA_ERR_ARG;
  if (num_tokens == 0) return MLA_OK;
  if (!kv_c || !k_pe || !slot_mapping || !cache) return MLA_ERR_ARG;

  WriteParams p;
  p.kv_c = kv_c;
  p.k_pe = k_pe;
  p.kv_c_stride = kv_c_row_stride;
  p.k_pe_stride = k_pe_row_stride;
  p.slots = slot_mapping;
  p.num_tokens = num_tokens;
  p.cache = cache;
  p.block_stride = block_stride;
  p.block_size = block_size;
  p.R = kv_lora_rank;
  p.P = rope_dim;
  p.scale = scale;
  p.tokens_per_wave = write_tokens_per_wave(num_tokens);
  p.positions = positions;
  p.rope = rope;
  p.max_position = max_position;

  const int ib = elem_bytes(in_dtype), cb = elem_bytes(cache_dtype);
  const int out_vec = 16 / ib * cb;   // bytes written per 16-byte input vector
  const bool vec = aligned16(kv_c) && aligned16(k_pe) &&
                   (kv_c_row_stride * ib) % 16 == 0 && (k_pe_row_stride * ib) % 16 == 0 &&
                   (reinterpret_cast<uintptr_t>(cache) % out_vec) == 0 &&
                   (block_stride * cb) % out_vec == 0 && ((int64_t)D * cb) % out_vec == 0 &&
                   ((int64_t)kv_lora_rank * cb) % out_vec == 0 && (rope == nullptr || aligned16(rope));
  (void)hipGetLastError();
  hipError_t e = launch_cache_write(in_dtype, cache_dtype, p, vec, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // namespace

extern "C" {

int mla_cache_write(const void* kv_c, int64_t kv_c_row_stride,
                    const void* k_pe, int64_t k_pe_row_stride, int in_dtype,
                    const int64_t* slot_mapping, int64_t num_tokens,
                    void* cache, int cache_dtype,
                    int64_t num_blocks, int block_size, int64_t block_stride,
                    int kv_lora_rank, int rope_dim,
                    const float* scale, void* stream) {
  return cache_write_impl(kv_c, kv_c_row_stride, k_pe, k_pe_row_stride, in_dtype, slot_mapping, num_tokens, cache,
                          cache_dtype, num_blocks, block_size, block_stride, kv_lora_rank, rope_dim, scale, nullptr,
                          nullptr, 0, stream);
}

int mla_cache_write_rope(const void* kv_c, int64_t kv_c_row_stride,
                         const void* k_pe, int64_t k_pe_row_stride, int in_dtype,
                         const int64_t* slot_mapping, int64_t num_tokens,
                         const int64_t* positions, const float* cos_sin_cache, int64_t max_position,
                         void* cache, int cache_dtype,
                         int64_t num_blocks, int block_size, int64_t block_stride,
                         int kv_lora_rank, int rope_dim,
                         const float* scale, void* stream) {
  if (max_position < 1) return MLA_ERR_ARG;
  if (num_tokens > 0 && (!positions || !cos_sin_cache)) return MLA_ERR_ARG;
  if (cos_sin_cache && reinterpret_cast<uintptr_t>(cos_sin_cache) % 4 != 0) return MLA_ERR_ARG;
  return cache_write_impl(kv_c, kv_c_row_stride, k_pe, k_pe_row_stride, in_dtype, slot_mapping, num_tokens, cache,
                          cache_dtype, num_blocks, block_size, block_stride, kv_lora_rank, rope_dim, scale, positions,
                          cos_sin_cache, max_position, stream);
}

int mla_rope_q(void* q, int64_t q_stride_n, int64_t q_stride_h, int q_dtype, int64_t num_tokens, int H,
               int kv_lora_rank, int rope_dim, const int64_t* positions, const float* cos_sin_cache,
               int64_t max_position, void* stream) {
  if (q_dtype != MLA_F32 && q_dtype != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  if (!shape_supported(kv_lora_rank, rope_dim)) return MLA_ERR_UNSUPPORTED;
  if (num_tokens < 0 || H < 1 || max_position < 1) return MLA_ERR_ARG;
  if (q_stride_h < kv_lora_rank + rope_dim || q_stride_n < (int64_t)H * q_stride_h) return MLA_ERR_ARG;
  if (num_tokens == 0) return MLA_OK;
  if (!q || !positions || !cos_sin_cache) return MLA_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(q) % elem_bytes(q_dtype) != 0 ||
      reinterpret_cast<uintptr_t>(cos_sin_cache) % 4 != 0)
    return MLA_ERR_ARG;
  RopeQParams p;
  p.q = q;
  p.q_sn = q_stride_n;
  p.q_sh = q_stride_h;
  p.N = num_tokens;
  p.H = H;
  p.R = kv_lora_rank;
  p.P = rope_dim;
  p.positions = positions;
  p.rope = cos_sin_cache;
  p.max_position = max_position;
  (void)hipGetLastError();
  const hipError_t e = launch_rope_q(q_dtype, p, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_decode_ex(const void* q, int64_t q_stride_b, int64_t q_stride_h, int q_dtype,
                  int B, int H,
                  const void* cache, int cache_dtype, int64_t num_blocks, int block_size,
                  int64_t block_stride, int kv_lora_rank, int rope_dim,
                  const int32_t* block_table, int64_t block_table_stride, int max_blocks_per_seq,
                  const int32_t* seq_lens,
                  float sm_scale, const float* kv_scale,
                  int num_kv_splits,
                  float* workspace, size_t workspace_bytes,
                  void* o, float* lse, void* stream,
                  const mla_decode_opts_t* opts) {
  mla_decode_opts_t op;
  memset(&op, 0, sizeof(op));
  if (opts) op = *opts;
  if (op.partition < 0 || op.partition > 3 || op.kernel < 0 || op.kernel > 3 || op.grid < 0 ||
      op.heads_per_group < 0 || op.piece_len < 0 || (op.partition == 3) != (op.piece_len > 0) || op.reserved[0] ||
      op.reserved[1])
    return MLA_ERR_ARG;

  const bool pair_ok = (q_dtype == MLA_F32 && cache_dtype == MLA_F32) ||
                       (q_dtype == MLA_BF16 && cache_dtype == MLA_BF16) ||
                       (q_dtype == MLA_BF16 && cache_dtype == MLA_FP8_E4M3);
  if (!pair_ok) return MLA_ERR_UNSUPPORTED;
  if (!shape_supported(kv_lora_rank, rope_dim)) return MLA_ERR_UNSUPPORTED;
  if (B < 0 || H < 1 || num_kv_splits < 1 || num_blocks < 1 || block_size < 1 || max_blocks_per_seq < 1)
    return MLA_ERR_ARG;
  const int D = kv_lora_rank + rope_dim;
  if (block_stride < (int64_t)block_size * D || block_table_stride < max_blocks_per_seq) return MLA_ERR_ARG;
  if (q_stride_b < 1 || q_stride_h < 1) return MLA_ERR_ARG;
  if (!isfinite(sm_scale)) return MLA_ERR_ARG;
  if ((cache_dtype == MLA_FP8_E4M3) != (kv_scale != nullptr)) return MLA_ERR_ARG;
  if (B == 0) return MLA_OK;
  if (!q || !cache || !block_table || !seq_lens || !workspace || !o || !lse) return MLA_ERR_ARG;
  if (!aligned16(workspace) || !aligned16(o)) return MLA_ERR_ARG;
  if (workspace_bytes < mla_decode_workspace_bytes(B, H, num_kv_splits, kv_lora_rank)) return MLA_ERR_WORKSPACE;
  // fixed-length pieces: a request of the longest length the table allows
  // must fit its num_kv_splits partial slots
  if (op.piece_len > 0 &&
      (long long)num_kv_splits * op.piece_len < (long long)max_blocks_per_seq * block_size)
    return MLA_ERR_ARG;

  // stage-1 kernel: MFMA for bf16 queries when the geometry allows it
  const bool mfma_ok = q_dtype == MLA_BF16 && mfma_supported(H, kv_lora_rank, cache_dtype) && aligned16(q) &&
                       (q_stride_b * 2) % 16 == 0 && (q_stride_h * 2) % 16 == 0 &&
                       aligned16(cache) && (block_stride * elem_bytes(cache_dtype)) % 16 == 0;
  bool use_mfma;
  if (op.kernel == 2 || op.kernel == 3) {
    if (!mfma_ok) return MLA_ERR_UNSUPPORTED;
    use_mfma = true;
  } else if (op.kernel == 1) {
    use_mfma = false;
  } else {
    use_mfma = mfma_ok;
  }

  DecodeParams p;
  p.q = q;
  p.q_sb = q_stride_b;
  p.q_sh = q_stride_h;
  p.cache = cache;
  p.block_stride = block_stride;
  p.block_table = block_table;
  p.bt_stride = block_table_stride;
  p.seq_lens = seq_lens;
  p.kv_scale = kv_scale;
  p.ws = workspace;
  p.o = o;
  p.lse = lse;
  p.sm_scale = sm_scale;
  p.B = B;
  p.H = H;
  p.S = num_kv_splits;
  p.block_size = block_size;
  p.bs_log2 = (block_size & (block_size - 1)) == 0 ? __builtin_ctz((unsigned)block_size) : -1;
  if (num_kv_splits == 1 || op.partition == 1 || op.partition == 3) p.partition = PART_LITERAL;
  else p.partition = PART_BALANCED;
  p.piece_len = op.piece_len;

  const int cus = device_cu_count();
  int groups;   // head groups per token chunk
  if (use_mfma) {
    const long long literal_items = p.partition == PART_LITERAL ? (long long)B * num_kv_splits : 0;
    p.heads_per_group = op.heads_per_group ? op.heads_per_group
                                           : mfma_heads_per_group(H, kv_lora_rank, cache_dtype, literal_items, cus,
                                                                  device_lds_per_cu());
    if (!mfma_group_ok(p.heads_per_group) || H % p.heads_per_group != 0) return MLA_ERR_ARG;
    groups = (H + p.heads_per_group - 1) / p.heads_per_group;
  } else {
    p.heads_per_group = 4;
    groups = (H + 3) / 4;
  }
  // 16- or 32-head groups: four waves split each token range (kernel 3)
  // instead of sharing each tile or one wave per range.  It sums a range's tiles in another order than the
  // one-wave kernels, so under the literal partition (whose results must not
  // depend on the batch) it is the default exactly when the head count
  // allows no group wider than 16, whatever the batch size: then every batch
  // runs it.  Measured against the one-wave kernel: 2.6x on batch-invariant
  // V2-Lite decode and 4-5% on 512 requests of 2048 tokens, 6% slower at
  // 1024 x 700 tokens and 8.6 us slower at 300 x 100 tokens.  Under the
  // balanced partition (no batch invariance to keep) it is the default for
  // 16-head groups while the batch is below two requests per four-wave
  // workgroup of the grid (one per CU and group): with the next tile
  // refilling each wave's slot it is faster on every such shape measured
  // (decode, H = 16: the V2-Lite mix 33.8 -> 33.1 us, 8 x 8192 44 -> 38,
  // 32 x 1024 58 -> 38, 384 x 2048 178 -> 172; R = 256: 32 x 1024 47 -> 27,
  // 512 x 2048 135 -> 126), while with more requests a chunk holds several
  // of them and the per-range merge of the four waves costs more than the
  // extra streams buy (R = 512: 512 x 2048 213 -> 219, 1024 x 700 176 -> 185).
  p.token_split = 0;
  p.len_min = 0;
  p.len_max = INT_MAX;
  if (op.kernel == 3) {
    if (!use_mfma || cache_dtype != MLA_BF16) return MLA_ERR_UNSUPPORTED;
    if (!op.heads_per_group) p.heads_per_group = 16;
    if ((p.heads_per_group != 16 && p.heads_per_group != 32) || H % p.heads_per_group != 0)
      return MLA_ERR_UNSUPPORTED;
    groups = H / p.heads_per_group;
    p.token_split = 1;
  } else if (use_mfma && p.heads_per_group == 16 && op.kernel == 0 && cache_dtype == MLA_BF16 && !op.grid &&
             H % 32 != 0) {
    if (p.partition == PART_LITERAL) p.token_split = 1;
    else p.token_split = (long long)B * groups < 2LL * cus ? 1 : 0;
  } else if (use_mfma && op.kernel == 0 && !op.heads_per_group && cache_dtype == MLA_BF16 && !op.grid &&
             p.partition == PART_BALANCED && kv_lora_rank == 512 && (H == 32 || H == 64) &&
             (long long)B * (H / 32) < 2LL * cus) {
    // the same rule for 32 and 64 heads at R = 512, with 32-head groups
    // (decode, default -> token split: H = 32, 64 x 8192 120.7 -> 111.0 us,
    // 128 x 2048 89.0 -> 70.3, 256 x 2048 130.2 -> 118.1; H = 64, 16 x 8192
    // 72.7 -> 57.6, 64 x 8192 154.2 -> 155.9; past the threshold, H = 32,
    // 512 x 1024 137.7 -> 142.8).  At R = 256 the one-wave kernel keeps
    // three workgroups per CU and stays ahead (H = 32: 60.0 against 66.5).
    p.heads_per_group = 32;
    groups = H / 32;
    p.token_split = 1;
  } else if (use_mfma && op.kernel == 0 && !op.heads_per_group && cache_dtype == MLA_BF16 && !op.grid &&
             p.partition == PART_BALANCED && kv_lora_rank == 512 && H == 128 && (long long)B * 4 <= cus &&
             (long long)B * max_blocks_per_seq * block_size <= 768LL * cus) {
    // 128 heads: the four 32-head groups of a token-split chunk each read
    // its tiles, so it only pays while the batch is small -- few requests
    // (the two-role kernel's chunks are then capped by the B * (S - 1)
    // partial slots and leave CUs idle) and a short context (bounded on the
    // host by the block table's width).  Decode, two-role -> token split:
    // 8 x 8192 76.2 -> 43.4 us, 4 x 32768 86.0 -> 64.1, 64 x 2048 86.2 ->
    // 63.3, 24 x 8192 100.4 -> 92.6, 48 x 4096 101.1 -> 99.4; beyond the
    // bounds 32 x 8192 99.2 -> 118.8 and 160 x 1024 92.6 -> 120.8.
    p.heads_per_group = 32;
    groups = 4;
    p.token_split = 1;
  }
  // Batch-invariant decode (one partial per request) with a head count that
  // 32 divides: a long request is served by four waves that each stream a
  // quarter of its tiles for 32 heads (its 32-head groups re-read each tile
  // from L2) instead of the fill rule's shared-tile groups, which leave SIMDs
  // idle when the requests are few.  The two kernels sum a request's tiles in
  // different orders, so the choice is made per request from its own length
  // (in the kernels: each launch skips the requests of the other), never from
  // the batch.  Measured (128 heads, R = 512, bf16): the token split takes
  // 234 us for 64 requests of 8192 tokens against 490 us, 789 against 1743
  // for 32 x 32768 and 1528 against 3457 for 16 x 65536, but 906 against
  // 582 for 256 x 8192, where the shared-tile groups alone fill the GPU;
  // below 4096 tokens it wins only for small batches (73 against 125 us for
  // 64 x 2048, 309 against 158 for 256 x 2048).
  int split_len = 0;
  const int want_split_len = op.split_len == 0 ? MLA_DEFAULT_SPLIT_LEN : op.split_len;
  if (use_mfma && op.kernel == 0 && !op.grid && !op.heads_per_group && cache_dtype == MLA_BF16 &&
      num_kv_splits == 1 && H % 32 == 0 && want_split_len > 0)
    split_len = want_split_len;
  if (op.grid) {
    p.G = op.grid;
  } else if (p.token_split) {
    p.G = cus / groups < 1 ? 1 : cus / groups;   // one four-wave workgroup per CU
  } else {
    // as many MFMA workgroups per compute unit as fit at once (one for the
    // 64- and 128-head shapes, whose tile ring fills the LDS; two or three of
    // the one-wave shapes); the vector kernel's grid is four workgroups per CU
    const int per_cu =
        use_mfma ? mfma_wgs_per_cu(p.heads_per_group, kv_lora_rank, cache_dtype, device_lds_per_cu()) : 4;
    int g = cus * per_cu / groups;
    p.G = g < 1 ? 1 : g;
  }
  // balanced: the chunks' partials must fit the B * S slots of the workspace
  // (slot of chunk c, request b is c + b)
  if (p.partition == PART_BALANCED) {
    const long long cap = (long long)B * (num_kv_splits - 1);
    if (p.G > cap) p.G = (int)cap;
  }

  (void)hipGetLastError();
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipEvent_t* ev = reinterpret_cast<hipEvent_t*>(op.stage_events);
  if (ev[0] && hipEventRecord(ev[0], st) != hipSuccess) return MLA_ERR_HIP;
  // KV tiles read by one or two head groups are streamed past the caches
  // (the second group's workgroup runs right after the first on the same
  // XCD and still finds the lines); tiles shared by more groups are meant to
  // meet in L2
  p.kv_nt = groups <= 2 ? 1 : 0;
  // one partial per request: stage 1 writes o and lse itself (the merge of a
  // single partial is the identity, bit for bit), so there is no stage 2 and
  // no workspace traffic
  p.direct = num_kv_splits == 1 ? 1 : 0;
  hipError_t e;
  if (split_len > 0) {
    DecodeParams pt = p;
    pt.heads_per_group = 32;
    pt.token_split = 1;
    pt.kv_nt = H <= 64 ? 1 : 0;
    pt.len_min = split_len;
    e = launch_stage1_mfma(cache_dtype, kv_lora_rank, pt, st);
    if (e != hipSuccess) return MLA_ERR_HIP;
    p.len_max = split_len;
  }
  e = use_mfma ? launch_stage1_mfma(cache_dtype, kv_lora_rank, p, st)
               : launch_stage1_valu(q_dtype, cache_dtype, kv_lora_rank, p, st);
  if (e != hipSuccess) return MLA_ERR_HIP;
  if (ev[1] && hipEventRecord(ev[1], st) != hipSuccess) return MLA_ERR_HIP;
  if (!p.direct) {
    e = launch_stage2(q_dtype, kv_lora_rank, p, st);
    if (e != hipSuccess) return MLA_ERR_HIP;
  }
  if (ev[2] && hipEventRecord(ev[2], st) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

size_t mla_linear_workspace_bytes(int M, int N, int K) {
  if (M < 1 || N < 16 || N % 16 != 0 || K < 64 || K % 64 != 0) return 0;
  const int rows = M < 64 ? M : 64;
  const int s = linear_splits(rows, N, K, device_cu_count());
  return s > 1 ? (size_t)s * rows * N * sizeof(float) : 0;
}

int mla_linear_bf16(const void* A, int64_t lda, const void* W, int64_t ldw, int M, int N, int K,
                    void* C, int64_t ldc, int c_dtype, float* workspace, size_t workspace_bytes, void* stream) {
  if (c_dtype != MLA_F32 && c_dtype != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  if (N < 16 || N % 16 != 0 || K < 64 || K % 64 != 0) return MLA_ERR_UNSUPPORTED;
  if (M < 0 || lda < K || ldw < K || ldc < N) return MLA_ERR_ARG;
  if (M == 0) return MLA_OK;
  if (!A || !W || !C) return MLA_ERR_ARG;
  if (!aligned16(A) || !aligned16(W) || lda % 8 != 0 || ldw % 8 != 0 || ldc % 4 != 0) return MLA_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(C) % (c_dtype == MLA_F32 ? 16 : 8) != 0) return MLA_ERR_ARG;
  const int rows = M < 64 ? M : 64;
  const int splits = linear_splits(rows, N, K, device_cu_count());
  if (splits > 1) {
    if (!workspace || !aligned16(workspace)) return MLA_ERR_ARG;
    if (workspace_bytes < (size_t)splits * rows * N * sizeof(float)) return MLA_ERR_WORKSPACE;
  }
  LinearParams p;
  p.W = W;
  p.ldw = ldw;
  p.lda = lda;
  p.ldc = ldc;
  p.N = N;
  p.K = K;
  p.ws = workspace;
  const int ksteps = K / 64;
  p.k_per_split = ((ksteps + splits - 1) / splits) * 64;
  p.splits = (K + p.k_per_split - 1) / p.k_per_split;
  (void)hipGetLastError();
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int cb = c_dtype == MLA_F32 ? 4 : 2;
  // 64 batch rows per launch; launches on one stream reuse the workspace in order
  for (int m0 = 0; m0 < M; m0 += 64) {
    p.M = M - m0 < 64 ? M - m0 : 64;
    p.A = static_cast<const uint16_t*>(A) + (int64_t)m0 * lda;
    p.C = static_cast<char*>(C) + (int64_t)m0 * ldc * cb;
    if (launch_linear(c_dtype, p, st) != hipSuccess) return MLA_ERR_HIP;
  }
  return MLA_OK;
}

int mla_merge_partials(const void* o_parts, const float* lse_parts, int G, int B, int H, int R, int dtype,
                       void* o, float* lse, void* stream) {
  if (R != 512 && R != 256) return MLA_ERR_UNSUPPORTED;
  if (dtype != MLA_F32 && dtype != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  if (G < 1 || B < 0 || H < 1) return MLA_ERR_ARG;
  if (B == 0) return MLA_OK;
  if (!o_parts || !lse_parts || !o || !lse) return MLA_ERR_ARG;
  if (!aligned16(o_parts) || !aligned16(o) || reinterpret_cast<uintptr_t>(lse_parts) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(lse) % 4 != 0)
    return MLA_ERR_ARG;
  (void)hipGetLastError();
  const hipError_t e = launch_shard_merge(dtype, R, o_parts, lse_parts, G, (long long)B * H, o, lse,
                                          reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_decode_noalloc(const void* q, int64_t q_stride_b, int64_t q_stride_h, int q_dtype,
                       int B, int H,
                       const void* cache, int cache_dtype, int64_t num_blocks, int block_size,
                       int64_t block_stride, int kv_lora_rank, int rope_dim,
                       const int32_t* block_table, int64_t block_table_stride, int max_blocks_per_seq,
                       const int32_t* seq_lens,
                       float sm_scale, const float* kv_scale,
                       int num_kv_splits,
                       void* o, float* lse, void* stream) {
  // the size check before the device lookup, so an oversized call fails the
  // same way on every device; argument errors are left to mla_decode_ex
  const size_t need = mla_decode_workspace_bytes(B, H, num_kv_splits, kv_lora_rank);
  if (need > MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_WORKSPACE;
  float* ws = device_scratch();
  if (!ws) return MLA_ERR_HIP;
  return mla_decode_ex(q, q_stride_b, q_stride_h, q_dtype, B, H, cache, cache_dtype, num_blocks, block_size,
                       block_stride, kv_lora_rank, rope_dim, block_table, block_table_stride, max_blocks_per_seq,
                       seq_lens, sm_scale, kv_scale, num_kv_splits, ws, MLA_NOALLOC_SCRATCH_BYTES, o, lse, stream,
                       nullptr);
}

int mla_decode(const void* q, int64_t q_stride_b, int64_t q_stride_h, int q_dtype,
               int B, int H,
               const void* cache, int cache_dtype, int64_t num_blocks, int block_size,
               int64_t block_stride, int kv_lora_rank, int rope_dim,
               const int32_t* block_table, int64_t block_table_stride, int max_blocks_per_seq,
               const int32_t* seq_lens,
               float sm_scale, const float* kv_scale,
               int num_kv_splits,
               float* workspace, size_t workspace_bytes,
               void* o, float* lse, void* stream) {
  return mla_decode_ex(q, q_stride_b, q_stride_h, q_dtype, B, H, cache, cache_dtype, num_blocks, block_size,
                       block_stride, kv_lora_rank, rope_dim, block_table, block_table_stride, max_blocks_per_seq,
                       seq_lens, sm_scale, kv_scale, num_kv_splits, workspace, workspace_bytes, o, lse, stream,
                       nullptr);
}

}  // extern "C"
