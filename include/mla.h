/*
 * mla.h — C ABI of libmla_amd.so: paged latent-KV cache write and split-KV
 * Multi-head Latent Attention (MLA) decode for AMD Instinct MI355X (gfx950).
 *
 * Sources (cited by page and section):
 *   [ESSAY] "Triton and MLA: portable attention and multi-head latent
 *           attention" (vLLM architecture notes, source version v0.25.1).
 *   [DIFF]  vLLM compare view whose commit is titled "fix TP": files
 *           csrc/cache_kernels.cu, csrc/torch_bindings.cpp,
 *           vllm/attention/ops/triton_decode_attention.py,
 *           vllm/attention/backends/triton_mla.py,
 *           vllm/attention/backends/mla/utils.py,
 *           vllm/model_executor/models/deepseek_v2.py.
 *   [API]   "vllm.v1.attention.backends.mla.triton_mla" API page,
 *           TritonMLAMetadataBuilder._reserve_attn_logits_workspace.
 *
 * Conventions for every call:
 *   - Every pointer argument is device memory owned by the caller unless the
 *     comment says otherwise.  The library never allocates, frees or
 *     synchronises inside these calls.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and the call returns without waiting.  No call reads device memory on
 *     the host, so the calls can be captured into a HIP graph.
 *   - Arguments are validated on the host before anything is enqueued.  A
 *     negative status means nothing was launched and no output was touched.
 *   - Device-resident values (seq_lens, block_table entries, slot_mapping) are
 *     not validated; their preconditions are stated per call.
 */
#ifndef MLA_AMD_MLA_H
#define MLA_AMD_MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  MLA_FP8_E4M3 is the OCP FP8 E4M3 ("e4m3fn") format: bias 7,
 * largest finite 448, NaN = S.1111.111, no infinities. */
typedef enum {
  MLA_F32 = 0,
  MLA_BF16 = 1,
  MLA_FP8_E4M3 = 2
} mla_dtype_t;

/* Status codes. */
enum {
  MLA_OK = 0,
  MLA_ERR_ARG = -1,          /* NULL required pointer, non-positive size, bad stride */
  MLA_ERR_UNSUPPORTED = -2,  /* shape or dtype combination outside the supported set */
  MLA_ERR_WORKSPACE = -3,    /* workspace smaller than mla_decode_workspace_bytes() */
  MLA_ERR_HIP = -4           /* a HIP runtime call or kernel launch failed */
};

/* Human-readable text for a status code (static storage). */
const char* mla_status_string(int status);

/*
 * Split count for a decode batch: one split per 512 tokens of the longest
 * sequence, clamped to [1, 2 * num_cus]; exactly 1 when batch_invariant is
 * non-zero, so that every request is reduced in one fixed order whatever else
 * is in the batch.  [ESSAY: Key files (_compute_num_kv_splits); Data flow]
 * Host-only.  Returns the split count, or MLA_ERR_ARG if max_seq_len < 0 or
 * num_cus < 1.
 */
int mla_num_kv_splits(int64_t max_seq_len, int num_cus, int batch_invariant);

/*
 * Bytes of the fp32 split workspace: B * H * num_kv_splits * (kv_lora_rank + 1)
 * values.  Only this size follows the pages (their workspace is
 * [B, H, num_kv_splits, kv_lora_rank + 1]: per request, head and split the
 * normalised partial output and its LSE).  The layout is this library's own
 * and internal: a pool of B * num_kv_splits partial slots per head, partial
 * rows [H, B * num_kv_splits, kv_lora_rank] followed by the natural-log LSEs
 * [H, B * num_kv_splits], so that every row starts on a cache line.
 * [ESSAY: Data flow (attn_logits shape, the "+1" LSE slot);
 * API: _reserve_attn_logits_workspace sizes it once at the worst case]
 * Host-only.  Returns 0 if any argument is < 1.
 */
size_t mla_decode_workspace_bytes(int B, int H, int num_kv_splits, int kv_lora_rank);

/*
 * Paged latent-KV cache write ("concat and cache").
 * [DIFF: csrc/cache_kernels.cu concat_and_cache_mla_kernel and its host
 *  launcher; csrc/torch_bindings.cpp op schema]
 *
 * For each token t < num_tokens with s = slot_mapping[t] >= 0, writes
 *   cache[s / block_size][s % block_size][0 : R)     = enc(kv_c[t][0 : R))
 *   cache[s / block_size][s % block_size][R : R + P) = enc(k_pe[t][0 : P))
 * Tokens with s < 0 are padding and are skipped.  num_tokens is the length of
 * slot_mapping; kv_c/k_pe may hold more rows (padding for graph capture).
 * enc is the identity (bit copy) when cache_dtype == in_dtype, and for
 * cache_dtype == MLA_FP8_E4M3 it is: x / (*scale) in IEEE fp32 (correctly
 * rounded), then round-to-nearest-even to E4M3, saturating finite values
 * beyond +-448 to +-448, NaN -> 0x7F with the sign kept.
 *
 *   kv_c, kv_c_row_stride : [>= num_tokens, R] rows, stride in elements
 *   k_pe, k_pe_row_stride : [>= num_tokens, P] rows, stride in elements
 *   in_dtype              : MLA_F32 or MLA_BF16 (both kv_c and k_pe)
 *   slot_mapping          : int64 [num_tokens]
 *   cache                 : [num_blocks, block_size, R + P], element type
 *                           cache_dtype, rows contiguous inside a block,
 *                           block_stride elements between blocks
 *   cache_dtype           : in_dtype, or MLA_FP8_E4M3
 *   kv_lora_rank R, rope_dim P : (512, 64) or (256, 64)  [ESSAY: Boundaries
 *                           and failure modes, head sizes 576 and 320]
 *   scale                 : device fp32 scalar; required iff the cache is fp8
 * Preconditions (device data): non-negative slots are unique and
 * < num_blocks * block_size.  Duplicate slots race.
 * Errors: MLA_ERR_ARG (NULL pointer, num_tokens < 0, num_blocks/block_size < 1,
 * strides too small), MLA_ERR_UNSUPPORTED (dtype pair, (R, P)), MLA_ERR_HIP.
 * num_tokens == 0 launches nothing and returns MLA_OK.
 */
int mla_cache_write(const void* kv_c, int64_t kv_c_row_stride,
                    const void* k_pe, int64_t k_pe_row_stride, int in_dtype,
                    const int64_t* slot_mapping, int64_t num_tokens,
                    void* cache, int cache_dtype,
                    int64_t num_blocks, int block_size, int64_t block_stride,
                    int kv_lora_rank, int rope_dim,
                    const float* scale, void* stream);

/*
 * Cache write with the rotary position embedding of k_pe fused in: the same
 * write as mla_cache_write, except that the k_pe columns of token t hold
 * enc(rot(k_pe[t], positions[t])).  rot turns each interleaved pair
 * (x[2i], x[2i+1]) by the angle whose cosine and sine are
 *   cos_sin_cache[positions[t] * P + i]  and  cos_sin_cache[positions[t] * P + P/2 + i]:
 *   (x[2i] cos - x[2i+1] sin,  x[2i+1] cos + x[2i] sin),
 * in fp32 with each product and sum rounded to fp32 (no fused multiply-add);
 * enc stores that fp32 value in the cache's type (bf16: round to nearest
 * even; fp8: divide by *scale, then as mla_cache_write).  kv_c is written
 * exactly as by mla_cache_write.  k_pe itself is not modified.
 * [DIFF: MLA decode path, rotary_emb(input_positions, q_pe, k_pe) ahead of
 *  the cache write; DeepSeek-V2 attention, get_rope with rope_type
 *  'deepseek_yarn' and is_neox_style=False (interleaved pairs)]
 *
 *   positions      : int64 [num_tokens], device; the position of each token
 *   cos_sin_cache  : fp32 [max_position, P], device, 4-byte aligned (16 for the
 *                    vectorised path): P/2 cosines then P/2 sines per row --
 *                    the caller's table (YaRN scaling, if any, is folded in)
 *   max_position   : rows in cos_sin_cache, >= 1
 *   other arguments: as mla_cache_write.
 * Preconditions (device data): 0 <= positions[t] < max_position for tokens
 * with a non-negative slot (a position outside is clamped to the nearest
 * row rather than read out of bounds); positions of padded tokens are not read.
 * Errors: as mla_cache_write; MLA_ERR_ARG also for max_position < 1 or a NULL
 * positions / cos_sin_cache when num_tokens > 0.
 */
int mla_cache_write_rope(const void* kv_c, int64_t kv_c_row_stride,
                         const void* k_pe, int64_t k_pe_row_stride, int in_dtype,
                         const int64_t* slot_mapping, int64_t num_tokens,
                         const int64_t* positions, const float* cos_sin_cache, int64_t max_position,
                         void* cache, int cache_dtype,
                         int64_t num_blocks, int block_size, int64_t block_stride,
                         int kv_lora_rank, int rope_dim,
                         const float* scale, void* stream);

/*
 * Rotary embedding of the query's rope part, in place: for every token n and
 * head h, q[n][h][R : R + P) is rotated by positions[n] exactly as k_pe is
 * in mla_cache_write_rope and stored back in q's dtype (bf16: round to
 * nearest even).  The first R columns are not touched.
 * [DIFF: MLA decode path, rotary_emb(input_positions, q_pe, k_pe)]
 *
 *   q                       : [num_tokens, H, R + P], device, element type q_dtype
 *   q_stride_n, q_stride_h  : strides in elements (q_stride_h >= R + P,
 *                             q_stride_n >= H * q_stride_h)
 *   q_dtype                 : MLA_F32 or MLA_BF16
 *   positions, cos_sin_cache, max_position : as mla_cache_write_rope
 * A query block of q_len tokens per request ([B, q_len, H, R + P]) is
 * num_tokens = B * q_len rows with a position per token.
 * Errors: MLA_ERR_ARG, MLA_ERR_UNSUPPORTED (dtype, (R, P)), MLA_ERR_HIP.
 * num_tokens == 0 launches nothing.
 */
int mla_rope_q(void* q, int64_t q_stride_n, int64_t q_stride_h, int q_dtype, int64_t num_tokens, int H,
               int kv_lora_rank, int rope_dim, const int64_t* positions, const float* cos_sin_cache,
               int64_t max_position, void* stream);

/*
 * Linear layer for the absorbed projections around the decode:
 *   C[m][n] = sum_k A[m][k] * W[n][k]
 * with bf16 A and W, fp32 accumulation, C in fp32 or bf16 (round to nearest
 * even).  With weight absorption the q side is q_nope = q_c W_Q_UK and the
 * output side is out = o W_UV_O, both plain products of a decode batch with
 * a precomputed weight [DIFF: MLACommonImpl docstring, decode steps 3, 7 and
 * 11; _q_proj_and_k_up_proj and _v_up_proj_and_o_proj;
 * process_weights_after_loading builds W_Q_UK and W_UV_O].
 *
 *   A, lda      : bf16 [M, K] rows (lda >= K, a multiple of 8), 16-byte aligned
 *   W, ldw      : bf16 [N, K] rows -- a linear layer's weight, one row per
 *                 output feature (ldw >= K, a multiple of 8), 16-byte aligned
 *   M, N, K     : M >= 0 (any; processed 64 rows per launch),
 *                 N a multiple of 16, K a multiple of 64
 *   C, ldc      : [M, N] rows of c_dtype (ldc >= N, a multiple of 4);
 *                 16-byte aligned for fp32, 8-byte for bf16
 *   c_dtype     : MLA_F32 or MLA_BF16
 *   workspace   : fp32 scratch of >= mla_linear_workspace_bytes(M, N, K)
 *                 bytes, 16-byte aligned (may be NULL when that is 0): when the
 *                 output features alone cannot fill the GPU, K is split over
 *                 workgroups and the partials are summed in a fixed order
 * The result does not depend on how the rows are batched.  Errors:
 * MLA_ERR_UNSUPPORTED (c_dtype, N, K), MLA_ERR_ARG (strides, alignment, NULL),
 * MLA_ERR_WORKSPACE, MLA_ERR_HIP.  M == 0 launches nothing.
 */
size_t mla_linear_workspace_bytes(int M, int N, int K);
int mla_linear_bf16(const void* A, int64_t lda, const void* W, int64_t ldw, int M, int N, int K,
                    void* C, int64_t ldc, int c_dtype, float* workspace, size_t workspace_bytes, void* stream);

/*
 * MLA decode over the paged latent cache: all H query heads attend to one
 * shared latent KV head (MQA form).
 * [ESSAY: Design motivation (single KV channel, head sizes 320/576, lse
 *  returned), Data flow (forward_mqa); DIFF: triton_decode_attention.py
 *  _fwd_grouped_kernel_stage1 and _fwd_kernel_stage2]
 *
 * For request b with n = seq_lens[b] tokens, token j's row is
 *   r_j = cache[block_table[b * block_table_stride + j / block_size]][j % block_size][:]
 * (times *kv_scale for an fp8 cache).  Head h scores
 *   s_hj = sm_scale * <q[b][h][0 : R + P), r_j>,
 * and returns o[b][h][:] = sum_j softmax_j(s_h) * r_j[0 : R)  (dtype q_dtype)
 * and lse[b][h] = ln sum_j exp(s_hj)  (fp32, natural log, includes sm_scale).
 * n == 0 gives o = 0 and lse = -inf.
 *
 * Multi-token rows.  A request whose q_len query tokens all attend, with no
 * causal mask among them, to the same n cached tokens (a non-causal
 * speculative block, which the pages flatten to one decode row per query
 * token [API: TritonMLAMetadataBuilder, non-causal multi-token decode]) is
 * passed as H = q_len * heads rows: q [B, q_len, heads, R + P] with
 * q_stride_h the head stride and a token stride of heads * q_stride_h; o and
 * lse then read as [B, q_len, heads, R] and [B, q_len, heads].  The rows of a
 * request are processed as its heads: a KV tile is read once per group of up
 * to 128 rows (groups of one token range share it through L2), not once per
 * query token.
 *
 * Two stages run on `stream`: stage 1 writes per-split normalised partial
 * outputs and LSEs into `workspace` (fp32; layout at
 * mla_decode_workspace_bytes); stage 2 merges each request's partials by
 * their LSEs.
 * num_kv_splits sets the workspace size: B * num_kv_splits partials.  With
 * num_kv_splits == 1 every request is one partial, reduced in a fixed order
 * independent of the rest of the batch (batch-invariant mode, [ESSAY: Data
 * flow]): the order depends on the request's own length only (for a bf16
 * cache with H a multiple of 32, requests of MLA_DEFAULT_SPLIT_LEN tokens or
 * more are cut among four waves of one workgroup; see split_len below), and
 * stage 1 then writes o and lse itself, with no stage 2.  With num_kv_splits > 1 the library cuts the whole batch into
 * equal token chunks across the GPU's compute units; each piece of a request
 * inside a chunk is one partial, and a long request may take more than
 * num_kv_splits of the B * num_kv_splits slots when shorter requests leave
 * them free.
 *
 *   q, q_stride_b, q_stride_h : [B, H, R + P], strides in elements, innermost
 *                               dimension contiguous
 *   q_dtype                   : MLA_F32 or MLA_BF16
 *   cache, cache_dtype        : as in mla_cache_write.  Supported pairs:
 *                               (q F32, cache F32), (q BF16, cache BF16),
 *                               (q BF16, cache FP8_E4M3)  [ESSAY: Boundaries
 *                               and failure modes, fp8 cache needs a bf16 query]
 *   block_table               : int32 [B, >= max_blocks_per_seq] with row
 *                               stride block_table_stride
 *   seq_lens                  : int32 [B]
 *   kv_scale                  : device fp32 scalar, required iff fp8 cache
 *                               (one scale for the whole row: k_scale == v_scale)
 *   workspace                 : >= mla_decode_workspace_bytes(B, H, num_kv_splits, R)
 *                               bytes, 16-byte aligned; contents on entry are ignored
 *   o                         : [B, H, R] contiguous, dtype q_dtype, 16-byte aligned
 *   lse                       : [B, H] contiguous fp32
 * Preconditions (device data): 0 <= seq_lens[b] <= max_blocks_per_seq *
 * block_size; the first ceil(seq_lens[b] / block_size) table entries of each
 * row lie in [0, num_blocks).
 * Errors: MLA_ERR_ARG, MLA_ERR_UNSUPPORTED ((R, P), dtype pair),
 * MLA_ERR_WORKSPACE (workspace_bytes too small, as the pages assert the
 * workspace split dimension equals num_kv_splits), MLA_ERR_HIP.
 * B == 0 launches nothing and returns MLA_OK.
 */
int mla_decode(const void* q, int64_t q_stride_b, int64_t q_stride_h, int q_dtype,
               int B, int H,
               const void* cache, int cache_dtype, int64_t num_blocks, int block_size,
               int64_t block_stride, int kv_lora_rank, int rope_dim,
               const int32_t* block_table, int64_t block_table_stride, int max_blocks_per_seq,
               const int32_t* seq_lens,
               float sm_scale, const float* kv_scale,
               int num_kv_splits,
               float* workspace, size_t workspace_bytes,
               void* o, float* lse, void* stream);

/*
 * Tuning and testing controls for mla_decode_ex.  Zero-initialise and set
 * only the fields you need; zero means "library default" for every field.
 *   partition  : 0 = default (balanced when num_kv_splits > 1),
 *                1 = the pages' literal partition: ceil(n / num_kv_splits)
 *                    tokens per split, empty splits skipped
 *                    [DIFF: triton_decode_attention.py, stage 1 split range],
 *                2 = balanced,
 *                3 = fixed-length pieces: request b is cut into
 *                    ceil(n_b / piece_len) pieces of piece_len tokens (the
 *                    last one shorter), each one partial, merged in piece
 *                    order.  The reduction order then depends on the
 *                    request's own length only: a batch-invariant decode
 *                    that still spreads a long request over several
 *                    workgroups (the pages' batch-invariant mode is
 *                    num_kv_splits = 1, one partial per request).  Requires
 *                    piece_len > 0 and num_kv_splits * piece_len >=
 *                    max_blocks_per_seq * block_size (MLA_ERR_ARG otherwise);
 *                    num_kv_splits sizes the workspace only, so a request
 *                    gives the same bits for any num_kv_splits that fits.
 *   kernel     : 0 = default, 1 = the generic vector-ALU stage 1,
 *                2 = the matrix-core (MFMA) stage 1 (bf16 query only),
 *                3 = the MFMA stage 1 with four waves splitting each token
 *                range of a 16- or 32-head group (bf16 cache; 16 heads per
 *                group unless heads_per_group is 32).  The default takes 3
 *                for a bf16 cache with the default grid: with 16-head
 *                groups when H is not a multiple of 32 (always under the
 *                literal partitions; under the balanced one while
 *                B * (H / 16) < 2 * compute units), and with 32-head groups
 *                for H = 32 or 64 at kv_lora_rank 512 under the balanced
 *                partition while B * (H / 32) < 2 * compute units, and
 *                for H = 128 at kv_lora_rank 512 under the balanced
 *                partition while 4 * B <= compute units and
 *                B * max_blocks_per_seq * block_size <= 768 * compute units
 *                (heads_per_group left at 0 in both).
 *   grid       : balanced partition only: number of token chunks the batch
 *                is cut into (0 = derived from the compute-unit count).
 *   heads_per_group : heads handled by one stage-1 workgroup (0 = default).
 *   stage_events : optional hipEvent_t handles (NULL entries are skipped),
 *                recorded on `stream` before stage 1, between stage 1 and
 *                stage 2, and after stage 2, for timing each stage.
 *   split_len  : batch-invariant decode (num_kv_splits == 1) of a bf16 cache
 *                with H a multiple of 32, under the default kernel, grid and
 *                head grouping: requests of at least split_len tokens run the
 *                32-head token-split stage 1 and shorter ones the stage 1
 *                whose waves share each tile (two launches, each skipping the
 *                other's requests).  The choice depends on the request's own
 *                length only, so a request decodes to the same bits in any
 *                batch that uses the same split_len.  The token split pays
 *                when the batch's requests are too few to fill the GPU with
 *                shared-tile workgroups and costs when they are many (each
 *                token-split workgroup of 32 heads reads every tile of its
 *                request; the shared-tile one reads it once for up to 128
 *                heads: about 1.5x for 256 requests of 8192 tokens at
 *                H = 128), which a batch-invariant rule cannot see.
 *                0 = MLA_DEFAULT_SPLIT_LEN, negative = off (every request on
 *                the shared-tile stage 1), positive = that threshold.
 *   piece_len  : partition 3 only (and required there): tokens per piece;
 *                a multiple of 32 keeps pieces on whole 32-token tiles.
 *   reserved   : must be zero.
 */
/* The length threshold of batch-invariant decode when split_len is 0. */
#define MLA_DEFAULT_SPLIT_LEN 4096

typedef struct {
  int partition;
  int kernel;
  int grid;
  int heads_per_group;
  void* stage_events[3];
  int split_len;
  int piece_len;
  int reserved[2];
} mla_decode_opts_t;

/* mla_decode with explicit controls (opts may be NULL = all defaults).
 * Same arguments, results within the documented tolerance of each other for
 * every opts value, and the same error behaviour, plus MLA_ERR_ARG for an
 * unknown opts value and MLA_ERR_UNSUPPORTED for a kernel that cannot run the
 * given dtype or head count.  [as mla_decode] */
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
                  const mla_decode_opts_t* opts);

/*
 * mla_decode without a caller-provided workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The split partials go to a scratch array
 * the library keeps on each GPU for the life of the process
 * (MLA_NOALLOC_SCRATCH_BYTES, allocated when the library's device code is
 * first loaded on that GPU); this call allocates nothing itself.
 *   Arguments, results, layouts and ownership: as mla_decode, minus
 *   workspace and workspace_bytes.  The results are the same bits as
 *   mla_decode's for the same arguments.
 *   Limit: mla_decode_workspace_bytes(B, H, num_kv_splits, kv_lora_rank) must
 *   not exceed MLA_NOALLOC_SCRATCH_BYTES, else MLA_ERR_WORKSPACE before any
 *   launch (a smaller num_kv_splits needs less).
 *   Every call on one GPU uses that GPU's one scratch array: calls that can
 *   overlap on a GPU (different streams without ordering between them, or
 *   different host threads) race and must be serialised by the caller.
 * Errors: as mla_decode, plus MLA_ERR_HIP when the scratch array cannot be
 * located on the current device.
 */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int mla_decode_noalloc(const void* q, int64_t q_stride_b, int64_t q_stride_h, int q_dtype,
                       int B, int H,
                       const void* cache, int cache_dtype, int64_t num_blocks, int block_size,
                       int64_t block_stride, int kv_lora_rank, int rope_dim,
                       const int32_t* block_table, int64_t block_table_stride, int max_blocks_per_seq,
                       const int32_t* seq_lens,
                       float sm_scale, const float* kv_scale,
                       int num_kv_splits,
                       void* o, float* lse, void* stream);

/*
 * Merge of partial attention results over disjoint key sets: combining the
 * per-shard outputs of a request whose tokens are split across GPUs (decode
 * context parallelism), here on one GPU's buffers.  For every (b, h):
 *   M = max_g lse_g,   w_g = exp(lse_g - M),
 *   o[b][h][:] = sum_g w_g o_g[b][h][:] / sum_g w_g,   lse[b][h] = M + ln sum_g w_g,
 * the same LSE merge as decode stage 2.  A shard with lse_g = -inf (no keys)
 * contributes nothing; if every shard is empty, o = 0 and lse = -inf.
 * [ESSAY: Design motivation (the decode returns the LSE because the
 *  cross-shard merge relies on it; natural-log LSE); API: DCP all-gathers the
 *  query heads before forward_mqa, so each shard holds every head]
 *   o_parts   : [G, B, H, R] contiguous, element type `dtype`, 16-byte aligned
 *   lse_parts : [G, B, H] contiguous fp32, natural log
 *   dtype     : MLA_F32 or MLA_BF16 (o_parts and o); accumulation is fp32
 *   o         : [B, H, R] contiguous, element type `dtype`, 16-byte aligned
 *   lse       : [B, H] contiguous fp32
 *   R         : 512 or 256
 * Errors: MLA_ERR_ARG (G < 1, B < 0, H < 1, a NULL pointer, misalignment),
 * MLA_ERR_UNSUPPORTED (R, dtype), MLA_ERR_HIP.  B == 0 launches nothing.
 */
int mla_merge_partials(const void* o_parts, const float* lse_parts, int G, int B, int H, int R, int dtype,
                       void* o, float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_AMD_MLA_H */
