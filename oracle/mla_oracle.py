"""CPU oracle for the paged latent-KV cache write and the MLA decode.

TEST INFRASTRUCTURE ONLY.  This module exists to check the HIP library.  Only
the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The product package never imports it, and the
product has no CPU fallback.  It imports nothing from the HIP path, and the HIP
path imports nothing from it.

Everything here is plain numpy.  Floating-point work is float64 unless the
method itself fixes a narrower step (the fp32 divide before fp8 encoding).

Array conventions (the same bit patterns the GPU sees):
  "f32"  -> numpy float32 values
  "bf16" -> numpy uint16 holding bfloat16 bit patterns
  "fp8"  -> numpy uint8 holding OCP FP8 E4M3 ("e4m3fn") codes

Sources, cited by page and section (no line numbers):
  [ESSAY] "Triton and MLA: portable attention and multi-head latent attention"
          (vLLM architecture notes, source version v0.25.1).
  [DIFF]  vLLM compare view whose commit is titled "fix TP" (MLA support for
          the V0 engine); the files it touches are named per citation.
  [API]   "vllm.v1.attention.backends.mla.triton_mla" API reference page.
  [OFP8]  OCP 8-bit Floating Point Specification (OFP8), E4M3 encoding.  The
          pages do not define the fp8 format; this is the published standard
          whose E4M3 flavour (largest finite value 448) matches a per-tensor
          scale of amax / 448.

Every function below is pinned by tests/test_oracle_*.py against closed forms,
brute force, library routines (torch's fp8 cast, torch SDPA and logsumexp in
float64) and invariances; none of those pins re-types a formula from here.
"""

from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

# ---------------------------------------------------------------------------
# Scalar formats
# ---------------------------------------------------------------------------

FP8_MAX = 448.0


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact).  A bfloat16 is the upper half
    of an IEEE binary32, so widening is a 16-bit shift."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f32_to_bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern, round-to-nearest-even on the 16 dropped
    bits (NaN kept quiet).  Used only to build expected bf16 outputs."""
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    r[nan] = np.uint16(0x7FC0) | ((u[nan] >> np.uint64(16)).astype(np.uint16) & np.uint16(0x8000))
    return r


def fp8_e4m3fn_decode_table() -> np.ndarray:
    """Value of each of the 256 E4M3 codes, from the format's definition [OFP8]:
    1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
    encodes subnormals m/8 * 2^(1-7); S.1111.111 is NaN; there is no infinity."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = math.nan
        elif e == 0:
            vals[code] = sign * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_FP8_TABLE = fp8_e4m3fn_decode_table()
# Non-negative finite codes 0x00..0x7E have strictly increasing values.
_FP8_POS = _FP8_TABLE[:0x7F].copy()


def fp8_e4m3fn_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes -> float64 values (exact)."""
    return _FP8_TABLE[np.asarray(codes, dtype=np.uint8)]


def fp8_e4m3fn_encode(x: np.ndarray) -> np.ndarray:
    """float32 -> E4M3 code by round-to-nearest, ties to the even code [OFP8].

    Finite magnitudes above the largest finite value 448 (and infinities)
    saturate to +-448: the pages name the conversion helper but do not show
    its body, and saturation is the reading taken here.  NaN maps to 0x7F with
    the input sign.  The sign bit is always kept, so tiny negatives become 0x80.

    Written as a nearest-neighbour search over the 127 non-negative finite
    values, which is the definition of rounding, not a bit trick.
    """
    x = np.asarray(x, dtype=np.float32)
    mag = np.abs(x.astype(np.float64))
    neg = np.signbit(x)
    out = np.empty(x.shape, dtype=np.uint8)

    nan = np.isnan(mag)
    sat = (~nan) & (mag >= FP8_MAX)
    reg = (~nan) & (~sat)

    m = mag[reg]
    hi = np.searchsorted(_FP8_POS, m, side="left")  # _FP8_POS[hi-1] < m <= _FP8_POS[hi]
    hi = np.clip(hi, 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = m - _FP8_POS[lo]
    d_hi = _FP8_POS[hi] - m
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(m == _FP8_POS[hi], hi, code)
    out[reg] = code.astype(np.uint8)
    out[sat] = 0x7E
    out[nan] = 0x7F
    out[neg] |= np.uint8(0x80)
    return out


def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Stored representation -> float64 values."""
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(arr)
    if dtype == "fp8":
        return fp8_e4m3fn_decode(arr)
    raise ValueError(dtype)


def to_f32_exact(arr: np.ndarray, dtype: str) -> np.ndarray:
    """f32/bf16 stored values -> float32 (exact widening)."""
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f64(arr).astype(np.float32)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# Cache write  [DIFF: csrc/cache_kernels.cu, concat_and_cache_mla_kernel and
#               its host launcher concat_and_cache_mla]
# ---------------------------------------------------------------------------

def cache_write(cache: np.ndarray, kv_c: np.ndarray, k_pe: np.ndarray,
                slot_mapping: np.ndarray, in_dtype: str, cache_dtype: str,
                scale: float | None = None) -> np.ndarray:
    """Return a copy of ``cache`` [num_blocks, block_size, R+P] after writing
    every token whose slot is non-negative.

    The token count is the length of slot_mapping (the kv_c/k_pe tensors may
    hold extra padded rows beyond it) [DIFF: host launcher].  Token t with slot
    s >= 0 lands in block s // block_size at offset s % block_size; columns
    [0, R) take kv_c[t] and [R, R+P) take k_pe[t].  Negative slots mark padded
    tokens and are skipped [DIFF: kernel].  With an fp8 cache each value is
    divided by the per-tensor scale in fp32 and encoded to E4M3.
    """
    out = np.array(cache, copy=True)
    nb, bs, D = out.shape
    R = kv_c.shape[1]
    P = k_pe.shape[1]
    if R + P != D:
        raise ValueError("cache row width must equal kv_lora_rank + rope_dim")
    T = len(slot_mapping)
    slots = np.asarray(slot_mapping, dtype=np.int64)[:T]
    tok = np.nonzero(slots >= 0)[0]
    blk = slots[tok] // bs
    off = slots[tok] % bs
    if cache_dtype == in_dtype:
        out[blk, off, :R] = kv_c[tok, :R]
        out[blk, off, R:] = k_pe[tok, :P]
    elif cache_dtype == "fp8":
        sc = np.float32(scale)
        out[blk, off, :R] = fp8_e4m3fn_encode(to_f32_exact(kv_c[tok, :R], in_dtype) / sc)
        out[blk, off, R:] = fp8_e4m3fn_encode(to_f32_exact(k_pe[tok, :P], in_dtype) / sc)
    else:
        raise ValueError("unsupported dtype pair")
    return out


# ---------------------------------------------------------------------------
# Rotary position embedding on the rope part, fused into the write
# [DIFF: MLA decode path, rotary_emb(input_positions, q_pe, k_pe) applied
#  before the cache write; DeepSeek-V2 attention, get_rope(...,
#  rope_type 'deepseek_yarn', is_neox_style=False)]
# ---------------------------------------------------------------------------

def rope_rotate_f32(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotary embedding in the non-NeoX form: element pairs (x[2i], x[2i+1])
    of the last axis (length P) are rotated by angle i, whose cosine and sine
    are cos[..., i] and sin[..., i] (P/2 each):
        x'[2i]   = x[2i] cos_i - x[2i+1] sin_i
        x'[2i+1] = x[2i+1] cos_i + x[2i] sin_i.
    The pages fix neither the precision nor the table; here the table is an
    input and the arithmetic is float32 with each product and each sum
    rounded to float32 (no fused multiply-add), the precision in which the
    stored value is then decided."""
    x = np.asarray(x, dtype=np.float32)
    c = np.asarray(cos, dtype=np.float32)
    s = np.asarray(sin, dtype=np.float32)
    a = x[..., 0::2]
    b = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = (a * c) - (b * s)
    out[..., 1::2] = (b * c) + (a * s)
    return out


def encode_f32(v: np.ndarray, dtype: str, scale: float | None = None) -> np.ndarray:
    """float32 values -> stored representation: fp32 as is, bf16 by
    round-to-nearest-even, fp8 as E4M3 of v / scale (fp32 divide)."""
    v = np.asarray(v, dtype=np.float32)
    if dtype == "f32":
        return v.copy()
    if dtype == "bf16":
        return f32_to_bf16_bits_rne(v)
    if dtype == "fp8":
        return fp8_e4m3fn_encode(v / np.float32(scale))
    raise ValueError(dtype)


def rope_table_rows(cos_sin_cache: np.ndarray, positions: np.ndarray, P: int):
    """cos and sin rows of a table laid out [max_position, P] as P/2 cosines
    followed by P/2 sines (the rotary module's cache layout)."""
    rows = np.asarray(cos_sin_cache, dtype=np.float32)[np.asarray(positions, dtype=np.int64)]
    return rows[..., :P // 2], rows[..., P // 2:P]


def cache_write_rope(cache: np.ndarray, kv_c: np.ndarray, k_pe: np.ndarray, positions: np.ndarray,
                     cos_sin_cache: np.ndarray, slot_mapping: np.ndarray, in_dtype: str, cache_dtype: str,
                     scale: float | None = None) -> np.ndarray:
    """``cache_write`` with the rotary embedding of each token's position
    applied to k_pe first: the kv_c columns are written as by ``cache_write``;
    the k_pe columns hold encode(rope_rotate_f32(k_pe, cos, sin)).  Tokens
    with a negative slot are skipped (their position is not read)."""
    out = cache_write(cache, kv_c, k_pe, slot_mapping, in_dtype, cache_dtype, scale)
    nb, bs, D = out.shape
    R = kv_c.shape[1]
    P = k_pe.shape[1]
    slots = np.asarray(slot_mapping, dtype=np.int64)
    tok = np.nonzero(slots >= 0)[0]
    c, s = rope_table_rows(cos_sin_cache, np.asarray(positions)[tok], P)
    rot = rope_rotate_f32(to_f32_exact(k_pe[tok, :P], in_dtype), c, s)
    out[slots[tok] // bs, slots[tok] % bs, R:] = encode_f32(rot, cache_dtype, scale)
    return out


def rope_q(q: np.ndarray, positions: np.ndarray, cos_sin_cache: np.ndarray, q_dtype: str,
           kv_lora_rank: int) -> np.ndarray:
    """q [N, H, R + P] with the rope part q[..., R:] of token n rotated by
    position positions[n] and stored back in q's dtype; the first R columns
    are unchanged."""
    out = np.array(q, copy=True)
    R = kv_lora_rank
    P = out.shape[-1] - R
    c, s = rope_table_rows(cos_sin_cache, positions, P)
    rot = rope_rotate_f32(to_f32_exact(out[..., R:], q_dtype), c[:, None, :], s[:, None, :])
    out[..., R:] = encode_f32(rot, q_dtype)
    return out


# ---------------------------------------------------------------------------
# Absorbed projections around the decode  [DIFF: MLACommonImpl docstring,
#  decode steps 3, 7 and 11 (weight absorption by associativity);
#  _q_proj_and_k_up_proj, _v_up_proj_and_o_proj and
#  process_weights_after_loading]
# ---------------------------------------------------------------------------

def linear(A: np.ndarray, W: np.ndarray, in_dtype: str = "bf16") -> np.ndarray:
    """C = A W^T in float64: A [M, K] and W [N, K] (a linear layer's weight,
    one row per output feature) in their stored representation."""
    return to_f64(A, in_dtype) @ to_f64(W, in_dtype).T


def absorb_q_weight(W_Q: np.ndarray, W_UK: np.ndarray) -> np.ndarray:
    """The q-side absorbed weight in linear-layer layout [N * Lkv, Lq]:
    row (n, l) is sum_p W_Q[:, n, p] W_UK[l, n, p], so that
    q_c W_Q_UK^T, viewed [B, N, Lkv], is q_nope after the k up-projection.
    W_Q [Lq, N, P] (the nope part of the q projection, input-major as the
    pages lay it out) and W_UK [Lkv, N, P], float64."""
    Lq, N, P = W_Q.shape
    Lkv = W_UK.shape[0]
    out = np.empty((N, Lkv, Lq))
    for n in range(N):
        out[n] = W_UK[:, n, :] @ W_Q[:, n, :].T
    return out.reshape(N * Lkv, Lq)


def absorb_o_weight(W_UV: np.ndarray, W_O: np.ndarray) -> np.ndarray:
    """The output-side absorbed weight in linear-layer layout [Hid, N * Lkv]:
    entry (h, (n, l)) is sum_v W_UV[l, n, v] W_O[h, n, v], so that the decode
    output [B, N, Lkv] flattened times its transpose is the o projection of
    the v up-projection.  W_UV [Lkv, N, V], W_O [Hid, N, V], float64."""
    Lkv, N, V = W_UV.shape
    Hid = W_O.shape[0]
    out = np.empty((Hid, N, Lkv))
    for n in range(N):
        out[:, n, :] = W_O[:, n, :] @ W_UV[:, n, :].T
    return out.reshape(Hid, N * Lkv)


def q_nope_unabsorbed(q_c: np.ndarray, W_Q: np.ndarray, W_UK: np.ndarray) -> np.ndarray:
    """q_nope [B, N, Lkv] the long way: x = q_c W_Q per head [B, N, P], then
    the k up-projection per head, q_nope[b, n, l] = sum_p x[b, n, p] W_UK[l, n, p]."""
    Lq, N, P = W_Q.shape
    x = (q_c @ W_Q.reshape(Lq, N * P)).reshape(-1, N, P)
    return np.einsum("bnp,lnp->bnl", x, W_UK)


def out_unabsorbed(o: np.ndarray, W_UV: np.ndarray, W_O: np.ndarray) -> np.ndarray:
    """Output projection the long way: v[b, n, :] = o[b, n, :] W_UV[:, n, :]
    per head, then out[b, h] = sum_{n, v} v[b, n, v] W_O[h, n, v]."""
    v = np.einsum("bnl,lnv->bnv", o, W_UV)
    return np.einsum("bnv,hnv->bh", v, W_O)


# ---------------------------------------------------------------------------
# Decode
# ---------------------------------------------------------------------------

def gather_rows(cache: np.ndarray, block_table_row: np.ndarray, n: int,
                cache_dtype: str, kv_scale: float | None = None) -> np.ndarray:
    """Logical rows 0..n-1 of one request as float64 [n, D].

    Token j lives in physical block block_table_row[j // block_size] at offset
    j % block_size [DIFF: vllm/attention/ops/triton_decode_attention.py,
    _fwd_grouped_kernel_stage1, page lookup].  fp8 codes are decoded exactly and
    multiplied by the per-tensor scale [ESSAY: Data flow, the k_scale/v_scale
    arguments]."""
    bs = cache.shape[1]
    j = np.arange(n)
    blocks = np.asarray(block_table_row, dtype=np.int64)[j // bs]
    rows = to_f64(cache[blocks, j % bs], cache_dtype).reshape(n, cache.shape[2])
    if cache_dtype == "fp8":
        rows *= float(np.float32(kv_scale))
    return rows


def attend(Q: np.ndarray, K: np.ndarray, R: int, sm_scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """MQA softmax attention of all heads against one shared latent row set.

    Q [H, D], K [n, D] (float64).  Each head scores every row over the full
    D = R+P width; the values are the first R columns of the same rows
    [ESSAY: Design motivation (single KV channel) and Data flow; DIFF:
    vllm/attention/backends/mla/utils.py, decode steps].  Returns o [H, R] and
    the natural-log LSE [H] of the scaled scores.  n == 0 gives o = 0 and
    lse = -inf (the pages would divide 0 by 0 there; this is the reading
    taken).
    """
    H = Q.shape[0]
    n = K.shape[0]
    if n == 0:
        return np.zeros((H, R)), np.full(H, -np.inf)
    s = sm_scale * (Q @ K.T)                      # [H, n]
    m = s.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
    p = np.exp(s - lse[:, None])
    o = p @ K[:, :R]
    return o, lse


def decode(q: np.ndarray, cache: np.ndarray, block_table: np.ndarray,
           seq_lens: np.ndarray, sm_scale: float, q_dtype: str, cache_dtype: str,
           kv_lora_rank: int, kv_scale: float | None = None) -> Tuple[np.ndarray, np.ndarray]:
    """Unsplit MLA decode for a batch: o [B, H, R] float64, lse [B, H] float64.

    This is what the split-KV two-stage pipeline computes, with the split and
    merge collapsed [DIFF: triton_decode_attention.py, stage 1 and stage 2;
    ESSAY: Data flow, forward_mqa returns (o, lse)]."""
    B, H, D = q.shape
    o = np.zeros((B, H, kv_lora_rank))
    lse = np.zeros((B, H))
    for b in range(B):
        n = int(seq_lens[b])
        K = gather_rows(cache, block_table[b], n, cache_dtype, kv_scale)
        Q = to_f64(q[b], q_dtype)
        o[b], lse[b] = attend(Q, K, kv_lora_rank, sm_scale)
    return o, lse


# ---------------------------------------------------------------------------
# Split-KV: partition, per-split partials, merge
# ---------------------------------------------------------------------------

def num_kv_splits(max_seq_len: int, num_cus: int, batch_invariant: bool = False) -> int:
    """Split count: one split per 512 tokens of the longest sequence, at most
    twice the compute-unit count; exactly one in batch-invariant mode
    [ESSAY: Key files, _compute_num_kv_splits; Data flow]."""
    if batch_invariant:
        return 1
    s = -(-int(max_seq_len) // 512)
    return max(1, min(s, 2 * int(num_cus)))


def split_bounds(n: int, num_splits: int) -> List[Tuple[int, int]]:
    """The pages' partition of one request: ceil(n / S) tokens per split,
    contiguous, empty splits dropped [DIFF: triton_decode_attention.py,
    stage 1 split range and the stage 2 skip of empty splits]."""
    kps = -(-n // num_splits) if n > 0 else 0
    out = []
    for s in range(num_splits):
        a = s * kps
        e = min(a + kps, n)
        if e > a:
            out.append((a, e))
    return out


def partials(Q: np.ndarray, K: np.ndarray, R: int, sm_scale: float,
             bounds: Sequence[Tuple[int, int]]) -> List[Tuple[np.ndarray, np.ndarray]]:
    """Per-split normalised partial output and partial LSE: attention of the
    heads against the split's rows alone [DIFF: stage 1 stores acc / e_sum and
    e_max + log(e_sum)]."""
    return [attend(Q, K[a:e], R, sm_scale) for (a, e) in bounds]


def merge(parts: Sequence[Tuple[np.ndarray, np.ndarray]]) -> Tuple[np.ndarray, np.ndarray]:
    """Combine split partials by their LSEs: weights exp(lse_s - M) with
    M = max_s lse_s; o = sum w_s o_s / sum w_s; lse = M + log(sum w_s)
    [DIFF: stage 2; ESSAY: Data flow (LogSumExp reduction)]."""
    if len(parts) == 0:
        raise ValueError("no non-empty splits")
    O = np.stack([p[0] for p in parts])          # [S, H, R]
    L = np.stack([p[1] for p in parts])          # [S, H]
    M = L.max(axis=0)
    w = np.exp(L - M)
    tot = w.sum(axis=0)
    o = (w[:, :, None] * O).sum(axis=0) / tot[:, None]
    return o, M + np.log(tot)


def decode_multi_token(q: np.ndarray, cache: np.ndarray, block_table: np.ndarray,
                       seq_lens: np.ndarray, sm_scale: float, q_dtype: str, cache_dtype: str,
                       kv_lora_rank: int, kv_scale: float | None = None) -> Tuple[np.ndarray, np.ndarray]:
    """Non-causal multi-token decode: q [B, T, H, D] holds T query tokens per
    request, each attending to all of the request's cached tokens.  As the
    pages do it, every query token becomes a decode row of its own that
    carries its request's block table and length [API:
    TritonMLAMetadataBuilder, non-causal multi-token decode]; then ``decode``.
    Returns o [B, T, H, R] and lse [B, T, H]."""
    B, T, H, D = q.shape
    rows = np.asarray(q).reshape(B * T, H, D)
    table = np.repeat(np.asarray(block_table), T, axis=0)
    lens = np.repeat(np.asarray(seq_lens), T)
    o, lse = decode(rows, cache, table, lens, sm_scale, q_dtype, cache_dtype, kv_lora_rank, kv_scale)
    return o.reshape(B, T, H, kv_lora_rank), lse.reshape(B, T, H)


def merge_shards(o_parts: np.ndarray, lse_parts: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Combine the results of G shards that attended to disjoint key sets of
    the same queries (decode context parallelism: each GPU holds part of a
    request's tokens and every head) [ESSAY: Design motivation (the LSE is
    returned for the cross-shard merge); API: DCP gathers all query heads].

    o_parts [G, B, H, R], lse_parts [G, B, H] (natural log).  Per (b, h) it is
    the same LSE-weighted mean as ``merge``; shards with lse = -inf hold no
    keys and get weight 0.  When every shard is empty the result is o = 0 and
    lse = -inf, the empty-request reading of ``attend``.
    """
    Op = np.asarray(o_parts, dtype=np.float64)
    L = np.asarray(lse_parts, dtype=np.float64)
    G, B, H = L.shape
    o = np.zeros(Op.shape[1:])
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        for h in range(H):
            live = [g for g in range(G) if L[g, b, h] != -np.inf]
            if live:
                ob, lb = merge([(Op[g, b, h][None], L[g, b, h][None]) for g in live])
                o[b, h], lse[b, h] = ob[0], lb[0]
    return o, lse


def decode_split_merge(q: np.ndarray, cache: np.ndarray, block_table: np.ndarray,
                       seq_lens: np.ndarray, sm_scale: float, q_dtype: str,
                       cache_dtype: str, kv_lora_rank: int, num_splits: int,
                       kv_scale: float | None = None) -> Tuple[np.ndarray, np.ndarray]:
    """The two-stage pipeline in float64 with the pages' partition."""
    B, H, D = q.shape
    o = np.zeros((B, H, kv_lora_rank))
    lse = np.zeros((B, H))
    for b in range(B):
        n = int(seq_lens[b])
        K = gather_rows(cache, block_table[b], n, cache_dtype, kv_scale)
        Q = to_f64(q[b], q_dtype)
        if n == 0:
            o[b], lse[b] = attend(Q, K, kv_lora_rank, sm_scale)
            continue
        o[b], lse[b] = merge(partials(Q, K, kv_lora_rank, sm_scale, split_bounds(n, num_splits)))
    return o, lse


def workspace_floats(B: int, H: int, num_splits: int, kv_lora_rank: int) -> int:
    """fp32 elements of the split workspace [B, H, S, R + 1]: the partial
    output followed by its LSE [ESSAY: Data flow, attn_logits shape;
    API: _reserve_attn_logits_workspace]."""
    return B * H * num_splits * (kv_lora_rank + 1)
