"""Thin ctypes binding over libmla_amd.so (include/mla.h).

Only argument marshalling lives here: tensor pointers, strides, dtypes and the
current HIP stream go to the C ABI; every step of the computation runs in the
library's kernels.  There is no CPU fallback: if the library is missing or
fails to load, calls raise.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))

MLA_F32, MLA_BF16, MLA_FP8_E4M3 = 0, 1, 2
STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported", -3: "workspace too small", -4: "HIP failure"}

EXPORTS = ["mla_status_string", "mla_num_kv_splits", "mla_decode_workspace_bytes", "mla_cache_write",
           "mla_decode", "mla_decode_ex", "mla_merge_partials", "mla_cache_write_rope", "mla_rope_q",
           "mla_linear_bf16", "mla_linear_workspace_bytes", "mla_decode_noalloc"]


class MLAError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status})")
        self.status = status


class DecodeOpts(ctypes.Structure):
    _fields_ = [("partition", ctypes.c_int), ("kernel", ctypes.c_int), ("grid", ctypes.c_int),
                ("heads_per_group", ctypes.c_int), ("stage_events", ctypes.c_void_p * 3),
                ("split_len", ctypes.c_int), ("piece_len", ctypes.c_int), ("reserved", ctypes.c_int * 2)]


_lib = None


def library_path() -> str:
    return os.path.join(HERE, "libmla_amd.so")


def load_library():
    """Load (once) and return the ctypes handle; raises if not built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path} is not built; run __graft_entry__.build() "
                                "or python -m mla_paged_decode_concat_amd.build")
    lib = ctypes.CDLL(path)
    vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_status_string.argtypes = [i32]
    lib.mla_num_kv_splits.restype = i32
    lib.mla_num_kv_splits.argtypes = [i64, i32, i32]
    lib.mla_decode_workspace_bytes.restype = sz
    lib.mla_decode_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.mla_cache_write.restype = i32
    lib.mla_cache_write.argtypes = [vp, i64, vp, i64, i32, vp, i64, vp, i32, i64, i32, i64, i32, i32, vp, vp]
    dec = [vp, i64, i64, i32, i32, i32, vp, i32, i64, i32, i64, i32, i32, vp, i64, i32, vp, f32, vp, i32,
           vp, sz, vp, vp, vp]
    lib.mla_decode.restype = i32
    lib.mla_decode.argtypes = dec
    lib.mla_decode_noalloc.restype = i32
    lib.mla_decode_noalloc.argtypes = dec[:20] + [vp, vp, vp]
    lib.mla_decode_ex.restype = i32
    lib.mla_decode_ex.argtypes = dec + [ctypes.POINTER(DecodeOpts)]
    lib.mla_cache_write_rope.restype = i32
    lib.mla_cache_write_rope.argtypes = [vp, i64, vp, i64, i32, vp, i64, vp, vp, i64, vp, i32, i64, i32, i64, i32,
                                         i32, vp, vp]
    lib.mla_rope_q.restype = i32
    lib.mla_rope_q.argtypes = [vp, i64, i64, i32, i64, i32, i32, i32, vp, vp, i64, vp]
    lib.mla_linear_workspace_bytes.restype = sz
    lib.mla_linear_workspace_bytes.argtypes = [i32, i32, i32]
    lib.mla_linear_bf16.restype = i32
    lib.mla_linear_bf16.argtypes = [vp, i64, vp, i64, i32, i32, i32, vp, i64, i32, vp, sz, vp]
    lib.mla_merge_partials.restype = i32
    lib.mla_merge_partials.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp]
    _lib = lib
    return lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MLA_F32
    if t.dtype == torch.bfloat16:
        return MLA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return MLA_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _same_gpu(*tensors: Optional[torch.Tensor]) -> None:
    """The library takes device pointers: every tensor must live on one GPU."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"tensor on {t.device}: the library takes GPU tensors only")
        if dev is not None and t.device != dev:
            raise ValueError(f"tensors on {dev} and {t.device}")
        dev = t.device


def _check(status: int, what: str) -> None:
    if status != 0:
        raise MLAError(status, what)


def num_kv_splits(max_seq_len: int, num_cus: Optional[int] = None, batch_invariant: bool = False) -> int:
    """Split count: ceil(max_seq_len / 512) clamped to [1, 2 * CUs]; 1 when batch-invariant."""
    if num_cus is None:
        num_cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    r = load_library().mla_num_kv_splits(int(max_seq_len), int(num_cus), int(bool(batch_invariant)))
    _check(r if r < 0 else 0, "mla_num_kv_splits")
    return r


def decode_workspace_bytes(B: int, H: int, num_kv_splits: int, kv_lora_rank: int) -> int:
    return int(load_library().mla_decode_workspace_bytes(B, H, num_kv_splits, kv_lora_rank))


def cache_write(kv_c: torch.Tensor, k_pe: torch.Tensor, kv_cache: torch.Tensor, slot_mapping: torch.Tensor,
                kv_cache_dtype: str = "auto", scale: Optional[torch.Tensor] = None,
                positions: Optional[torch.Tensor] = None, cos_sin_cache: Optional[torch.Tensor] = None) -> None:
    """Scatter kv_c [T', R] and k_pe [T', P] into kv_cache [num_blocks, block_size, R+P]
    at slot_mapping [T] (T <= T'; slot -1 = skip).  kv_cache_dtype "auto" stores
    the input dtype; "fp8"/"fp8_e4m3" encodes with the device fp32 scalar ``scale``.
    With ``positions`` (int64 [T]) and ``cos_sin_cache`` (fp32 [max_position, P]:
    cosines then sines) k_pe is rotated (interleaved pairs) before it is stored."""
    in_dt = _dtype_code(kv_c)
    cache_dt = _dtype_code(kv_cache)
    if kv_cache_dtype.startswith("fp8") != (cache_dt == MLA_FP8_E4M3):
        raise ValueError("kv_cache_dtype does not match the cache tensor's dtype")
    if k_pe.dtype != kv_c.dtype or slot_mapping.dtype != torch.int64:
        raise TypeError("k_pe must match kv_c's dtype and slot_mapping must be int64")
    if kv_c.stride(-1) != 1 or k_pe.stride(-1) != 1 or kv_cache.stride(-1) != 1 or kv_cache.stride(1) != kv_cache.shape[2]:
        raise ValueError("rows must be contiguous")
    if not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be contiguous")
    if k_pe.shape[0] != kv_c.shape[0] or slot_mapping.numel() > kv_c.shape[0]:
        raise ValueError("kv_c and k_pe need one row per slot_mapping entry")
    if kv_cache.dim() != 3 or kv_cache.shape[2] != kv_c.shape[1] + k_pe.shape[1]:
        raise ValueError("kv_cache must be [num_blocks, block_size, R + P]")
    if scale is not None and scale.numel() < 1:
        raise ValueError("scale must hold one fp32 value")
    _same_gpu(kv_c, k_pe, kv_cache, slot_mapping, scale, positions, cos_sin_cache)
    if (positions is None) != (cos_sin_cache is None):
        raise ValueError("positions and cos_sin_cache go together")
    lib = load_library()
    if positions is None:
        st = lib.mla_cache_write(
            kv_c.data_ptr(), kv_c.stride(0), k_pe.data_ptr(), k_pe.stride(0), in_dt,
            slot_mapping.data_ptr(), slot_mapping.numel(),
            kv_cache.data_ptr(), cache_dt, kv_cache.shape[0], kv_cache.shape[1], kv_cache.stride(0),
            kv_c.shape[1], k_pe.shape[1],
            scale.data_ptr() if scale is not None else None, _stream(kv_c.device))
        _check(st, "mla_cache_write")
        return
    _check_rope_args(positions, cos_sin_cache, slot_mapping.numel(), k_pe.shape[1])
    st = lib.mla_cache_write_rope(
        kv_c.data_ptr(), kv_c.stride(0), k_pe.data_ptr(), k_pe.stride(0), in_dt,
        slot_mapping.data_ptr(), slot_mapping.numel(), positions.data_ptr(), cos_sin_cache.data_ptr(),
        cos_sin_cache.shape[0],
        kv_cache.data_ptr(), cache_dt, kv_cache.shape[0], kv_cache.shape[1], kv_cache.stride(0),
        kv_c.shape[1], k_pe.shape[1],
        scale.data_ptr() if scale is not None else None, _stream(kv_c.device))
    _check(st, "mla_cache_write_rope")


def _check_rope_args(positions: torch.Tensor, cos_sin_cache: torch.Tensor, n: int, P: int) -> None:
    if positions.dtype != torch.int64 or not positions.is_contiguous() or positions.numel() < n:
        raise ValueError("positions must be contiguous int64 with one entry per token")
    if cos_sin_cache.dtype != torch.float32 or not cos_sin_cache.is_contiguous() or cos_sin_cache.dim() != 2 \
            or cos_sin_cache.shape[1] != P:
        raise ValueError("cos_sin_cache must be contiguous fp32 [max_position, rope_dim]")


def rope_q(q: torch.Tensor, positions: torch.Tensor, cos_sin_cache: torch.Tensor, kv_lora_rank: int = 512) -> torch.Tensor:
    """Rotate the rope part q[..., R:] of q [N, H, R+P] (or [B, q_len, H, R+P],
    one position per token) in place; returns q."""
    if q.dim() == 4:
        if q.stride(0) != q.shape[1] * q.stride(1):
            raise ValueError("a [B, q_len, H, D] query needs batch stride q_len * token stride")
        flat = torch.as_strided(q, (q.shape[0] * q.shape[1], q.shape[2], q.shape[3]),
                                (q.stride(1), q.stride(2), q.stride(3)))
        rope_q(flat, positions, cos_sin_cache, kv_lora_rank)
        return q
    N, H, D = q.shape
    if q.stride(-1) != 1:
        raise ValueError("rows must be contiguous")
    _check_rope_args(positions, cos_sin_cache, N, D - kv_lora_rank)
    _same_gpu(q, positions, cos_sin_cache)
    st = load_library().mla_rope_q(q.data_ptr(), q.stride(0), q.stride(1), _dtype_code(q), N, H, kv_lora_rank,
                                   D - kv_lora_rank, positions.data_ptr(), cos_sin_cache.data_ptr(),
                                   cos_sin_cache.shape[0], _stream(q.device))
    _check(st, "mla_rope_q")
    return q


def decode(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
           sm_scale: float, num_kv_splits: int, kv_lora_rank: int = 512,
           kv_scale: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
           o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
           partition: int = 0, kernel: int = 0, grid: int = 0, heads_per_group: int = 0,
           stage_events=None, split_len: int = 0, piece_len: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """MLA decode of q [B, H, R+P] against the paged latent cache.  Returns
    o [B, H, R] (q's dtype) and the natural-log lse [B, H] (fp32).

    q may also be [B, q_len, H, R+P]: q_len query tokens per request that all
    attend to the request's whole cached sequence (non-causal multi-token
    decode); they run as q_len * H rows of one request, and o and lse come
    back as [B, q_len, H, R] and [B, q_len, H].

    partition, kernel, grid, heads_per_group, split_len and piece_len are
    the mla_decode_opts_t controls of include/mla.h (0 = library default;
    partition 3 with piece_len > 0 cuts every request into fixed-length
    pieces, a batch-invariant split);
    stage_events are three events recorded around the two stages."""
    if isinstance(q, tuple):
        q = torch.cat(q, dim=-1)
    if q.dim() == 4:
        B, T, H, D = q.shape
        if q.stride(1) != H * q.stride(2):
            raise ValueError("a [B, q_len, H, D] query needs token stride H * head stride")
        flat = torch.as_strided(q, (B, T * H, D), (q.stride(0), q.stride(2), q.stride(3)))
        o_flat = o.view(B, T * H, -1) if o is not None else None
        lse_flat = lse.view(B, T * H) if lse is not None else None
        of, lf = decode(flat, kv_cache, block_table, seq_lens, sm_scale, num_kv_splits, kv_lora_rank, kv_scale,
                        workspace, o_flat, lse_flat, partition, kernel, grid, heads_per_group, stage_events,
                        split_len, piece_len)
        return of.view(B, T, H, -1), lf.view(B, T, H)
    B, H, D = q.shape
    R = kv_lora_rank
    P = D - R
    lib = load_library()
    o, lse = _decode_outputs(q, kv_cache, block_table, seq_lens, kv_scale, o, lse, R)
    need = lib.mla_decode_workspace_bytes(max(B, 1), H, num_kv_splits, R)
    if workspace is None:
        workspace = torch.empty((need + 3) // 4, dtype=torch.float32, device=q.device)
    _same_gpu(q, kv_cache, block_table, seq_lens, kv_scale, workspace, o, lse)
    opts = DecodeOpts(partition, kernel, grid, heads_per_group)
    opts.split_len = split_len
    opts.piece_len = piece_len
    if stage_events is not None:   # three torch.cuda.Event (or None) recorded around the two stages
        for i, ev in enumerate(stage_events):
            opts.stage_events[i] = ev.cuda_event if ev is not None else None
    st = lib.mla_decode_ex(
        q.data_ptr(), q.stride(0), q.stride(1), _dtype_code(q), B, H,
        kv_cache.data_ptr(), _dtype_code(kv_cache), kv_cache.shape[0], kv_cache.shape[1], kv_cache.stride(0),
        R, P, block_table.data_ptr(), block_table.stride(0), block_table.shape[1], seq_lens.data_ptr(),
        float(sm_scale), kv_scale.data_ptr() if kv_scale is not None else None, int(num_kv_splits),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), o.data_ptr(), lse.data_ptr(),
        _stream(q.device), ctypes.byref(opts))
    _check(st, "mla_decode")
    return o, lse


def decode_noalloc(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                   sm_scale: float, num_kv_splits: int, kv_lora_rank: int = 512,
                   kv_scale: Optional[torch.Tensor] = None, o: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """decode through mla_decode_noalloc: the split partials go to the
    library's per-GPU scratch array, so the library call allocates nothing
    (o and lse are allocated here only when not given).  q is [B, H, R+P]."""
    B, H, D = q.shape
    R = kv_lora_rank
    lib = load_library()
    o, lse = _decode_outputs(q, kv_cache, block_table, seq_lens, kv_scale, o, lse, R)
    _same_gpu(q, kv_cache, block_table, seq_lens, kv_scale, o, lse)
    st = lib.mla_decode_noalloc(
        q.data_ptr(), q.stride(0), q.stride(1), _dtype_code(q), B, H,
        kv_cache.data_ptr(), _dtype_code(kv_cache), kv_cache.shape[0], kv_cache.shape[1], kv_cache.stride(0),
        R, D - R, block_table.data_ptr(), block_table.stride(0), block_table.shape[1], seq_lens.data_ptr(),
        float(sm_scale), kv_scale.data_ptr() if kv_scale is not None else None, int(num_kv_splits),
        o.data_ptr(), lse.data_ptr(), _stream(q.device))
    _check(st, "mla_decode_noalloc")
    return o, lse


def _decode_outputs(q, kv_cache, block_table, seq_lens, kv_scale, o, lse, R):
    """Argument checks shared by the decode calls; returns (o, lse), new
    tensors where None was given."""
    B, H, D = q.shape
    if q.stride(-1) != 1 or kv_cache.stride(-1) != 1 or kv_cache.stride(1) != kv_cache.shape[2]:
        raise ValueError("rows must be contiguous")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous():
        raise TypeError("block_table and seq_lens must be int32 (seq_lens contiguous)")
    if block_table.stride(-1) != 1:
        raise ValueError("block_table rows must be contiguous")
    if seq_lens.numel() != B or block_table.dim() != 2 or block_table.shape[0] < B:
        raise ValueError("seq_lens must hold B entries and block_table B rows")
    if kv_cache.dim() != 3 or kv_cache.shape[2] != D:
        raise ValueError("kv_cache must be [num_blocks, block_size, R + P]")
    if kv_scale is not None and kv_scale.numel() < 1:
        raise ValueError("kv_scale must hold one fp32 value")
    if o is None:
        o = torch.empty((B, H, R), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    if not (o.is_contiguous() and lse.is_contiguous() and lse.dtype == torch.float32 and o.dtype == q.dtype):
        raise ValueError("o must be contiguous in q's dtype and lse contiguous fp32")
    if tuple(o.shape) != (B, H, R) or tuple(lse.shape) != (B, H):
        raise ValueError("o must be [B, H, R] and lse [B, H]")
    return o, lse


def merge_partials(o_parts: torch.Tensor, lse_parts: torch.Tensor, o: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Merge G shard results o_parts [G, B, H, R] (fp32 or bf16) with their
    natural-log LSEs lse_parts [G, B, H] into o [B, H, R] and lse [B, H]."""
    G, B, H, R = o_parts.shape
    if tuple(lse_parts.shape) != (G, B, H) or lse_parts.dtype != torch.float32:
        raise ValueError("lse_parts must be fp32 [G, B, H]")
    if not (o_parts.is_contiguous() and lse_parts.is_contiguous()):
        raise ValueError("o_parts and lse_parts must be contiguous")
    if o is None:
        o = torch.empty((B, H, R), dtype=o_parts.dtype, device=o_parts.device)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=o_parts.device)
    if not (o.is_contiguous() and lse.is_contiguous() and o.dtype == o_parts.dtype and lse.dtype == torch.float32):
        raise ValueError("o must be contiguous in o_parts' dtype and lse contiguous fp32")
    if tuple(o.shape) != (B, H, R) or tuple(lse.shape) != (B, H):
        raise ValueError("o must be [B, H, R] and lse [B, H]")
    _same_gpu(o_parts, lse_parts, o, lse)
    st = load_library().mla_merge_partials(o_parts.data_ptr(), lse_parts.data_ptr(), G, B, H, R,
                                           _dtype_code(o_parts), o.data_ptr(), lse.data_ptr(),
                                           _stream(o_parts.device))
    _check(st, "mla_merge_partials")
    return o, lse


def linear_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(load_library().mla_linear_workspace_bytes(M, N, K))


def linear(A: torch.Tensor, W: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = A W^T for bf16 A [M, K] and a bf16 weight W [N, K] (linear-layer
    layout), fp32 accumulation, C [M, N] in ``out_dtype`` (fp32 or bf16)."""
    M, K = A.shape
    N, K2 = W.shape
    if K2 != K or A.dtype != torch.bfloat16 or W.dtype != torch.bfloat16:
        raise ValueError("A [M, K] and W [N, K] must both be bf16")
    if A.stride(-1) != 1 or W.stride(-1) != 1:
        raise ValueError("rows must be contiguous")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=A.device)
    if tuple(out.shape) != (M, N) or out.stride(-1) != 1:
        raise ValueError("out must be [M, N] with contiguous rows")
    lib = load_library()
    need = lib.mla_linear_workspace_bytes(M, N, K)
    if need and workspace is None:
        workspace = torch.empty((need + 3) // 4, dtype=torch.float32, device=A.device)
    _same_gpu(A, W, out, workspace)
    st = lib.mla_linear_bf16(A.data_ptr(), A.stride(0), W.data_ptr(), W.stride(0), M, N, K, out.data_ptr(),
                             out.stride(0), _dtype_code(out), workspace.data_ptr() if workspace is not None else None,
                             workspace.numel() * 4 if workspace is not None else 0, _stream(A.device))
    _check(st, "mla_linear_bf16")
    return out
