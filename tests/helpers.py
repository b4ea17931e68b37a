"""Shared test helpers: run the oracle on a workload batch and compare a GPU
result with it.  The oracle's inputs always come from the workload generator,
never from the HIP path."""

from __future__ import annotations

import numpy as np
import torch

from mla_paged_decode_concat_amd import workloads as W
from oracle import mla_oracle as O

# Tolerances: fp32 path max-abs 1e-5 on o and lse; bf16/fp8 inputs with fp32
# accumulation max-abs 1e-2 on o and 1e-3 on lse.
TOL = {"f32": (1e-5, 1e-5), "bf16": (1e-2, 1e-3)}


def check_slots(slot_mapping, num_blocks: int, block_size: int) -> None:
    """Debug validation pass of a cache write's slot mapping (tests only):
    every non-negative slot lies in [0, num_blocks * block_size) and none
    repeats.  The write gives each token its own wave with no ordering
    between them, so a repeated slot would leave whichever row lands last
    (the library states unique slots as a precondition and does not check
    device data)."""
    s = slot_mapping.cpu().numpy() if isinstance(slot_mapping, torch.Tensor) else np.asarray(slot_mapping)
    real = s[s >= 0]
    if real.size and int(real.max()) >= num_blocks * block_size:
        raise ValueError(f"slot {int(real.max())} out of range for {num_blocks} blocks of {block_size}")
    if np.unique(real).size != real.size:
        raise ValueError("repeated slot in slot_mapping")


def oracle_cache(bt: W.Batch) -> np.ndarray:
    scale = float(bt.scale[0].cpu()) if bt.scale is not None else None
    return O.cache_write(W.bits(bt.cache), W.bits(bt.kv_c), W.bits(bt.k_pe), bt.slot_mapping.cpu().numpy(),
                         bt.spec.in_dtype, bt.spec.cache_dtype, scale)


def oracle_decode(bt: W.Batch, cache: np.ndarray, sm_scale: float, requests=None):
    spec = bt.spec
    scale = float(bt.scale[0].cpu()) if bt.scale is not None else None
    q = W.bits(bt.q)
    table = bt.block_table.cpu().numpy()
    lens = bt.seq_lens.cpu().numpy()
    if requests is not None:
        q, table, lens = q[requests], table[requests], lens[requests]
    return O.decode(q, cache, table, lens, sm_scale, spec.in_dtype, spec.cache_dtype, spec.R, scale)


def logical_rows_f64(bt: W.Batch, b: int) -> np.ndarray:
    """Request b's token rows [n, R+P] from the generator's inputs, as the
    oracle write would store and the oracle gather would read them."""
    spec = bt.spec
    slots = bt.slot_mapping.cpu().numpy()
    valid = np.nonzero(slots >= 0)[0]
    start = sum(bt.seq_lens_list[:b])
    rows = valid[start:start + bt.seq_lens_list[b]]
    idx = torch.from_numpy(rows).to(bt.kv_c.device)
    kc = W.bits(bt.kv_c.index_select(0, idx))
    kp = W.bits(bt.k_pe.index_select(0, idx))
    if spec.cache_dtype == "fp8":
        sc = np.float32(bt.scale[0].cpu())
        enc = lambda x: O.fp8_e4m3fn_decode(O.fp8_e4m3fn_encode(O.to_f32_exact(x, spec.in_dtype) / sc)) * float(sc)
        return np.concatenate([enc(kc), enc(kp)], axis=1)
    return np.concatenate([O.to_f64(kc, spec.in_dtype), O.to_f64(kp, spec.in_dtype)], axis=1)


def oracle_decode_sampled(bt: W.Batch, sm_scale: float, requests):
    """Oracle o/lse for selected requests at full size, from the inputs."""
    spec = bt.spec
    q = W.bits(bt.q[torch.as_tensor(requests, device=bt.q.device)])
    o = np.zeros((len(requests), bt.H, spec.R))
    lse = np.zeros((len(requests), bt.H))
    for i, b in enumerate(requests):
        K = logical_rows_f64(bt, b)
        o[i], lse[i] = O.attend(O.to_f64(q[i], spec.in_dtype), K, spec.R, sm_scale)
    return o, lse


def margins(o_gpu: torch.Tensor, lse_gpu: torch.Tensor, o_ref: np.ndarray, lse_ref: np.ndarray, in_dtype: str):
    """Plain errors against the oracle: max |o - oracle|, max |o - oracle
    rounded to o's dtype| (bf16 outputs; the same as the first for fp32),
    max |lse - oracle| over finite LSEs, the largest error in excess of half
    a bf16 ulp of the exact value (bf16 outputs), and max |oracle o|."""
    og = o_gpu.detach().float().cpu().numpy().astype(np.float64)
    lg = lse_gpu.detach().cpu().numpy().astype(np.float64)
    fin = np.isfinite(lse_ref)
    err_l = float(np.max(np.abs(lg[fin] - lse_ref[fin]))) if fin.any() else 0.0
    err_o = float(np.max(np.abs(og - o_ref))) if og.size else 0.0
    err_or = err_o
    excess = err_o
    if in_dtype == "bf16" and og.size:
        ref_r = O.bf16_bits_to_f64(O.f32_to_bf16_bits_rne(o_ref.astype(np.float32)))
        err_or = float(np.max(np.abs(og - ref_r)))
        half_ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(o_ref), 2.0 ** -126))) - 8)
        excess = float(np.max(np.abs(og - o_ref) - half_ulp))
    return err_o, err_or, err_l, excess, float(np.max(np.abs(o_ref))) if og.size else 0.0


def compare(o_gpu: torch.Tensor, lse_gpu: torch.Tensor, o_ref: np.ndarray, lse_ref: np.ndarray, in_dtype: str):
    """Max-abs errors (o, lse) against the oracle.  fp32: max-abs <= 1e-5 on
    both.  bf16/fp8 inputs: lse max-abs <= 1e-3; o max-abs <= 1e-2 beyond the
    half bf16 ulp that rounding the stored bf16 output costs, and o within
    1e-2 (or one bf16 ulp) of the oracle rounded to bf16."""
    tol_o, tol_l = TOL["f32" if in_dtype == "f32" else "bf16"]
    og = o_gpu.detach().float().cpu().numpy().astype(np.float64)
    lg = lse_gpu.detach().cpu().numpy().astype(np.float64)
    assert og.shape == o_ref.shape and lg.shape == lse_ref.shape
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lg), fin), "lse finiteness differs"
    assert np.all(lg[~fin] == lse_ref[~fin])
    err_l = float(np.max(np.abs(lg[fin] - lse_ref[fin]))) if fin.any() else 0.0
    assert np.all(np.isfinite(og)), "non-finite o"
    err_o = float(np.max(np.abs(og - o_ref))) if og.size else 0.0
    if in_dtype == "bf16":
        # o is stored in bf16: no bf16 result can be closer to the oracle than
        # half a bf16 unit in the last place, so the bar applies to the error
        # in excess of that (it is what the 1e-2 bound can mean for a bf16
        # output; elements with |o| < 2 see at most 2^-9 of it).
        mag = np.maximum(np.abs(o_ref), 2.0 ** -126)
        half_ulp = np.exp2(np.floor(np.log2(mag)) - 8)
        excess = float(np.max(np.abs(og - o_ref) - half_ulp)) if og.size else 0.0
        assert excess <= tol_o, f"o vs oracle beyond bf16 output rounding {excess}"
        # and against the oracle rounded to bf16: within the bar, or one bf16
        # ulp where the exact value lies next to a rounding boundary (above
        # |o| = 2 the bf16 grid is coarser than 1e-2, so an fp32 result a hair
        # across the boundary rounds to the neighbouring grid point)
        ref_r = O.bf16_bits_to_f64(O.f32_to_bf16_bits_rne(o_ref.astype(np.float32)))
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref_r), 2.0 ** -126))) - 7)
        bad = np.abs(og - ref_r) > np.maximum(tol_o, ulp)
        assert not bad.any(), f"o vs the oracle rounded to bf16: {float(np.max(np.abs(og - ref_r)))}"
    else:
        assert err_o <= tol_o, f"o vs oracle {err_o}"
    assert err_l <= tol_l, f"lse vs oracle {err_l}"
    return err_o, err_l
