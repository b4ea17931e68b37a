"""GPU parity: the HIP cache write is bit-exact with the oracle's and the HIP
decode is within tolerance of the oracle's fp64 decode, on every workload
(reduced sizes that the oracle finishes in seconds, spanning many tiles and
ragged tails), both stage-1 kernels, both partitions and several split
counts.  Calls go through the C ABI (ctypes binding)."""

import math

import numpy as np
import pytest
import torch

import mla_paged_decode_concat_amd as M
from mla_paged_decode_concat_amd import workloads as W
from oracle import mla_oracle as O

from helpers import compare, oracle_cache, oracle_decode

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SM = W.SM_SCALE


def _print(*a):
    print(*a, flush=True)


def gpu_write(bt: W.Batch):
    kv_dtype = "fp8" if bt.spec.cache_dtype == "fp8" else "auto"
    M.cache_write(bt.kv_c, bt.k_pe, bt.cache, bt.slot_mapping, kv_dtype, bt.scale)
    torch.cuda.synchronize()


def _cache_bytes(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.uint8).numpy()


def check_write(bt: W.Batch) -> np.ndarray:
    ref = oracle_cache(bt)
    gpu_write(bt)
    got = _cache_bytes(bt.cache)
    assert np.array_equal(got.reshape(-1), ref.view(np.uint8).reshape(-1)), "cache write differs from oracle"
    return ref


CASES = [
    # (workload, overrides)
    (0, {}),
    (1, dict(B=8, max_len=1500)),
    (2, dict(B=3)),
    (3, dict(B=16, max_len=3000)),
    (4, dict(B=4, max_len=5000)),
]


@pytest.mark.parametrize("index,kw", CASES)
def test_cache_write_bit_exact(index, kw):
    _print(f"[write] workload {index} {kw}")
    bt = W.make_batch(index, DEV, **kw)
    check_write(bt)


def _splits_for(bt):
    mx = max(bt.seq_lens_list)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    s = M.num_kv_splits(mx, cus)
    return sorted({1, 2, s, min(512, 3 * s + 1)})


@pytest.mark.parametrize("index,kw", CASES)
def test_decode_parity(index, kw):
    bt = W.make_batch(index, DEV, **kw)
    cache_ref = check_write(bt)
    o_ref, lse_ref = oracle_decode(bt, cache_ref, SM)
    kernels = [1] if bt.spec.in_dtype == "f32" else [1, 0]
    for S in _splits_for(bt):
        for partition in [1, 2]:
            for kernel in kernels:
                _print(f"[decode] workload {index} {kw} S={S} partition={partition} kernel={kernel}")
                o, lse = M.decode(bt.q, bt.cache, bt.block_table, bt.seq_lens, SM, S, bt.spec.R,
                                  kv_scale=bt.scale, partition=partition, kernel=kernel)
                torch.cuda.synchronize()
                eo, el = compare(o, lse, o_ref, lse_ref, bt.spec.in_dtype)
                _print(f"    max|do|={eo:.3e} max|dlse|={el:.3e}")


def test_tiny_f32_exact_pages_configuration():
    """The tiny fp32 workload at num_kv_splits 1 and 2 with the pages' own
    partition (ceil(n / S) tokens per split)."""
    bt = W.make_batch(0, DEV)
    cache_ref = check_write(bt)
    o_ref, lse_ref = oracle_decode(bt, cache_ref, SM)
    for S in [1, 2]:
        o, lse = M.decode(bt.q, bt.cache, bt.block_table, bt.seq_lens, SM, S, 512, partition=1)
        torch.cuda.synchronize()
        compare(o, lse, o_ref, lse_ref, "f32")
