"""Non-causal multi-token decode: q_len query tokens per request, every one
attending to the request's whole cached sequence, run as q_len * H rows of
one request (one KV read for all of them) and checked against the oracle,
which decodes each query token as a row of its own."""

import numpy as np
import pytest
import torch

import mla_paged_decode_concat_amd as M
from mla_paged_decode_concat_amd import workloads as W
from oracle import mla_oracle as O

from helpers import compare, oracle_cache

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SM = W.SM_SCALE


def _print(*a):
    print(*a, flush=True)


def _oracle(bt, ref_cache, q):
    scale = float(bt.scale[0].cpu()) if bt.scale is not None else None
    return O.decode_multi_token(W.bits(q), ref_cache, bt.block_table.cpu().numpy(), bt.seq_lens.cpu().numpy(),
                                SM, bt.spec.in_dtype, bt.spec.cache_dtype, bt.spec.R, scale)


CASES = [
    # (workload, q_len, seq_lens): bf16 H=16 (q_len*H = 32..128), V3 H=128
    # (several head groups per request), the fp8 cache, fp32 (vector ALU
    # kernel), kv_lora_rank 256
    (1, 2, [700, 1, 0, 4096, 65]),
    (1, 8, [3000, 129, 64]),
    (2, 2, [2500, 1, 900]),
    (2, 4, [1200, 333]),
    (4, 3, [4000, 70, 1025]),
    (0, 5, [37, 100, 0]),
    (3, 4, [600, 17, 2049]),
]


@pytest.mark.parametrize("index,q_len,lens", CASES)
def test_multi_token_rows_against_oracle(index, q_len, lens):
    bt = W.make_batch(index, DEV, seq_lens=lens)
    q = W.multi_token_q(bt, q_len)
    _print(f"[mtok] workload {index} q_len={q_len} H={bt.H} lens={lens}")
    ref_cache = oracle_cache(bt)
    M.cache_write(bt.kv_c, bt.k_pe, bt.cache, bt.slot_mapping, "fp8" if bt.spec.cache_dtype == "fp8" else "auto",
                  bt.scale)
    o_ref, lse_ref = _oracle(bt, ref_cache, q)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for S in sorted({1, 3, M.num_kv_splits(max(lens), cus)}):
        o, lse = M.decode(q, bt.cache, bt.block_table, bt.seq_lens, SM, S, bt.spec.R, kv_scale=bt.scale)
        torch.cuda.synchronize()
        assert tuple(o.shape) == (bt.B, q_len, bt.H, bt.spec.R) and tuple(lse.shape) == (bt.B, q_len, bt.H)
        err = compare(o, lse, o_ref, lse_ref, bt.spec.in_dtype)
        _print(f"[mtok] S={S} max |o err| {err[0]:.3g} max |lse err| {err[1]:.3g}")


def test_multi_token_strided_query_view():
    """A query block that is a view with padded rows (token stride = H * head
    stride, head stride > R+P) gives the same result as its contiguous copy."""
    bt = W.make_batch(1, DEV, seq_lens=[300, 1000])
    q_len, H, D = 4, bt.H, bt.spec.D
    big = W.multi_token_q(bt, q_len)
    store = torch.zeros((bt.B, q_len, H, D + 64), dtype=big.dtype, device=DEV)
    store[..., :D] = big
    view = store[..., :D]
    M.cache_write(bt.kv_c, bt.k_pe, bt.cache, bt.slot_mapping)
    o1, l1 = M.decode(view, bt.cache, bt.block_table, bt.seq_lens, SM, 2, bt.spec.R)
    o2, l2 = M.decode(big.contiguous(), bt.cache, bt.block_table, bt.seq_lens, SM, 2, bt.spec.R)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
