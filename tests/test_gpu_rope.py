"""Rotary embedding fused into the cache write, and the query's rope part
rotated in place: bit-exact against the oracle (both sides decide the stored
value from the same fp32 arithmetic), on every dtype pair, the element-wise
path for unaligned views, and end to end through the decode."""

import numpy as np
import pytest
import torch

import mla_paged_decode_concat_amd as M
from mla_paged_decode_concat_amd import workloads as W
from oracle import mla_oracle as O

from helpers import compare

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SM = W.SM_SCALE


def _print(*a):
    print(*a, flush=True)


def _oracle_rope_cache(bt, pos, tab):
    scale = float(bt.scale[0].cpu()) if bt.scale is not None else None
    return O.cache_write_rope(W.bits(bt.cache), W.bits(bt.kv_c), W.bits(bt.k_pe), pos.cpu().numpy(),
                              tab.cpu().numpy(), bt.slot_mapping.cpu().numpy(), bt.spec.in_dtype,
                              bt.spec.cache_dtype, scale)


def _same_bits(a, b):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


def _mode(bt):
    return "fp8" if bt.spec.cache_dtype == "fp8" else "auto"


@pytest.mark.parametrize("index,B,max_len", [(0, 2, None), (1, 6, 900), (3, 20, 600), (4, 4, 2000)])
def test_cache_write_rope_bit_exact(index, B, max_len):
    bt = W.make_batch(index, DEV, B=B, max_len=max_len) if index else W.make_batch(0, DEV)
    _print(f"[rope] write workload {index} lens={bt.seq_lens_list}")
    pos = W.token_positions(bt)
    tab = W.rope_table(max(bt.seq_lens_list) + 1, bt.spec.P).to(DEV)
    want = _oracle_rope_cache(bt, pos, tab)
    M.cache_write(bt.kv_c, bt.k_pe, bt.cache, bt.slot_mapping, _mode(bt), bt.scale, positions=pos, cos_sin_cache=tab)
    torch.cuda.synchronize()
    assert _same_bits(W.bits(bt.cache), want)


def test_cache_write_rope_unaligned_view():
    """Rows that are not 16-byte aligned take the element-wise kernel."""
    bt = W.make_batch(1, DEV, B=4, max_len=300)
    T = bt.kv_c.shape[0]
    pos = W.token_positions(bt)
    tab = W.rope_table(301, 64).to(DEV)
    want = _oracle_rope_cache(bt, pos, tab)
    odd = torch.zeros((T, 580), dtype=torch.bfloat16, device=DEV)
    odd[:, 1:513] = bt.kv_c
    odd[:, 513:577] = bt.k_pe
    M.cache_write(odd[:, 1:513], odd[:, 513:577], bt.cache, bt.slot_mapping, "auto", positions=pos,
                  cos_sin_cache=tab)
    torch.cuda.synchronize()
    assert _same_bits(W.bits(bt.cache), want)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_rope_q_bit_exact(dtype):
    g = torch.Generator(device=DEV).manual_seed(11)
    N, H = 37, 128
    q = torch.randn((N, H, 576), generator=g, device=DEV).to(dtype)
    pos = torch.randint(0, 4096, (N,), generator=g, device=DEV)
    tab = W.rope_table(4096, 64).to(DEV)
    want = O.rope_q(W.bits(q), pos.cpu().numpy(), tab.cpu().numpy(), "f32" if dtype == torch.float32 else "bf16",
                    512)
    M.rope_q(q, pos, tab, 512)
    torch.cuda.synchronize()
    assert _same_bits(W.bits(q), want)


def test_rope_q_multi_token_block():
    """A [B, q_len, H, D] query block with one position per token."""
    bt = W.make_batch(1, DEV, B=3, max_len=500)
    q = W.multi_token_q(bt, 4)
    pos = torch.arange(12, dtype=torch.int64, device=DEV) + 100
    tab = W.rope_table(200, 64).to(DEV)
    want = O.rope_q(W.bits(q).reshape(12, bt.H, 576), pos.cpu().numpy(), tab.cpu().numpy(), "bf16", 512)
    M.rope_q(q, pos, tab, 512)
    torch.cuda.synchronize()
    assert _same_bits(W.bits(q).reshape(12, bt.H, 576), want)


@pytest.mark.parametrize("index", [1, 4])
def test_roped_write_then_decode(index):
    """The decode step with RoPE: the cache written with rotated k_pe, the
    query's rope part rotated at each request's newest position, then the
    decode -- against the oracle's decode over its own rotated cache and q."""
    bt = W.make_batch(index, DEV, B=5, max_len=1500)
    pos = W.token_positions(bt)
    tab = W.rope_table(max(bt.seq_lens_list) + 1, 64).to(DEV)
    ref_cache = _oracle_rope_cache(bt, pos, tab)
    qpos = torch.tensor([max(n - 1, 0) for n in bt.seq_lens_list], dtype=torch.int64, device=DEV)
    ref_q = O.rope_q(W.bits(bt.q), qpos.cpu().numpy(), tab.cpu().numpy(), bt.spec.in_dtype, bt.spec.R)
    M.cache_write(bt.kv_c, bt.k_pe, bt.cache, bt.slot_mapping, _mode(bt), bt.scale, positions=pos, cos_sin_cache=tab)
    M.rope_q(bt.q, qpos, tab, bt.spec.R)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    o, lse = M.decode(bt.q, bt.cache, bt.block_table, bt.seq_lens, SM, M.num_kv_splits(max(bt.seq_lens_list), cus),
                      bt.spec.R, kv_scale=bt.scale)
    torch.cuda.synchronize()
    assert _same_bits(W.bits(bt.cache), ref_cache) and _same_bits(W.bits(bt.q), ref_q)
    scale = float(bt.scale[0].cpu()) if bt.scale is not None else None
    o_ref, lse_ref = O.decode(ref_q, ref_cache, bt.block_table.cpu().numpy(), bt.seq_lens.cpu().numpy(), SM,
                              bt.spec.in_dtype, bt.spec.cache_dtype, bt.spec.R, scale)
    compare(o, lse, o_ref, lse_ref, bt.spec.in_dtype)
