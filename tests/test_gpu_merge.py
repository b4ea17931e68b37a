"""Shard merge (decode context parallelism on one GPU's buffers): the merge of
G shard results against the oracle's merge, and end to end -- each request's
blocks dealt out over G shards, every shard decoded on its own, the shard
results merged -- against the oracle's decode over all of the tokens.
"""

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


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("G,B,H,R", [(1, 3, 16, 512), (3, 5, 128, 512), (8, 7, 5, 256), (70, 2, 3, 512)])
def test_merge_partials_against_oracle(dtype, G, B, H, R):
    _print(f"[merge] dtype={dtype} G={G} B={B} H={H} R={R}")
    gen = torch.Generator().manual_seed(G * 1000 + B)
    o_parts = torch.randn((G, B, H, R), generator=gen).to(dtype)
    lse_parts = torch.randn((G, B, H), generator=gen) * 4.0
    empty = torch.rand((G, B, H), generator=gen) < 0.3      # shards that hold no keys
    lse_parts[empty] = -torch.inf
    lse_parts[:, 0, 0] = -torch.inf                           # a (b, h) no shard holds keys for
    if G > 1:
        lse_parts[0, -1, -1] = 80.0                           # one shard dominates
    o_bits = W.bits(o_parts)
    o_ref, lse_ref = O.merge_shards(O.to_f64(o_bits, "f32" if dtype == torch.float32 else "bf16"),
                                    lse_parts.numpy())
    o, lse = M.merge_partials(o_parts.to(DEV), lse_parts.to(DEV))
    torch.cuda.synchronize()
    assert o.dtype == dtype and tuple(o.shape) == (B, H, R)
    compare(o, lse, o_ref, lse_ref, "f32" if dtype == torch.float32 else "bf16")
    assert torch.all(o[0, 0] == 0)


def _shard(bt, G, g):
    """Shard g's view of the cache when the logical blocks of every request
    are dealt round-robin over G shards: its block table (the blocks it owns,
    in order) and its token counts.  Only a request's last block can be
    partial, and it is the last block of the shard that owns it."""
    bs = bt.spec.block_size
    table = bt.block_table.cpu()
    lens = []
    rows = []
    for b, n in enumerate(bt.seq_lens_list):
        nblk = -(-n // bs)
        mine = list(range(g, nblk, G))
        lens.append(sum(min(bs, n - j * bs) for j in mine))
        rows.append([int(table[b, j]) for j in mine])
    width = max(1, max(len(r) for r in rows))
    t = torch.full((len(rows), width), bt.spare_block, dtype=torch.int32)
    for b, r in enumerate(rows):
        t[b, :len(r)] = torch.tensor(r, dtype=torch.int32)
    return t.to(DEV), torch.tensor(lens, dtype=torch.int32, device=DEV)


def _half_ulp(x):
    mag = np.maximum(np.abs(x), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(mag)) - 8)


def _oracle_shard(bt, ref_cache, table, seq):
    """The oracle's decode of one shard's tokens (its own table and lengths)."""
    scale = float(bt.scale[0].cpu()) if bt.scale is not None else None
    return O.decode(W.bits(bt.q), ref_cache, table.cpu().numpy(), seq.cpu().numpy(), SM, bt.spec.in_dtype,
                    bt.spec.cache_dtype, bt.spec.R, scale)


@pytest.mark.parametrize("index,G", [(0, 2), (2, 3), (2, 8), (4, 4)])
def test_decode_shards_then_merge(index, G):
    lens = {0: [300, 17, 0, 1000], 2: [3000, 64, 1, 700, 0, 2049], 4: [5000, 130, 65, 2500]}[index]
    bt = W.make_batch(index, DEV, seq_lens=lens)
    _print(f"[dcp] workload {index} G={G} lens={lens}")
    ref_cache = oracle_cache(bt)
    M.cache_write(bt.kv_c, bt.k_pe, bt.cache, bt.slot_mapping, "fp8" if bt.spec.cache_dtype == "fp8" else "auto",
                  bt.scale)
    o_ref, lse_ref = oracle_decode(bt, ref_cache, SM)
    o_parts, lse_parts = [], []
    shard_ref = []
    for g in range(G):
        table, seq = _shard(bt, G, g)
        S = M.num_kv_splits(int(seq.max()), torch.cuda.get_device_properties(0).multi_processor_count)
        o_g, lse_g = M.decode(bt.q, bt.cache, table, seq, SM, S, bt.spec.R, kv_scale=bt.scale)
        o_parts.append(o_g)
        lse_parts.append(lse_g)
        shard_ref.append(_oracle_shard(bt, ref_cache, table, seq))
    o, lse = M.merge_partials(torch.stack(o_parts), torch.stack(lse_parts))
    torch.cuda.synchronize()
    if bt.spec.in_dtype == "f32":
        compare(o, lse, o_ref, lse_ref, "f32")
        return
    # Each shard's output is stored in bf16 before the merge, as the decode
    # returns it; the merge carries that rounding (the LSE-weighted mean of
    # half a bf16 unit of every shard output) on top of the final output's.
    # The 1e-2 bar applies beyond both.
    og = o.float().cpu().numpy().astype(np.float64)
    lg = lse.cpu().numpy().astype(np.float64)
    Lg = np.stack([r[1] for r in shard_ref])
    Mx = np.max(Lg, axis=0)
    live = np.isfinite(Mx)
    w = np.where(np.isfinite(Lg), np.exp(Lg - np.where(live, Mx, 0.0)), 0.0)
    w = w / np.maximum(w.sum(axis=0), 1e-300)
    carried = sum(w[g][..., None] * _half_ulp(shard_ref[g][0]) for g in range(G))
    excess = np.abs(og - o_ref) - _half_ulp(o_ref) - carried
    assert np.array_equal(np.isfinite(lg), np.isfinite(lse_ref))
    fin = np.isfinite(lse_ref)
    assert np.max(np.abs(lg[fin] - lse_ref[fin])) <= 1e-3
    _print(f"[dcp] max excess over bf16 roundings {excess.max():.3g}, max carried {carried.max():.3g}")
    assert excess.max() <= 1e-2
