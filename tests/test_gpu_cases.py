"""GPU edge cases and invariances, each against the oracle (or bit-exact
against another GPU run where the property is exact):

* every stage-1 kernel configuration (heads per workgroup 16/32/64/128),
  both partitions, several grids, for a bf16 and an fp8 cache;
* a late token whose score jumps far above the earlier maximum (the decode
  must redo the range with a larger softmax reference);
* block sizes 1, 16, 48, 64 (1 exceeds the staged block-table window);
* empty and single-token requests, head counts that are not multiples of 16;
* strided kv_c/k_pe views (the projection-output layout) and an unaligned view;
* NaN in every unwritten cache slot never reaching o or lse;
* bit-exact invariance to the physical block permutation (same split count)
  and batch invariance with num_kv_splits = 1.
"""

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


def _write(bt):
    M.cache_write(bt.kv_c, bt.k_pe, bt.cache, bt.slot_mapping, "fp8" if bt.spec.cache_dtype == "fp8" else "auto",
                  bt.scale)
    torch.cuda.synchronize()


def _decode(bt, S, **kw):
    o, lse = M.decode(bt.q, bt.cache, bt.block_table, bt.seq_lens, SM, S, bt.spec.R, kv_scale=bt.scale, **kw)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("hpg", [16, 32, 64, 128])
@pytest.mark.parametrize("partition", [1, 2])
def test_mfma_head_groups_v3_shape(hpg, partition):
    bt = W.make_batch(2, DEV, B=2, seq_lens=[1000, 777])
    ref_cache = oracle_cache(bt)
    _write(bt)
    o_ref, lse_ref = oracle_decode(bt, ref_cache, SM)
    for S in [1, 3, 16]:
        _print(f"[mfma] hpg={hpg} partition={partition} S={S}")
        o, lse = _decode(bt, S, kernel=2, heads_per_group=hpg, partition=partition)
        compare(o, lse, o_ref, lse_ref, "bf16")


@pytest.mark.parametrize("hpg", [16, 32, 64, 128])
@pytest.mark.parametrize("partition", [1, 2])
def test_mfma_head_groups_fp8_cache(hpg, partition):
    """The matrix-core path with an fp8 cache (tiles converted to bf16 in LDS)."""
    bt = W.make_batch(4, DEV, B=3, seq_lens=[1000, 777, 33])
    ref_cache = oracle_cache(bt)
    _write(bt)
    assert np.array_equal(bt.cache.cpu().numpy(), ref_cache)
    o_ref, lse_ref = oracle_decode(bt, ref_cache, SM)
    for S in [1, 3, 16]:
        _print(f"[mfma fp8] hpg={hpg} partition={partition} S={S}")
        o, lse = _decode(bt, S, kernel=2, heads_per_group=hpg, partition=partition)
        compare(o, lse, o_ref, lse_ref, "bf16")


@pytest.mark.parametrize("grid", [1, 7, 64, 1000])
def test_balanced_grid_sizes(grid):
    bt = W.make_batch(1, DEV, B=9, max_len=2500)
    ref_cache = oracle_cache(bt)
    _write(bt)
    o_ref, lse_ref = oracle_decode(bt, ref_cache, SM)
    for S in [2, 5, 8]:
        _print(f"[grid] G={grid} S={S}")
        for kernel in [1, 2]:
            o, lse = _decode(bt, S, kernel=kernel, partition=2, grid=grid)
            compare(o, lse, o_ref, lse_ref, "bf16")


@pytest.mark.parametrize("index", [2, 4])
def test_late_dominant_token_forces_redo(index):
    """Scores of the last tokens sit far above every earlier score: the
    decode's softmax reference set on the first tile cannot represent them,
    so the range is redone; results still match the oracle (bf16 cache:
    every stage-1 shape; fp8 cache: 32- and 128-head groups)."""
    bt = W.make_batch(index, DEV, B=2, seq_lens=[700, 1500])
    # q and the rows' rope part aligned on a few late tokens: score ~ +200
    with torch.no_grad():
        n0 = bt.seq_lens_list[0]
        rows = bt.last_token_rows  # last token of each request
        for b in range(2):
            r = int(rows[b])
            for back in [0, 5, 33]:          # three late tokens per request
                bt.k_pe[r - back] = 0
                bt.k_pe[r - back, :16] = 4.0
        bt.q[:, :, 512:] = 0
        bt.q[:, :, 512:528] = 4.0            # 16 * 4 * 4 = 256 raw -> ~18 after sm_scale
        bt.q[:, :, 512:528] *= 12.0          # -> raw 3072, score ~ 222 (natural units)
    ref_cache = oracle_cache(bt)
    _write(bt)
    o_ref, lse_ref = oracle_decode(bt, ref_cache, SM)
    assert np.all(lse_ref > 150)
    shapes = [(32, 2), (128, 2), (16, 3), (32, 3)] if index == 2 else [(32, 2), (128, 2)]
    for hpg, kernel in shapes:
        for S in [1, 4]:
            _print(f"[redo] workload {index} hpg={hpg} kernel={kernel} S={S}")
            o, lse = _decode(bt, S, kernel=kernel, heads_per_group=hpg)
            compare(o, lse, o_ref, lse_ref, bt.spec.in_dtype)


@pytest.mark.parametrize("bs,H", [(1, 32), (16, 32), (48, 32), (64, 32), (16, 128), (48, 128)])
@pytest.mark.parametrize("index", [1, 4])
def test_block_sizes(bs, H, index):
    spec = W.SPECS[index]
    lens = [1, 31, 33, 1500, 2049]
    bt = W.make_batch(index, DEV, seq_lens=lens, H=H)
    # rebuild the paging with block size bs over the same token rows
    nblk = [-(-n // bs) for n in lens]
    g = torch.Generator().manual_seed(bs)
    perm = torch.randperm(sum(nblk) + 1, generator=g)
    table = torch.full((len(lens), max(nblk)), int(perm[-1]), dtype=torch.int32)
    slots, off = [], 0
    for b, n in enumerate(lens):
        ids = perm[off:off + nblk[b]]
        off += nblk[b]
        table[b, :nblk[b]] = ids.to(torch.int32)
        j = torch.arange(n)
        slots.append(ids[j // bs] * bs + j % bs)
    bt.block_table = table.to(DEV)
    bt.slot_mapping = torch.cat(slots).to(DEV)
    if spec.cache_dtype == "fp8":
        bt.cache = torch.full((sum(nblk) + 1, bs, spec.D), W.NAN_FP8, dtype=torch.uint8, device=DEV)
    else:
        bt.cache = torch.full((sum(nblk) + 1, bs, spec.D), W.NAN_BF16, dtype=torch.int16,
                              device=DEV).view(torch.bfloat16)
    scale = float(bt.scale[0].cpu()) if bt.scale is not None else None
    ref_cache = O.cache_write(W.bits(bt.cache), W.bits(bt.kv_c), W.bits(bt.k_pe), bt.slot_mapping.cpu().numpy(),
                              "bf16", spec.cache_dtype, scale)
    _write(bt)
    assert np.array_equal(W.bits(bt.cache), ref_cache)
    o_ref, lse_ref = oracle_decode(bt, ref_cache, SM)
    # the token-split kernels (bf16 cache only) with 16- and 32-head groups;
    # block size 1 stages the table of a 2049-token request in three windows.
    # At 128 heads: the two-role kernels (128-head groups), whose tile
    # addresses take the division path for block size 48 and the shift for 16
    if H == 128:
        runs = [(2, 128)]
    else:
        runs = [(1, 0), (2, 0)] + ([(3, 16), (3, 32)] if spec.cache_dtype == "bf16" else [])
    for S in [1, 4]:
        for kernel, hpg in runs:
            for partition in [1, 2]:
                _print(f"[bs] bs={bs} S={S} kernel={kernel} hpg={hpg} partition={partition}")
                o, lse = _decode(bt, S, kernel=kernel, heads_per_group=hpg, partition=partition)
                compare(o, lse, o_ref, lse_ref, "bf16")


def test_empty_and_single_token_requests():
    bt = W.make_batch(2, DEV, seq_lens=[0, 1, 0, 65, 1])
    ref_cache = oracle_cache(bt)
    _write(bt)
    o_ref, lse_ref = oracle_decode(bt, ref_cache, SM)
    assert np.isneginf(lse_ref[0]).all() and np.isneginf(lse_ref[2]).all()
    for S in [1, 2, 7]:
        for kernel in [1, 2]:
            for partition in [1, 2]:
                o, lse = _decode(bt, S, kernel=kernel, partition=partition)
                compare(o, lse, o_ref, lse_ref, "bf16")
                assert torch.all(o[0] == 0) and torch.all(o[2] == 0)


@pytest.mark.parametrize("H", [1, 5, 24, 40, 48])
def test_head_counts_not_multiple_of_16(H):
    bt = W.make_batch(1, DEV, B=3, max_len=300, H=H)
    ref_cache = oracle_cache(bt)
    _write(bt)
    o_ref, lse_ref = oracle_decode(bt, ref_cache, SM)
    for S in [1, 3]:
        o, lse = _decode(bt, S)            # auto picks a kernel that supports H
        compare(o, lse, o_ref, lse_ref, "bf16")


def test_strided_inputs_and_unaligned_view():
    """kv_c and k_pe as column slices of one [T, 576] projection output, and
    a view whose rows are not 16-byte aligned (element-wise write path)."""
    bt = W.make_batch(1, DEV, B=4, max_len=200)
    T = bt.kv_c.shape[0]
    big = torch.cat([bt.kv_c, bt.k_pe], dim=1).contiguous()
    ref_cache = oracle_cache(bt)
    M.cache_write(big[:, :512], big[:, 512:], bt.cache, bt.slot_mapping, "auto")
    torch.cuda.synchronize()
    assert np.array_equal(bt.cache.cpu().view(torch.int16).numpy().view(np.uint16), ref_cache)
    odd = torch.zeros((T, 577 + 3), dtype=torch.bfloat16, device=DEV)
    odd[:, 1:513] = bt.kv_c
    odd[:, 513:577] = bt.k_pe
    bt.cache.view(torch.int16).fill_(W.NAN_BF16)
    M.cache_write(odd[:, 1:513], odd[:, 513:577], bt.cache, bt.slot_mapping, "auto")
    torch.cuda.synchronize()
    assert np.array_equal(bt.cache.cpu().view(torch.int16).numpy().view(np.uint16), ref_cache)


def test_nan_poison_never_leaks():
    """Unwritten slots (tails of last pages, the spare block used as table
    padding) hold NaN; outputs stay finite and match the oracle."""
    bt = W.make_batch(3, DEV, B=12, max_len=700)      # block 16, ragged tails, 10% pad rows
    ref_cache = oracle_cache(bt)
    _write(bt)
    c = bt.cache.float()
    assert torch.isnan(c).any()                       # poison is present
    o_ref, lse_ref = oracle_decode(bt, ref_cache, SM)
    for S in [1, 5]:
        o, lse = _decode(bt, S)
        assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
        compare(o, lse, o_ref, lse_ref, "bf16")


def test_block_permutation_invariance_bit_exact():
    """The same logical sequences under two different physical block
    assignments decode to identical bits (same num_kv_splits)."""
    a = W.make_batch(2, DEV, B=3, seq_lens=[800, 1500, 64], seed=5)
    b = W.make_batch(2, DEV, B=3, seq_lens=[800, 1500, 64], seed=5)
    # re-assign b's physical blocks with another permutation
    g = torch.Generator().manual_seed(99)
    perm = torch.randperm(b.num_blocks, generator=g).to(DEV)
    old_table = b.block_table.long()
    b.block_table = perm[old_table].to(torch.int32)
    bsz = b.spec.block_size
    b.slot_mapping = perm[b.slot_mapping // bsz] * bsz + b.slot_mapping % bsz
    _write(a)
    _write(b)
    for S in [1, 4, 16]:
        for kernel in [1, 2]:
            oa, la = _decode(a, S, kernel=kernel)
            ob, lb = _decode(b, S, kernel=kernel)
            assert torch.equal(oa, ob) and torch.equal(la, lb)


def _alone(bt, b):
    """Request b of the batch decoded as a batch of one (num_kv_splits = 1)."""
    o1, l1 = M.decode(bt.q[b:b + 1].contiguous(), bt.cache, bt.block_table[b:b + 1].contiguous(),
                      bt.seq_lens[b:b + 1].contiguous(), SM, 1, bt.spec.R, kv_scale=bt.scale)
    torch.cuda.synchronize()
    return o1[0], l1[0]


# 16 heads; 128 heads with requests on both sides of the default token-split
# threshold; 32 heads of 320-wide rows; 128 heads on an fp8 cache
INVARIANCE_CASES = [(1, dict(B=6, max_len=3000)), (2, dict(seq_lens=[5000, 4096, 17, 9000, 300, 4095])),
                    (3, dict(B=6, max_len=6000)), (4, dict(B=6, max_len=6000))]


@pytest.mark.parametrize("index,kw", INVARIANCE_CASES)
def test_batch_invariance_single_split(index, kw):
    """num_kv_splits = 1: a request decodes to the same bits alone and inside
    a batch, and the batch matches the oracle."""
    full = W.make_batch(index, DEV, **kw)
    _write(full)
    o, lse = _decode(full, 1)
    o_ref, lse_ref = oracle_decode(full, oracle_cache(full), SM)
    compare(o, lse, o_ref, lse_ref, full.spec.in_dtype)
    for b in [0, 1, 3, 5]:
        o1, l1 = _alone(full, b)
        assert torch.equal(o1, o[b]) and torch.equal(l1, lse[b]), b


@pytest.mark.parametrize("index,H", [(1, 16), (4, 128)])
def test_batch_invariance_single_split_large_batch(index, H):
    """num_kv_splits = 1 with more requests than compute units: the stage-1
    kernel choice (head grouping) must not depend on the batch size, so a
    request decodes to the same bits alone and inside a batch of 300
    (16 heads on a bf16 cache; 128 heads on an fp8 cache, where a batch of
    300 takes 128-head groups and a batch of one 16-head groups)."""
    full = W.make_batch(index, DEV, seq_lens=[(37 * i) % 400 + 1 for i in range(300)], H=H)
    _write(full)
    o, lse = _decode(full, 1)
    for b in [0, 7, 150, 299]:
        o1, l1 = _alone(full, b)
        assert torch.equal(o1, o[b]) and torch.equal(l1, lse[b]), b


def test_fp8_write_every_bf16_pattern():
    """All 65536 bf16 bit patterns through the fp8 write, compared with the
    oracle's encoder (covers subnormals, ties, saturation and NaN)."""
    pats = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    T = 65536 // 512
    kv_c = pats.reshape(T, 512).to(DEV)
    k_pe = pats[:T * 64].reshape(T, 64).to(DEV)
    cache = torch.full((T, 1, 576), 0x7F, dtype=torch.uint8, device=DEV)
    slots = torch.arange(T, dtype=torch.int64, device=DEV)
    for sc in [1.0, 9.5 / 448.0, 0.0213, 3.7, 1e-30]:
        scale = torch.tensor([sc], dtype=torch.float32, device=DEV)
        M.cache_write(kv_c, k_pe, cache, slots, "fp8", scale)
        torch.cuda.synchronize()
        ref = O.cache_write(np.full((T, 1, 576), 0x7F, np.uint8), W.bits(kv_c), W.bits(k_pe), slots.cpu().numpy(),
                            "bf16", "fp8", float(np.float32(sc)))
        assert np.array_equal(cache.cpu().numpy(), ref), sc


@pytest.mark.parametrize("lens,S,grid", [([5000, 1, 1], 2, 0), ([3000, 40, 0, 900], 3, 0), ([4096] + [7] * 31, 8, 0),
                                         ([700, 2000], 2, 1000)])
def test_long_request_takes_free_partial_slots(lens, S, grid):
    """Balanced partition: the workspace's B*S partial slots are one pool, so
    a long request next to short ones is cut into more than S pieces (the
    host caps the chunk count at B*(S-1), also for an explicit grid)."""
    bt = W.make_batch(2, DEV, seq_lens=lens)
    ref_cache = oracle_cache(bt)
    _write(bt)
    o_ref, lse_ref = oracle_decode(bt, ref_cache, SM)
    for kernel in [1, 2]:
        o, lse = _decode(bt, S, kernel=kernel, partition=2, grid=grid)
        compare(o, lse, o_ref, lse_ref, "bf16")


@pytest.mark.parametrize("index", [2, 4])
def test_single_split_result_independent_of_head_grouping(index):
    """With num_kv_splits = 1 the library picks smaller head groups for small
    batches; every head's result must not depend on the grouping, so a
    request decodes to the same bits in any batch (bf16 and fp8 caches)."""
    bt = W.make_batch(index, DEV, seq_lens=[3000, 17, 900], seed=11)
    _write(bt)
    outs = [_decode(bt, 1, kernel=2, heads_per_group=hpg) for hpg in [128, 64, 32, 16]]
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])



@pytest.mark.parametrize("hpg", [16, 32])
@pytest.mark.parametrize("index", [1, 3])
def test_token_split_kernel(index, hpg):
    """Four waves splitting each token range of a 16- or 32-head group
    (kernel 3): ragged, empty, one-token and long requests, both partitions,
    several split counts, one or two head groups, against the oracle."""
    lens = [0, 1, 31, 33, 700, 2500, 129, 5000]
    bt = W.make_batch(index, DEV, seq_lens=lens, H=32)    # block 64 (R=512) and block 16 (R=256)
    ref_cache = oracle_cache(bt)
    _write(bt)
    o_ref, lse_ref = oracle_decode(bt, ref_cache, SM)
    for S in [1, 3, 9]:
        for partition in [1, 2]:
            _print(f"[ts] workload {index} hpg={hpg} S={S} partition={partition}")
            o, lse = _decode(bt, S, kernel=3, heads_per_group=hpg, partition=partition)
            compare(o, lse, o_ref, lse_ref, "bf16")


def test_token_split_rejects_what_it_cannot_run():
    bt = W.make_batch(4, DEV, B=2, max_len=300, H=16)     # fp8 cache
    with pytest.raises(M.MLAError):
        M.decode(bt.q, bt.cache, bt.block_table, bt.seq_lens, SM, 2, 512, kv_scale=bt.scale, kernel=3)
    bt = W.make_batch(1, DEV, B=2, max_len=300, H=64)
    with pytest.raises(M.MLAError):
        M.decode(bt.q, bt.cache, bt.block_table, bt.seq_lens, SM, 2, 512, kernel=3, heads_per_group=64)
    bt = W.make_batch(1, DEV, B=2, max_len=300, H=48)
    with pytest.raises(M.MLAError):
        M.decode(bt.q, bt.cache, bt.block_table, bt.seq_lens, SM, 2, 512, kernel=3, heads_per_group=32)


@pytest.mark.parametrize("index,H,split_len", [(2, 128, 4096), (2, 128, 600), (2, 64, 600), (3, 32, 600)])
def test_single_split_length_classes(index, H, split_len):
    """num_kv_splits = 1 with a length threshold (128 or 64 heads of
    576-wide rows, 32 heads of 320-wide rows): requests of at least
    split_len tokens take the 32-head token-split kernel and the others the
    shared-tile kernel, in two launches over the same batch.  Results match
    the oracle, and a request decodes to the same bits alone and inside the
    batch, on both sides of the threshold."""
    lens = [4500, 599, 600, 1, 0, 4096, 4095, 1300]
    bt = W.make_batch(index, DEV, seq_lens=lens, seed=21, H=H)
    R = bt.spec.R
    ref_cache = oracle_cache(bt)
    _write(bt)
    o_ref, lse_ref = oracle_decode(bt, ref_cache, SM)
    o, lse = _decode(bt, 1, split_len=split_len)
    compare(o, lse, o_ref, lse_ref, "bf16")
    for b in range(len(lens)):
        o1, l1 = M.decode(bt.q[b:b + 1].contiguous(), bt.cache, bt.block_table[b:b + 1].contiguous(),
                          bt.seq_lens[b:b + 1].contiguous(), SM, 1, R, split_len=split_len)
        torch.cuda.synchronize()
        assert torch.equal(o1[0], o[b]) and torch.equal(l1[0], lse[b]), b
    # with the threshold off every request takes the shared-tile kernel, which
    # differs from the token-split one only in rounding
    o2, l2 = _decode(bt, 1, split_len=-1)
    compare(o2, l2, o_ref, lse_ref, "bf16")
    assert torch.equal(o2[1], o[1]) and torch.equal(l2[1], lse[1])   # 599 tokens: shared-tile either way


@pytest.mark.parametrize("index,H", [(2, 128), (3, 32)])
def test_single_split_default_threshold(index, H):
    """num_kv_splits = 1 with split_len left at 0 is the library's threshold
    of 4096 tokens: bit for bit the explicit split_len = 4096 run, for a
    batch with requests on both sides of it (also through the plain entry
    point, which takes every default)."""
    lens = [4500, 4096, 4095, 1, 0, 9000, 300]
    bt = W.make_batch(index, DEV, seq_lens=lens, seed=23, H=H)
    R = bt.spec.R
    _write(bt)
    o_ref, lse_ref = oracle_decode(bt, oracle_cache(bt), SM)
    o, lse = _decode(bt, 1)
    compare(o, lse, o_ref, lse_ref, "bf16")
    o4, l4 = _decode(bt, 1, split_len=4096)
    assert torch.equal(o, o4) and torch.equal(lse, l4)
    on, ln = M.decode_noalloc(bt.q, bt.cache, bt.block_table, bt.seq_lens, SM, 1, R)
    torch.cuda.synchronize()
    assert torch.equal(o, on) and torch.equal(lse, ln)


@pytest.mark.parametrize("index,H,piece_len", [(2, 128, 2048), (2, 128, 96), (4, 128, 1024), (3, 32, 512),
                                               (1, 16, 256), (0, 4, 32)])
def test_fixed_piece_partition(index, H, piece_len):
    """Partition 3: every request is cut into ceil(n / piece_len) pieces of
    piece_len tokens, each one partial, merged in order.  Results match the
    oracle, and a request gives the same bits alone (with a larger
    num_kv_splits) as inside the batch: the split depends on its own length
    only (fp32 on the vector-ALU kernel, 16 heads on the token-split kernel,
    32 and 128 heads on the shared-tile kernels, bf16 and fp8 caches)."""
    lens = [5000, 1, 0, piece_len, piece_len + 1, 3 * piece_len - 7, 700]
    bt = W.make_batch(index, DEV, seq_lens=lens, H=H, seed=31)
    _write(bt)
    o_ref, lse_ref = oracle_decode(bt, oracle_cache(bt), SM)
    max_len = bt.block_table.shape[1] * bt.spec.block_size
    S = -(-max_len // piece_len)
    _print(f"[pieces] workload {index} H={H} piece_len={piece_len} S={S}")
    o, lse = _decode(bt, S, partition=3, piece_len=piece_len)
    compare(o, lse, o_ref, lse_ref, bt.spec.in_dtype)
    for b in [0, 1, 2, 4, 5]:
        o1, l1 = M.decode(bt.q[b:b + 1].contiguous(), bt.cache, bt.block_table[b:b + 1].contiguous(),
                          bt.seq_lens[b:b + 1].contiguous(), SM, S + 3, bt.spec.R, kv_scale=bt.scale, partition=3,
                          piece_len=piece_len)
        torch.cuda.synchronize()
        assert torch.equal(o1[0], o[b]) and torch.equal(l1[0], lse[b]), b


def test_fixed_piece_partition_rejects_short_cover():
    """num_kv_splits pieces of piece_len tokens must cover the table's
    longest request."""
    bt = W.make_batch(2, DEV, seq_lens=[1000, 300], H=32)
    _write(bt)
    max_len = bt.block_table.shape[1] * bt.spec.block_size
    with pytest.raises(M.MLAError):
        _decode(bt, 1, partition=3, piece_len=max_len - 1)
    o, lse = _decode(bt, 1, partition=3, piece_len=max_len)     # one piece per request: fits
    assert torch.isfinite(lse).all()


@pytest.mark.parametrize("index,H,below", [(1, 16, True), (1, 16, False), (3, 16, True), (2, 32, True),
                                           (2, 32, False), (2, 64, True), (2, 128, True), (2, 128, False)])
def test_default_stage1_for_small_head_counts_under_balanced(index, H, below):
    """bf16 cache, num_kv_splits > 1 (balanced partition), 16 heads (any
    rank) or 32 and 64 heads (R = 512): the default stage 1 is the token
    split (16- or 32-head groups) while B * groups < 2 * CUs, and for 128
    heads (R = 512) while 4 * B <= CUs and the table's width bounds the
    batch's tokens by 768 per CU; the shared-tile kernels from there on --
    the same bits as the explicit choice on either side of the threshold."""
    cus = torch.cuda.get_device_properties(DEV).multi_processor_count
    hpg = 16 if H % 32 else 32
    groups = H // hpg
    if H == 128:
        B = cus // 4 if below else cus // 4 + 1
    else:
        B = (2 * cus + groups - 1) // groups - 1 if below else (2 * cus + groups - 1) // groups
    bt = W.make_batch(index, DEV, B=B, max_len=200, H=H)
    assert B * bt.block_table.shape[1] * bt.spec.block_size <= 768 * cus
    _write(bt)
    _print(f"[default-small-H] workload {index} H={H} B={B} cus={cus}")
    o, lse = _decode(bt, 2)
    ts = dict(kernel=3, heads_per_group=hpg)
    oe, le = _decode(bt, 2, **(ts if below else dict(kernel=2)))
    assert torch.equal(o, oe) and torch.equal(lse, le)
    other = _decode(bt, 2, **(dict(kernel=2) if below else ts))
    assert not torch.equal(o, other[0])      # the two kernels sum in different orders
