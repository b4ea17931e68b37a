"""Seeded random decode configurations against the oracle: batch size, head
count (including counts only the vector kernel takes), lengths (empty, one
token, ragged, one long request), num_kv_splits, partition and cache type
drawn per case, and, from a second generator, the stage-1 choice (library
default, the token-split kernel with 16 or 32 heads, or batch-invariant
length classes) and from a third whether the batch is cut into fixed-length
pieces -- combinations the targeted tests do not enumerate.
MLA_RANDOM_CASES sets the number of cases (100 by default; seeds 42 and 65
once exceeded the bound on an fp8 cache, before its P carried the bf16
rounding remainder)."""

import os

import numpy as np
import pytest
import torch

import mla_paged_decode_concat_amd as M
from mla_paged_decode_concat_amd import workloads as W

from helpers import compare, oracle_cache, oracle_decode

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SM = W.SM_SCALE


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    index = int(rng.choice([1, 2, 3, 4]))
    B = int(rng.integers(1, 10))
    H = int(rng.choice([16, 32, 48, 64, 128, 5, 24]))
    lens = [int(x) for x in rng.integers(0, 1500, B)]
    if rng.random() < 0.3:
        lens[int(rng.integers(0, B))] = int(rng.integers(3000, 9000))
    if rng.random() < 0.3:
        lens[int(rng.integers(0, B))] = int(rng.choice([0, 1]))
    S = int(rng.choice([1, 2, 3, 8, 17]))
    partition = int(rng.choice([0, 1, 2]))
    # stage-1 choice, from its own generator so the draws above stay as they were
    r2 = np.random.default_rng(5000 + seed)
    mode = r2.choice(["default", "token_split", "length_classes"], p=[0.5, 0.25, 0.25])
    opts = {}
    if mode == "token_split" and index != 4 and H % 16 == 0:      # bf16 cache
        opts = dict(kernel=3, heads_per_group=32 if H % 32 == 0 and r2.random() < 0.5 else 16)
    elif mode == "length_classes" and index != 4 and H % 32 == 0:
        S, partition = 1, 0
        opts = dict(split_len=int(r2.choice([1, 300, 1000])))
    # fixed-length pieces (partition 3), from a third generator; num_kv_splits
    # is then set from the batch's table width
    r3 = np.random.default_rng(9000 + seed)
    if "split_len" not in opts and r3.random() < 0.25:
        partition = 3
        opts = dict(opts, piece_len=int(r3.choice([32, 100, 512, 2048])))
    return index, H, lens, S, partition, opts


@pytest.mark.parametrize("seed", range(int(os.environ.get("MLA_RANDOM_CASES", "100"))))
def test_random_configuration_against_oracle(seed):
    index, H, lens, S, partition, opts = _case(seed)
    print(f"[random {seed}] workload {index} H={H} S={S} partition={partition} {opts} lens={lens}", flush=True)
    bt = W.make_batch(index, DEV, seq_lens=lens, H=H, seed=seed)
    if partition == 3:
        S = -(-bt.block_table.shape[1] * bt.spec.block_size // opts["piece_len"])
        print(f"[random {seed}] fixed pieces: num_kv_splits={S}", flush=True)
    ref_cache = oracle_cache(bt)
    M.cache_write(bt.kv_c, bt.k_pe, bt.cache, bt.slot_mapping, "fp8" if bt.spec.cache_dtype == "fp8" else "auto",
                  bt.scale)
    o_ref, lse_ref = oracle_decode(bt, ref_cache, SM)
    o, lse = M.decode(bt.q, bt.cache, bt.block_table, bt.seq_lens, SM, S, bt.spec.R, kv_scale=bt.scale,
                      partition=partition, **opts)
    torch.cuda.synchronize()
    compare(o, lse, o_ref, lse_ref, bt.spec.in_dtype)
