"""Limits and capture: the split-count cap (num_kv_splits = 2 x CUs for a
request of a quarter million tokens, every partition and kernel), and the
whole step -- cache write, decode (with a workspace, without allocation, with
one partial per request and with fixed pieces), shard merge, RoPE, linear
layer -- captured in a HIP graph and replayed several times with eager work
in between, each replay equal to the eager result."""

import numpy as np
import pytest
import torch

import mla_paged_decode_concat_amd as M
from mla_paged_decode_concat_amd import workloads as W
from oracle import mla_oracle as O

from helpers import compare, oracle_decode_sampled

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SM = W.SM_SCALE


def _print(*a):
    print(*a, flush=True)


def test_split_count_cap_long_request():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n_long = 512 * 2 * cus + 777           # ceil(n / 512) exceeds the cap
    bt = W.make_batch(1, DEV, seq_lens=[n_long, 5, 1], H=16)
    S = M.num_kv_splits(n_long, cus)
    assert S == 2 * cus
    _print(f"[limits] n={n_long} S={S}")
    M.cache_write(bt.kv_c, bt.k_pe, bt.cache, bt.slot_mapping)
    o_ref, lse_ref = oracle_decode_sampled(bt, SM, [0, 1, 2])
    for kernel in [1, 2]:
        for partition in [1, 2]:
            o, lse = M.decode(bt.q, bt.cache, bt.block_table, bt.seq_lens, SM, S, bt.spec.R, kernel=kernel,
                              partition=partition)
            torch.cuda.synchronize()
            _print(f"[limits] kernel={kernel} partition={partition}")
            compare(o, lse, o_ref, lse_ref, "bf16")


def test_graph_capture_and_replay():
    bt = W.make_batch(1, DEV, B=6, max_len=2000)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    S = M.num_kv_splits(max(bt.seq_lens_list), cus)
    R = bt.spec.R
    pos = W.token_positions(bt)
    tab = W.rope_table(max(bt.seq_lens_list) + 1, 64).to(DEV)
    ws = torch.empty(M.decode_workspace_bytes(bt.B, bt.H, S, R) // 4, dtype=torch.float32, device=DEV)
    o = torch.empty((bt.B, bt.H, R), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((bt.B, bt.H), dtype=torch.float32, device=DEV)
    om = torch.empty_like(o)
    lm = torch.empty_like(lse)
    g = torch.Generator(device=DEV).manual_seed(3)
    A = torch.randn((bt.B, 1024), generator=g, device=DEV).to(torch.bfloat16)
    Wt = torch.randn((4096, 1024), generator=g, device=DEV).to(torch.bfloat16)
    C = torch.empty((bt.B, 4096), dtype=torch.bfloat16, device=DEV)
    q0 = bt.q.clone()
    qr = bt.q.clone()
    qpos = torch.tensor([n - 1 for n in bt.seq_lens_list], dtype=torch.int64, device=DEV)
    # the other decode forms: no allocation (library scratch), one partial
    # per request, fixed pieces of 256 tokens
    o_na, l_na = torch.empty_like(o), torch.empty_like(lse)
    ws1 = torch.empty(M.decode_workspace_bytes(bt.B, bt.H, 1, R) // 4, dtype=torch.float32, device=DEV)
    o1, l1 = torch.empty_like(o), torch.empty_like(lse)
    S_pc = -(-bt.block_table.shape[1] * bt.spec.block_size // 256)
    ws_pc = torch.empty(M.decode_workspace_bytes(bt.B, bt.H, S_pc, R) // 4, dtype=torch.float32, device=DEV)
    o_pc, l_pc = torch.empty_like(o), torch.empty_like(lse)

    def step():
        M.cache_write(bt.kv_c, bt.k_pe, bt.cache, bt.slot_mapping, positions=pos, cos_sin_cache=tab)
        qr.copy_(q0)
        M.rope_q(qr, qpos, tab, R)
        M.decode(qr, bt.cache, bt.block_table, bt.seq_lens, SM, S, R, workspace=ws, o=o, lse=lse)
        M.merge_partials(torch.stack([o, o]), torch.stack([lse, lse]), om, lm)
        M.linear(A, Wt, out=C)
        M.decode_noalloc(qr, bt.cache, bt.block_table, bt.seq_lens, SM, 2, R, o=o_na, lse=l_na)
        M.decode(qr, bt.cache, bt.block_table, bt.seq_lens, SM, 1, R, workspace=ws1, o=o1, lse=l1)
        M.decode(qr, bt.cache, bt.block_table, bt.seq_lens, SM, S_pc, R, workspace=ws_pc, o=o_pc, lse=l_pc,
                 partition=3, piece_len=256)

    outs = (qr, o, lse, om, lm, C, o_na, l_na, o1, l1, o_pc, l_pc)
    blank = bt.cache.clone()                   # NaN in every slot
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (bt.cache,) + outs]
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                 # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        bt.cache.copy_(blank)                  # eager work that resets or scrambles every output
        for t in outs:
            t.view(torch.uint8).fill_(0x55)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip((bt.cache,) + outs, ref)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}, output {i}"
    _print("[limits] 4 replays equal to the eager step")
