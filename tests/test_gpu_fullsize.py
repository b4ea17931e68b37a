"""Parity at the workloads' full sizes, in the launch configuration the
benchmark uses: num_kv_splits from the library's rule for the batch's longest
request and this GPU's compute-unit count, the default kernel, partition and
grid.  At these sizes the oracle is run on sampled requests, each one
computed on its own in fp64 from the generator's inputs; the cache write is
checked bit-exactly on sampled tokens against the oracle's write.

Workload 2 (DeepSeek-V3 shape, B=64, H=128, 8192 tokens each) is the one the
benchmark times; it is also checked with num_kv_splits = 1, the benchmark's
batch-invariant run, and with fixed pieces of 2048 tokens (partition 3).
"""

import os

import numpy as np
import pytest
import torch

import mla_paged_decode_concat_amd as M
from mla_paged_decode_concat_amd import workloads as W
from oracle import mla_oracle as O

from helpers import compare, margins, oracle_decode_sampled

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SM = W.SM_SCALE


def _print(*a):
    print(*a, flush=True)


def _sampled_requests(bt):
    lens = bt.seq_lens_list
    picks = {0, bt.B // 2, bt.B - 1, int(np.argmax(lens)), int(np.argmin(lens))}
    return sorted(picks)


def _check_write_sampled(bt, n_tokens=512, seed=7):
    """The GPU cache rows of sampled real tokens equal the oracle's write of
    those tokens (bit for bit)."""
    spec = bt.spec
    slots = bt.slot_mapping.cpu().numpy()
    real = np.nonzero(slots >= 0)[0]
    rng = np.random.default_rng(seed)
    toks = np.sort(rng.choice(real, size=min(n_tokens, real.size), replace=False))
    idx = torch.from_numpy(toks).to(bt.kv_c.device)
    kv_c = W.bits(bt.kv_c.index_select(0, idx))
    k_pe = W.bits(bt.k_pe.index_select(0, idx))
    # the oracle writes the sampled tokens into a small cache of their own
    empty = W.bits(W.nan_cache(spec, len(toks), "cpu"))[:, :1, :]
    scale = float(bt.scale[0].cpu()) if bt.scale is not None else None
    want = O.cache_write(empty, kv_c, k_pe, np.arange(len(toks), dtype=np.int64), spec.in_dtype,
                         spec.cache_dtype, scale)[:, 0, :]
    s = torch.from_numpy(slots[toks]).to(bt.cache.device)
    bs = spec.block_size
    got = W.bits(bt.cache[s // bs, s % bs])
    assert np.array_equal(got, want)


@pytest.mark.parametrize("index", [0, 1, 2, 3, 4])
def test_full_size_default_launch(index):
    spec = W.SPECS[index]
    _print(f"[full] workload {index} {spec.name}: drawing inputs")
    bt = W.make_batch(index, DEV)
    M.cache_write(bt.kv_c, bt.k_pe, bt.cache, bt.slot_mapping, "fp8" if spec.cache_dtype == "fp8" else "auto",
                  bt.scale)
    torch.cuda.synchronize()
    _check_write_sampled(bt)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    S = M.num_kv_splits(max(bt.seq_lens_list), cus)
    reqs = _sampled_requests(bt)
    _print(f"[full] workload {index}: B={bt.B} tokens={sum(bt.seq_lens_list)} S={S} sampled requests {reqs}")
    o, lse = M.decode(bt.q, bt.cache, bt.block_table, bt.seq_lens, SM, S, spec.R, kv_scale=bt.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(lse).all()
    o_ref, lse_ref = oracle_decode_sampled(bt, SM, reqs)
    compare(o[reqs], lse[reqs], o_ref, lse_ref, spec.in_dtype)
    _margin_line(index, spec, S, reqs, margins(o[reqs], lse[reqs], o_ref, lse_ref, spec.in_dtype))
    if index == 2:
        _print("[full] workload 2: num_kv_splits = 1")
        o1, lse1 = M.decode(bt.q, bt.cache, bt.block_table, bt.seq_lens, SM, 1, spec.R)
        torch.cuda.synchronize()
        compare(o1[reqs], lse1[reqs], o_ref, lse_ref, spec.in_dtype)
        _margin_line(index, spec, 1, reqs, margins(o1[reqs], lse1[reqs], o_ref, lse_ref, spec.in_dtype))
        _print("[full] workload 2: fixed pieces of 2048 tokens, num_kv_splits = 4")
        o2, lse2 = M.decode(bt.q, bt.cache, bt.block_table, bt.seq_lens, SM, 4, spec.R, partition=3, piece_len=2048)
        torch.cuda.synchronize()
        compare(o2[reqs], lse2[reqs], o_ref, lse_ref, spec.in_dtype)
        _margin_line(index, spec, 4, reqs, margins(o2[reqs], lse2[reqs], o_ref, lse_ref, spec.in_dtype))


def _margin_line(index, spec, S, reqs, m):
    """Print the plain errors; with MLA_PARITY_MARGINS set, also append them
    to that file (the committed margins table is made this way)."""
    line = (f"workload {index} {spec.name} num_kv_splits={S} requests={reqs}: max|o-oracle|={m[0]:.4g} "
            f"max|o-bf16(oracle)|={m[1]:.4g} max(|o-oracle|-half_bf16_ulp)={m[3]:.4g} max|oracle o|={m[4]:.4g} "
            f"max|lse-oracle|={m[2]:.4g}")
    _print("[margins] " + line)
    path = os.environ.get("MLA_PARITY_MARGINS")
    if path:
        with open(path, "a") as f:
            f.write(line + "\n")
