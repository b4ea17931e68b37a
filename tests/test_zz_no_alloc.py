"""mla_decode_noalloc (the decode for callers that cannot allocate: its
partials go to the library's per-GPU scratch array) against mla_decode on the
same inputs, through the C ABI: the same bits, on two calls in a row whose
second one is smaller, so that the scratch left behind by the first call
cannot leak into the second."""

import pytest
import torch

import mla_paged_decode_concat_amd as M
from mla_paged_decode_concat_amd import binding, workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
NOALLOC_SCRATCH_BYTES = 64 << 20     # MLA_NOALLOC_SCRATCH_BYTES in include/mla.h


def _pair(bt, S):
    spec = bt.spec
    assert binding.decode_workspace_bytes(bt.B, bt.H, S, spec.R) <= NOALLOC_SCRATCH_BYTES
    o1, l1 = M.decode(bt.q, bt.cache, bt.block_table, bt.seq_lens, W.SM_SCALE, S, spec.R, kv_scale=bt.scale)
    o2, l2 = M.decode_noalloc(bt.q, bt.cache, bt.block_table, bt.seq_lens, W.SM_SCALE, S, spec.R,
                              kv_scale=bt.scale)
    torch.cuda.synchronize()
    same_o = torch.equal(o1.view(torch.int16), o2.view(torch.int16)) if o1.dtype == torch.bfloat16 else \
        torch.equal(o1, o2)
    assert same_o and torch.equal(l1, l2), (spec.name, bt.B, S)


@pytest.mark.parametrize("first,second", [
    ((2, dict(B=6, max_len=3000), 3), (2, dict(B=2, max_len=700), 2)),      # 128 heads (two-role stage 1)
    ((1, dict(B=16, max_len=4096), 8), (1, dict(B=3, max_len=300), 4)),     # 16 heads
    ((4, dict(B=3, max_len=5000), 6), (0, {}, 2)),                          # fp8 cache, then the fp32 path
])
def test_noalloc_matches_decode_on_two_calls(first, second):
    for index, kw, S in (first, second):
        print(f"noalloc workload {index} {kw} S={S}", flush=True)
        bt = W.make_batch(index, DEV, **kw)
        M.cache_write(bt.kv_c, bt.k_pe, bt.cache, bt.slot_mapping, "fp8" if bt.spec.cache_dtype == "fp8" else "auto",
                      bt.scale)
        _pair(bt, S)
