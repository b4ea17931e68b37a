"""Pins for the oracle's cache write: it is an exact scatter through
slot_mapping (read-back inverse), padded rows (slot -1) land nowhere, untouched
slots keep their NaN fill, only len(slot_mapping) tokens are written, and the
fp8 write equals torch's own cast of x / scale."""

import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from mla_paged_decode_concat_amd import workloads as W


def _check_scatter(cache_in, cache_out, kv_c, k_pe, slots, enc):
    nb, bs, D = cache_out.shape
    R = kv_c.shape[1]
    written = np.zeros((nb, bs), dtype=bool)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        row = cache_out[s // bs, s % bs]
        assert np.array_equal(row[:R], enc(kv_c[t])) and np.array_equal(row[R:], enc(k_pe[t]))
        written[s // bs, s % bs] = True
    # everything else is untouched, bit for bit
    a = cache_in.reshape(nb * bs, D)[~written.reshape(-1)]
    b = cache_out.reshape(nb * bs, D)[~written.reshape(-1)]
    assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    return written


@pytest.mark.parametrize("index,kw", [(0, {}), (3, dict(B=6, max_len=90)), (1, dict(B=3, max_len=200))])
def test_write_is_exact_scatter(index, kw):
    bt = W.make_batch(index, "cpu", **kw)
    spec = bt.spec
    cin = W.bits(bt.cache)
    kv_c, k_pe, slots = W.bits(bt.kv_c), W.bits(bt.k_pe), bt.slot_mapping.numpy()
    out = O.cache_write(cin, kv_c, k_pe, slots, spec.in_dtype, spec.cache_dtype)
    written = _check_scatter(cin, out, kv_c, k_pe, slots, lambda x: x)
    assert written.sum() == (slots >= 0).sum() == sum(bt.seq_lens_list)
    if spec.pad_frac:
        frac = (slots < 0).mean()
        assert 0.08 < frac < 0.12
        # padded rows' values appear nowhere in the cache
        pad_rows = kv_c[slots < 0]
        flat = out.reshape(-1, spec.D)[:, :spec.R]
        assert not any(np.array_equal(flat[i], pad_rows[0]) for i in range(flat.shape[0]))


def test_num_tokens_is_len_of_slot_mapping():
    bt = W.make_batch(0, "cpu")
    kv_c, k_pe = W.bits(bt.kv_c), W.bits(bt.k_pe)
    slots = bt.slot_mapping.numpy()[:50]
    out = O.cache_write(W.bits(bt.cache), kv_c, k_pe, slots, "f32", "f32")
    assert np.isfinite(out.reshape(-1, 576)).all(axis=1).sum() == 50


def test_fp8_write_matches_torch_cast():
    bt = W.make_batch(4, "cpu", B=2, max_len=1030)
    scale = np.float32(bt.scale[0])
    kv_c, k_pe, slots = W.bits(bt.kv_c), W.bits(bt.k_pe), bt.slot_mapping.numpy()
    cin = W.bits(bt.cache)
    out = O.cache_write(cin, kv_c, k_pe, slots, "bf16", "fp8", float(scale))

    def enc(x):
        y = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float() / torch.tensor(scale)
        return y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()

    _check_scatter(cin, out, kv_c, k_pe, slots, enc)
    # scale = amax/448 puts the largest magnitude exactly on 448
    assert (out[np.isin(out, [0x7E, 0xFE])]).size >= 1


def test_slot_validation_pass():
    """The tests' debug validation of a slot mapping: padding (-1) is
    allowed, a repeated or out-of-range slot is rejected."""
    import pytest
    from helpers import check_slots
    check_slots(np.array([3, -1, 0, 7, -1], dtype=np.int64), 2, 4)
    with pytest.raises(ValueError):
        check_slots(np.array([3, -1, 3], dtype=np.int64), 2, 4)
    with pytest.raises(ValueError):
        check_slots(np.array([0, 8], dtype=np.int64), 2, 4)
    check_slots(np.array([], dtype=np.int64), 2, 4)
