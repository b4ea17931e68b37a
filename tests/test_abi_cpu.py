"""C-ABI checks that need no GPU: the library loads, exports every function
include/mla.h declares, the host-only calls compute the documented values,
and invalid arguments are rejected before anything is launched (no compute
call reaches a kernel here)."""

import ctypes
import os
import re

import pytest

from mla_paged_decode_concat_amd import binding
from oracle import mla_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")

pytestmark = pytest.mark.skipif(not os.path.exists(binding.library_path()),
                                reason="libmla_amd.so not built (run __graft_entry__.build())")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_header_functions_are_exported():
    lib = binding.load_library()
    names = _declared_functions()
    assert set(binding.EXPORTS) <= set(names)
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings():
    lib = binding.load_library()
    for code in [0, -1, -2, -3, -4]:
        assert lib.mla_status_string(code)
    assert lib.mla_status_string(12345) == b"unknown status"


@pytest.mark.parametrize("max_len,cus,bi", [(0, 256, 0), (1, 256, 0), (512, 256, 0), (513, 256, 0), (8192, 256, 0),
                                            (65536, 256, 0), (10 ** 8, 256, 0), (4096, 8, 0), (8192, 256, 1)])
def test_num_kv_splits_matches_oracle(max_len, cus, bi):
    lib = binding.load_library()
    assert lib.mla_num_kv_splits(max_len, cus, bi) == O.num_kv_splits(max_len, cus, bool(bi))


def test_num_kv_splits_rejects_bad_args():
    lib = binding.load_library()
    assert lib.mla_num_kv_splits(-1, 256, 0) == -1
    assert lib.mla_num_kv_splits(10, 0, 0) == -1


def test_workspace_bytes():
    lib = binding.load_library()
    for B, H, S, R in [(64, 128, 16, 512), (2, 4, 2, 512), (128, 32, 64, 256), (1, 1, 1, 1)]:
        assert lib.mla_decode_workspace_bytes(B, H, S, R) == 4 * O.workspace_floats(B, H, S, R)
    assert lib.mla_decode_workspace_bytes(0, 1, 1, 512) == 0
    assert lib.mla_decode_workspace_bytes(1, 1, 0, 512) == 0


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def _write(**kw):
    a = dict(kv_c=FAKE, kvs=512, k_pe=FAKE, kps=64, in_dt=1, slots=FAKE, T=10, cache=FAKE, cache_dt=1,
             nb=4, bs=16, bstride=16 * 576, R=512, P=64, scale=None, stream=None)
    a.update(kw)
    return binding.load_library().mla_cache_write(*a.values())


def test_cache_write_validation():
    assert _write(in_dt=2) == -2                    # fp8 input is not an input dtype
    assert _write(cache_dt=0) == -2                 # bf16 in, f32 cache
    assert _write(R=128) == -2 and _write(P=32) == -2
    assert _write(T=-1) == -1
    assert _write(nb=0) == -1 and _write(bs=0) == -1
    assert _write(bstride=16 * 576 - 1) == -1
    assert _write(kvs=511) == -1 and _write(kps=63) == -1
    assert _write(cache_dt=2) == -1                 # fp8 cache without a scale
    assert _write(scale=FAKE) == -1                 # scale given for a bf16 cache
    assert _write(kv_c=None) == -1 and _write(slots=None) == -1 and _write(cache=None) == -1
    assert _write(T=0) == 0                         # nothing to do, nothing launched


def _decode(opts=None, **kw):
    a = dict(q=FAKE, qsb=128 * 576, qsh=576, q_dt=1, B=4, H=128, cache=FAKE, cache_dt=1, nb=100, bs=64,
             bstride=64 * 576, R=512, P=64, bt=FAKE, bts=10, maxblk=10, seq=FAKE, sm=0.07, kvs=None, S=4,
             ws=FAKE, wsb=4 * 128 * 4 * 513 * 4, o=FAKE, lse=FAKE, stream=None)
    a.update(kw)
    lib = binding.load_library()
    if opts is None:
        return lib.mla_decode(*a.values())
    return lib.mla_decode_ex(*a.values(), ctypes.byref(opts))


def test_decode_validation():
    assert _decode(q_dt=0) == -2                    # f32 q with bf16 cache
    assert _decode(q_dt=0, cache_dt=2) == -2        # fp8 cache needs a bf16 query
    assert _decode(R=128) == -2 and _decode(P=0) == -2
    assert _decode(B=-1) == -1 and _decode(H=0) == -1 and _decode(S=0) == -1
    assert _decode(bs=0) == -1 and _decode(nb=0) == -1 and _decode(maxblk=0) == -1
    assert _decode(bstride=100) == -1 and _decode(bts=5) == -1
    assert _decode(qsb=0) == -1 and _decode(qsh=0) == -1
    assert _decode(sm=float("nan")) == -1 and _decode(sm=float("inf")) == -1
    assert _decode(cache_dt=2) == -1                # fp8 cache without kv_scale
    assert _decode(kvs=FAKE) == -1                  # kv_scale with a bf16 cache
    for k in ["q", "cache", "bt", "seq", "ws", "o", "lse"]:
        assert _decode(**{k: None}) == -1, k
    assert _decode(ws=FAKE + 2) == -1               # misaligned workspace
    assert _decode(ws=FAKE + 4) == -1               # workspace not 16-byte aligned
    assert _decode(o=FAKE + 8) == -1                # output not 16-byte aligned
    assert _decode(wsb=4 * 128 * 4 * 513 * 4 - 4) == -3
    assert _decode(S=5) == -3                       # workspace sized for 4 splits
    assert _decode(B=0) == 0                        # empty batch: nothing launched


def test_decode_ex_validation():
    O_ = binding.DecodeOpts
    assert _decode(O_(3, 0, 0, 0)) == -1
    assert _decode(O_(0, 4, 0, 0)) == -1
    assert _decode(O_(0, 0, -1, 0)) == -1
    assert _decode(O_(0, 2, 0, 0), q_dt=0, cache_dt=0) == -2   # MFMA kernel needs a bf16 query
    assert _decode(O_(0, 0, 0, 0), B=0) == 0
    bad = O_(0, 0, 0, 0)
    bad.reserved[1] = 7
    assert _decode(bad) == -1                                  # reserved fields must be zero
    assert _decode(O_(0, 3, 0, 64)) == -2                      # token split takes 16- or 32-head groups
    assert _decode(O_(0, 3, 0, 32), H=48) == -1                # a head group must divide the head count
    assert _decode(O_(0, 3, 0, 16), cache_dt=2, kvs=FAKE) == -2   # ... of a bf16 cache


def test_decode_ex_piece_partition_validation():
    """Fixed-length pieces (partition 3): piece_len is required there and
    only there, and num_kv_splits pieces of piece_len tokens must cover the
    longest request the table allows (maxblk 10 x block 64 = 640 tokens)."""
    O_ = binding.DecodeOpts
    def opts(partition, piece_len):
        o = O_(partition, 0, 0, 0)
        o.piece_len = piece_len
        return o
    assert _decode(opts(3, 0)) == -1                           # partition 3 needs a piece length
    assert _decode(opts(0, 160)) == -1                         # a piece length needs partition 3
    assert _decode(opts(1, 160)) == -1
    assert _decode(opts(3, -32)) == -1
    assert _decode(opts(3, 159)) == -1                         # 4 x 159 < 640
    assert _decode(opts(3, 64), S=9, wsb=4 * 128 * 9 * 513 * 4) == -1   # 9 x 64 < 640
    assert _decode(opts(3, 160), B=0) == 0                     # 4 x 160 = 640: valid (empty batch launches nothing)
    assert _decode(opts(3, 64), S=10, B=0, wsb=4 * 128 * 10 * 513 * 4) == 0


def _merge(**kw):
    a = dict(o_parts=FAKE, lse_parts=FAKE, G=4, B=8, H=16, R=512, dt=1, o=FAKE, lse=FAKE, stream=None)
    a.update(kw)
    return binding.load_library().mla_merge_partials(*a.values())


def test_merge_partials_validation():
    assert _merge(R=576) == -2 and _merge(dt=2) == -2   # R must be 512/256; fp8 is no output dtype
    assert _merge(G=0) == -1 and _merge(H=0) == -1 and _merge(B=-1) == -1
    assert _merge(o_parts=None) == -1 and _merge(lse_parts=None) == -1
    assert _merge(o=None) == -1 and _merge(lse=None) == -1
    assert _merge(o_parts=FAKE + 8) == -1               # not 16-byte aligned
    assert _merge(o=FAKE + 4) == -1
    assert _merge(lse=FAKE + 2) == -1
    assert _merge(B=0) == 0                             # nothing launched


def test_binding_rejects_host_tensors_and_bad_shapes():
    """The binding refuses tensors the library cannot address (host memory)
    and shapes that do not match, before any call into the library."""
    import torch
    import mla_paged_decode_concat_amd as M
    q = torch.zeros((2, 4, 576), dtype=torch.bfloat16)
    cache = torch.zeros((3, 16, 576), dtype=torch.bfloat16)
    table = torch.zeros((2, 3), dtype=torch.int32)
    lens = torch.ones(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU tensors"):
        M.decode(q, cache, table, lens, 0.1, 1)
    with pytest.raises(ValueError, match="B entries"):
        M.decode(q, cache, table, torch.ones(3, dtype=torch.int32), 0.1, 1)
    with pytest.raises(ValueError, match="R \\+ P"):
        M.decode(q, torch.zeros((3, 16, 512), dtype=torch.bfloat16), table, lens, 0.1, 1)
    kv_c = torch.zeros((5, 512), dtype=torch.bfloat16)
    k_pe = torch.zeros((5, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensors"):
        M.cache_write(kv_c, k_pe, cache, torch.zeros(5, dtype=torch.int64))
    with pytest.raises(ValueError, match="one row per"):
        M.cache_write(kv_c, k_pe, cache, torch.zeros(6, dtype=torch.int64))
    with pytest.raises(ValueError, match="GPU tensors"):
        M.merge_partials(torch.zeros((2, 2, 4, 512)), torch.zeros((2, 2, 4)))
    with pytest.raises(ValueError, match="fp32 \\[G, B, H\\]"):
        M.merge_partials(torch.zeros((2, 2, 4, 512)), torch.zeros((2, 2, 5)))


def _wrope(**kw):
    a = dict(kv_c=FAKE, kvs=512, k_pe=FAKE, kps=64, in_dt=1, slots=FAKE, T=10, pos=FAKE, tab=FAKE, maxpos=100,
             cache=FAKE, cache_dt=1, nb=4, bs=16, bstride=16 * 576, R=512, P=64, scale=None, stream=None)
    a.update(kw)
    return binding.load_library().mla_cache_write_rope(*a.values())


def test_cache_write_rope_validation():
    assert _wrope(maxpos=0) == -1
    assert _wrope(pos=None) == -1 and _wrope(tab=None) == -1
    assert _wrope(tab=FAKE + 2) == -1                 # table not 4-byte aligned
    assert _wrope(in_dt=2) == -2 and _wrope(R=128) == -2
    assert _wrope(cache_dt=2) == -1                   # fp8 cache without a scale
    assert _wrope(T=0, pos=None, tab=None) == 0       # nothing to do


def _ropeq(**kw):
    a = dict(q=FAKE, sn=128 * 576, sh=576, dt=1, N=4, H=128, R=512, P=64, pos=FAKE, tab=FAKE, maxpos=100,
             stream=None)
    a.update(kw)
    return binding.load_library().mla_rope_q(*a.values())


def test_rope_q_validation():
    assert _ropeq(dt=2) == -2 and _ropeq(P=32) == -2
    assert _ropeq(H=0) == -1 and _ropeq(N=-1) == -1 and _ropeq(maxpos=0) == -1
    assert _ropeq(sh=575) == -1 and _ropeq(sn=127 * 576) == -1
    assert _ropeq(q=None) == -1 and _ropeq(pos=None) == -1 and _ropeq(tab=None) == -1
    assert _ropeq(q=FAKE + 1) == -1 and _ropeq(tab=FAKE + 2) == -1
    assert _ropeq(N=0) == 0


def _lin(**kw):
    a = dict(A=FAKE, lda=1536, W=FAKE, ldw=1536, M=8, N=256, K=1536, C=FAKE, ldc=256, dt=1, ws=None, wsb=0,
             stream=None)
    a.update(kw)
    return binding.load_library().mla_linear_bf16(*a.values())


def test_linear_validation():
    assert _lin(dt=2) == -2
    assert _lin(N=24) == -2 and _lin(N=0) == -2 and _lin(K=96) == -2 and _lin(K=0) == -2
    assert _lin(M=-1) == -1 and _lin(lda=1535) == -1 and _lin(ldw=1000) == -1 and _lin(ldc=255) == -1
    assert _lin(A=None) == -1 and _lin(W=None) == -1 and _lin(C=None) == -1
    assert _lin(A=FAKE + 8) == -1 and _lin(W=FAKE + 2) == -1 and _lin(lda=1544 + 4) == -1
    assert _lin(C=FAKE + 4) == -1                    # bf16 output needs 8-byte alignment
    assert _lin(C=FAKE + 8, dt=0) == -1              # fp32 output needs 16-byte alignment
    assert _lin(M=0) == 0
    lib = binding.load_library()
    assert lib.mla_linear_workspace_bytes(8, 24, 1536) == 0          # unsupported N
    assert lib.mla_linear_workspace_bytes(0, 256, 1536) == 0


def test_decode_noalloc_rejects_sizes_beyond_its_scratch():
    """mla_decode_noalloc checks the workspace the call needs against its
    fixed scratch size before anything else (no device is touched)."""
    lib = binding.load_library()
    v, i = ctypes.c_void_p, ctypes
    args = [FAKE, 128 * 576, 576, 1, 64, 128, FAKE, 1, 9000, 64, 64 * 576, 512, 64, FAKE, 128, 128, FAKE,
            ctypes.c_float(0.07), None, 16, FAKE, FAKE, None]
    # 64 * 128 * 16 * 513 * 4 bytes = 269 MB > 64 MiB
    assert lib.mla_decode_noalloc(*args) == -3
    args[19] = 64                    # still more than the scratch holds
    assert lib.mla_decode_noalloc(*args) == -3
