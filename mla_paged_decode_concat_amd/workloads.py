"""Seeded synthetic workloads for the paged MLA cache write and decode.

This module only draws inputs: sequence lengths, physical block assignment,
block tables, slot maps and random tensors.  It holds none of the method's
arithmetic, imports neither the HIP binding nor the oracle, and is shared by
the tests, ``bench.py`` and ``__graft_entry__.smoke()``.

The five workloads are the DeepSeek-V2/V3 MLA head geometries the decode path
serves (kv_lora_rank 512 or 256, rope_dim 64, row width 576 or 320):

  0 tiny_f32       fp32, B=2, H=4, block 16, seq_lens [37, 100], 16 blocks
  1 v2lite_bf16    bf16, B=32, H=16, block 64, seq_lens ~ U{1..4096}
  2 v3_bf16        bf16, B=64, H=128, block 64, every seq_len 8192
  3 r256_bf16      bf16, kv_lora_rank 256, B=128, H=32, block 16,
                   seq_lens ~ round(LogNormal(ln 2048, 1)) clipped to [1, 32768],
                   10% of slot_mapping entries are -1 (padded rows)
  4 fp8_long       fp8 E4M3 cache, bf16 q, B=128, H=128, block 64,
                   seq_lens ~ U{1024..65536}, kv ~ 2*N(0,1) in bf16,
                   per-tensor scale = amax / 448

Recipe: a CPU ``torch.Generator`` seeded ``1000 + index`` draws the lengths,
the block permutation and the pad positions; a generator on the target device
with the same seed draws kv_c, then k_pe, then q, as N(0, sigma^2) float32,
cast to bf16 with round-to-nearest-even where the workload is bf16.  Every
request owns whole physical blocks taken in order from a random permutation;
one extra block is never written and is filled, like every unwritten slot,
with NaN so that a read of it shows up.  Block-table rows are padded with that
spare block (parity runs) or with block 0 (timing runs).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import torch

SM_SCALE = 1.0 / math.sqrt(192.0)   # 1/sqrt(qk_nope_head_dim + qk_rope_head_dim) of DeepSeek-V2/V3

NAN_BF16 = 0x7FC0
NAN_FP8 = 0x7F


@dataclass(frozen=True)
class Spec:
    index: int
    name: str
    in_dtype: str       # dtype of q, kv_c and k_pe: "f32" | "bf16"
    cache_dtype: str    # "f32" | "bf16" | "fp8"
    B: int
    H: int
    R: int
    P: int
    block_size: int
    sigma: float = 1.0
    pad_frac: float = 0.0

    @property
    def D(self) -> int:
        return self.R + self.P


SPECS: List[Spec] = [
    Spec(0, "tiny_f32", "f32", "f32", B=2, H=4, R=512, P=64, block_size=16),
    Spec(1, "v2lite_bf16", "bf16", "bf16", B=32, H=16, R=512, P=64, block_size=64),
    Spec(2, "v3_bf16", "bf16", "bf16", B=64, H=128, R=512, P=64, block_size=64),
    Spec(3, "r256_bf16", "bf16", "bf16", B=128, H=32, R=256, P=64, block_size=16, pad_frac=0.10),
    Spec(4, "fp8_long", "bf16", "fp8", B=128, H=128, R=512, P=64, block_size=64, sigma=2.0),
]


def torch_dtype(d: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[d]


def draw_seq_lens(spec: Spec, gen: torch.Generator, B: int, max_len: Optional[int]) -> List[int]:
    """Sequence lengths of the workload; ``max_len`` clips them for reduced
    parity cases (the distribution shape below the clip is unchanged)."""
    i = spec.index
    if i == 0:
        lens = [37, 100][:B] + [100] * max(0, B - 2)
    elif i == 1:
        lens = torch.randint(1, 4097, (B,), generator=gen).tolist()
    elif i == 2:
        lens = [8192] * B
    elif i == 3:
        z = torch.randn(B, generator=gen, dtype=torch.float64)
        lens = [int(min(32768, max(1, round(math.exp(math.log(2048.0) + float(v)))))) for v in z]
    elif i == 4:
        lens = torch.randint(1024, 65537, (B,), generator=gen).tolist()
    else:
        raise ValueError(i)
    if max_len is not None:
        lens = [min(n, max_len) for n in lens]
    return lens


@dataclass
class Batch:
    """One synthetic batch.  Tensors live on ``device``."""
    spec: Spec
    seq_lens_list: List[int]
    seq_lens: torch.Tensor        # int32 [B]
    block_table: torch.Tensor     # int32 [B, max_blocks]
    slot_mapping: torch.Tensor    # int64 [T]   (-1 = padded row)
    kv_c: torch.Tensor            # [T, R]  in_dtype
    k_pe: torch.Tensor            # [T, P]  in_dtype
    q: torch.Tensor               # [B, H, R+P]  in_dtype
    cache: torch.Tensor           # [num_blocks, block_size, R+P] cache dtype (uint8 for fp8), NaN-filled
    scale: Optional[torch.Tensor] # fp32 [1] (fp8 only)
    spare_block: int
    num_blocks: int
    last_token_rows: torch.Tensor # int64 [B]: row index in kv_c/k_pe of each request's last token
    extra: Dict[str, object] = field(default_factory=dict)

    @property
    def B(self) -> int:
        return len(self.seq_lens_list)

    @property
    def H(self) -> int:
        return self.q.shape[1]


def nan_cache(spec: Spec, num_blocks: int, device) -> torch.Tensor:
    shape = (num_blocks, spec.block_size, spec.D)
    if spec.cache_dtype == "f32":
        return torch.full(shape, float("nan"), dtype=torch.float32, device=device)
    if spec.cache_dtype == "bf16":
        return torch.full(shape, NAN_BF16, dtype=torch.int16, device=device).view(torch.bfloat16)
    return torch.full(shape, NAN_FP8, dtype=torch.uint8, device=device)


def make_batch(index: int, device="cpu", B: Optional[int] = None, max_len: Optional[int] = None,
               seq_lens: Optional[List[int]] = None, H: Optional[int] = None,
               pad_table_with_spare: bool = True, seed: Optional[int] = None) -> Batch:
    """Draw workload ``index`` (0..4).  ``B``, ``max_len``, ``H`` and
    ``seq_lens`` override the full-size shape for reduced parity cases."""
    spec = SPECS[index]
    if H is not None:
        spec = Spec(spec.index, spec.name, spec.in_dtype, spec.cache_dtype, spec.B, H, spec.R,
                    spec.P, spec.block_size, spec.sigma, spec.pad_frac)
    B = spec.B if B is None else B
    s = 1000 + index if seed is None else seed
    gen = torch.Generator(device="cpu")
    gen.manual_seed(s)
    lens = list(seq_lens) if seq_lens is not None else draw_seq_lens(spec, gen, B, max_len)
    B = len(lens)
    bs = spec.block_size
    nblk = [-(-n // bs) for n in lens]
    used = sum(nblk)
    if index == 0 and seq_lens is None and B == 2:
        num_blocks = 16           # the tiny workload fixes a pool of 16 blocks
    else:
        num_blocks = used + 1     # one never-written spare block
    perm = torch.randperm(num_blocks, generator=gen)
    spare = int(perm[used]) if num_blocks > used else int(perm[-1])
    max_blocks = max(1, max(nblk) if nblk else 1)
    pad_id = spare if pad_table_with_spare else 0
    table = torch.full((B, max_blocks), pad_id, dtype=torch.int32)
    slots: List[torch.Tensor] = []
    off = 0
    for b, n in enumerate(lens):
        ids = perm[off:off + nblk[b]]
        off += nblk[b]
        table[b, :nblk[b]] = ids.to(torch.int32)
        j = torch.arange(n, dtype=torch.int64)
        slots.append(ids.to(torch.int64)[j // bs] * bs + j % bs)
    slot = torch.cat(slots) if slots else torch.zeros(0, dtype=torch.int64)
    T_real = slot.numel()
    # row index of each request's last token, before padding rows are inserted
    ends = torch.tensor([sum(lens[:b + 1]) - 1 for b in range(B)], dtype=torch.int64)
    if spec.pad_frac > 0 and T_real > 0:
        T_pad = int(round(T_real * spec.pad_frac / (1.0 - spec.pad_frac)))
        T = T_real + T_pad
        pos = torch.randperm(T, generator=gen)
        real_pos = torch.sort(pos[:T_real]).values
        full = torch.full((T,), -1, dtype=torch.int64)
        full[real_pos] = slot
        slot = full
        ends = real_pos[ends]
    T = slot.numel()

    dgen = torch.Generator(device=device)
    dgen.manual_seed(s)
    td = torch_dtype(spec.in_dtype)
    kv_c = (torch.randn((T, spec.R), generator=dgen, device=device, dtype=torch.float32) * spec.sigma).to(td)
    k_pe = (torch.randn((T, spec.P), generator=dgen, device=device, dtype=torch.float32) * spec.sigma).to(td)
    q = torch.randn((B, spec.H, spec.D), generator=dgen, device=device, dtype=torch.float32).to(td)
    scale = None
    if spec.cache_dtype == "fp8":
        amax = torch.maximum(kv_c.float().abs().amax(), k_pe.float().abs().amax())
        scale = (amax / 448.0).reshape(1).to(torch.float32)
    return Batch(spec=spec, seq_lens_list=lens,
                 seq_lens=torch.tensor(lens, dtype=torch.int32).to(device),
                 block_table=table.to(device), slot_mapping=slot.to(device),
                 kv_c=kv_c, k_pe=k_pe, q=q, cache=nan_cache(spec, num_blocks, device),
                 scale=scale, spare_block=spare, num_blocks=num_blocks,
                 last_token_rows=ends.to(device))


def bits(t: torch.Tensor):
    """Host numpy view of a tensor's stored bits in the oracle's convention
    (float32 values, bf16 as uint16, fp8 as uint8)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def multi_token_q(bt: Batch, q_len: int, seed: Optional[int] = None) -> torch.Tensor:
    """Query block of ``q_len`` tokens per request, [B, q_len, H, R+P], drawn
    like the batch's q: N(0, 1) float32 on a generator on the batch's device
    (seeded 2000 + workload index unless given), cast to the input dtype."""
    spec = bt.spec
    dev = bt.q.device
    g = torch.Generator(device=dev)
    g.manual_seed(2000 + spec.index if seed is None else seed)
    shape = (bt.B, q_len, spec.H, spec.D)
    return torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch_dtype(spec.in_dtype))


ROPE_THETA = 10000.0   # rope_theta of DeepSeek-V2/V3


def rope_table(max_position: int, P: int = 64, theta: float = ROPE_THETA) -> torch.Tensor:
    """A rotary table [max_position, P] float32: P/2 cosines then P/2 sines of
    position * theta^(-2i/P), evaluated in float64 on the CPU.  It stands in
    for the model's (YaRN-scaled) table, which is an input of the rotary
    step; any table of angles exercises the same arithmetic."""
    pos = torch.arange(max_position, dtype=torch.float64)[:, None]
    inv = theta ** (-torch.arange(0, P, 2, dtype=torch.float64) / P)
    ang = pos * inv[None, :]
    return torch.cat([torch.cos(ang), torch.sin(ang)], dim=1).to(torch.float32)


def token_positions(bt: Batch) -> torch.Tensor:
    """Position of every row of kv_c/k_pe within its request (int64 [T]);
    padded rows (slot -1) get position 0."""
    pos = torch.zeros(bt.slot_mapping.numel(), dtype=torch.int64)
    slots = bt.slot_mapping.cpu()
    real = torch.nonzero(slots >= 0).flatten()
    within = torch.cat([torch.arange(n, dtype=torch.int64) for n in bt.seq_lens_list]) if real.numel() else real
    pos[real] = within
    return pos.to(bt.slot_mapping.device)


# DeepSeek-V3 projection sizes around the decode: q_lora_rank, heads,
# qk_nope_head_dim, kv_lora_rank, v_head_dim, hidden size
V3_PROJ = dict(Lq=1536, N=128, P=128, Lkv=512, V=128, Hid=7168)


def projection_inputs(B: int, Lq: int, N: int, P: int, Lkv: int, V: int, Hid: int, seed: int = 3000,
                      device="cpu"):
    """Random bf16 projection weights in the pages' layouts and a q_c batch:
    W_Q [Lq, N, P], W_UK [Lkv, N, P], W_UV [Lkv, N, V], W_O [Hid, N, V] with
    N(0, 1/fan_in) entries, and q_c [B, Lq] ~ N(0, 1).  Drawn in float32 on a
    CPU generator and cast to bf16 (round to nearest even)."""
    g = torch.Generator().manual_seed(seed)
    bf = torch.bfloat16
    q_c = torch.randn((B, Lq), generator=g).to(bf)
    W_Q = (torch.randn((Lq, N, P), generator=g) / math.sqrt(Lq)).to(bf)
    W_UK = (torch.randn((Lkv, N, P), generator=g) / math.sqrt(P)).to(bf)
    W_UV = (torch.randn((Lkv, N, V), generator=g) / math.sqrt(Lkv)).to(bf)
    W_O = (torch.randn((Hid, N, V), generator=g) / math.sqrt(N * V)).to(bf)
    return {k: v.to(device) for k, v in dict(q_c=q_c, W_Q=W_Q, W_UK=W_UK, W_UV=W_UV, W_O=W_O).items()}
