"""The skinny bf16 linear layer of the absorbed projections, against the
oracle's float64 product: small shapes spanning ragged feature blocks, one to
two 64-row launches and the split-K path; the DeepSeek-V3 q-side and
output-side absorbed shapes on sampled features; and absorption end to end.

Tolerance, from the arithmetic: the products of two bf16 values are exact in
fp32; the sum is accumulated in fp32 over K/32 matrix-core steps (each adding
32 products) plus up to `splits` partials, so |error| <= (K/16 + 16) * 2^-24 *
sum_k |a_k w_k| with a margin of two; a bf16 output adds half a unit in the
last place of the result."""

import numpy as np
import pytest
import torch

import mla_paged_decode_concat_amd as M
from mla_paged_decode_concat_amd import workloads as W
from oracle import mla_oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _print(*a):
    print(*a, flush=True)


def _half_ulp_bf16(x):
    mag = np.maximum(np.abs(x), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(mag)) - 8)


def _check(C, A_bits, W_bits, out_dtype, cols=None):
    """C (GPU) against the oracle on the given feature columns."""
    Wb = W_bits if cols is None else W_bits[cols]
    exact = O.linear(A_bits, Wb, "bf16")
    absum = np.abs(O.to_f64(A_bits, "bf16")) @ np.abs(O.to_f64(Wb, "bf16")).T
    K = A_bits.shape[1]
    bound = (K / 16 + 16) * 2.0 ** -24 * absum
    got = C.float().cpu().numpy().astype(np.float64)
    if cols is not None:
        got = got[:, cols]
    if out_dtype == torch.bfloat16:
        bound = bound + _half_ulp_bf16(exact)
    err = np.abs(got - exact)
    assert np.all(np.isfinite(got))
    assert np.all(err <= bound), f"max excess {np.max(err - bound):.3g}"
    return float(err.max())


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("Mr,N,K", [(1, 16, 64), (5, 48, 192), (16, 272, 640), (33, 1024, 1536),
                                    (64, 256, 256), (100, 96, 4096), (7, 16, 8192)])
def test_linear_small_against_oracle(Mr, N, K, out_dtype):
    g = torch.Generator().manual_seed(Mr * 7 + N + K)
    A = torch.randn((Mr, K), generator=g).to(torch.bfloat16)
    Wt = torch.randn((N, K), generator=g).to(torch.bfloat16)
    _print(f"[linear] M={Mr} N={N} K={K} out={out_dtype} workspace={M.linear_workspace_bytes(Mr, N, K)}")
    C = M.linear(A.to(DEV), Wt.to(DEV), out_dtype)
    torch.cuda.synchronize()
    _check(C, W.bits(A), W.bits(Wt), out_dtype)


def test_linear_strided_rows():
    """Row strides larger than K (views into wider buffers)."""
    g = torch.Generator().manual_seed(1)
    A_store = torch.randn((20, 1600), generator=g).to(torch.bfloat16).to(DEV)
    W_store = torch.randn((64, 1600), generator=g).to(torch.bfloat16).to(DEV)
    C_store = torch.zeros((20, 80), dtype=torch.float32, device=DEV)
    A, Wt, C = A_store[:, :1536], W_store[:, 8:1544], C_store[:, :64]
    M.linear(A, Wt, torch.float32, out=C)
    torch.cuda.synchronize()
    _check(C, W.bits(A), W.bits(Wt), torch.float32)
    assert torch.all(C_store[:, 64:] == 0)


@pytest.mark.parametrize("which", ["q", "o"])
def test_linear_v3_absorbed_shapes_sampled(which):
    """DeepSeek-V3 per-GPU shapes, batch 64: q_c [64, 1536] -> [64, 128*512]
    (one feature block per CU, no split) and the decode output [64, 128*512]
    -> [64, 7168] (split K); random weights, features sampled."""
    g = torch.Generator(device=DEV).manual_seed(5)
    Mr, N, K = (64, 65536, 1536) if which == "q" else (64, 7168, 65536)
    A = torch.randn((Mr, K), generator=g, device=DEV).to(torch.bfloat16)
    Wt = (torch.randn((N, K), generator=g, device=DEV) / K ** 0.5).to(torch.bfloat16)
    _print(f"[linear] V3 {which}: M={Mr} N={N} K={K} workspace={M.linear_workspace_bytes(Mr, N, K)}")
    C = M.linear(A, Wt, torch.bfloat16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    cols = np.sort(rng.choice(N, size=512, replace=False))
    cols[0], cols[-1] = 0, N - 1
    cols_t = torch.from_numpy(cols).to(DEV)
    Ws = W.bits(Wt.index_select(0, cols_t))
    err = _check(C.index_select(1, cols_t), W.bits(A), Ws, torch.bfloat16, cols=None)
    _print(f"[linear] max |err| {err:.3g}")


def test_absorbed_q_projection_end_to_end():
    """q_nope by the absorbed weight (computed once from W_Q and W_UK, as the
    weights are prepared after loading, and stored in bf16) against the
    two-step path in float64.  The bound adds the rounding of the absorbed
    weight to bf16: sum_k |q_c[k]| * half a bf16 unit of W_Q_UK[n, k]."""
    d = W.projection_inputs(B=8, Lq=256, N=4, P=32, Lkv=512, V=32, Hid=64)
    q_c, W_Q, W_UK = (O.to_f64(W.bits(d[k]), "bf16") for k in ("q_c", "W_Q", "W_UK"))
    Wa = O.absorb_q_weight(W_Q, W_UK)                       # [N * Lkv, Lq] float64
    Wa_bits = O.f32_to_bf16_bits_rne(Wa.astype(np.float32))
    want = O.q_nope_unabsorbed(q_c, W_Q, W_UK).reshape(8, -1)
    Wa_t = torch.from_numpy(Wa_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    C = M.linear(d["q_c"].to(DEV), Wa_t, torch.float32)
    torch.cuda.synchronize()
    got = C.cpu().numpy().astype(np.float64)
    wround = np.abs(q_c) @ _half_ulp_bf16(Wa).T
    acc = (256 / 16 + 16) * 2.0 ** -24 * (np.abs(q_c) @ np.abs(O.to_f64(Wa_bits, "bf16")).T)
    assert np.all(np.abs(got - want) <= wround + acc + 2.0 ** -24 * np.abs(want))
