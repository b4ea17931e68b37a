"""Pins for the absorbed projections: the linear layer against pure-Python
brute force, and absorption itself -- by associativity, the absorbed weight
applied once equals the two-step (up-projection per head, then projection)
path that the pages start from."""

import math

import numpy as np

from oracle import mla_oracle as O


def test_linear_brute_force():
    rng = np.random.default_rng(1)
    A = rng.standard_normal((3, 7)).astype(np.float32)
    W = rng.standard_normal((5, 7)).astype(np.float32)
    C = O.linear(A, W, "f32")
    for m in range(3):
        for n in range(5):
            assert abs(C[m, n] - math.fsum(float(A[m, k]) * float(W[n, k]) for k in range(7))) < 1e-12


def test_linear_reads_bf16_bits():
    rng = np.random.default_rng(2)
    a = rng.standard_normal((2, 32)).astype(np.float32)
    w = rng.standard_normal((3, 32)).astype(np.float32)
    ab, wb = O.f32_to_bf16_bits_rne(a), O.f32_to_bf16_bits_rne(w)
    C = O.linear(ab, wb, "bf16")
    assert np.max(np.abs(C - O.bf16_bits_to_f64(ab) @ O.bf16_bits_to_f64(wb).T)) == 0


def test_q_absorption_equals_two_step_path():
    rng = np.random.default_rng(3)
    B, Lq, N, P, Lkv = 4, 24, 3, 8, 16
    q_c = rng.standard_normal((B, Lq))
    W_Q = rng.standard_normal((Lq, N, P))
    W_UK = rng.standard_normal((Lkv, N, P))
    Wa = O.absorb_q_weight(W_Q, W_UK)
    assert Wa.shape == (N * Lkv, Lq)
    absorbed = (q_c @ Wa.T).reshape(B, N, Lkv)
    assert np.max(np.abs(absorbed - O.q_nope_unabsorbed(q_c, W_Q, W_UK))) < 1e-11
    # one entry by hand: head 2, latent column 5 of request 1
    want = sum(sum(q_c[1, i] * W_Q[i, 2, p] for i in range(Lq)) * W_UK[5, 2, p] for p in range(P))
    assert abs(absorbed[1, 2, 5] - want) < 1e-11


def test_o_absorption_equals_two_step_path():
    rng = np.random.default_rng(4)
    B, N, Lkv, V, Hid = 3, 4, 16, 8, 10
    o = rng.standard_normal((B, N, Lkv))
    W_UV = rng.standard_normal((Lkv, N, V))
    W_O = rng.standard_normal((Hid, N, V))
    Wa = O.absorb_o_weight(W_UV, W_O)
    assert Wa.shape == (Hid, N * Lkv)
    absorbed = o.reshape(B, N * Lkv) @ Wa.T
    assert np.max(np.abs(absorbed - O.out_unabsorbed(o, W_UV, W_O))) < 1e-11
    want = sum(sum(o[2, n, l] * W_UV[l, n, v] for l in range(Lkv)) * W_O[7, n, v] for n in range(N) for v in range(V))
    assert abs(absorbed[2, 7] - want) < 1e-11
