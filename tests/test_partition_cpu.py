"""The balanced partition's slot rule, modelled on the host: on random
batches, the pieces (chunk c, request b) get distinct slots c + b below
B * S, each request's pieces take consecutive slots, and the pieces tile every
request exactly -- the invariants the two decode stages rely on."""

import numpy as np
import pytest


def pieces(lens, S, G):
    pad = [(n + 31) // 32 * 32 for n in lens]
    total = sum(pad)
    G = max(1, min(G, len(lens) * (S - 1)))
    Q = max(32, ((total + G - 1) // G + 31) // 32 * 32)
    out = []
    start = 0
    for b, n in enumerate(lens):
        if n > 0:
            for c in range(start // Q, (start + n - 1) // Q + 1):
                a = max(c * Q - start, 0)
                e = min((c + 1) * Q - start, n)
                out.append((b, c, a, e, c + b))
        start += pad[b]
    return out, G


@pytest.mark.parametrize("seed", range(40))
def test_slots_distinct_bounded_and_tiling(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 70))
    S = int(rng.integers(2, 40))
    lens = [int(x) for x in rng.integers(0, 20000, B)]
    if rng.random() < 0.3:
        lens[int(rng.integers(0, B))] = int(rng.integers(50000, 300000))
    G = int(rng.integers(1, 600))
    ps, G = pieces(lens, S, G)
    slots = [p[4] for p in ps]
    assert len(set(slots)) == len(slots)
    assert all(0 <= s < B * S for s in slots)
    for b, n in enumerate(lens):
        mine = sorted((p for p in ps if p[0] == b), key=lambda p: p[2])
        if n == 0:
            assert not mine
            continue
        assert [p[4] for p in mine] == list(range(mine[0][4], mine[0][4] + len(mine)))
        assert mine[0][2] == 0 and mine[-1][3] == n
        assert all(mine[i][3] == mine[i + 1][2] for i in range(len(mine) - 1))
        assert all(p[2] < p[3] for p in mine)
    assert max(p[1] for p in ps) < G
