"""The tiled online-softmax recurrence equals the oracle's three-step result (CPU).

The oracle evaluates attention as the plain three-step definition.  This test
runs the other route the pages describe -- the tiled forward of AIInfraGuide 6.2
"FlashAttention V2 explained", section 6 (the complete forward algorithm): for
each block of Br query rows, walk key blocks of Bc, keep the running maximum m,
the row sum l and the unnormalised output, rescale l and O by exp(m_old - m_new)
whenever the maximum moves, and divide by l once at the end with
LSE = m + ln l -- in fp64, and requires it to equal the oracle to 1e-12 for
Br, Bc in {1, 3, 16} with Bc not dividing Nk, causal and not, Nq != Nk.

Two readings the pseudocode leaves open are taken as the rest of the pages
fix them: causal visibility is bottom-right (key j visible to query i iff
j <= i + Nk - Nq; LLM Infra Atlas "FA2: parallelism", section 4), and a row whose
block holds no visible key keeps m = -inf and uses 0 as the exponent reference
(so exp(-inf - -inf) never occurs).  Masks are applied only to blocks that cross
the diagonal or lie past the key tail, and blocks past the diagonal are never
visited (section 5.3 of the same page): equality then also shows that the block
classification loses no visible key.

The variant that does not rescale l by exp(m_old - m_new) (KingOfEgg "Flash
Attention (4)", section 3.1 reports that omission as a real bug; one page says
the factor touches only the output accumulator) must fail.
"""
import itertools
import math

import numpy as np
import pytest
import torch

SEEDS = {(7, 50): 11, (33, 50): 12, (33, 33): 13, (50, 33): 14, (5, 1): 15}


def tiled_forward(q, k, v, causal, scale, Br, Bc, alpha_on_l=True, mask_everywhere=False):
    """fp64 tiled forward over one head: q [Nq, d], k and v [Nk, d] (float64)."""
    Nq, d = q.shape
    Nk = k.shape[0]
    off = Nk - Nq
    O = np.zeros((Nq, d))
    L = np.full(Nq, -np.inf)
    for i0 in range(0, Nq, Br):
        rows = np.arange(i0, min(Nq, i0 + Br))
        m = np.full(rows.size, -np.inf)
        l = np.zeros(rows.size)
        acc = np.zeros((rows.size, d))
        kv_end = Nk if not causal else max(0, min(Nk, rows[-1] + off + 1))   # later blocks fully masked
        for j0 in range(0, kv_end, Bc):
            cols = np.arange(j0, min(Nk, j0 + Bc))
            s = scale * (q[rows] @ k[cols].T)
            crosses = causal and cols[-1] > rows[0] + off
            if crosses or mask_everywhere:
                vis = np.ones_like(s, dtype=bool)
                if causal:
                    vis = cols[None, :] <= rows[:, None] + off
                s = np.where(vis, s, -np.inf)
            m_new = np.maximum(m, s.max(axis=1))
            ref = np.where(np.isneginf(m_new), 0.0, m_new)
            p = np.exp(s - ref[:, None])
            alpha = np.exp(m - ref)
            l = (alpha * l if alpha_on_l else l) + p.sum(axis=1)
            acc = alpha[:, None] * acc + p @ v[cols]
            m = m_new
        seen = l > 0
        O[rows[seen]] = acc[seen] / l[seen, None]
        L[rows[seen]] = m[seen] + np.log(l[seen])
    return O, L


def _inputs(Nq, Nk, d, seed, dtype=torch.float16):
    g = torch.Generator().manual_seed(seed)
    return [(torch.randn(shape, generator=g) * 1.5).to(dtype) for shape in ((1, 2, Nq, d), (1, 2, Nk, d), (1, 2, Nk, d))]


CASES = [(Nq, Nk, Br, Bc, causal)
         for (Nq, Nk), Br, Bc, causal in itertools.product([(7, 50), (33, 50), (33, 33), (50, 33), (5, 1)],
                                                           [1, 3, 16], [1, 3, 16], [False, True])]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "q{}k{}-Br{}-Bc{}-c{}".format(*c[:4], int(c[4])))
def test_tiled_recurrence_equals_oracle(oracle_lib, case):
    Nq, Nk, Br, Bc, causal = case
    d = 8
    scale = 1 / math.sqrt(d)
    q, k, v = _inputs(Nq, Nk, d, SEEDS[(Nq, Nk)])
    ro, rl = oracle_lib.attention(q, k, v, causal, scale, nthreads=1)
    sigma = float(np.float32(scale))
    for h in range(2):
        qd, kd, vd = (t[0, h].double().numpy() for t in (q, k, v))
        o, lse = tiled_forward(qd, kd, vd, causal, sigma, Br, Bc)
        assert np.array_equal(np.isneginf(lse), np.isneginf(rl[0, h])), "empty rows differ"
        fin = np.isfinite(lse)
        assert np.max(np.abs(o - ro[0, h]), initial=0.0) <= 1e-12
        assert np.max(np.abs(lse[fin] - rl[0, h][fin]), initial=0.0) <= 1e-12
        assert np.all(o[~fin] == 0)


@pytest.mark.parametrize("Br,Bc", [(1, 3), (3, 16), (16, 3), (3, 1)])
def test_masking_only_crossing_blocks_loses_nothing(Br, Bc):
    q, k, v = (t[0, 0].double().numpy() for t in _inputs(33, 50, 8, 21))
    a = tiled_forward(q, k, v, True, 0.35, Br, Bc)
    b = tiled_forward(q, k, v, True, 0.35, Br, Bc, mask_everywhere=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("Br,Bc", [(1, 3), (3, 16), (16, 3), (3, 1), (16, 16)])
@pytest.mark.parametrize("causal", [False, True])
def test_without_alpha_on_l_fails(oracle_lib, Br, Bc, causal):
    """Scores that grow along the keys move the maximum in every block, so a row
    sum that is not rescaled keeps stale terms and the result must differ."""
    Nq, Nk, d = 33, 50, 8
    q = torch.zeros((1, 1, Nq, d))
    k = torch.zeros((1, 1, Nk, d))
    q[..., 0] = 1.0
    k[0, 0, :, 0] = torch.arange(Nk) * 0.25
    v = torch.randn((1, 1, Nk, d), generator=torch.Generator().manual_seed(3))
    q, k, v = q.half(), k.half(), v.half()
    ro, rl = oracle_lib.attention(q, k, v, causal, 1.0, nthreads=1)
    args = [t[0, 0].double().numpy() for t in (q, k, v)]
    good = tiled_forward(*args, causal, 1.0, Br, Bc)
    bad = tiled_forward(*args, causal, 1.0, Br, Bc, alpha_on_l=False)
    assert np.max(np.abs(good[0] - ro[0, 0])) <= 1e-12 and np.max(np.abs(good[1] - rl[0, 0])) <= 1e-12
    if Bc >= Nk:
        pytest.skip("one key block: the maximum never moves")
    assert np.max(np.abs(bad[0] - ro[0, 0])) > 1e-3, "dropping alpha on l must change O"
    assert np.max(np.abs(bad[1] - rl[0, 0])) > 1e-3, "dropping alpha on l must change LSE"
