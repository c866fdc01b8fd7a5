"""GPU parity of the backward pass (fa_bwd, fa_bwd_gqa) through the C ABI against
the fp64 oracle.

The library's own forward supplies o and lse (the intended use); the oracle
computes exact gradients from q, k, v and dout alone.  Small shapes (several
tiles, ragged tails, Nq != Nk, rows that see no key, a single query row) are
compared on every element; the causal_d128 workload, a grouped-head causal
prefill and the benchmark's long_causal backward are compared at full size on
sampled query and key rows.
"""
import math

import numpy as np
import pytest
import torch

from exact_attention_22_amd import fa
from exact_attention_22_amd.inputs import BY_NAME, make_qkv
from tests import parity

pytestmark = pytest.mark.gpu
F16, BF16 = torch.float16, torch.bfloat16


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def rnd(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(dtype)


def say(msg):
    print(f"[case] {msg}", flush=True)


def run(dev, q, k, v, g, causal, scale=None):
    qd, kd, vd, gd = (t.to(dev) for t in (q, k, v, g))
    o, lse = fa.fwd(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, gd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


SMALL = [  # B, H, Nq, Nk, d, causal, dtype
    (1, 2, 128, 128, 64, False, F16),
    (1, 2, 200, 333, 128, True, BF16),
    (2, 1, 257, 257, 128, True, F16),
    (1, 1, 333, 100, 64, True, BF16),     # Nq > Nk: leading rows see no key
    (1, 1, 100, 333, 128, True, F16),     # Nq < Nk: bottom-right diagonal
    (1, 2, 64, 65, 128, False, BF16),
    (1, 1, 1, 77, 64, False, F16),
    (1, 1, 1000, 1000, 128, True, BF16),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "x".join(map(str, c[:5])) + f"-c{int(c[5])}-{('bf16' if c[6] == BF16 else 'f16')}")
def test_bwd_small(dev, oracle_lib, case):
    B, H, Nq, Nk, d, causal, dt = case
    q, k, v = rnd((B, H, Nq, d), dt, 1), rnd((B, H, Nk, d), dt, 2), rnd((B, H, Nk, d), dt, 3)
    g = rnd((B, H, Nq, d), dt, 4)
    say(f"fa_bwd {case}")
    dq, dk, dv = run(dev, q, k, v, g, causal)
    rq, rk, rv = oracle_lib.attention_bwd(q, k, v, g, causal, 1 / math.sqrt(d))
    parity.check_grads((dq, dk, dv), (rq, rk, rv), dt, f"bwd {case}")


@pytest.mark.parametrize("scale", [0.0, -0.3, 1.5])
def test_bwd_scales(dev, oracle_lib, scale):
    B, H, N, d = 1, 2, 150, 64
    q, k, v, g = (rnd((B, H, N, d), F16, s) for s in (5, 6, 7, 8))
    for causal in (False, True):
        say(f"fa_bwd scale={scale} causal={causal}")
        dq, dk, dv = run(dev, q, k, v, g, causal, scale=scale)
        rq, rk, rv = oracle_lib.attention_bwd(q, k, v, g, causal, scale)
        parity.check_grads((dq, dk, dv), (rq, rk, rv), F16, f"bwd scale {scale} causal {causal}")


WIDE_DQ = [  # B, H, N, causal, dtype: dQ workgroups of 256 rows (1024 keys or more, 256 such workgroups)
    (2, 32, 1100, False, BF16),
    (4, 32, 1500, True, F16),
]


@pytest.mark.parametrize("case", WIDE_DQ, ids=lambda c: "x".join(map(str, c[:3])) + f"-c{int(c[3])}-{('bf16' if c[4] == BF16 else 'f16')}")
def test_bwd_wide_dq_sampled(dev, oracle_lib, case):
    """Eight-wavefront dQ workgroups with ragged tails: the first and last rows of
    every head and 128 seeded random query and key rows against the oracle."""
    B, H, N, causal, dt = case
    d = 128
    q, k, v, g = (rnd((B, H, N, d), dt, s) for s in (21, 22, 23, 24))
    say(f"fa_bwd eight-wavefront dQ workgroups {case}")
    dq, dk, dv = run(dev, q, k, v, g, causal)
    rng = np.random.default_rng(N)
    heads = np.arange(B * H)
    qr = np.unique(np.concatenate([heads * N, heads * N + N - 1, rng.integers(0, B * H * N, 128)]))
    kr = np.unique(np.concatenate([heads * N, heads * N + N - 1, rng.integers(0, B * H * N, 128)]))
    rq, rk, rv = oracle_lib.attention_bwd(q, k, v, g, causal, 1 / math.sqrt(d), q_rows=qr, k_rows=kr)
    qi, ki = torch.from_numpy(qr).to(dev), torch.from_numpy(kr).to(dev)
    parity.check_grads((dq.reshape(-1, d)[qi], dk.reshape(-1, d)[ki], dv.reshape(-1, d)[ki]),
                       (rq, rk, rv), dt, f"bwd wide dQ {case} sampled")


def test_bwd_workload(dev, oracle_lib):
    """causal_d128 (B=4 H=16 N=2048 d=128 fp16 causal) at full size, sampled rows of two heads."""
    w = BY_NAME["causal_d128"]
    q, k, v = make_qkv(w)
    g = rnd(tuple(q.shape), w.dtype, 9)
    say(f"fa_bwd {w.name}")
    dq, dk, dv = run(dev, q, k, v, g, w.causal, scale=w.scale)
    rng = np.random.default_rng(11)
    heads = np.array([0, w.B * w.H - 1])
    qr = np.unique(np.concatenate([heads * w.Nq, heads * w.Nq + w.Nq - 1,
                                   heads[rng.integers(0, 2, 96)] * w.Nq + rng.integers(0, w.Nq, 96)]))
    kr = np.unique(np.concatenate([heads * w.Nk, heads * w.Nk + w.Nk - 1,
                                   heads[rng.integers(0, 2, 96)] * w.Nk + rng.integers(0, w.Nk, 96)]))
    rq, rk, rv = oracle_lib.attention_bwd(q, k, v, g, w.causal, w.scale, q_rows=qr, k_rows=kr)
    qi, ki = torch.from_numpy(qr).to(dev), torch.from_numpy(kr).to(dev)
    parity.check_grads((dq.reshape(-1, w.d)[qi], dk.reshape(-1, w.d)[ki], dv.reshape(-1, w.d)[ki]),
                       (rq, rk, rv), w.dtype, f"bwd {w.name} sampled")


GQA_SMALL = [  # B, H, H_kv, Nq, Nk, d, causal, dtype
    (1, 4, 2, 200, 200, 128, True, BF16),
    (2, 4, 1, 129, 300, 64, True, F16),      # MQA, Nq < Nk
    (1, 8, 2, 300, 129, 128, True, F16),     # Nq > Nk: leading rows see no key
    (1, 6, 3, 64, 65, 64, False, BF16),
    (1, 4, 4, 150, 150, 128, True, BF16),    # H_kv = H through the grouped entry point
    (1, 8, 1, 1, 77, 128, False, F16),
]


def run_gqa(dev, q, k, v, g, causal, scale=None):
    qd, kd, vd, gd = (t.to(dev) for t in (q, k, v, g))
    o, lse = fa.fwd_gqa(qd, kd, vd, causal=causal, scale=scale)
    grads = fa.bwd_gqa(qd, kd, vd, o, lse, gd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return grads


@pytest.mark.parametrize("case", GQA_SMALL, ids=lambda c: "x".join(map(str, c[:6])) + f"-c{int(c[6])}-{('bf16' if c[7] == BF16 else 'f16')}")
def test_bwd_gqa_small(dev, oracle_lib, case):
    B, H, H_kv, Nq, Nk, d, causal, dt = case
    q, g = rnd((B, H, Nq, d), dt, 21), rnd((B, H, Nq, d), dt, 22)
    k, v = rnd((B, H_kv, Nk, d), dt, 23), rnd((B, H_kv, Nk, d), dt, 24)
    say(f"fa_bwd_gqa {case}")
    grads = run_gqa(dev, q, k, v, g, causal)
    refs = oracle_lib.attention_bwd_gqa(q, k, v, g, causal, 1 / math.sqrt(d))
    parity.check_grads(grads, refs, dt, f"bwd gqa {case}")


def test_bwd_gqa_matches_bwd_when_ungrouped(dev):
    """With H_kv = H, fa_bwd_gqa and fa_bwd run the same kernels in the same order:
    the gradients agree bit for bit."""
    B, H, N, d = 1, 3, 260, 128
    q, k, v, g = (rnd((B, H, N, d), BF16, s).to(dev) for s in (31, 32, 33, 34))
    say("fa_bwd_gqa vs fa_bwd, H_kv = H")
    o, lse = fa.fwd(q, k, v, causal=True)
    a = fa.bwd(q, k, v, o, lse, g, causal=True)
    b = fa.bwd_gqa(q, k, v, o, lse, g, causal=True)
    torch.cuda.synchronize()
    for x, y, n in zip(a, b, ("dq", "dk", "dv")):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16)), n


def test_bwd_gqa_workload(dev, oracle_lib):
    """Grouped-head causal prefill at full size (B=1, H=32, H_kv=8, N=4096, d=128,
    bf16), sampled rows of the first and last query and K/V heads."""
    B, H, H_kv, N, d, dt = 1, 32, 8, 4096, 128, BF16
    q, g = rnd((B, H, N, d), dt, 41), rnd((B, H, N, d), dt, 42)
    k, v = rnd((B, H_kv, N, d), dt, 43), rnd((B, H_kv, N, d), dt, 44)
    scale = 1 / math.sqrt(d)
    say(f"fa_bwd_gqa B={B} H={H} H_kv={H_kv} N={N} d={d} bf16 causal")
    dq, dk, dv = run_gqa(dev, q, k, v, g, True)
    rng = np.random.default_rng(12)
    qh, kh = np.array([0, B * H - 1]), np.array([0, B * H_kv - 1])
    qr = np.unique(np.concatenate([qh * N, qh * N + N - 1, qh[rng.integers(0, 2, 48)] * N + rng.integers(0, N, 48)]))
    kr = np.unique(np.concatenate([kh * N, kh * N + N - 1, kh[rng.integers(0, 2, 48)] * N + rng.integers(0, N, 48)]))
    rq, rk, rv = oracle_lib.attention_bwd_gqa(q, k, v, g, True, scale, q_rows=qr, k_rows=kr)
    qi, ki = torch.from_numpy(qr).to(dev), torch.from_numpy(kr).to(dev)
    parity.check_grads((dq.reshape(-1, d)[qi], dk.reshape(-1, d)[ki], dv.reshape(-1, d)[ki]),
                       (rq, rk, rv), dt, "bwd gqa H32/8 N4096 sampled")


def test_bwd_long_causal_benchmark_shape(dev, oracle_lib):
    """The backward the benchmark times: long_causal (B=1 H=32 N=8192 d=128 bf16
    causal, inputs N(0,1) x 0.5), dO ~ N(0,1), o and lse from fa_fwd.  Rows from
    all 32 heads: 8 random query rows and the last query row per head (dQ); for
    dK and dV the last key and 2 random keys among the last 1024 per head, plus
    keys near the start of 4 heads, whose gradients sum over almost every query
    row (the oracle needs the statistics of every query row that sees a key)."""
    w = BY_NAME["long_causal"]
    q, k, v = make_qkv(w)
    g = rnd(tuple(q.shape), w.dtype, 19)
    say(f"fa_bwd {w.name} (the benchmark's shape)")
    dq, dk, dv = run(dev, q, k, v, g, w.causal, scale=w.scale)
    G = w.B * w.H
    heads = np.arange(G)
    rng = np.random.default_rng(23)
    qr = np.unique(np.concatenate([heads * w.Nq + w.Nq - 1, np.repeat(heads, 8) * w.Nq + rng.integers(0, w.Nq, 8 * G)]))
    early = np.array([0 * w.Nk + 0, 9 * w.Nk + 5, 20 * w.Nk + 3000, 31 * w.Nk + 129])
    kr = np.unique(np.concatenate([heads * w.Nk + w.Nk - 1, early,
                                   np.repeat(heads, 2) * w.Nk + w.Nk - 1 - rng.integers(0, 1024, 2 * G)]))
    say(f"oracle bwd {len(qr)} query rows, {len(kr)} key rows")
    rq, rk, rv = oracle_lib.attention_bwd(q, k, v, g, w.causal, w.scale, q_rows=qr, k_rows=kr)
    qi, ki = torch.from_numpy(qr).to(dev), torch.from_numpy(kr).to(dev)
    parity.check_grads((dq.reshape(-1, w.d)[qi], dk.reshape(-1, w.d)[ki], dv.reshape(-1, w.d)[ki]),
                       (rq, rk, rv), w.dtype, f"bwd {w.name} (all 32 heads sampled)")
