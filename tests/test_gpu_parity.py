"""GPU parity: the HIP library through its C ABI against the fp64 oracle.

Small shapes (several tiles plus ragged tails) are compared on every output
element; the named workloads are compared at full size through the same calls
the benchmark times (every row of the tiny, prefill_d64, causal_d128 and
decode workloads; four whole heads and samples of every other head of
long_causal).  Two invariants of the method are checked on the GPU without the
oracle: key-shift invariance and value-shift equivariance.
"""
import math

import numpy as np
import pytest
import torch

from exact_attention_22_amd import fa
from exact_attention_22_amd.inputs import BY_NAME, WORKLOADS, make_partials, make_qkv
from tests import parity

pytestmark = pytest.mark.gpu
F16, BF16 = torch.float16, torch.bfloat16


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def rnd(shape, dtype, seed, mult=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * mult).to(dtype)


def say(msg):
    print(f"[case] {msg}", flush=True)


SMALL = [  # B, H, Nq, Nk, d, causal, dtype
    (1, 1, 128, 128, 64, False, F16),
    (1, 2, 129, 200, 64, False, F16),
    (2, 1, 257, 257, 128, True, F16),
    (1, 2, 300, 300, 128, True, BF16),
    (1, 1, 1, 77, 128, False, F16),
    (1, 1, 1, 1, 64, True, F16),
    (1, 1, 17, 1, 64, False, BF16),
    (1, 2, 100, 333, 128, True, F16),     # Nq < Nk: bottom-right diagonal
    (1, 1, 333, 100, 64, True, BF16),     # Nq > Nk: leading rows see nothing
    (1, 1, 127, 129, 64, True, F16),
    (3, 2, 64, 65, 128, False, BF16),
    (1, 1, 1000, 1000, 128, True, BF16),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "x".join(map(str, c[:5])) + f"-c{int(c[5])}-{str(c[6])[-4:]}")
def test_fwd_small(dev, oracle_lib, case):
    B, H, Nq, Nk, d, causal, dt = case
    q, k, v = rnd((B, H, Nq, d), dt, 1), rnd((B, H, Nk, d), dt, 2), rnd((B, H, Nk, d), dt, 3)
    say(f"fa_fwd {case}")
    o, lse = fa.fwd(q.to(dev), k.to(dev), v.to(dev), causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle_lib.attention(q, k, v, causal, 1 / math.sqrt(d))
    parity.check(o, lse, ro, rl, dt, f"fwd {case}")


# Shapes that take 256-row workgroups of eight wavefronts: at d = 128 from 2048
# keys on with at least 128 such workgroups, at d = 64 without the mask with at
# least 256 of them; tails ragged against both 256 rows and 64 keys.
WIDE = [  # B, H, H_kv, Nq, Nk, d, causal, dtype
    (1, 32, 32, 2100, 2100, 128, True, F16),
    (1, 32, 32, 1900, 2300, 128, True, BF16),    # Nq < Nk: bottom-right diagonal
    (1, 16, 16, 2200, 2049, 128, False, F16),
    (2, 16, 16, 2000, 2000, 64, False, F16),
    (1, 32, 32, 2049, 777, 64, False, BF16),
    (1, 32, 8, 2100, 2100, 64, False, F16),      # grouped K/V heads
    (1, 32, 8, 2100, 2100, 128, True, BF16),
]


@pytest.mark.parametrize("case", WIDE, ids=lambda c: "x".join(map(str, c[:6])) + f"-c{int(c[6])}-{str(c[7])[-4:]}")
def test_fwd_wide(dev, oracle_lib, case):
    B, H, Hkv, Nq, Nk, d, causal, dt = case
    q, k, v = rnd((B, H, Nq, d), dt, 11), rnd((B, Hkv, Nk, d), dt, 12), rnd((B, Hkv, Nk, d), dt, 13)
    say(f"fa_fwd{'_gqa' if Hkv != H else ''} 8-wavefront workgroups {case}")
    if Hkv == H:
        o, lse = fa.fwd(q.to(dev), k.to(dev), v.to(dev), causal=causal)
    else:
        o, lse = fa.fwd_gqa(q.to(dev), k.to(dev), v.to(dev), causal=causal)
    torch.cuda.synchronize()
    if Hkv == H:
        ro, rl = oracle_lib.attention(q, k, v, causal, 1 / math.sqrt(d))
    else:
        ro, rl = oracle_lib.attention_gqa(q, k, v, causal, 1 / math.sqrt(d))
    parity.check(o, lse, ro, rl, dt, f"wide {case}")


@pytest.mark.parametrize("scale", [0.0, -0.3, 2.5])
def test_fwd_scales(dev, oracle_lib, scale):
    B, H, N, d = 1, 2, 130, 64
    q, k, v = (rnd((B, H, N, d), F16, s) for s in (4, 5, 6))
    for causal in (False, True):
        say(f"fa_fwd scale={scale} causal={causal}")
        o, lse = fa.fwd(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale)
        torch.cuda.synchronize()
        ro, rl = oracle_lib.attention(q, k, v, causal, scale)
        parity.check(o, lse, ro, rl, F16, f"scale {scale} causal {causal}")


def test_fwd_closed_forms(dev):
    """Identical keys give the running mean of V; the first causal row is v_0."""
    B, H, N, d = 1, 2, 200, 128
    q = rnd((B, H, N, d), F16, 7)
    k = rnd((B, H, 1, d), F16, 8).expand(B, H, N, d).contiguous()
    v = rnd((B, H, N, d), F16, 9)
    say("fa_fwd identical keys")
    o, lse = fa.fwd(q.to(dev), k.to(dev), v.to(dev), causal=True)
    torch.cuda.synchronize()
    vd = v.double()
    running_mean = vd.cumsum(2) / torch.arange(1, N + 1, dtype=torch.float64)[:, None]
    assert (o.cpu().double() - running_mean).abs().max().item() <= 2e-3
    s = (q.double() * k.double()).sum(-1) / math.sqrt(d)
    exp_l = s + torch.log(torch.arange(1, N + 1, dtype=torch.float64))
    assert ((lse.cpu().double() - exp_l).abs() / exp_l.abs().clamp(min=1)).max().item() <= 1e-4
    assert torch.equal(o.cpu()[:, :, 0], v[:, :, 0]), "first causal row must be exactly v_0"


def test_fwd_deterministic_and_in_bounds(dev):
    B, H, Nq, Nk, d = 2, 2, 190, 190, 128
    q, k, v = (rnd((B, H, n, d), BF16, s).to(dev) for n, s in ((Nq, 10), (Nk, 11), (Nk, 12)))
    pad = 4096
    o_buf = torch.full((B * H * Nq * d + pad,), 12345.0, dtype=BF16, device=dev)
    l_buf = torch.full((B * H * Nq + pad,), 777.0, dtype=torch.float32, device=dev)
    o = o_buf[: B * H * Nq * d].view(B, H, Nq, d)
    l = l_buf[: B * H * Nq].view(B, H, Nq)
    say("fa_fwd canary")
    fa.fwd(q, k, v, causal=True, out=o, lse=l)
    o2, l2 = fa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.all(o_buf[B * H * Nq * d:] == 12345.0) and torch.all(l_buf[B * H * Nq:] == 777.0)
    assert torch.equal(o, o2) and torch.equal(l, l2), "two runs differ"


# Rows compared per prefill workload: every row of tiny, prefill_d64 and
# causal_d128; for long_causal four whole heads (0, 11, 22, 31: 32,768 rows) plus
# the first, last and 16 seeded random rows of every other head.
LONG_HEADS = (0, 11, 22, 31)


def long_causal_rows(w):
    rng = np.random.default_rng(17)
    whole = [np.arange(h * w.Nq, (h + 1) * w.Nq) for h in LONG_HEADS]
    rest = np.array([h for h in range(w.B * w.H) if h not in LONG_HEADS])
    some = [rest * w.Nq, rest * w.Nq + w.Nq - 1, np.repeat(rest, 16) * w.Nq + rng.integers(0, w.Nq, 16 * rest.size)]
    return np.unique(np.concatenate(whole + some))


@pytest.mark.parametrize("w", [w for w in WORKLOADS if not w.splits and not w.H_kv and not w.seqlens], ids=lambda w: w.name)
def test_workload_prefill(dev, oracle_lib, w):
    say(f"workload {w.name} inputs")
    q, k, v = make_qkv(w, device=dev)
    say(f"workload {w.name} fa_fwd")
    o, lse = fa.fwd(q, k, v, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    rows = long_causal_rows(w) if w.name == "long_causal" else None
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    say(f"workload {w.name} oracle ({'all' if rows is None else len(rows)} rows)")
    ro, rl = oracle_lib.attention(qc, kc, vc, w.causal, w.scale, rows=rows)
    if rows is None:
        parity.check(o, lse, ro, rl, w.dtype, f"{w.name} (every row)")
    else:
        idx = torch.from_numpy(rows)
        parity.check(o.reshape(-1, w.d).cpu()[idx], lse.reshape(-1).cpu()[idx], ro, rl, w.dtype,
                     f"{w.name} ({len(rows)} rows: {len(LONG_HEADS)} whole heads + samples of the rest)")


def grid(shape, step, lo, hi, seed, dtype):
    """Values on a grid of `step` in [lo, hi], exact in fp16 and bf16 here."""
    g = torch.Generator().manual_seed(seed)
    n = torch.randint(int(round(lo / step)), int(round(hi / step)) + 1, shape, generator=g)
    return (n.double() * step).to(dtype)


@pytest.mark.parametrize("dt", [F16, BF16], ids=["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_key_shift_invariance(dev, dt, causal):
    """Adding one vector u to every key adds sigma q_i.u to every score of row i:
    O is unchanged and LSE_i moves by exactly sigma q_i.u (Ringi, "Lecture 25",
    section 2.1: softmax is invariant to a per-row constant).  Queries are
    positive and u = 16 in every coordinate, so the shift is about +100 per row
    and exp of an unshifted score would overflow fp32: the maximum subtraction
    is exercised.  Keys and u lie on a grid of 1/8, so K + u is exact."""
    B, H, N, d = 1, 2, 777, 128
    q = grid((B, H, N, d), 1 / 8, 0.0, 1.5, 61, dt)
    k = grid((B, H, N, d), 1 / 8, -2.0, 2.0, 62, dt)
    v = rnd((B, H, N, d), dt, 63)
    ks = (k.double() + 16.0).to(dt)
    assert torch.equal(ks.double(), k.double() + 16.0), "shifted keys must be exact"
    scale = 1 / math.sqrt(d)
    say(f"key shift invariance causal={causal} {dt}")
    o, lse = fa.fwd(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale)
    o2, lse2 = fa.fwd(q.to(dev), ks.to(dev), v.to(dev), causal=causal, scale=scale)
    torch.cuda.synchronize()
    shift = float(np.float32(scale)) * 16.0 * q.double().sum(-1)
    assert shift.min().item() > 89, "the shift must exceed exp's fp32 range (e^89 > 3.4e38)"
    do = (o2.double() - o.double()).abs().max().item()
    dl = ((lse2.double().cpu() - lse.double().cpu() - shift).abs() / lse2.double().cpu().abs().clamp(min=1)).max().item()
    print(f"[parity] key shift {dt} causal={causal} max|dO|={do:.3e} max rel dLSE={dl:.3e}", flush=True)
    assert do <= parity.O_TOL[dt], f"O changed by {do:.3e} under a key shift"
    assert dl <= parity.LSE_TOL, f"LSE moved by the wrong amount ({dl:.3e})"


@pytest.mark.parametrize("dt", [F16, BF16], ids=["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_value_shift_equivariance(dev, dt, causal):
    """O(V + 1 w^T) = O(V) + w^T, since each row's weights sum to one; LSE does
    not change.  V and w lie on a grid of 1/8 in [-2, 2] and [-1, 1], so V + w is
    exact."""
    B, H, N, d = 2, 1, 555, 64
    q, k = rnd((B, H, N, d), dt, 71), rnd((B, H, N, d), dt, 72)
    v = grid((B, H, N, d), 1 / 8, -2.0, 2.0, 73, dt)
    wv = grid((1, 1, 1, d), 1 / 8, -1.0, 1.0, 74, dt)
    vs = (v.double() + wv.double()).to(dt)
    assert torch.equal(vs.double(), v.double() + wv.double()), "shifted values must be exact"
    say(f"value shift equivariance causal={causal} {dt}")
    o, lse = fa.fwd(q.to(dev), k.to(dev), v.to(dev), causal=causal)
    o2, lse2 = fa.fwd(q.to(dev), k.to(dev), vs.to(dev), causal=causal)
    torch.cuda.synchronize()
    do = (o2.double().cpu() - o.double().cpu() - wv.double()).abs().max().item()
    print(f"[parity] value shift {dt} causal={causal} max|dO - w|={do:.3e}", flush=True)
    assert do <= parity.O_TOL[dt], f"O(V + w) - O(V) differs from w by {do:.3e}"
    assert torch.equal(lse, lse2), "LSE must not depend on V"


def test_workload_decode(dev, oracle_lib):
    w = BY_NAME["decode"]
    say("workload decode inputs")
    q, k, v = make_qkv(w, device=dev)
    say("workload decode fa_fwd_splitkv + combine")
    o, lse = fa.decode(q, k, v, num_splits=w.splits, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    ro, rl = oracle_lib.attention(qc, kc, vc, w.causal, w.scale)
    parity.check(o, lse, ro, rl, w.dtype, "decode (all rows)")


SPLIT_CASES = [  # B, H, Nq, Nk, d, causal, dtype
    (2, 2, 1, 1000, 128, False, F16),
    (1, 2, 1, 333, 64, True, BF16),
    (1, 1, 1, 20, 128, False, BF16),
    (1, 2, 70, 300, 128, True, F16),
    (1, 1, 129, 129, 64, False, BF16),
    (1, 1, 40, 20, 64, True, F16),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "x".join(map(str, c[:5])) + f"-c{int(c[5])}")
@pytest.mark.parametrize("S", [1, 2, 16, 17])
def test_splitkv(dev, oracle_lib, case, S):
    B, H, Nq, Nk, d, causal, dt = case
    q, k, v = rnd((B, H, Nq, d), dt, 21), rnd((B, H, Nk, d), dt, 22), rnd((B, H, Nk, d), dt, 23)
    scale = 1 / math.sqrt(d)
    say(f"fa_fwd_splitkv {case} S={S}")
    op, lp = fa.fwd_splitkv(q.to(dev), k.to(dev), v.to(dev), S, causal=causal)
    say(f"fa_splitkv_combine {case} S={S}")
    o, lse = fa.splitkv_combine(op, lp, dt)
    torch.cuda.synchronize()
    rop, rlp = oracle_lib.split_partials(q, k, v, causal, scale, S)
    parity.check(op, lp, rop, rlp, dt, f"partials {case} S={S}")
    ro, rl = oracle_lib.attention(q, k, v, causal, scale)
    parity.check(o, lse, ro, rl, dt, f"split+combine {case} S={S}")


@pytest.mark.parametrize("empty_every", [0, 3, 1])
@pytest.mark.parametrize("d,dt", [(64, F16), (128, BF16)])
@pytest.mark.parametrize("S", [5, 64, 67, 130])
def test_combine_alone(dev, oracle_lib, empty_every, d, dt, S):
    """Split counts below, at and past the 64 splits the combine weighs per pass
    and not a multiple of the 8 it loads per round; an empty split's partial row
    holds NaN, which must not reach the result (its weight is zero)."""
    B, H, Nq = 2, 3, 7
    op, lp = make_partials(S, B, H, Nq, d, seed=31, empty_every=empty_every)
    op[torch.isinf(lp)] = float("nan")
    say(f"fa_splitkv_combine partials S={S} d={d} empty_every={empty_every}")
    o, lse = fa.splitkv_combine(op.to(dev), lp.to(dev), dt)
    torch.cuda.synchronize()
    ro, rl = oracle_lib.combine(op.double().numpy(), lp.double().numpy())
    parity.check(o, lse, ro, rl, dt, f"combine alone d={d} empty_every={empty_every}")
