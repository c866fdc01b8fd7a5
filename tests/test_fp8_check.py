"""The FP8 output checks (tests/fp8_check.py) on the CPU, at long_causal's shape.

An O emulating the kernel's arithmetic (P lifted and rounded to e4m3 with round
to nearest even, fp32 row sum of the unrounded weights, V scale applied once,
bf16 output) must pass; an all-zero O, an O with the V scale dropped and an O
whose P was truncated instead of rounded must fail.  The inputs are long_causal's
shape and distribution (one head, N = 8192, d = 128, N(0,1) x 0.5 in bf16,
quantized per block by the oracle's quantizer).
"""
import math

import numpy as np
import pytest
import torch

from oracle import fp8 as ofp8
from tests import fp8_check

N, D = 8192, 128


@pytest.fixture(scope="module")
def case():
    g = torch.Generator().manual_seed(4242)
    q, k, v = ((torch.randn((1, N, D), generator=g) * 0.5).bfloat16() for _ in range(3))
    q8, qd = ofp8.quantize_blocks(q, 128)
    k8, kd = ofp8.quantize_blocks(k, 128)
    v8, vd = ofp8.quantize_blocks(v, N)
    shp = (1, 1, N, D)
    q8, k8, v8 = q8.reshape(shp), k8.reshape(shp), v8.reshape(shp)
    qd, kd, vd = qd.reshape(1, 1, -1), kd.reshape(1, 1, -1), vd.reshape(1, 1)
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 1, 2, 7, 100, 1000, 4000, N - 1], rng.integers(0, N, 40)]))
    scale = 1 / math.sqrt(D)
    ro, rl, A, U, R = ofp8.attention_fp8(q8, k8, v8, qd, kd, vd, True, scale, rows=rows, spread=True)
    return dict(q8=q8, k8=k8, v8=v8, qd=qd, kd=kd, vd=vd, rows=rows, scale=scale, ro=ro, A=A, U=U, R=R)


def emulate(c, lift_log2, rounding):
    """O as the kernel forms it: P = 2^lift * exp(s - m) rounded to e4m3
    ('nearest': ties to even; 'truncate': toward zero), l summed from the
    unrounded weights, O = (sum P v8) / (2^lift l) * v_scale, rounded to bf16."""
    kx = ofp8.dequantize(c["k8"][0], c["kd"][0], 128)[0]
    v8 = ofp8.decode_e4m3(c["v8"][0, 0])
    sigma = float(np.float32(c["scale"]))
    out = np.zeros((len(c["rows"]), D))
    pos = ofp8.decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    for r, i in enumerate(c["rows"]):
        qrow = ofp8.decode_e4m3(c["q8"][0, 0, i]) * float(c["qd"][0, 0, i // 128])
        s = sigma * (kx[: i + 1] @ qrow)
        p = np.exp(s - s.max())
        lifted = p * 2.0 ** lift_log2
        if rounding == "nearest":
            pr = ofp8.decode_e4m3(ofp8.encode_e4m3(lifted))
        else:
            pr = pos[np.searchsorted(pos, lifted, side="right") - 1]
        out[r] = (pr @ v8[: i + 1]) / (2.0 ** lift_log2 * np.sum(p)) * float(c["vd"][0, 0])
    return torch.from_numpy(out).bfloat16().double().numpy()


@pytest.mark.parametrize("lift", [4, 8])
def test_kernel_like_output_passes(case, lift):
    o = emulate(case, lift, "nearest")
    fp8_check.check(o, case["ro"], case["A"], case["U"], case["R"], f"emulated kernel, lift 2^{lift}")


def test_zero_output_fails(case):
    mz2, _ = fp8_check.statistical(np.zeros_like(case["ro"]), case["ro"], case["R"])
    assert mz2 > 50 * fp8_check.MEAN_Z2_BAR, f"O = 0 must fail the statistical check (mean z^2 {mz2:.2f})"
    with pytest.raises(AssertionError):
        fp8_check.check(np.zeros_like(case["ro"]), case["ro"], case["A"], case["U"], case["R"], "O = 0")


def test_dropped_v_scale_fails(case):
    bad = case["ro"] / float(case["vd"][0, 0])
    with pytest.raises(AssertionError):
        fp8_check.check(bad, case["ro"], case["A"], case["U"], case["R"], "V scale dropped")
    mz2, _ = fp8_check.statistical(bad, case["ro"], case["R"])
    assert mz2 > 1e3


def test_truncated_p_fails(case):
    o = emulate(case, 4, "truncate")
    mz2, _ = fp8_check.statistical(o, case["ro"], case["R"])
    assert mz2 > fp8_check.MEAN_Z2_BAR, f"P truncated toward zero must fail (mean z^2 {mz2:.3f})"


def test_zero_output_was_accepted_by_worst_case_alone(case):
    """Why the statistical check exists: at this shape the worst-case bound alone
    accepts O = 0 on most compared elements."""
    a = np.zeros_like(case["ro"])
    bound = 2.0 ** -4 * case["A"] + 2.0 ** -14 * case["U"] + 2.0 ** -8 * np.abs(case["ro"]) + 1e-5 * case["A"]
    assert np.mean(np.abs(a - case["ro"]) <= bound) > 0.5
