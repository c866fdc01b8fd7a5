"""fp64 CPU reference for the FP8 (e4m3) attention forward with per-block scales.

TEST INFRASTRUCTURE ONLY: imported by the tests and the smoke check -- never by
the product path.  It shares no code with the HIP kernels.

What the pages fix (Ringi, "Lecture 25", section 5.4, and the FP8 underflow
question of section 8.3): Q K^T and P V run on FP8 (e4m3) operands, and
per-block scale factors keep the data inside the narrow e4m3 range.  The reference is the
plain definition of attention evaluated on the *dequantized* inputs:

    x = code * descale(block of the row)          (exact, in double)
    S = scale * Q K^T,  P = softmax(S + mask),  O = P V,  LSE = m + ln l

with the blocks of this library: 128 query rows per Q scale, 128 keys per K
scale, one V scale per (batch, K/V head).

The e4m3 format (OCP 8-bit floating point, "E4M3FN"): 1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits; exponent 0 holds subnormals m * 2^-9; the
pattern S.1111.111 is NaN; there are no infinities; the largest finite value is
1.75 * 2^8 = 448.

Quantization (the library's block quantizer, reproduced in the same fp32 steps
so that its integer codes can be compared exactly): per block, amax = max |x|
in fp32; descale = amax / 448 (1 when amax is 0); each value is x * (448 /
amax) in fp32, clamped to [-448, 448] and rounded to the nearest e4m3 value,
ties to the even code.
"""
import math

import numpy as np
import torch

E4M3_MAX = 448.0
Q_BLOCK = 128      # query rows per Q scale
K_BLOCK = 128      # keys per K scale


def decode_e4m3(codes):
    """e4m3 codes (uint8 array) -> float64 values, from the format definition."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    expo = (c >> 3) & 0xF
    mant = c & 0x7
    normal = sign * np.ldexp(1.0 + mant / 8.0, expo - 7)
    sub = sign * np.ldexp(mant.astype(np.float64), -9)
    out = np.where(expo == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


# the 127 non-negative finite values, ascending, indexed by code 0x00..0x7E
_POS = decode_e4m3(np.arange(0x7F, dtype=np.uint8))


def encode_e4m3(x):
    """float values (already within [-448, 448]) -> nearest e4m3 code, ties to
    the even code (the one whose lowest mantissa bit is 0); the sign bit is the
    input's."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(a > E4M3_MAX) or np.any(np.isnan(a)):
        raise ValueError("encode_e4m3 takes finite values within [-448, 448]")
    hi = np.searchsorted(_POS, a, side="left")          # first value >= a
    hi = np.minimum(hi, len(_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - _POS[lo], _POS[hi] - a
    pick = np.where(d_hi < d_lo, hi, lo)
    tie = d_hi == d_lo
    pick = np.where(tie & (lo != hi), np.where(hi % 2 == 0, hi, lo), pick)
    pick = np.where(a == _POS[hi], hi, pick)
    code = pick.astype(np.uint8)
    # the sign bit follows the input's sign, negative zero included
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def quantize_blocks(x, block_rows):
    """Quantize x [G, N, d] (fp16/bf16 tensor or array) block by block along N.

    Returns codes uint8 [G, N, d] and descale float32 [G, ceil(N / block_rows)],
    following the fp32 steps in the module docstring."""
    xf = np.asarray(torch.as_tensor(x).float().numpy(), dtype=np.float32)
    G, N, d = xf.shape
    nb = -(-N // block_rows)
    codes = np.empty((G, N, d), dtype=np.uint8)
    descale = np.empty((G, nb), dtype=np.float32)
    for g in range(G):
        for b in range(nb):
            blk = xf[g, b * block_rows:(b + 1) * block_rows]
            amax = np.float32(np.max(np.abs(blk))) if blk.size else np.float32(0)
            if amax == 0:
                descale[g, b] = np.float32(1.0)
                codes[g, b * block_rows:(b + 1) * block_rows] = 0
                continue
            inv = np.float32(E4M3_MAX) / amax
            y = np.clip(blk * inv, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
            codes[g, b * block_rows:(b + 1) * block_rows] = encode_e4m3(y)
            descale[g, b] = amax / np.float32(E4M3_MAX)
    return codes, descale


def dequantize(codes, descale, block_rows):
    """codes [G, N, d] and descale [G, nb] -> float64 values [G, N, d]."""
    vals = decode_e4m3(codes)
    G, N, d = vals.shape
    rows = np.arange(N) // block_rows
    return vals * np.asarray(descale, dtype=np.float64)[:, rows][:, :, None]


def attention_fp8(q8, k8, v8, q_descale, k_descale, v_descale, causal, scale, rows=None, spread=False):
    """fp64 attention of dequantized e4m3 inputs.

    q8 [B, H, Nq, d], k8 and v8 [B, H_kv, Nk, d] (uint8 codes); q_descale
    [B, H, ceil(Nq/128)], k_descale [B, H_kv, ceil(Nk/128)], v_descale [B, H_kv]
    (float32).  Query head h reads K/V head h // (H // H_kv); causal key j is
    visible to query i iff j <= i + Nk - Nq.  rows: optional flat indices
    (b*H + h)*Nq + i; then o is [len(rows), d] and lse [len(rows)], else o
    [B, H, Nq, d] and lse [B, H, Nq].

    Also returns, for the error bound of a kernel that rounds P to e4m3, two
    arrays shaped like o: A[r, t] = sum_j p_j |v_jt| / l (the weight-averaged
    magnitude) and U[r, t] = sum over keys with p_j / max p < 2^-10 of |v_jt|,
    divided by l (the magnitude carried by weights small enough to reach e4m3's
    subnormal range); p_j = exp(s_j - m).

    With spread=True a fifth array shaped like o is returned:
    R[r, t] = sqrt(sum_j (e_j v_jt)^2) / l with e_j = max(2^-4 p_j, 2^-14), the
    largest absolute error of p_j rounded to e4m3 (relative 2^-4 for normals;
    below 2^-10 of the row maximum the absolute spacing takes over, 2^-14 in
    units of the largest weight).  If each weight's rounding error is spread
    evenly over that interval, independently of the others, the output error
    O_t - O_exact,t has a standard deviation of at most R / sqrt(3).
    """
    q8, k8, v8 = (np.asarray(t, dtype=np.uint8) for t in (q8, k8, v8))
    B, H, Nq, d = q8.shape
    H_kv, Nk = k8.shape[1], k8.shape[2]
    G = H // H_kv
    sigma = float(np.float32(scale))
    qd = np.asarray(q_descale, dtype=np.float32)
    kd = np.asarray(k_descale, dtype=np.float32)
    vd = np.asarray(v_descale, dtype=np.float32)
    flat = np.arange(B * H * Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((flat.size, d))
    lse = np.full(flat.size, -np.inf)
    amag = np.zeros((flat.size, d))
    umag = np.zeros((flat.size, d))
    rms = np.zeros((flat.size, d))
    cache = {}
    for r, f in enumerate(flat):
        bh, i = divmod(int(f), Nq)
        b, hq = divmod(bh, H)
        hk = hq // G
        if (b, hk) not in cache:
            kx = dequantize(k8[b, hk][None], kd[b, hk][None], K_BLOCK)[0]
            vx = decode_e4m3(v8[b, hk]) * float(vd[b, hk])
            cache = {(b, hk): (kx, vx)}
        kx, vx = cache[(b, hk)]
        qrow = decode_e4m3(q8[b, hq, i]) * float(qd[b, hq, i // Q_BLOCK])
        hi = Nk if not causal else max(0, min(Nk, i + (Nk - Nq) + 1))
        if hi == 0:
            continue
        s = sigma * (kx[:hi] @ qrow)
        m = np.max(s)
        p = np.exp(s - m)
        l = np.sum(p)
        o[r] = (p @ vx[:hi]) / l
        lse[r] = m + math.log(l)
        amag[r] = (p @ np.abs(vx[:hi])) / l
        umag[r] = np.abs(vx[:hi])[p < 2.0 ** -10].sum(axis=0) / l
        if spread:
            e = np.maximum(2.0 ** -4 * p, 2.0 ** -14)
            rms[r] = np.sqrt((e * e) @ (vx[:hi] * vx[:hi])) / l
    if rows is None:
        sh = (B, H, Nq, d)
        out = (o.reshape(sh), lse.reshape(B, H, Nq), amag.reshape(sh), umag.reshape(sh), rms.reshape(sh))
    else:
        out = (o, lse, amag, umag, rms)
    return out if spread else out[:4]
