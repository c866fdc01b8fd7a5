"""CPU checks of the parity helpers the GPU tests build their references with.

d_rounding_shift claims to give the exact change of dQ and dK when D =
rowsum(dO o O) is formed from O rounded to the output type; here that claim is
checked against the backward written out by brute force in fp64 with the rounded
D (Ringi, "Lecture 25", section 3.3: dS = P o (dP - D), dQ = scale dS K, dK =
scale dS^T Q), and varlen_bwd_refs against the dense helper on one sequence.
"""
import math

import numpy as np
import torch

from tests import parity


def _rand(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(dtype)


def _brute_grads_rounded_d(q, k, v, g, causal, scale, dtype):
    qd, kd, vd, gd = (t.double().numpy() for t in (q, k, v, g))
    Nq, Nk = qd.shape[2], kd.shape[2]
    s = scale * np.einsum("bhid,bhjd->bhij", qd, kd)
    if causal:
        vis = np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + (Nk - Nq)
        s = np.where(vis, s, -np.inf)
    p = np.exp(s - s.max(axis=-1, keepdims=True))
    p /= p.sum(axis=-1, keepdims=True)
    o = np.einsum("bhij,bhjd->bhid", p, vd)
    o_r = torch.from_numpy(o).to(dtype).double().numpy()
    dd = np.sum(gd * o_r, axis=-1)
    dp = np.einsum("bhid,bhjd->bhij", gd, vd)
    ds = p * (dp - dd[..., None])
    return scale * np.einsum("bhij,bhjd->bhid", ds, kd), scale * np.einsum("bhij,bhid->bhjd", ds, qd), o, p


def test_d_rounding_shift_matches_brute_force(oracle_lib):
    for causal, dt, (Nq, Nk) in ((True, torch.bfloat16, (5, 7)), (False, torch.float16, (6, 4))):
        B, H, d, scale = 1, 2, 16, 0.625       # exact in fp32, the type the library takes
        q, g = _rand((B, H, Nq, d), dt, 1), _rand((B, H, Nq, d), dt, 2)
        k, v = _rand((B, H, Nk, d), dt, 3), _rand((B, H, Nk, d), dt, 4)
        bq, bk, _, _ = _brute_grads_rounded_d(q, k, v, g, causal, scale, dt)
        rq, rk, _ = oracle_lib.attention_bwd(q, k, v, g, causal, scale)
        ro, rl = oracle_lib.attention(q, k, v, causal, scale)
        ddq, ddk = parity.d_rounding_shift(q, k, g, ro, rl, causal, scale, dt)
        assert np.max(np.abs(ddq)) > 0      # the rounding does move the gradients here
        np.testing.assert_allclose(rq + ddq.reshape(rq.shape), bq, rtol=0, atol=1e-12)
        np.testing.assert_allclose(rk + ddk.reshape(rk.shape), bk, rtol=0, atol=1e-12)


def test_varlen_refs_match_dense_on_one_sequence(oracle_lib):
    N, H, H_kv, d, dt, scale = 9, 4, 2, 16, torch.bfloat16, 1 / math.sqrt(16)
    q, g = _rand((N, H, d), dt, 5), _rand((N, H, d), dt, 6)
    k, v = _rand((N, H_kv, d), dt, 7), _rand((N, H_kv, d), dt, 8)
    cu = torch.tensor([0, N], dtype=torch.int32)
    rq, rk, rv = parity.varlen_bwd_refs(oracle_lib, q, k, v, g, cu, cu, True, scale, dt)

    def hm(t):
        return t.permute(1, 0, 2).unsqueeze(0).contiguous()

    dq, dk, dv = oracle_lib.attention_bwd_gqa(hm(q), hm(k), hm(v), hm(g), True, scale)
    ro, rl = oracle_lib.attention_gqa(hm(q), hm(k), hm(v), True, scale)
    ddq, ddk = parity.d_rounding_shift(hm(q), oracle_lib.expand_kv_heads(hm(k), H), hm(g), ro, rl, True, scale, dt)
    dq = dq + ddq.reshape(dq.shape)
    dk = dk + ddk.reshape(1, H_kv, H // H_kv, N, d).sum(axis=2)
    np.testing.assert_allclose(rq, dq[0].transpose(1, 0, 2), rtol=0, atol=1e-12)
    np.testing.assert_allclose(rk, dk[0].transpose(1, 0, 2), rtol=0, atol=1e-12)
    np.testing.assert_allclose(rv, dv[0].transpose(1, 0, 2), rtol=0, atol=1e-12)
