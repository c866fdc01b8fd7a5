"""Comparison of the HIP library's outputs with the fp64 oracle.

Tolerances (the spec contract for this path): O max-abs 2e-3 for fp16 and
1e-2 for bf16 outputs; LSE max |dLSE| / max(1, |LSE|) <= 1e-4.  Rows the oracle
marks empty (LSE = -inf) must be exactly -inf with O exactly 0; NaN fails.
"""
import numpy as np
import torch

O_TOL = {torch.float16: 2e-3, torch.bfloat16: 1e-2, torch.float32: 2e-5}
LSE_TOL = 1e-4


def errors(o_gpu, lse_gpu, o_ref, lse_ref, out_dtype):
    o = o_gpu.detach().double().cpu().numpy().reshape(o_ref.shape)
    l = lse_gpu.detach().double().cpu().numpy().reshape(lse_ref.shape)
    assert not np.isnan(o).any(), "NaN in O"
    assert not np.isnan(l).any(), "NaN in LSE"
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(l), empty), "empty rows differ"
    assert np.all(o[empty] == 0.0), "empty rows must have O = 0"
    fin = ~empty
    o_err = float(np.max(np.abs(o - o_ref), initial=0.0))
    lse_err = float(np.max(np.abs(l[fin] - lse_ref[fin]) / np.maximum(1.0, np.abs(lse_ref[fin])), initial=0.0))
    ref_rounded = torch.from_numpy(np.ascontiguousarray(o_ref)).to(out_dtype).double().numpy()
    o_err_rounded = float(np.max(np.abs(o - ref_rounded), initial=0.0))
    return {"o_err": o_err, "lse_err": lse_err, "o_err_vs_rounded_oracle": o_err_rounded}


def check(o_gpu, lse_gpu, o_ref, lse_ref, out_dtype, what=""):
    e = errors(o_gpu, lse_gpu, o_ref, lse_ref, out_dtype)
    print(f"[parity] {what} {e}", flush=True)
    assert e["o_err"] <= O_TOL[out_dtype], f"{what}: O error {e}"
    assert e["lse_err"] <= LSE_TOL, f"{what}: LSE error {e}"
    return e


def sample_rows(B, H, Nq, n_random=256, seed=0):
    """Flat row indices (b*H + h)*Nq + i: the first and last rows of every head
    plus seeded random rows."""
    rng = np.random.default_rng(seed)
    bh = np.arange(B * H)
    rows = [bh * Nq, bh * Nq + (Nq - 1), rng.integers(0, B * H * Nq, n_random)]
    if Nq > 1:
        rows.append(bh * Nq + 1)
    return np.unique(np.concatenate(rows))


# Gradients: max |g - g_oracle| / max |g_oracle| per tensor.  The backward rounds
# P and dS to the input type before its products, reads the forward's rounded O
# and rounds its outputs, each a relative error of at most the unit roundoff u
# (2^-11 fp16, 2^-8 bf16); the bar is 4u of the largest gradient.
GRAD_TOL = {torch.float16: 4 * 2.0 ** -11, torch.bfloat16: 4 * 2.0 ** -8}


def d_rounding_shift(q, k, dout, o_ref, lse_ref, causal, scale, dtype):
    """Exact effect on dQ and dK of forming D = rowsum(dO o O) from O rounded to the
    output type (the pages' recipe: the backward reads the forward's stored O)
    instead of the exact O.  With dD_i = sum_t dO_it (round(O_it) - O_it), dS moves
    by -P_ij dD_i, so dq_i moves by -scale dD_i sum_j P_ij k_j and dk_j by
    -scale sum_i P_ij dD_i q_i.  dP - D can cancel to far below the gradient's own
    size, so this term is not covered by a tolerance relative to the gradient;
    adding it to the oracle's exact gradients compares like with like.  O is the
    oracle's, rounded here; P is formed in fp64 from the oracle's LSE."""
    qd, kd, gd = (t.double().cpu().numpy() for t in (q, k, dout))
    o = np.asarray(o_ref, dtype=np.float64).reshape(qd.shape)
    o_r = torch.from_numpy(np.ascontiguousarray(o)).to(dtype).double().numpy()
    lse = np.asarray(lse_ref, dtype=np.float64).reshape(qd.shape[:3])
    dD = np.sum(gd * (o_r - o), axis=-1)                                       # [B, H, Nq]
    Nq, Nk = qd.shape[2], kd.shape[2]
    fin = np.isfinite(lse)
    vis = np.broadcast_to(fin[..., None], fin.shape + (Nk,)).copy()
    if causal:
        vis &= (np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + (Nk - Nq))[None, None]
    s = scale * np.einsum("bhid,bhjd->bhij", qd, kd) - np.where(fin, lse, 0.0)[..., None]
    p = np.where(vis, np.exp(np.where(vis, s, 0.0)), 0.0)
    ddq = -scale * dD[..., None] * np.einsum("bhij,bhjd->bhid", p, kd)
    ddk = -scale * np.einsum("bhij,bhi,bhid->bhjd", p, dD, qd)
    return ddq, ddk


def grad_errors(grads, refs):
    """Max error of each gradient normalised by its reference's largest value.

    dQ and dK vanish exactly when every softmax row is one-hot (a query that sees
    a single key): dP - D is then zero in exact arithmetic, and the kernel returns
    the fp32 rounding of that difference.  So their normaliser never drops below
    2^-10 of dV's largest value (dV = P^T dO keeps the size of dO): that noise is
    about d * 2^-24 * |dO| |V|, far below the bound this leaves."""
    out = {}
    dv_max = float(np.max(np.abs(refs[2]), initial=0.0))
    for name, g, r in zip(("dq", "dk", "dv"), grads, refs):
        a = g.detach().double().cpu().numpy().reshape(r.shape)
        assert not np.isnan(a).any(), f"NaN in {name}"
        scale = max(float(np.max(np.abs(r), initial=0.0)), 1e-30)
        if name != "dv":
            scale = max(scale, 2.0 ** -10 * dv_max)
        out[name] = float(np.max(np.abs(a - r), initial=0.0)) / scale
    return out


def check_grads(grads, refs, dtype, what=""):
    e = grad_errors(grads, refs)
    print(f"[parity] {what} {e}", flush=True)
    for name, err in e.items():
        assert err <= GRAD_TOL[dtype], f"{what}: {name} normalised error {err:.3e}"
    return e


def varlen_bwd_refs(orc, q, k, v, g, cq, ck, causal, scale, dt):
    """Oracle gradients plus, per sequence, the exact effect of D from rounded O."""
    rq, rk, rv = orc.attention_bwd_varlen(q, k, v, g, cq.numpy(), ck.numpy(), causal, scale)
    ro, rl = orc.attention_varlen(q, k, v, cq.numpy(), ck.numpy(), causal, scale)
    H, H_kv, d = q.shape[1], k.shape[1], q.shape[2]
    for b in range(len(cq) - 1):
        q0, q1, k0, k1 = int(cq[b]), int(cq[b + 1]), int(ck[b]), int(ck[b + 1])
        if q1 == q0 or k1 == k0:
            continue
        hm = lambda t, a, z: t[a:z].permute(1, 0, 2).unsqueeze(0).contiguous()
        ke = orc.expand_kv_heads(hm(k, k0, k1), H)
        ddq, ddk = d_rounding_shift(hm(q, q0, q1), ke, hm(g, q0, q1),
                                    np.asarray(ro)[q0:q1].transpose(1, 0, 2)[None],
                                    np.asarray(rl)[:, q0:q1][None], causal, scale, dt)
        rq[q0:q1] += ddq[0].transpose(1, 0, 2)
        rk[k0:k1] += ddk[0].reshape(H_kv, H // H_kv, k1 - k0, d).sum(axis=1).transpose(1, 0, 2)
    return rq, rk, rv
