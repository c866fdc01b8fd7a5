"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
at least one pin catches each: evidence that the pins constrain every part of
the oracle -- the scores, the mask, the softmax, the LSE, the decoders and the
split merge."""
import os

import numpy as np
import torch

import pytest

from oracle import build, oracle
from tests import oracle_pins

MUTANTS = [
    ("drop_scale", "s[j - lo] = sigma * acc;", "s[j - lo] = acc;"),
    ("score_sign", "acc += qrow[t] * decode", "acc -= qrow[t] * decode"),
    ("causal_off_by_one", "(int64_t)i + (Nk - Nq) + 1;", "(int64_t)i + (Nk - Nq);"),
    ("causal_offset_sign", "(int64_t)i + (Nk - Nq) + 1;", "(int64_t)i - (Nk - Nq) + 1;"),
    ("causal_top_left", "(int64_t)i + (Nk - Nq) + 1;", "(int64_t)i + 1;"),
    ("no_max_subtraction", "double p = exp(s[j - lo] - m);", "double p = exp(s[j - lo]);"),
    ("lse_without_max", "*lse_out = m + log(l);", "*lse_out = log(l);"),
    ("lse_without_log", "*lse_out = m + log(l);", "*lse_out = m + l;"),
    ("unnormalised_output", "for (int t = 0; t < d; ++t) o_row[t] /= l;", "for (int t = 0; t < d; ++t) o_row[t] /= 1.0;"),
    ("k_row_stride", "const uint16_t *kj = kp + (size_t)j * kstride;", "const uint16_t *kj = kp + (size_t)j;"),
    ("v_row_of_first_key", "const uint16_t *vj = vp + (size_t)j * kstride;", "const uint16_t *vj = vp + (size_t)lo * kstride;"),
    ("q_row_of_key", "*qp = jb->q + ((size_t)bh * Nq + i) * d;", "*qp = jb->q + ((size_t)bh * Nq) * d;"),
    ("head_stride", "i) * d;\n    const uint16_t *kp = jb->k + (size_t)bh * Nk * d;\n    const uint16_t *vp = jb->v + (size_t)bh * Nk * d;\n\n    int lo",
     "i) * d;\n    const uint16_t *kp = jb->k;\n    const uint16_t *vp = jb->v + (size_t)bh * Nk * d;\n\n    int lo"),
    ("f16_exponent_bias", "expo - 25", "expo - 24"),
    ("f16_subnormal", "ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    ("bf16_exponent_bias", "expo - 134", "expo - 133"),
    ("key_range_ignored", "int lo = jb->key_begin < 0 ? 0 : jb->key_begin;", "int lo = 0;"),
    ("combine_weight_sign", "double w = exp(ls - M);", "double w = exp(M - ls);"),
    ("combine_lse_missing_max", "lse[r] = M + log(wsum);", "lse[r] = log(wsum);"),
    ("combine_skip_normalise", "for (int t = 0; t < d; ++t) orow[t] /= wsum;", "for (int t = 0; t < d; ++t) orow[t] /= 1.0;"),
    ("varlen_group_modulo", "const int g = h / (H / H_kv);", "const int g = h % H_kv;"),
    ("varlen_key_offset_of_queries", "const uint16_t *kp = jb->k + ((size_t)jb->cu_k[b] * H_kv + g) * d;",
     "const uint16_t *kp = jb->k + ((size_t)jb->cu_q[b] * H_kv + g) * d;"),
    ("varlen_value_head", "const uint16_t *vp = jb->v + ((size_t)jb->cu_k[b] * H_kv + g) * d;",
     "const uint16_t *vp = jb->v + ((size_t)jb->cu_k[b] * H_kv) * d;"),
    ("varlen_key_stride", "row_core(qp, kp, vp, (size_t)H_kv * d,", "row_core(qp, kp, vp, (size_t)d,"),
    ("varlen_key_count", "const int Nk = jb->cu_k[b + 1] - jb->cu_k[b];", "const int Nk = jb->cu_q[b + 1] - jb->cu_q[b];"),
    ("varlen_query_head", "const uint16_t *qp = jb->q + ((size_t)token * H + h) * d;",
     "const uint16_t *qp = jb->q + ((size_t)token * H) * d;"),
    ("varlen_sequence_search", "while (b + 1 < jb->B && jb->cu_q[b + 1] <= token) ++b;",
     "while (b + 1 < jb->B && jb->cu_q[b + 1] < token) ++b;"),
    ("bwd_rowsum_without_p", "D += p * dot_rows(gi, vp", "D += dot_rows(gi, vp"),
    ("bwd_dq_without_scale", "dq[t] += jb->sigma * ds * decode(kj[t], jb->dtype);", "dq[t] += ds * decode(kj[t], jb->dtype);"),
    ("bwd_dk_without_scale", "dk[t] += jb->sigma * ds * decode(qi[t], jb->dtype);", "dk[t] += ds * decode(qi[t], jb->dtype);"),
    ("bwd_dk_from_keys", "dk[t] += jb->sigma * ds * decode(qi[t], jb->dtype);", "dk[t] += jb->sigma * ds * decode(kj[t], jb->dtype);"),
    ("bwd_dv_from_ds", "dv[t] += p * decode(gi[t], jb->dtype);", "dv[t] += ds * decode(gi[t], jb->dtype);"),
    ("bwd_causal_off_by_one", "if (j >= row_visible_end(i, Nq, Nk, jb->causal)) continue;", "if (j > row_visible_end(i, Nq, Nk, jb->causal)) continue;"),
    ("bwd_ds_sign", "double ds = p * (dot_rows(gi, vp + (size_t)j * d, d, jb->dtype) - jb->D[slot]);", "double ds = p * (dot_rows(gi, vp + (size_t)j * d, d, jb->dtype) + jb->D[slot]);"),
    ("empty_row_lse_zero", "if (hi <= lo) { *lse_out = -INFINITY; return; }", "if (hi <= lo) { *lse_out = 0.0; return; }"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    with open(build.SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"pattern for {name} must occur exactly once"
    mpath = os.path.join(tmp_path, f"{name}.c")
    with open(mpath, "w") as f:
        f.write(src.replace(old, new))
    # a mutant may leave a parameter unused: warnings stay warnings here
    lib = build.build(src=mpath, out=os.path.join(tmp_path, f"lib{name}.so"), extra_flags=("-Wno-error",))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, RuntimeError, FloatingPointError) as e:
            caught.append(f"{pin.__name__}: {str(e)[:80]}")
    assert caught, f"no pin catches the mutant {name}"


def test_dense_grouped_heads_mapping_mutant_is_caught():
    """Tiling K/V heads (h -> h % H_kv) instead of repeating them per group fails
    the dense grouped-heads pin."""
    class Tiled(oracle.Oracle):
        @staticmethod
        def expand_kv_heads(t, H):
            return t.repeat(1, H // t.shape[1], 1, 1).contiguous()

    with pytest.raises(AssertionError):
        oracle_pins.pin_dense_grouped_heads(Tiled())


@pytest.mark.parametrize("kind", ["row_page_swapped", "first_table_row", "page_off_by_one"])
def test_paged_gather_mutants_are_caught(kind):
    """Plausible mistakes in the page-table gather fail the paged pins."""
    class Broken(oracle.Oracle):
        @staticmethod
        def gather_pages(cache, block_table, seqlens):
            ps = cache.shape[1]
            table = np.asarray(block_table, dtype=np.int64)
            rows = []
            for b in range(table.shape[0]):
                for t in range(int(seqlens[b])):
                    if kind == "row_page_swapped":
                        page, row = int(table[b, t % table.shape[1]]), (t // table.shape[1]) % ps
                    elif kind == "first_table_row":
                        page, row = int(table[0, t // ps]), t % ps
                    else:
                        page, row = int(table[b, t // ps]), (t + 1) % ps
                    rows.append(cache[page, row])
            if not rows:
                return cache.new_empty((0,) + tuple(cache.shape[2:]))
            return torch.stack(rows).contiguous()

    orc = Broken()
    caught = 0
    for pin in (oracle_pins.pin_paged_matches_contiguous, oracle_pins.pin_paged_brute_force,
                oracle_pins.pin_paged_splits):
        try:
            pin(orc)
        except (AssertionError, IndexError, RuntimeError):
            caught += 1
    assert caught, f"no paged pin catches the {kind} mutant"


@pytest.mark.parametrize("kind", ["first_sequence", "offset_of_next", "one_split"])
def test_varlen_decode_mutants_are_caught(kind):
    """Plausible mistakes in locating a packed sequence's keys, or in its split
    rule, fail the packed-decode pins."""
    class Broken(oracle.Oracle):
        def split_partials_varlen(self, q, k, v, cu_seqlens_k, scale, num_splits, nthreads=None):
            B, H, d = q.shape
            cu = [int(x) for x in cu_seqlens_k]
            o_part = np.zeros((num_splits, B, H, 1, d))
            lse_part = np.full((num_splits, B, H, 1), -np.inf)
            for b in range(B):
                lo, hi = cu[b], cu[b + 1]
                if kind == "first_sequence":
                    lo, hi = cu[0], cu[1]
                elif kind == "offset_of_next":
                    lo, hi = min(lo + 1, cu[-1] - 1), min(hi + 1, cu[-1])
                if hi <= lo:
                    continue
                kb = k[lo:hi].permute(1, 0, 2).unsqueeze(0).contiguous()
                vb = v[lo:hi].permute(1, 0, 2).unsqueeze(0).contiguous()
                S = 1 if kind == "one_split" else num_splits
                ob, lb = self.split_partials(q[b:b + 1, :, None, :].contiguous(), kb, vb, False, scale, S,
                                             nthreads=nthreads)
                o_part[:S, b] = ob[:, 0]
                lse_part[:S, b] = lb[:, 0]
            return o_part, lse_part

    orc = Broken()
    caught = 0
    for pin in oracle_pins.VARLEN_DECODE_PINS:
        try:
            pin(orc)
        except (AssertionError, IndexError, RuntimeError):
            caught += 1
    assert caught, f"no packed-decode pin catches the {kind} mutant"


FP8_MUTANTS = {
    # decoder: exponent bias 8 instead of 7
    "decode_bias": ("normal = sign * np.ldexp(1.0 + mant / 8.0, expo - 7)",
                    "normal = sign * np.ldexp(1.0 + mant / 8.0, expo - 8)"),
    # decoder: subnormals scaled as 2^-10
    "decode_subnormal": ("sub = sign * np.ldexp(mant.astype(np.float64), -9)",
                         "sub = sign * np.ldexp(mant.astype(np.float64), -10)"),
    # encoder: ties away from zero
    "encode_ties_away": ("pick = np.where(tie & (lo != hi), np.where(hi % 2 == 0, hi, lo), pick)",
                         "pick = np.where(tie & (lo != hi), hi, pick)"),
    # quantizer: descale of the block taken as 448 / amax
    "descale_inverted": ("descale[g, b] = amax / np.float32(E4M3_MAX)",
                         "descale[g, b] = np.float32(E4M3_MAX) / amax"),
    # attention: K scale looked up per 64 keys
    "k_block": ("kx = dequantize(k8[b, hk][None], kd[b, hk][None], K_BLOCK)[0]",
                "kx = dequantize(k8[b, hk][None], kd[b, hk][None], 64)[0]"),
    # attention: V scale ignored
    "v_scale": ("vx = decode_e4m3(v8[b, hk]) * float(vd[b, hk])", "vx = decode_e4m3(v8[b, hk])"),
    # attention: causal bound off by one
    "causal": ("hi = Nk if not causal else max(0, min(Nk, i + (Nk - Nq) + 1))",
               "hi = Nk if not causal else max(0, min(Nk, i + (Nk - Nq)))"),
    # error terms: U weighted by the small weights instead of counting their |v|
    "u_weighted": ("umag[r] = np.abs(vx[:hi])[p < 2.0 ** -10].sum(axis=0) / l",
                   "umag[r] = (p[p < 2.0 ** -10] @ np.abs(vx[:hi])[p < 2.0 ** -10]) / l"),
    # error terms: subnormal threshold 2^-9 instead of 2^-10
    "u_threshold": ("umag[r] = np.abs(vx[:hi])[p < 2.0 ** -10].sum(axis=0) / l",
                    "umag[r] = np.abs(vx[:hi])[p < 2.0 ** -9].sum(axis=0) / l"),
    # error terms: A without the absolute value of v
    "a_signed": ("amag[r] = (p @ np.abs(vx[:hi])) / l", "amag[r] = (p @ vx[:hi]) / l"),
    # error terms: R without the absolute floor of the smallest weights
    "r_no_floor": ("e = np.maximum(2.0 ** -4 * p, 2.0 ** -14)", "e = 2.0 ** -4 * p"),
    # error terms: R summed linearly instead of in quadrature
    "r_linear": ("rms[r] = np.sqrt((e * e) @ (vx[:hi] * vx[:hi])) / l", "rms[r] = (e @ np.abs(vx[:hi])) / l"),
}


@pytest.mark.parametrize("name", sorted(FP8_MUTANTS))
def test_fp8_oracle_mutants_are_caught(name, tmp_path, oracle_lib):
    """Plausible mistakes in the FP8 oracle (decoder, encoder, quantizer,
    scales, mask) each fail at least one FP8 pin."""
    import importlib.util
    from oracle import fp8
    old, new = FP8_MUTANTS[name]
    src = open(fp8.__file__).read()
    assert src.count(old) == 1, f"pattern for {name} must occur exactly once"
    path = tmp_path / f"fp8_{name}.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"fp8_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    import sys
    saved = sys.modules.get("oracle.fp8")
    import oracle as oracle_pkg
    saved_attr = getattr(oracle_pkg, "fp8", None)
    sys.modules["oracle.fp8"] = mod
    oracle_pkg.fp8 = mod
    caught = []
    try:
        for pin in oracle_pins.FP8_PINS:
            try:
                pin(oracle_lib)
            except (AssertionError, ValueError, IndexError) as e:
                caught.append(f"{pin.__name__}: {str(e)[:60]}")
    finally:
        sys.modules["oracle.fp8"] = saved
        oracle_pkg.fp8 = saved_attr
    assert caught, f"no FP8 pin catches the mutant {name}"
