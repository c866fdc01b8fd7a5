"""Error checks for the FP8 forward's output against the fp64 FP8 oracle.

The kernel rounds the softmax weights P to e4m3 before the P.V product (Ringi,
"Lecture 25", section 5.4: both products on FP8 operands).  Two checks bound
what that rounding, bf16 output rounding and fp32 accumulation may change:

* worst case, per element:
      |dO_t| <= 2^-4 A_t + 2^-14 U_t + 2^-8 |O_t| + 1e-5 A_t
  (A_t = sum_j w_j |v_jt|, U_t the |v| mass of weights below 2^-10 of the row
  maximum; both from the oracle).  It assumes every rounding error points the
  same way, so on a long row with nearly uniform weights it is far larger than
  |O| itself and would accept O = 0.

* statistical, over all compared elements: round-to-nearest errors are spread
  evenly over [-e_j, e_j] and independent from key to key, so
      z_t = dO_t / sqrt((R_t^2 + (2^-8 O_t)^2) / 3 + 1e-12)
  (R from the oracle: sqrt(sum_j (e_j v_jt)^2) / l) has E[z^2] <= 1; the
  check requires mean(z^2) <= 1 and max |z| <= 8.  On long_causal's rows R is
  about 30 times smaller than |O|, so O = 0 or a dropped V scale fails it.
"""
import numpy as np

MEAN_Z2_BAR = 1.0
MAX_Z_BAR = 8.0


def worst_case_ratio(a, ro, A, U):
    """max |dO| / bound of the worst-case per-element bound (must be <= 1)."""
    bound = 2.0 ** -4 * A + 2.0 ** -14 * U + 2.0 ** -8 * np.abs(ro) + 1e-5 * A + 1e-7
    return float(np.max(np.abs(a - ro) / bound))


def z_scores(a, ro, R):
    sd = np.sqrt((R * R + (2.0 ** -8 * ro) ** 2) / 3.0 + 1e-12)
    return (a - ro) / sd


def statistical(a, ro, R):
    """(mean z^2, max |z|) of the output error against the rounding spread."""
    z = z_scores(np.asarray(a, dtype=np.float64), ro, R)
    return float(np.mean(z * z)), float(np.max(np.abs(z)))


def check(a, ro, A, U, R, what):
    a = np.asarray(a, dtype=np.float64).reshape(ro.shape)
    assert not np.isnan(a).any(), f"{what}: NaN in O"
    ratio = worst_case_ratio(a, ro, A, U)
    mz2, mz = statistical(a, ro, R)
    print(f"[parity] {what} max|dO|={np.max(np.abs(a - ro)):.3e} worst-case ratio={ratio:.3f} "
          f"mean z^2={mz2:.3f} max|z|={mz:.2f}", flush=True)
    assert ratio <= 1.0, f"{what}: O outside the worst-case e4m3 rounding bound (ratio {ratio:.3f})"
    assert mz2 <= MEAN_Z2_BAR, f"{what}: mean z^2 {mz2:.3f} > {MEAN_Z2_BAR} (errors larger than e4m3 rounding of P)"
    assert mz <= MAX_Z_BAR, f"{what}: max |z| {mz:.2f} > {MAX_Z_BAR}"
