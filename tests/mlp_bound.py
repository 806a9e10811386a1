"""Tolerance of the MLP feature kernel against the plain fp64 definition.

The kernel (rma_phi_mlp_features) rounds the input x, every weight matrix, h0,
the activation and h1 to bfloat16 (round to nearest even: relative error at
most u_b = 2^-8) and sums the matrix-core products in fp32.  A worst-case
first-order bound, with |W| |x| products through the two 512-wide layers, is
uselessly loose (it allows errors of e^100).  The measured errors behave as
the standard rounding model says: independent relative errors, spread like a
sum of many small independent terms.  So the tolerance follows that model:

  * every rounding point of oracle.phi_mlp gets an independent relative
    perturbation drawn uniformly from [-u_b, u_b] (RNE's relative error is
    at most u_b and at least u_b / 2 at its extremes, so the uniform law
    over-states its spread), and the plain forward pass is repeated with
    fresh draws;
  * sigma = the root mean square, over the trials, of the change of each
    output exponent z = W_o h1 + b_o;
  * each feature phi = e^z may then differ from the plain value by
    |log phi_kernel - z| <= 8 sigma + 1e-4 + u_store, with 1e-4 for fp32
    summation and exp (gamma_512 = 3e-5 of the magnitude) and u_store =
    2^-8 for bf16 rows (one more rounding), 2^-24 for fp32 rows.

With 24 trials sigma is estimated to about 15 %; 8 sigma stays above 6.5
true standard deviations, whose two-sided tail (1e-10) is negligible over
the rows a test checks.
"""
import numpy as np

import oracle as O

U_B = 2.0 ** -8
TRIALS = 24
N_SIGMA = 8.0


def sigma_z(x, params, trials=TRIALS, seed=0):
    """Per-feature RMS change of z under the rounding model."""
    rng = np.random.default_rng(seed)

    def perturb(a):
        a = np.asarray(a, dtype=np.float64)
        return a * (1.0 + rng.uniform(-U_B, U_B, a.shape))

    _, T = O.phi_mlp(x, params, return_terms=True)
    acc = np.zeros_like(T["z"])
    for _ in range(trials):
        _, Tp = O.phi_mlp(x, params, return_terms=True, operand_round=perturb)
        acc += (Tp["z"] - T["z"]) ** 2
    return T["z"], np.sqrt(acc / trials)


def check_rows(phi_kernel, x, params, bf16_rows):
    """Asserts every feature of the kernel's rows is within the model's
    tolerance of the plain definition; returns (worst ratio to the tolerance,
    median relative error)."""
    z, sig = sigma_z(x, params)
    got = np.asarray(phi_kernel, dtype=np.float64)
    assert (got > 0).all(), "non-positive feature"
    tol = N_SIGMA * sig + 1e-4 + (U_B if bf16_rows else 2.0 ** -24)
    dev = np.abs(np.log(got) - z)
    ratio = float((dev / tol).max())
    assert ratio <= 1.0, f"feature off the plain definition by {ratio:.2f} x its tolerance"
    return ratio, float(np.median(np.abs(np.expm1(np.log(got) - z))))
