"""Parity bar between the HIP path and the fp64 oracle.

Tolerances on O: fp32 inputs, max |O - O_ref| <= 1e-5; bf16 inputs, max |O - O_ref| <= 2e-2 and
relative RMS ||O - O_ref|| / ||O_ref|| <= 5e-3.

LSE (the pages fix no bar for it): |LSE - LSE_ref| <= 1e-4 for bf16 inputs and 1e-5 for fp32
inputs, absolute.  The scores are exact products of the inputs summed in fp32 and the row sum
adds fp32 probabilities, so on the specified workloads (scale = 1/sqrt(d), N(0, 1) inputs, unit
variance scores, |LSE| below about 16) the fp32 rounding stays near 1e-6.  Rows that see no key
must be exactly O = 0 and LSE = -inf.

Stress tests outside the specified workloads multiply the scores by a factor f (a scale of 2,
inputs times 30): fp32 rounding of a score grows with its magnitude, and LSE is close to the
row's largest score, so such a test passes ``magnitude=f`` and ``lse_relative=True``.  Then the
fp32 O bound is multiplied by max(1, f) and the LSE bound becomes tau * max(1, |LSE_ref|) (the bf16
O bounds are dominated by the bf16 rounding of P and O and do not change).  The named workloads
never use this relaxation.

Gradients (attn_bwd, bf16) have no specified bar; it is derived the same way.  The inputs are
exact in both paths; the GPU rounds P and dS = P (dP - D) to bf16 before the products that use
them, takes D = rowsum(dO * O) from the forward's bf16 O, and rounds the results to bf16.  Each
rounding has a relative RMS of about 2^-8 / sqrt(3) ~ 2.3e-3 and the products sum many such
terms with independent errors, so a gradient's relative RMS error is about 2.5e-3 (the output
rounding dominates).  The bar is relative RMS <= 5e-3 per gradient tensor and
max |g - g_ref| <= 1e-2 * max(1, max |g_ref|) (the largest entries carry the largest rounding,
u * |g| with u = 2^-8, plus the accumulated share)."""
import sys

import numpy as np

O_TOL = {"f32": 1e-5, "bf16": 2e-2}
RMS_TOL = {"bf16": 5e-3}
LSE_TOL = {"f32": 1e-5, "bf16": 1e-4}
GRAD_RMS_TOL = 5e-3
GRAD_MAX_TOL = 1e-2


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


# Errors measured on the named workloads, printed by tests/conftest.py at the end of a run.
SUMMARY: list = []


def record(name: str, stats: dict) -> dict:
    """Keep the measured errors of a named workload for the end-of-run summary; returns them."""
    SUMMARY.append((name, dict(stats)))
    say(name, stats)
    return stats


# FP8 inputs (attn_fwd_fp8): S = Q K^T runs on v_mfma_f32_32x32x64_f8f6f4, which adds its 64
# products with fewer bits than fp32 carries.  A score may therefore be off by up to
# FP8_MFMA_EPS * |scale| * sum_i |q_i k_i|, and so may the LSE; check() adds that per row
# (``lse_abs_extra``) to the LSE bar and reports the raw LSE error beside it.  The bound is
# measured, not assumed: tests/test_fp8_gpu.py::test_fp8_score_accumulation_error reads single
# scores back through the LSE of one-key rows over full-range random codes and requires every
# error to stay within it.  O is not affected beyond the bf16 bar (the score error stays below
# the bf16 rounding of P).
FP8_MFMA_EPS = 2.0 ** -12


def check(o, o_ref, lse, lse_ref, dtype: str, label: str = "", magnitude: float = 1.0, lse_relative: bool = False,
          lse_abs_extra=None):
    """O and LSE against the oracle; returns the measured errors (max_abs, rel_rms, lse_err, and
    lse_bound_used when an FP8 allowance applies)."""
    o = np.asarray(o, np.float64)
    o_ref = np.asarray(o_ref, np.float64)
    assert o.shape == o_ref.shape, (label, o.shape, o_ref.shape)
    stats = {}
    if lse_ref is not None:
        lse_ref = np.asarray(lse_ref, np.float64)
        empty = np.isneginf(lse_ref)
        if lse is not None:
            lse = np.asarray(lse, np.float64)
            assert np.all(np.isneginf(lse[empty])), (label, "rows that see no key need LSE = -inf")
            fin = ~empty
            assert np.all(np.isfinite(lse[fin])), (label, "non-finite LSE")
            diff = np.abs(lse[fin] - lse_ref[fin])
            bound = np.full(diff.shape, LSE_TOL[dtype])
            if lse_relative:
                bound = bound * np.maximum(1.0, np.abs(lse_ref[fin]))
            if lse_abs_extra is not None:
                extra = np.broadcast_to(np.asarray(lse_abs_extra, np.float64), lse.shape)[fin]
                bound = bound + extra
                stats["lse_bound_max"] = float(np.max(bound, initial=0.0))
            stats["lse_err"] = float(np.max(diff, initial=0.0))
            worst = int(np.argmax(diff - bound)) if diff.size else 0
            assert diff.size == 0 or diff[worst] <= bound[worst], (label, "LSE error", float(diff[worst]),
                                                                   "bound", float(bound[worst]))
        assert np.all(o[empty] == 0.0), (label, "rows that see no key need O = 0")
    assert np.all(np.isfinite(o)), (label, "non-finite output")
    err = float(np.max(np.abs(o - o_ref), initial=0.0))
    stats["max_abs"] = err
    o_tol = O_TOL[dtype] * (max(1.0, magnitude) if dtype == "f32" else 1.0)
    assert err <= o_tol, (label, "max abs error", err, o_tol)
    if dtype in RMS_TOL:
        nref = float(np.linalg.norm(o_ref))
        if nref > 0:
            rms = float(np.linalg.norm(o - o_ref)) / nref
            stats["rel_rms"] = rms
            assert rms <= RMS_TOL[dtype], (label, "relative RMS", rms)
    return stats


def check_grad(g, g_ref, label: str = ""):
    """A bf16 gradient tensor against the fp64 oracle's (see the module docstring for the bar)."""
    g = np.asarray(g, np.float64)
    g_ref = np.asarray(g_ref, np.float64)
    assert g.shape == g_ref.shape, (label, g.shape, g_ref.shape)
    assert np.all(np.isfinite(g)), (label, "non-finite gradient")
    err = float(np.max(np.abs(g - g_ref), initial=0.0))
    bound = GRAD_MAX_TOL * max(1.0, float(np.max(np.abs(g_ref), initial=0.0)))
    stats = {"max_abs": err}
    assert err <= bound, (label, "max abs error", err, bound)
    # An exactly zero reference (one key per row: dP = D, so dS = 0) leaves the fp32 rounding of
    # dP - D, which only the absolute bound covers.
    nref = float(np.linalg.norm(g_ref))
    if nref > 0:
        rms = float(np.linalg.norm(g - g_ref)) / nref
        stats["rel_rms"] = rms
        assert rms <= GRAD_RMS_TOL, (label, "relative RMS", rms)
    return stats
