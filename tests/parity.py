"""Comparison rules between the HIP path and the CPU oracle.

(a) quantized codes: |delta| <= 1 LSB everywhere, mismatch rate <= 1e-4 (fp32 rotation sums may
    round differently from the oracle's fp64 sums right at a rounding edge);
(b) integer accumulators, given identical codes: bit-exact;
(c) fp32 scales: within 1e-6 relative.  fp16 group scales: both sides round max|group|/7 once
    to fp16 from an fp32 group maximum, so they are bit-equal unless the two fp32 maxima differ
    (the rotation sums' rounding order) right at an fp16 rounding edge; such a scale is then
    1 ulp (2^-10 relative) away, which 1e-6 cannot express, so the rule for fp16 scales is
    "equal, except at most 1 ulp apart at a mismatch rate <= 1e-4" (measured on 32k-64k scales
    by the large-sample test);
(d) bf16 output: max|y_gpu - y_oracle| / max|y_oracle| <= 1e-2, against the oracle's quantized
    result (not the exact product), plus a tighter check that almost every element is within a
    couple of bf16 ulps of it.
"""
import sys

import numpy as np
import torch

CODE_MISMATCH_RATE = 1e-4
SCALE_RTOL = 1e-6
F16_SCALE_MISMATCH_RATE = 1e-4
Y_REL_TOL = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def allowed_mismatches(n: int, rate: float) -> float:
    """Mismatch count compatible with `rate` on a sample of n codes: the expectation plus a
    3-sigma Poisson margin and 2 events, so a small sample is not failed by one or two edge
    cases (exact half-integer quotients do occur with bf16 inputs) while large samples are held
    to the rate itself."""
    lam = rate * n
    return lam + 3.0 * np.sqrt(lam) + 2.0


def check_codes(gpu: np.ndarray, ref: np.ndarray, what: str = "codes", rate: float = CODE_MISMATCH_RATE,
                slack: bool = True):
    gpu = gpu.astype(np.int64)
    ref = ref.astype(np.int64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    d = np.abs(gpu - ref)
    mism = np.count_nonzero(d)
    assert d.max(initial=0) <= 1, "%s: max |delta| = %d" % (what, d.max())
    limit = allowed_mismatches(d.size, rate) if slack else rate * d.size
    assert mism <= limit, "%s: %d mismatches of %d (rate %.2e, limit %.1f)" % (
        what, mism, d.size, mism / max(d.size, 1), limit)
    return mism


def check_scales_f32(gpu: np.ndarray, ref: np.ndarray, what: str = "scales"):
    gpu = gpu.astype(np.float64)
    ref = ref.astype(np.float64)
    err = np.abs(gpu - ref)
    bad = err > SCALE_RTOL * np.abs(ref)
    assert not bad.any(), "%s: %d scales off by more than %g relative (max rel %.3e)" % (
        what, bad.sum(), SCALE_RTOL, (err / np.maximum(np.abs(ref), 1e-300)).max())


def check_scales_f16(gpu: np.ndarray, ref: np.ndarray, what: str = "fp16 scales", slack: bool = True):
    g = gpu.astype(np.float16).view(np.uint16).astype(np.int64)
    r = ref.astype(np.float16).view(np.uint16).astype(np.int64)
    d = np.abs(g - r)
    assert d.max(initial=0) <= 1, "%s: scales differ by %d fp16 ulps" % (what, d.max())
    mism = np.count_nonzero(d)
    limit = allowed_mismatches(d.size, F16_SCALE_MISMATCH_RATE) if slack else F16_SCALE_MISMATCH_RATE * d.size
    assert mism <= limit, "%s: %d of %d differ (limit %.1f)" % (what, mism, d.size, limit)
    return mism


def check_y(gpu: np.ndarray, ref: np.ndarray, what: str = "y", strict_frac: float = 1e-3):
    gpu = gpu.astype(np.float64)
    ref = ref.astype(np.float64)
    scale = np.abs(ref).max()
    err = np.abs(gpu - ref)
    rel = err.max() / scale if scale > 0 else err.max()
    assert rel <= Y_REL_TOL, "%s: max error %.3e of max|y| (tol %g)" % (what, rel, Y_REL_TOL)
    # bf16 has 8 significant bits: rounding alone gives <= 2^-9 |y|; allow 4 ulps + a tiny floor
    loose = err > (2.0 ** -6) * np.abs(ref) + 1e-4 * scale
    assert loose.mean() <= strict_frac, "%s: %d of %d elements beyond 4 bf16 ulps" % (what, loose.sum(), loose.size)
    return rel
