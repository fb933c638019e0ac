"""Pins for the CPU oracle: each test checks it against something other than itself --
closed forms, a library routine, brute force, a hand-worked example, or a property the pages
state -- so that a dropped term, a wrong sign/index or a transposed operand fails one of them.
"""
import os

import numpy as np
import pytest
import scipy.linalg

from int4_quantized_linear_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_example_g4.txt")
POW2 = [1, 2, 4, 8, 16, 32, 64, 128, 256]


def _golden():
    d = {}
    for line in open(GOLDEN, encoding="utf-8"):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, *v = line.split()
        d[k] = v
    return d


# ------------------------------------------------------------------ Hadamard / rotation pins

@pytest.mark.parametrize("g", POW2)
def test_hadamard_orthogonal_exact(oracle, g):
    H = np.array([[oracle.hadamard_entry(i, j) for j in range(g)] for i in range(g)], np.int64)
    assert np.array_equal(H @ H.T, g * np.eye(g, dtype=np.int64))
    assert np.array_equal(H, H.T)


@pytest.mark.parametrize("g", POW2)
def test_rotation_matrix_is_blockdiag_sylvester(oracle, g):
    """rotate(I) is R itself; sqrt(g) R must be blockdiag(scipy's Sylvester Hadamard)."""
    K = max(2 * g, 8)
    R = oracle.rotate(np.eye(K), g)
    ref = scipy.linalg.block_diag(*([scipy.linalg.hadamard(g)] * (K // g))).astype(np.float64)
    assert np.allclose(R * np.sqrt(g), ref, rtol=0, atol=1e-12)


def test_rotation_of_unit_vector(oracle):
    K, g = 512, 256
    e0 = np.zeros((1, K))
    e0[0, 0] = 1.0
    y = oracle.rotate(e0, g)
    assert np.array_equal(y[0, :g], np.full(g, 1.0 / 16.0))     # 1/sqrt(256) exactly
    assert np.array_equal(y[0, g:], np.zeros(K - g))


def test_rotation_involution_parseval_locality(oracle):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((5, 1024))
    for g in (2, 16, 128, 256):
        y = oracle.rotate(x, g)
        assert np.allclose(oracle.rotate(y, g), x, rtol=0, atol=1e-12)     # (H/sqrt g)^2 = I
        assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
        # Perturbing one channel only moves outputs inside that channel's group.
        x2 = x.copy()
        x2[:, 300] += 1.0
        d = np.abs(oracle.rotate(x2, g) - y).max(axis=0)
        lo = (300 // g) * g
        assert np.all(d[:lo] == 0) and np.all(d[lo + g:] == 0) and np.all(d[lo:lo + g] > 0)


def test_rotation_identity_for_group_one(oracle):
    x = np.random.default_rng(1).standard_normal((3, 40))
    assert np.array_equal(oracle.rotate(x, 1), x)


def test_rotated_product_equals_plain_product(oracle):
    """(XR)(WR)^T = X W^T in fp64 to 1e-10 relative (tiny workload)."""
    x, w = workloads.tiny_inputs()
    x = x.double().numpy()
    w = w.double().numpy()
    ref = x @ w.T
    got = oracle.rotate(x, 256) @ oracle.rotate(w, 256).T
    assert np.abs(got - ref).max() / np.abs(ref).max() < 1e-10


def test_group_divides_workload_dims():
    for K in (5120, 5376, 8192, 25600, 512):
        assert K % 256 == 0


# ------------------------------------------------------------------ hand-worked example

def test_golden_hand_example(oracle):
    d = _golden()
    g = int(d["g"][0])
    x = np.array([float(v) for v in d["x"]])[None, :]
    y = oracle.rotate(x, g)
    assert np.array_equal(y[0], np.array([float(v) for v in d["rotated"]]))
    q, s = oracle.quantize_rows_i8(y)
    num, den = (float(v) for v in d["i8_scale_num_den"])
    assert s[0] == np.float32(num / den)
    assert q[0].tolist() == [int(v) for v in d["i8_codes"]]
    c, s4 = oracle.quantize_groups_i4(y, g)
    assert s4.view(np.uint16)[0].tolist() == [int(v, 16) for v in d["i4_scale_fp16_bits"]]
    assert c[0].tolist() == [int(v) for v in d["i4_codes"]]
    p = oracle.pack_i4(c)
    assert p[0].tolist() == [int(v, 16) for v in d["i4_packed"]]
    ones = np.ones((1, 8), np.int8)
    assert oracle.gemm_i32(q, ones)[0, 0] == int(d["dot_ones"][0])
    b = np.array([[int(v) for v in d["dot_b"]]], np.int8)
    assert oracle.gemm_i32(q, b)[0, 0] == int(d["dot_b_value"][0])


# ------------------------------------------------------------------ INT8 quantizer pins

def test_quantizer_brute_force_nearest_level(oracle):
    """Each code is the level s*q (q in [-127,127]) nearest to the value (exhaustive search)."""
    rng = np.random.default_rng(3)
    y = rng.standard_t(4, size=(40, 64)) * rng.uniform(0.01, 10, size=(40, 1))
    q, s = oracle.quantize_rows_i8(y)
    levels = np.arange(-127, 128)
    y32 = y.astype(np.float32).astype(np.float64)
    for r in range(y.shape[0]):
        dist = np.abs(y32[r][:, None] - float(s[r]) * levels[None, :])
        best = levels[np.argmin(dist, axis=1)]
        assert np.array_equal(best, q[r].astype(np.int64))


def test_quantizer_invariants(oracle):
    rng = np.random.default_rng(4)
    y = rng.standard_normal((64, 300)) * np.exp(rng.uniform(-5, 5, size=(64, 1)))
    q, s = oracle.quantize_rows_i8(y)
    assert q.min() >= -127 and q.max() <= 127
    y32 = y.astype(np.float32).astype(np.float64)
    amax = np.abs(y32).max(axis=1)
    # scale is max|y|/127 rounded once to fp32
    assert np.all(np.abs(s.astype(np.float64) * 127.0 - amax) <= amax * 2.0 ** -23)
    # the largest element maps to +-127 and every element is within half a step
    arg = np.abs(y32).argmax(axis=1)
    assert np.all(np.abs(q[np.arange(64), arg]) == 127)
    err = np.abs(y32 - q * s.astype(np.float64)[:, None])
    assert np.all(err <= s.astype(np.float64)[:, None] * (0.5 + 1e-6))
    # a power-of-two rescale changes only the scale
    q2, s2 = oracle.quantize_rows_i8(y * 8.0)
    assert np.array_equal(q2, q) and np.array_equal(s2, s * np.float32(8.0))


def test_quantizer_zero_row(oracle):
    y = np.zeros((2, 16))
    y[1, 3] = -2.5
    q, s = oracle.quantize_rows_i8(y)
    assert s[0] == 0 and np.all(q[0] == 0)
    assert q[1, 3] == -127 and np.count_nonzero(q[1]) == 1


# ------------------------------------------------------------------ GEMM / dequant pins

def test_gemm_matches_numpy_int64_and_fp64(oracle):
    rng = np.random.default_rng(5)
    a = rng.integers(-127, 128, size=(37, 300), dtype=np.int8)
    b = rng.integers(-127, 128, size=(53, 300), dtype=np.int8)
    ref = a.astype(np.int64) @ b.astype(np.int64).T
    got = oracle.gemm_i32(a, b)
    assert np.array_equal(got.astype(np.int64), ref)
    assert np.array_equal(got.astype(np.float64), a.astype(np.float64) @ b.astype(np.float64).T)
    ms = rng.integers(0, 37, 100)
    ns = rng.integers(0, 53, 100)
    assert np.array_equal(oracle.gemm_i32_pairs(a, b, ms, ns), got[ms, ns])


def test_gemm_int32_range_bound(oracle):
    """|acc| <= 127^2 K fits int32 for K <= floor((2^31-1)/127^2) = 133144 and not beyond."""
    assert (2 ** 31 - 1) // (127 * 127) == 133144
    for K, ok in ((133144, True), (133145, False)):
        a = np.full((1, K), 127, np.int8)
        if ok:
            assert oracle.gemm_i32(a, a)[0, 0] == 127 * 127 * K
        else:
            with pytest.raises(oracle.OracleError):
                oracle.gemm_i32(a, a)


def test_dequant_closed_form(oracle):
    acc = np.array([[2, -3], [5, 0]], np.int32)
    y = oracle.dequant(acc, np.array([0.5, 2.0], np.float32), np.array([0.25, 4.0], np.float32),
                       np.array([1.0, -1.0], np.float32))
    assert np.array_equal(y, np.array([[2 * 0.5 * 0.25 + 1, -3 * 0.5 * 4 - 1], [5 * 2 * 0.25 + 1, -1.0]]))
    assert np.array_equal(oracle.dequant(acc, np.ones(2, np.float32), np.ones(2, np.float32), None), acc)


def test_w8a8_error_within_closed_form_bound(oracle):
    """|y_hat - XW^T| <= s_x/2 |w_rot|_1 + s_w/2 |x_rot|_1 + K s_x s_w / 4 per output."""
    x, w = workloads.tiny_inputs()
    x = x.double().numpy()
    w = w.double().numpy()
    r = oracle.linear_w8a8(x, w, None, 256)
    exact = x @ w.T
    xr = oracle.rotate(x, 256)
    wr = oracle.rotate(w, 256)
    sx = r["sx"].astype(np.float64)[:, None]
    sw = r["sw"].astype(np.float64)[None, :]
    K = x.shape[1]
    bound = sx / 2 * np.abs(wr).sum(1)[None, :] + sw / 2 * np.abs(xr).sum(1)[:, None] + K * sx * sw / 4
    assert np.all(np.abs(r["y"] - exact) <= bound * (1 + 1e-5) + 1e-12)


def test_convrot_flattens_outliers_better_than_plain_int8(oracle):
    """The pages' claim: the rotation spreads outlier energy so INT8 holds it better.
    Plain per-token/per-channel W8A8 is the g = 1 special case (rotation = identity)."""
    x, w = workloads.tiny_inputs()
    x = x.double().numpy()
    w = w.double().numpy()
    exact = x @ w.T
    err = {}
    for g in (1, 256):
        y = oracle.linear_w8a8(x, w, None, g)["y"]
        err[g] = np.abs(y - exact).max() / np.abs(exact).max()
    assert err[256] < 0.5 * err[1]
    assert err[256] < 2e-2


# ------------------------------------------------------------------ fp16 / INT4 pins

def test_f16_rounding_matches_numpy(oracle):
    rng = np.random.default_rng(6)
    vals = np.concatenate([
        rng.standard_normal(2000) * np.exp(rng.uniform(-20, 11, 2000)),
        [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e9, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14,
         1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 2047.0 / 2048, 5 / 7, 4.5 / 7],
    ])
    for v in vals:
        assert oracle.f16_from_double(v) == int(np.float16(v).view(np.uint16)), v
    for h in range(0, 65536, 7):
        ref = float(np.uint16(h).view(np.float16))
        got = oracle.f16_to_double(h)
        assert (np.isnan(ref) and np.isnan(got)) or ref == got


def test_int4_pack_roundtrip(oracle):
    allbytes = np.arange(256, dtype=np.uint8)[None, :]
    assert np.array_equal(oracle.pack_i4(oracle.unpack_i4(allbytes)), allbytes)
    codes = np.array([[-8, -7, -1, 0, 1, 7, 3, -4]], np.int8)
    assert np.array_equal(oracle.unpack_i4(oracle.pack_i4(codes)), codes)
    assert oracle.pack_i4(np.array([[1, 2]], np.int8))[0, 0] == 0x21


def test_int4_quantizer_brute_force_and_bounds(oracle):
    rng = np.random.default_rng(8)
    g = 32
    y = rng.standard_normal((6, 4 * g)) * np.exp(rng.uniform(-3, 3, size=(6, 4 * g // g))).repeat(g, 1)
    c, s = oracle.quantize_groups_i4(y, g)
    assert c.min() >= -7 and c.max() <= 7
    y32 = y.astype(np.float32).astype(np.float64)
    levels = np.arange(-7, 8)
    s64 = s.astype(np.float64)
    for r in range(y.shape[0]):
        for j in range(y.shape[1] // g):
            seg = y32[r, j * g:(j + 1) * g]
            # scale = fp16(max|.|/7), checked against numpy's fp16 rounding
            assert s[r, j] == np.float16(np.abs(seg).max() / 7.0)
            best = levels[np.argmin(np.abs(seg[:, None] - s64[r, j] * levels[None, :]), axis=1)]
            assert np.array_equal(best, c[r, j * g:(j + 1) * g].astype(np.int64))


@pytest.mark.parametrize("g", [256, 128])
def test_int4_group_sums_and_unit_scales(oracle, g):
    """With all scales 1 the W4A4 output is the plain integer product (exact), and each group
    partial sum is bounded by g * 7 * 7; 128 is the dynamic group of widths 256 does not divide."""
    rng = np.random.default_rng(9)
    cx = rng.integers(-7, 8, size=(5, 2 * g), dtype=np.int8)
    cw = rng.integers(-7, 8, size=(9, 2 * g), dtype=np.int8)
    ones = np.ones((5, 2), np.float16), np.ones((9, 2), np.float16)
    y = oracle.linear_i4(cx, ones[0], cw, ones[1], None, g)
    assert np.array_equal(y, (cx.astype(np.int64) @ cw.astype(np.int64).T).astype(np.float64))
    for j in range(2):
        part = cx[:, j * g:(j + 1) * g].astype(np.int64) @ cw[:, j * g:(j + 1) * g].astype(np.int64).T
        assert np.abs(part).max() <= g * 49
    # a scale on one group only scales that group's contribution
    sx = np.ones((5, 2), np.float16)
    sx[:, 1] = 0.5
    y2 = oracle.linear_i4(cx, sx, cw, ones[1], None, g)
    p0 = cx[:, :g].astype(np.int64) @ cw[:, :g].astype(np.int64).T
    p1 = cx[:, g:].astype(np.int64) @ cw[:, g:].astype(np.int64).T
    assert np.array_equal(y2, p0 + 0.5 * p1)


def test_w4a4_loses_more_than_w8a8(oracle):
    """The pages: full W4A4 loses quality relative to INT8 ConvRot (qualitative)."""
    x, w = workloads.tiny_inputs()
    x = x.double().numpy()
    w = w.double().numpy()
    exact = x @ w.T
    e8 = np.abs(oracle.linear_w8a8(x, w, None, 256)["y"] - exact).max()
    e4 = np.abs(oracle.linear_w4a4(x, w, None, 256)["y"] - exact).max()
    assert e4 > 2 * e8
    assert e4 / np.abs(exact).max() < 0.2


def test_w4a8_integer_core_and_group_scales(oracle):
    """W4A8 with unit scales is the plain integer product of INT8 tokens and INT4 weights
    (numpy int64); a per-group weight scale multiplies only that group's integer dot product,
    and the token scale multiplies the whole row (checked against numpy block products)."""
    rng = np.random.default_rng(11)
    g = 256
    qx = rng.integers(-127, 128, size=(6, 768), dtype=np.int8)
    cw = rng.integers(-7, 8, size=(10, 768), dtype=np.int8)
    y = oracle.linear_w4a8_codes(qx, np.ones(6, np.float32), cw, np.ones((10, 3), np.float16), None, g)
    assert np.array_equal(y, (qx.astype(np.int64) @ cw.astype(np.int64).T).astype(np.float64))
    sw = np.ones((10, 3), np.float16)
    sw[:, 1] = 0.25
    sw[:, 2] = 2.0
    sx = np.full(6, 0.5, np.float32)
    y2 = oracle.linear_w4a8_codes(qx, sx, cw, sw, None, g)
    parts = [qx[:, j * g:(j + 1) * g].astype(np.int64) @ cw[:, j * g:(j + 1) * g].astype(np.int64).T for j in range(3)]
    assert np.array_equal(y2, 0.5 * (parts[0] + 0.25 * parts[1] + 2.0 * parts[2]))
    # per-group integer sums stay far inside int32: 256 * 127 * 7
    assert max(np.abs(p).max() for p in parts) <= g * 127 * 7


def test_w4a8_error_sits_between_w8a8_and_w4a4(oracle):
    """4-bit weights with 8-bit tokens lose more than W8A8 and less than W4A4 on the same data."""
    x, w = workloads.tiny_inputs()
    x = x.double().numpy()
    w = w.double().numpy()
    exact = x @ w.T
    err = {name: np.abs(fn(x, w, None, 256)["y"] - exact).max()
           for name, fn in (("w8a8", oracle.linear_w8a8), ("w4a8", oracle.linear_w4a8), ("w4a4", oracle.linear_w4a4))}
    assert err["w8a8"] < err["w4a8"] < err["w4a4"], err


def test_w4a8_matches_its_definition_on_a_hand_case(oracle):
    """Brute force on a tiny case: g = 2, two groups, hand-written codes and scales."""
    qx = np.array([[3, -1, 2, 5]], np.int8)
    cw = np.array([[1, 2, -3, 4], [-7, 0, 7, 1]], np.int8)
    sw = np.array([[0.5, 2.0], [1.0, 0.25]], np.float16)
    sx = np.array([0.125], np.float32)
    b = np.array([1.0, -2.0], np.float32)
    # row 0: group 0: 3*1 + (-1)*2 = 1; group 1: 2*(-3) + 5*4 = 14 -> 0.125 * (0.5*1 + 2*14) + 1
    # row 1: group 0: 3*(-7) + 0 = -21; group 1: 2*7 + 5*1 = 19 -> 0.125 * (-21 + 0.25*19) - 2
    y = oracle.linear_w4a8_codes(qx, sx, cw, sw, b, 2)
    assert np.array_equal(y, np.array([[0.125 * (0.5 + 28.0) + 1.0, 0.125 * (-21.0 + 4.75) - 2.0]]))


def test_bias_is_added_once(oracle):
    x, w = workloads.tiny_inputs()
    x = x.double().numpy()
    w = w.double().numpy()
    b = np.arange(256, dtype=np.float32) * 0.125
    for fn in (oracle.linear_w8a8, oracle.linear_w4a4, oracle.linear_w4a8):
        assert np.allclose(fn(x, w, b, 256)["y"] - fn(x, w, None, 256)["y"], b[None, :], rtol=0, atol=1e-12)


def test_dynamic_group_pins(oracle):
    """Dynamic group choice: the pages' qkv layers (in_features 5376) keep 256 (nvfp4-convrot
    page, section 四, detail 3), the adaln projection weight [96768, 2688] of the pruning section
    (2688 = 2^7 * 21) gets 128; the Qwen3 widths keep 256."""
    assert oracle.dynamic_group(5376) == 256
    assert oracle.dynamic_group(2688) == 128
    for K in (5120, 8192, 25600):
        assert oracle.dynamic_group(K) == 256
    assert oracle.dynamic_group(2688, 64) == 64
    assert oracle.dynamic_group(96) == 32 and oracle.dynamic_group(7) == 1


def test_dynamic_group_brute_force(oracle):
    """Against an independent reading of the rule (largest power of two <= 256 among K's
    divisors, found by listing them) for every K up to 3000."""
    for K in range(1, 3001):
        divisors = [d for d in range(1, K + 1) if K % d == 0]
        best = max(d for d in divisors if d <= 256 and d & (d - 1) == 0)
        assert oracle.dynamic_group(K) == best, K
    with pytest.raises(ValueError):
        oracle.dynamic_group(0)
    with pytest.raises(ValueError):
        oracle.dynamic_group(512, 96)
