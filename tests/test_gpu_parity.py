"""HIP path vs CPU oracle, element by element, on seeded inputs (rules in tests/parity.py).

Sizes are chosen so the oracle finishes in seconds while the kernels still run several tiles
plus ragged tails; the full-size workloads are checked on sampled rows / outputs.
"""
import numpy as np
import pytest
import torch

from int4_quantized_linear_amd import workloads
from oracle import oracle as orc
from tests import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def cr():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from int4_quantized_linear_amd import convrot
    convrot.load()
    return convrot


def _np(t):
    return t.detach().cpu().numpy()


def _x64(t):
    return P.to_np64(t)


# ------------------------------------------------------------------ rotate + quantize (INT8)

QUANT_CASES = [
    # rows, K, g, dtype
    (4, 512, 256, torch.float32),
    (37, 320, 64, torch.bfloat16),
    (37, 320, 1, torch.bfloat16),
    (29, 320, 8, torch.float32),
    (64, 768, 128, torch.bfloat16),
    (65, 768, 32, torch.bfloat16),
    (300, 5376, 256, torch.bfloat16),
    (12, 5120, 256, torch.bfloat16),
    (5, 25600, 256, torch.bfloat16),
    (3, 40960, 256, torch.bfloat16),
    (2, 131072, 256, torch.bfloat16),
    (130, 2688, 128, torch.bfloat16),
]


@pytest.mark.parametrize("rows,K,g,dtype", QUANT_CASES)
def test_quantize_int8_parity(cr, rows, K, g, dtype):
    P.say("quantize_act int8 rows=%d K=%d g=%d %s" % (rows, K, g, dtype))
    x, _, _ = workloads.ragged_case(rows, K, 8, seed=rows + K + g, dtype=dtype)
    q, s = cr.quantize_act(x.to(DEV), group=g, bits=8)
    torch.cuda.synchronize()
    qr, sr = orc.quantize_act_i8(_x64(x), g)
    P.check_scales_f32(_np(s), sr)
    P.check_codes(_np(q), qr)


@pytest.mark.parametrize("g", [1, 128, 256])
def test_quantize_code_mismatch_rate_large_sample(cr, g):
    """Rule (a) held to the rate itself (no small-sample allowance) on 2M codes; g = 128 is the
    dynamic group, whose 1/sqrt(128) is inexact in fp32."""
    x, _, _ = workloads.ragged_case(512, 4096, 8, seed=77 + g)
    q, s = cr.quantize_act(x.to(DEV), group=g, bits=8)
    torch.cuda.synchronize()
    qr, sr = orc.quantize_act_i8(_x64(x), g)
    P.check_scales_f32(_np(s), sr)
    n = P.check_codes(_np(q), qr, slack=False)
    P.say("g=%d: %d mismatches in %d codes" % (g, n, qr.size))


@pytest.mark.parametrize("g", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_prepare_weight_bf16_rows_mismatch_rate_large_sample(cr, g):
    """bf16 N(0, 0.02) weight rows at every group, rule (a)'s rate with no allowance on 2.2M
    codes.  Small groups sum few bf16 values, so exact half-integer quotients are common there
    (a randomized shape sweep found 808 mismatches in 2.19M codes at g = 2 when those codes came
    from a rounded reciprocal).  Codes are the rint of the correctly rounded quotient, so groups
    of <= 16 channels, whose sums of bf16 values are exact in fp32, are held to 1e-6."""
    x, w, _ = workloads.ragged_case(10, 3584, 623, seed=2000 + g)
    wq, ws = cr.prepare_weight(w.to(DEV), g, 8)
    torch.cuda.synchronize()
    qr, sr = orc.prepare_weight_i8(_x64(w), g)
    P.check_scales_f32(_np(ws), sr)
    n = P.check_codes(_np(wq), qr, "weight codes", rate=1e-6 if g <= 16 else P.CODE_MISMATCH_RATE, slack=False)
    P.say("bf16 weight rows g=%d: %d mismatches in %d codes" % (g, n, qr.size))


@pytest.mark.parametrize("g", [1, 64, 128, 256])
def test_quantize_small_integer_inputs_ties(cr, g):
    """Integer-valued activations (|x| <= 3): the rotated values carry few significant bits, so
    exact half-integer quotients are common at every group (an fp32 model of a code taken as the
    product with a rounded reciprocal misses 6.7e-4 of them at g = 256).  The codes are the rint of
    the correctly rounded quotient on both sides, so they must agree everywhere (1e-6 on 2M INT8
    codes; INT4 at the groups it supports)."""
    x = torch.from_numpy(np.random.default_rng(500 + g).integers(-3, 4, size=(512, 4096)).astype(np.float32))
    xd = x.bfloat16().to(DEV)
    q, s = cr.quantize_act(xd, group=g, bits=8)
    torch.cuda.synchronize()
    qr, sr = orc.quantize_act_i8(x.double().numpy(), g)
    P.check_scales_f32(_np(s), sr)
    n = P.check_codes(_np(q), qr, "int8 codes", rate=1e-6, slack=False)
    P.say("small-integer inputs g=%d: %d INT8 mismatches in %d codes" % (g, n, qr.size))
    if g in (128, 256):
        q4, s4 = cr.quantize_act(xd, group=g, bits=4)
        torch.cuda.synchronize()
        c, sr4, _ = orc.prepare_i4(x.double().numpy(), g)
        P.check_scales_f16(_np(s4).T, sr4, "fp16 scales", slack=False)
        n4 = P.check_codes(orc.unpack_i4(_np(q4)), c, "int4 codes", rate=1e-6, slack=False)
        P.say("small-integer inputs g=%d: %d INT4 mismatches in %d codes" % (g, n4, c.size))


@pytest.mark.parametrize("g", [128, 256])
def test_quantize_int4_mismatch_rates_large_sample(cr, g):
    """INT4 codes held to rule (a)'s rate itself (no small-sample allowance) on 8M codes, and the
    fp16 group scales to their own rate on 32k-64k scales: both sides round max|group|/7 once to
    fp16 from the same fp32 group maximum, so a scale differs only where the fp32 rotation sums
    give a different maximum right at an fp16 rounding edge."""
    x, _, _ = workloads.ragged_case(2048, 4096, 8, seed=88 + g)
    q, s = cr.quantize_act(x.to(DEV), group=g, bits=4)
    torch.cuda.synchronize()
    c, sr, _ = orc.prepare_i4(_x64(x), g)
    ns = P.check_scales_f16(_np(s).T, sr, "fp16 scales", slack=False)
    n = P.check_codes(orc.unpack_i4(_np(q)), c, "int4 codes", slack=False)
    P.say("int4 g=%d: %d code mismatches in %d codes, %d scale mismatches in %d scales" % (
        g, n, c.size, ns, sr.size))


# Larger row counts (several persistent rounds of row groups, ragged last round) at K of 9..32
# slots of 256 channels, even and odd log2 g; a zero row and one huge outlier in each.
LARGE_QUANT_CASES = [
    (1024, 5376, 256),
    (1100, 2304, 128),
    (1031, 4096, 2),
    (1030, 6144, 32),
    (2048, 5120, 128),
    (1500, 8192, 256),
]


@pytest.mark.parametrize("rows,K,g", LARGE_QUANT_CASES)
def test_quantize_int8_parity_many_rows(cr, rows, K, g):
    P.say("quantize_act int8 rows=%d K=%d g=%d" % (rows, K, g))
    x, _, _ = workloads.ragged_case(rows, K, 8, seed=rows + K + g)
    x[3] = 0                    # a zero row: scale 0, codes 0
    x[rows - 1, 5] = 3.0e4      # one huge outlier
    q, s = cr.quantize_act(x.to(DEV), group=g, bits=8)
    torch.cuda.synchronize()
    qr, sr = orc.quantize_act_i8(_x64(x), g)
    assert _np(s)[3] == 0 and np.all(_np(q)[3] == 0)
    P.check_scales_f32(_np(s), sr)
    P.check_codes(_np(q), qr)


@pytest.mark.parametrize("rows,K,g", LARGE_QUANT_CASES)
def test_quantize_bf16_and_fp32_inputs_agree(cr, rows, K, g):
    """The same bf16 values given as fp32: the two input widths share every arithmetic step
    after the load, so codes and scales are equal bit for bit."""
    x, _, _ = workloads.ragged_case(rows, K, 8, seed=3 * rows + K + g)
    xd = x.to(DEV)
    q16, s16 = cr.quantize_act(xd, group=g, bits=8)
    q32, s32 = cr.quantize_act(xd.float(), group=g, bits=8)
    torch.cuda.synchronize()
    assert torch.equal(q16, q32)
    assert torch.equal(s16.view(torch.int32), s32.view(torch.int32))


@pytest.mark.parametrize("g", [128, 256])
def test_quantize_prefill_width_mismatch_rate_large_sample(cr, g):
    """Rule (a) held to the rate itself on 5.5M codes at the prefill activations' K."""
    x, _, _ = workloads.ragged_case(1024, 5376, 8, seed=99 + g)
    q, s = cr.quantize_act(x.to(DEV), group=g, bits=8)
    torch.cuda.synchronize()
    qr, sr = orc.quantize_act_i8(_x64(x), g)
    P.check_scales_f32(_np(s), sr)
    n = P.check_codes(_np(q), qr, slack=False)
    P.say("K=5376 g=%d: %d mismatches in %d codes" % (g, n, qr.size))


def test_quantize_zero_rows_and_single_outlier(cr):
    x = torch.zeros(6, 512)
    x[1, 7] = 1000.0
    x[3] = torch.linspace(-1, 1, 512)
    x[4, :] = 1e-3
    q, s = cr.quantize_act(x.to(DEV), group=256, bits=8)
    torch.cuda.synchronize()
    qr, sr = orc.quantize_act_i8(x.double().numpy(), 256)
    assert _np(s)[0] == 0 and np.all(_np(q)[0] == 0)
    P.check_scales_f32(_np(s), sr)
    P.check_codes(_np(q), qr, rate=0.0)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("g", [128, 256])
def test_quantize_tiny_rows(cr, g, dtype):
    """Rows of tiny magnitude: an fp32 scale below 2^-100 (1/s would overflow past 2^-128) is
    handled with v and s scaled by 2^64, exactly, so the codes are those of the same row at
    ordinary magnitude and equal the oracle's."""
    x, _, _ = workloads.ragged_case(8, 1024, 8, seed=31 + g)
    x = x.float()
    x[1] *= 2.0 ** -110          # scale near 2^-109
    x[2] *= 2.0 ** -118          # scale near 2^-117
    x[3] = 0.0
    x[4] = 0.0
    x[4, 7] = 2.0 ** -112        # one tiny value
    x[5] *= 2.0 ** 100           # large, for contrast
    x = x.to(dtype)
    q, s = cr.quantize_act(x.to(DEV), group=g, bits=8)
    torch.cuda.synchronize()
    qr, sr = orc.quantize_act_i8(_x64(x), g)
    P.check_scales_f32(_np(s), sr)
    P.check_codes(_np(q), qr, "codes", rate=0.0)
    # a row scaled by a power of two has the codes of the unscaled row
    q0, _ = cr.quantize_act((x[0:1].float() * 2.0 ** -110).to(dtype).to(DEV), group=g, bits=8)
    q1, _ = cr.quantize_act(x[0:1].to(DEV), group=g, bits=8)
    torch.cuda.synchronize()
    assert torch.equal(q0, q1)


def test_prepare_weight_same_as_quantize_act(cr):
    w = workloads.gaussian_weights(300, 768, cfg=99)
    a = cr.prepare_weight(w.to(DEV), 256, 8)
    b = cr.quantize_act(w.to(DEV), 256, 8)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ------------------------------------------------------------------ integer core (rule b)

GEMM_CASES = [
    # M, N, K  (M <= 16 runs the decode GEMV kernel)
    (1, 64, 64), (12, 1000, 5120), (16, 264, 320), (12, 8192, 5120), (3, 5120, 25600),
    (17, 8, 64), (300, 264, 320), (513, 1000, 5376), (256, 256, 128), (1000, 1280, 1024),
    # N % 8 != 0 (element stores; N % 4 != 0 too): GEMV and GEMM
    (12, 1003, 5120), (12, 7, 320), (17, 7, 64), (33, 1001, 320), (300, 262, 5376),
    # the longest K the ABI takes (CONVROT_MAX_K): GEMV and GEMM
    (5, 40, 131072), (17, 72, 131072),
]


@pytest.mark.parametrize("M,N,K", GEMM_CASES)
def test_gemm_i32_bit_exact(cr, M, N, K):
    P.say("gemm_i8_i32 M=%d N=%d K=%d" % (M, N, K))
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    a = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    b = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    acc = cr.gemm_i8_i32(torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV))
    torch.cuda.synchronize()
    ref = orc.gemm_i32(a, b)
    assert np.array_equal(_np(acc), ref)


def test_gemm_i32_extreme_values(cr):
    """All-(+-127) operands reach the largest accumulators."""
    M, N, K = 40, 72, 5376
    a = np.full((M, K), 127, np.int8)
    a[1::2] = -127
    b = np.full((N, K), -127, np.int8)
    acc = cr.gemm_i8_i32(torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(_np(acc), orc.gemm_i32(a, b))
    assert abs(int(_np(acc)[0, 0])) == 127 * 127 * K


# ------------------------------------------------------------------ full INT8 linear (rules a-d)

def _linear_case(cr, x, w, b, g):
    xd, wd = x.to(DEV), w.to(DEV)
    bd = None if b is None else b.to(DEV)
    wq, ws = cr.prepare_weight(wd, g, 8)
    y = cr.linear(xd, wq, ws, bd, group=g)
    xq, xs = cr.quantize_act(xd, g, 8)
    y2 = cr.linear(None, wq, ws, bd, group=g, xq=xq, x_scale=xs)
    torch.cuda.synchronize()
    ref = orc.linear_w8a8(_x64(x), _x64(w), None if b is None else b.numpy(), g)
    P.check_codes(_np(wq), ref["qw"], "qw")
    P.check_scales_f32(_np(ws), ref["sw"], "sw")
    P.check_codes(_np(xq), ref["qx"], "qx")
    P.check_scales_f32(_np(xs), ref["sx"], "sx")
    # y against the oracle's dequant of the GPU's own codes (exact integer part; only fp32 and
    # bf16 rounding differ) ...
    bn = None if b is None else b.numpy()
    yown = orc.dequant(orc.gemm_i32(_np(xq), _np(wq)), _np(xs), _np(ws), bn)
    P.check_y(_x64(y), yown, "y (own codes)", strict_frac=1e-4)
    # ... and rule (d) against the oracle end to end: a code that rule (a) lets differ moves a
    # whole output row (an activation code) or column (a weight code) by one code step, so the
    # element-wise bf16-ulp count is loose here, as in the W4A4 and W4A8 cases
    P.check_y(_x64(y), ref["y"], "y (oracle codes)", strict_frac=2e-2)
    assert torch.equal(y, y2), "pre-quantized path differs from the fused path"
    return y, ref


def test_linear_tiny_config(cr):
    x, w = workloads.tiny_inputs()
    _linear_case(cr, x, w, None, 256)
    b = torch.from_numpy(np.linspace(-1, 1, 256).astype(np.float32))
    _linear_case(cr, x, w, b, 256)


LINEAR_CASES = [
    (12, 1000, 320, 64), (16, 1024, 5120, 256), (1, 200, 512, 256), (17, 264, 320, 32),
    (300, 1000, 768, 128), (257, 520, 1024, 256), (600, 264, 2688, 128),
    # N % 8 != 0: the element-store epilogues of the GEMV and the GEMM
    (12, 1001, 320, 64), (40, 1003, 512, 256), (257, 517, 1024, 256),
]


@pytest.mark.parametrize("M,N,K,g", LINEAR_CASES)
def test_linear_ragged(cr, M, N, K, g):
    P.say("linear M=%d N=%d K=%d g=%d" % (M, N, K, g))
    x, w, b = workloads.ragged_case(M, K, N, seed=3)
    _linear_case(cr, x, w, b, g)


@pytest.mark.parametrize("K,N", workloads.DECODE_SHAPES)
def test_linear_decode_shapes(cr, K, N):
    P.say("decode linear M=12 K=%d N=%d" % (K, N))
    x, w = workloads.decode_inputs(K, N)
    _linear_case(cr, x, w, None, 256)


def test_linear_dynamic_group_adaln_width(cr):
    """A layer whose in_features (2688, the adaln projection's) 256 does not divide: the dynamic
    group (128) through prepare / quantize / linear, against the oracle at the same group."""
    K = 2688
    g = cr.dynamic_group(K)
    assert g == 128
    for M, N in [(12, 1000), (300, 2048)]:
        P.say("dynamic-group linear M=%d N=%d K=%d g=%d" % (M, N, K, g))
        x, w, b = workloads.ragged_case(M, K, N, seed=11)
        _linear_case(cr, x, w, b, g)
    # W4A4 takes the same group (128-channel rotation and scale groups), against the oracle
    for M, N in [(12, 1000), (300, 2048)]:
        P.say("dynamic-group W4A4 M=%d N=%d K=%d g=%d" % (M, N, K, g))
        _w4a4_case(cr, *workloads.ragged_case(M, K, N, seed=12), g)
    # and the W4A8 decode path (two scale sets per 256-channel block, a zero upper half in the
    # last one); the group-256 re-layout still rejects the width, nothing is silently regrouped
    P.say("dynamic-group W4A8 M=12 N=1000 K=%d g=%d" % (K, g))
    _w4a8_case(cr, *workloads.ragged_case(12, K, 1000, seed=13), "w4a8 dynamic-group y", g=g)
    w4 = workloads.gaussian_weights(64, K, cfg=94).to(DEV)
    wq4, ws4 = cr.prepare_weight(w4, g, 4)
    assert ws4.shape == (K // g, 64)
    with pytest.raises(cr.ConvRotError, match="SHAPE|GROUP"):
        cr.pack_weight_w4a8(wq4, ws4)
    # weights packed with one scale group and called with the other are rejected on the host
    # (the two layouts differ in size), never read past their end or misread
    w5 = workloads.gaussian_weights(64, 5120, cfg=94).to(DEV)
    for gp, gc in ((256, 128), (128, 256)):
        wq5, ws5 = cr.prepare_weight(w5, gp, 4)
        wp5 = cr.pack_weight_w4a8(wq5, ws5, gp)
        x5 = workloads.heavy_tailed_acts(12, 5120, cfg=94, layer=1).to(DEV)
        with pytest.raises(cr.ConvRotError, match="SHAPE"):
            cr.linear_w4a8(x5, wp5, 64, group=gc)


def test_linear_prefill_full_size_sampled(cr):
    """Full 4096 x 5376 x 16128 workload; oracle on 384 sampled token rows / weight rows and
    4096 sampled outputs."""
    M, K, N = workloads.PREFILL["M"], workloads.PREFILL["K"], workloads.PREFILL["N"]
    x, w, b = workloads.prefill_inputs()
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    wq, ws = cr.prepare_weight(wd, 256, 8)
    y = cr.linear(xd, wq, ws, bd, group=256)
    xq, xs = cr.quantize_act(xd, 256, 8)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    mr = np.sort(rng.choice(M, 384, replace=False))
    nr = np.sort(rng.choice(N, 384, replace=False))
    qx, sx = orc.quantize_act_i8(_x64(x[mr]), 256)
    qw, sw = orc.prepare_weight_i8(_x64(w[nr]), 256)
    P.check_codes(_np(xq)[mr], qx, "qx rows")
    P.check_scales_f32(_np(xs)[mr], sx, "sx rows")
    P.check_codes(_np(wq)[nr], qw, "qw rows")
    P.check_scales_f32(_np(ws)[nr], sw, "sw rows")
    ii = rng.integers(0, 384, 4096)
    jj = rng.integers(0, 384, 4096)
    acc = orc.gemm_i32_pairs(qx, qw, ii, jj)
    yref = acc.astype(np.float64) * sx[ii].astype(np.float64) * sw[jj].astype(np.float64) + b.numpy()[nr[jj]]
    ygpu = _x64(y)[mr[ii], nr[jj]]
    P.check_y(ygpu, yref, "sampled y")
    # integer core at full size on the GPU's own codes for the same pairs
    accg = _np(cr.gemm_i8_i32(xq, wq))
    assert np.array_equal(accg[mr[ii], nr[jj]], orc.gemm_i32_pairs(_np(xq), _np(wq), mr[ii], nr[jj]))


def _stack_groups():
    """The layer stack's linears grouped by shared input, as the bench fuses them."""
    groups = []
    for i, (name, K, N) in enumerate(workloads.STACK_MATRICES):
        inp = workloads.STACK_INPUT_OF[name]
        if groups and groups[-1][0] == inp:
            groups[-1][2].append((i, N))
        else:
            groups.append((inp, K, [(i, N)]))
    return groups


STACK_TEST_LAYERS = [0, 31, 63]


@pytest.mark.parametrize("layer", STACK_TEST_LAYERS)
@pytest.mark.parametrize("inp,K,members", _stack_groups(), ids=[g[0] for g in _stack_groups()])
def test_linear_stack_shapes_full_size_sampled(cr, inp, K, members, layer):
    """The layer stack's GEMMs at their full size (M = 2048; q|k|v and gate|up as one GEMM over the
    concatenated weight rows, o with K = 8192, down with K = 25600), on the device-drawn inputs of
    the first, a middle and the last layer; the oracle on 256 sampled token rows / weight rows and
    4096 sampled outputs."""
    M = workloads.STACK_M
    j = [name for name, _ in workloads.STACK_INPUTS].index(inp)
    P.say("stack layer %d %s: M=%d K=%d N=%d" % (layer, inp, M, K, sum(N for _, N in members)))
    x = workloads.stack_acts(layer, j, M, K, DEV)
    w = torch.cat([workloads.stack_weight(layer, i, N, K, DEV) for i, N in members])
    N = w.shape[0]
    wq, ws = cr.prepare_weight(w, 256, 8)
    y = cr.linear(x, wq, ws, group=256)
    xq, xs = cr.quantize_act(x, 256, 8)
    torch.cuda.synchronize()
    rng = np.random.default_rng(K + N + 1000 * layer)
    mr = np.sort(rng.choice(M, 256, replace=False))
    nr = np.sort(rng.choice(N, 256, replace=False))
    x_h, w_h = x[torch.from_numpy(mr).to(DEV)].cpu(), w[torch.from_numpy(nr).to(DEV)].cpu()
    qx, sx = orc.quantize_act_i8(_x64(x_h), 256)
    qw, sw = orc.prepare_weight_i8(_x64(w_h), 256)
    P.check_codes(_np(xq)[mr], qx, "qx rows")
    P.check_scales_f32(_np(xs)[mr], sx, "sx rows")
    P.check_codes(_np(wq)[nr], qw, "qw rows")
    P.check_scales_f32(_np(ws)[nr], sw, "sw rows")
    ii = rng.integers(0, 256, 4096)
    jj = rng.integers(0, 256, 4096)
    acc = orc.gemm_i32_pairs(qx, qw, ii, jj)
    yref = acc.astype(np.float64) * sx[ii].astype(np.float64) * sw[jj].astype(np.float64)
    P.check_y(_x64(y)[mr[ii], nr[jj]], yref, "sampled y")
    # the integer core on the GPU's own codes, bit-exact on the same pairs
    accg = cr.gemm_i8_i32(xq, wq)
    torch.cuda.synchronize()
    ti, tj = torch.from_numpy(mr[ii]).to(DEV), torch.from_numpy(nr[jj]).to(DEV)
    got = accg[ti, tj].cpu().numpy()
    del accg
    assert np.array_equal(got, orc.gemm_i32_pairs(_np(xq), _np(wq), mr[ii], nr[jj]))


# Shapes whose tiles leave the last round of the persistent GEMM partly idle, so the tail tiles
# are split in K (int32 partial sums in the workspace, then a second kernel): mid-size M, ragged
# M, long K, and the layer stack's k/v projection (N = 1024 at M = 2048: 32 tiles).
SPLIT_CASES = [(64, 8192, 5120, True), (17, 520, 1024, False), (300, 1000, 4096, True), (130, 1000, 2048, True),
               (513, 1000, 5376, False), (200, 5120, 25600, True), (2048, 1024, 5120, True)]


@pytest.mark.parametrize("M,N,K,with_bias", SPLIT_CASES)
def test_linear_split_k_tail_bit_identical(cr, M, N, K, with_bias):
    P.say("split-K tail M=%d N=%d K=%d" % (M, N, K))
    # the workspace the binding passes has a split region for these shapes
    assert cr.workspace_bytes(M, N, K, 8) > _r256(M * K) + _r256(4 * M)
    x = workloads.heavy_tailed_acts(M, K, cfg=95, layer=M).to(DEV)
    w = workloads.gaussian_weights(N, K, cfg=95, layer=N).to(DEV)
    b = torch.randn(N, generator=torch.Generator().manual_seed(N)).to(DEV) if with_bias else None
    xq, xs = cr.quantize_act(x, 256, 8)
    wq, ws = cr.prepare_weight(w, 256, 8)
    y_split = cr.linear(None, wq, ws, b, xq=xq, x_scale=xs)
    y_whole = cr.linear(None, wq, ws, b, xq=xq, x_scale=xs, split_k=False)
    y_again = cr.linear(x, wq, ws, b)
    torch.cuda.synchronize()
    assert torch.equal(y_split, y_whole)
    assert torch.equal(y_again, y_whole)
    # and against the oracle on the GPU's own codes
    rng = np.random.default_rng(M + N + K)
    ii, jj = rng.integers(0, M, 2048), rng.integers(0, N, 2048)
    acc = orc.gemm_i32_pairs(_np(xq), _np(wq), ii, jj)
    yref = acc.astype(np.float64) * _np(xs)[ii].astype(np.float64) * _np(ws)[jj].astype(np.float64)
    if b is not None:
        yref += b.cpu().numpy().astype(np.float64)[jj]
    P.check_y(_x64(y_split)[ii, jj], yref, "sampled y")


def _r256(n):
    return (n + 255) // 256 * 256


def test_linear_concatenated_rows_equal_separate(cr):
    # Linears sharing an input can run as one GEMM over their concatenated weight rows: row-wise
    # scales make the concatenation's preparation the concatenation of the separate ones, and
    # every output is computed the same way, so the results are bit-identical.
    M, K = 300, 1024
    x = workloads.heavy_tailed_acts(M, K, cfg=97, layer=0).to(DEV)
    parts = [workloads.gaussian_weights(N, K, cfg=97 + i).to(DEV) for i, N in enumerate((512, 128, 128))]
    xq, xs = cr.quantize_act(x, 256, 8)
    sep = []
    for w in parts:
        wq, ws = cr.prepare_weight(w, 256, 8)
        sep.append(cr.linear(None, wq, ws, xq=xq, x_scale=xs))
    wq, ws = cr.prepare_weight(torch.cat(parts), 256, 8)
    fused = cr.linear(None, wq, ws, xq=xq, x_scale=xs)
    torch.cuda.synchronize()
    assert torch.equal(fused, torch.cat(sep, dim=1))


def test_linear_empty_and_repeat(cr):
    w = workloads.gaussian_weights(64, 256, cfg=98).to(DEV)
    wq, ws = cr.prepare_weight(w, 256, 8)
    y = cr.linear(torch.empty(0, 256, dtype=torch.bfloat16, device=DEV), wq, ws)
    assert y.shape == (0, 64)
    # two decode calls in a row with different inputs
    for seed in (1, 2):
        x = workloads.heavy_tailed_acts(12, 256, cfg=98, layer=seed).to(DEV)
        y = cr.linear(x, wq, ws)
        torch.cuda.synchronize()
        ref = orc.linear_w8a8(_x64(x), _x64(w), None, 256)
        P.check_y(_x64(y), ref["y"])


# ------------------------------------------------------------------ W4A4

W4_QUANT_CASES = [(4, 512, 256), (37, 768, 256), (300, 5376, 256), (12, 25600, 256), (37, 2688, 128),
                  (5, 384, 128), (64, 1024, 128)]


@pytest.mark.parametrize("rows,K,g", W4_QUANT_CASES)
def test_quantize_int4_parity(cr, rows, K, g):
    P.say("quantize int4 rows=%d K=%d g=%d" % (rows, K, g))
    x, _, _ = workloads.ragged_case(rows, K, 8, seed=rows + K)
    q, s = cr.quantize_act(x.to(DEV), g, 4)
    torch.cuda.synchronize()
    assert s.shape == (K // g, rows)
    c, sr, pr = orc.prepare_i4(_x64(x), g)
    P.check_scales_f16(_np(s).T, sr)
    P.check_codes(orc.unpack_i4(_np(q)), c, "int4 codes")


W4_GEMM_CASES = [(17, 256, 256), (130, 264, 512), (300, 520, 5376), (1, 8, 256)]


@pytest.mark.parametrize("M,N,K", W4_GEMM_CASES)
def test_gemm_i4_bit_exact(cr, M, N, K):
    P.say("gemm_i4_i32 M=%d N=%d K=%d" % (M, N, K))
    rng = np.random.default_rng(M + N + K)
    cx = rng.integers(-8, 8, size=(M, K), dtype=np.int8)
    cw = rng.integers(-8, 8, size=(N, K), dtype=np.int8)
    acc = cr.gemm_i4_i32(torch.from_numpy(orc.pack_i4(cx)).to(DEV), torch.from_numpy(orc.pack_i4(cw)).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(_np(acc), orc.gemm_i32(cx, cw))


def test_gemm_i4_every_code_at_max_k(cr):
    # Rows of one constant code each (all 16 nibbles, -8..7) against the same on the weight side
    # plus random rows, at the largest K: every code's matrix-core encoding is exercised and the
    # sums reach 64 * 131072 = 2^23 in magnitude.
    M, N, K = 16, 40, 131072
    P.say("gemm_i4_i32 every code M=%d N=%d K=%d" % (M, N, K))
    rng = np.random.default_rng(16)
    cx = np.repeat(np.arange(-8, 8, dtype=np.int8)[:, None], K, axis=1)
    cw = np.concatenate([cx, rng.integers(-8, 8, size=(N - M, K), dtype=np.int8)])
    acc = cr.gemm_i4_i32(torch.from_numpy(orc.pack_i4(cx)).to(DEV), torch.from_numpy(orc.pack_i4(cw)).to(DEV))
    torch.cuda.synchronize()
    ref = orc.gemm_i32(cx, cw)
    assert ref[0, 0] == 64 * K and ref[0, 15] == -56 * K
    assert np.array_equal(_np(acc), ref)


# FP6 E3M2 (OCP Microscaling Formats v1.0): sign bit 5, exponent bits 2..4 with bias 3, mantissa
# bits 0..1; exponent 0 is subnormal (m/4 * 2^-2).
def _e3m2_value(c: np.ndarray) -> np.ndarray:
    c = c.astype(np.int64)
    e, m = (c >> 2) & 7, c & 3
    mag = np.where(e == 0, m / 4.0 * 2.0 ** -2, (1 + m / 4.0) * 2.0 ** (e - 3.0))
    return np.where(c >> 5 == 1, -mag, mag)


def _unpack_w4a4_tiles(buf: np.ndarray, N: int, K: int) -> np.ndarray:
    """Codes [N, K] from the pre-encoded W4A4 buffer: per 32-row block and 64-channel step a
    1536-byte piece; lane l = r + 32 h holds row r, channels 64 step + 32 h + s at bit 6 s of
    bytes 16 l .. 16 l + 15 followed by 1024 + 8 l .. 1024 + 8 l + 7."""
    RB, KS = -(-N // 32), K // 64
    pieces = buf[:RB * KS * 1536].reshape(RB, KS, 1536)
    s24 = np.concatenate([pieces[:, :, :1024].reshape(RB, KS, 64, 16), pieces[:, :, 1024:].reshape(RB, KS, 64, 8)],
                         axis=3)
    bits = np.unpackbits(s24, axis=3, bitorder="little").reshape(RB, KS, 64, 32, 6).astype(np.int64)
    codes = (bits << np.arange(6)).sum(axis=4)                       # [RB, KS, lane, s]
    vals = _e3m2_value(codes).reshape(RB, KS, 2, 32, 32)             # [RB, KS, h, r, s]
    out = vals.transpose(0, 3, 1, 2, 4).reshape(RB * 32, K)          # row 32 rb + r, channel 64 ks + 32 h + s
    assert np.all(out == np.round(out))
    assert np.all(out[N:] == 0), "rows past N must be zeros"
    return out[:N].astype(np.int64)


@pytest.mark.parametrize("N,K", [(32, 256), (200, 512), (1000, 5376)])
def test_pack_w4a4_layout(cr, N, K):
    P.say("pack_weight_w4a4 N=%d K=%d" % (N, K))
    rng = np.random.default_rng(N + K)
    cw = rng.integers(-8, 8, size=(N, K), dtype=np.int8)
    wp = cr.pack_weight_w4a4(torch.from_numpy(orc.pack_i4(cw)).to(DEV))
    torch.cuda.synchronize()
    assert wp.numel() == cr.packed_bytes_w4a4(N, K)
    assert np.array_equal(_unpack_w4a4_tiles(_np(wp), N, K), cw.astype(np.int64))


W4_LINEAR_CASES = [(4, 256, 512, 256), (130, 264, 768, 256), (257, 1024, 5376, 256), (12, 1024, 5120, 256),
                   (130, 264, 384, 128), (257, 520, 2688, 128)]


@pytest.mark.parametrize("M,N,K,g", W4_LINEAR_CASES)
def test_linear_w4a4_packed_matches(cr, M, N, K, g):
    # the pre-encoded weights give the per-call path's result bit for bit, with x and with xq
    P.say("linear_w4a4_packed M=%d N=%d K=%d g=%d" % (M, N, K, g))
    x, w, b = workloads.ragged_case(M, K, N, seed=6)
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    wq, ws = cr.prepare_weight(wd, g, 4)
    wp = cr.pack_weight_w4a4(wq)
    xq, xs = cr.quantize_act(xd, g, 4)
    y1 = cr.linear_w4a4(xd, wq, ws, bd, group=g)
    y2 = cr.linear_w4a4_packed(xd, wp, ws, bd, group=g)
    y3 = cr.linear_w4a4_packed(None, wp, ws, bd, group=g, xq=xq, x_scale=xs)
    y4 = cr.linear_w4a4_packed(None, wp, ws, None, group=g, xq=xq, x_scale=xs)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(y1, y3)
    yown = orc.linear_i4(orc.unpack_i4(_np(xq)), _np(xs).T, orc.unpack_i4(_np(wq)), _np(ws).T, None, g)
    P.check_y(_x64(y4), yown, "y (no bias, own codes)", strict_frac=1e-4)


FUSED_W4_CASES = [(M, K, g) for M in (1, 31, 33, 100) for K, g in ((256, 256), (384, 128), (2688, 128), (5376, 256))]
# the largest K, and the largest K with a half 256-block at the end (group 128)
FUSED_W4_CASES += [(33, 131072, 256), (40, 130944, 128)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("M,K,g", FUSED_W4_CASES)
def test_linear_w4a4_x_given_matches_codes_path(cr, M, K, g, dtype):
    """With x given, the W4A4 linear rotates and quantizes straight into the GEMM's FP6 token tiles
    (rows padded to the 32-row block with zero codes); the result must equal, bit for bit, the
    linear on the packed INT4 codes and fp16 scales that quantize_act makes from the same x."""
    N = 72
    P.say("linear_w4a4 x given vs codes M=%d N=%d K=%d g=%d %s" % (M, N, K, g, dtype))
    x, w, b = workloads.ragged_case(M, K, N, seed=9, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    wq, ws = cr.prepare_weight(wd, g, 4)
    wp = cr.pack_weight_w4a4(wq)
    xq, xs = cr.quantize_act(xd, g, 4)
    y_x = cr.linear_w4a4(xd, wq, ws, bd, group=g)
    y_q = cr.linear_w4a4(None, wq, ws, bd, group=g, xq=xq, x_scale=xs)
    yp_x = cr.linear_w4a4_packed(xd, wp, ws, None, group=g)
    yp_q = cr.linear_w4a4_packed(None, wp, ws, None, group=g, xq=xq, x_scale=xs)
    torch.cuda.synchronize()
    assert torch.equal(y_x, y_q)
    assert torch.equal(yp_x, yp_q)
    yown = orc.linear_i4(orc.unpack_i4(_np(xq)), _np(xs).T, orc.unpack_i4(_np(wq)), _np(ws).T, b.numpy(), g)
    P.check_y(_x64(y_x), yown, "y (own codes)", strict_frac=1e-4)


W4_WHOLE_TILE_CASES = [(1000, 4000, 512, 256), (1100, 8200, 512, 256), (1100, 8200, 384, 128)]


@pytest.mark.parametrize("M,N,K,g", W4_WHOLE_TILE_CASES)
def test_linear_w4a4_whole_tile_grids(cr, M, N, K, g):
    """Ragged shapes whose grids take several rounds of the persistent walk (8 x 16 and 9 x 33
    tiles of 256 x 128), against the oracle on the GPU's own codes and end to end."""
    P.say("linear_w4a4 whole-tile grid M=%d N=%d K=%d g=%d" % (M, N, K, g))
    _w4a4_case(cr, *workloads.ragged_case(M, K, N, seed=12), g)


def _w4a4_case(cr, x, w, b, g):
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    wq, ws = cr.prepare_weight(wd, g, 4)
    y = cr.linear_w4a4(xd, wq, ws, bd, group=g)
    xq, xs = cr.quantize_act(xd, g, 4)
    torch.cuda.synchronize()
    ref = orc.linear_w4a4(_x64(x), _x64(w), b.numpy(), g)
    P.check_scales_f16(_np(ws).T, ref["sw"], "sw16")
    P.check_scales_f16(_np(xs).T, ref["sx"], "sx16")
    # y against the oracle evaluated on the GPU's own codes and scales (exact integer part) ...
    yown = orc.linear_i4(orc.unpack_i4(_np(xq)), _np(xs).T, orc.unpack_i4(_np(wq)), _np(ws).T, b.numpy(), g)
    P.check_y(_x64(y), yown, "y (own codes)", strict_frac=1e-4)
    # ... and against the oracle end to end
    P.check_y(_x64(y), ref["y"], "y (oracle codes)", strict_frac=2e-2)


@pytest.mark.parametrize("M,N,K,g", W4_LINEAR_CASES)
def test_linear_w4a4_parity(cr, M, N, K, g):
    P.say("linear_w4a4 M=%d N=%d K=%d g=%d" % (M, N, K, g))
    _w4a4_case(cr, *workloads.ragged_case(M, K, N, seed=5), g)


def test_linear_w4a4_full_size_sampled(cr):
    """Full 4096 x 5376 x 10752 W4A4 workload, per-call and pre-encoded weights (the bench's
    serving path); the oracle on 384 sampled token rows x 384 sampled weight rows."""
    M, K, N = workloads.W4A4_SHAPE["M"], workloads.W4A4_SHAPE["K"], workloads.W4A4_SHAPE["N"]
    P.say("linear_w4a4 full size M=%d N=%d K=%d" % (M, N, K))
    x, w, b = workloads.prefill_inputs(M, K, N, cfg=workloads.CFG_W4A4)
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    wq, ws = cr.prepare_weight(wd, 256, 4)
    del wd
    xq, xs = cr.quantize_act(xd, 256, 4)
    y = cr.linear_w4a4(xd, wq, ws, bd)
    yp = cr.linear_w4a4_packed(None, cr.pack_weight_w4a4(wq), ws, bd, xq=xq, x_scale=xs)
    torch.cuda.synchronize()
    assert torch.equal(y, yp)
    rng = np.random.default_rng(12)
    mr = np.sort(rng.choice(M, 384, replace=False))
    nr = np.sort(rng.choice(N, 384, replace=False))
    ys = _x64(y)[np.ix_(mr, nr)]
    # scales and codes of the sampled rows
    cx, sxr, _ = orc.prepare_i4(_x64(x[mr]), 256)
    cw, swr, _ = orc.prepare_i4(_x64(w[nr]), 256)
    P.check_scales_f16(_np(xs).T[mr], sxr, "sx16 rows")
    P.check_scales_f16(_np(ws).T[nr], swr, "sw16 rows")
    P.check_codes(orc.unpack_i4(_np(xq)[mr]), cx, "x int4 codes")
    P.check_codes(orc.unpack_i4(_np(wq)[nr]), cw, "w int4 codes")
    # exact integer part on the GPU's own codes and scales, then the oracle end to end
    yown = orc.linear_i4(orc.unpack_i4(_np(xq)[mr]), _np(xs).T[mr], orc.unpack_i4(_np(wq)[nr]), _np(ws).T[nr],
                         b.numpy()[nr], 256)
    P.check_y(ys, yown, "sampled y (own codes)", strict_frac=1e-4)
    ref = orc.linear_w4a4(_x64(x[mr]), _x64(w[nr]), b.numpy()[nr], 256)
    P.check_y(ys, ref["y"], "sampled y (oracle codes)", strict_frac=2e-2)


def test_mixed_profile_schedule_sampled(cr):
    """The mixed W4A4 / W8A8 schedule at the full W4A4 shape (4096 x 5376 x 10752): four instances
    with their own device-drawn weights, instances 1 and 2 promoted to W8A8, dispatched in order;
    one instance of each kind checked against the oracle on 256 sampled token rows x 256 sampled
    weight rows, and the schedule's W4A4 instance equal to the plain W4A4 linear."""
    from int4_quantized_linear_amd.mixed import MixedSchedule
    M, K, N = workloads.W4A4_SHAPE["M"], workloads.W4A4_SHAPE["K"], workloads.W4A4_SHAPE["N"]
    P.say("mixed schedule M=%d K=%d N=%d" % (M, K, N))
    b = workloads.bias_vector(N, workloads.CFG_W4A4).to(DEV)
    sched = MixedSchedule(M, K, N, 4, [1, 2], lambda i: workloads.mixed_weight(i, N, K, DEV), bias=b)
    assert sched.kinds() == ["w4a4", "w8a8", "w8a8", "w4a4"]
    xs = [workloads.mixed_acts(j, M, K, DEV) for j in range(2)]
    ys = [torch.empty((M, N), dtype=torch.bfloat16, device=DEV) for _ in range(4)]
    sched.run(xs, ys)
    torch.cuda.synchronize()
    rng = np.random.default_rng(240)
    mr = np.sort(rng.choice(M, 256, replace=False))
    nr = np.sort(rng.choice(N, 256, replace=False))
    bn = b.cpu().numpy()[nr]
    for inst, kind in ((1, "w8a8"), (0, "w4a4")):
        w = workloads.mixed_weight(inst, N, K, DEV)
        x = xs[inst % len(xs)]
        x_h, w_h = _x64(x[torch.from_numpy(mr).to(DEV)]), _x64(w[torch.from_numpy(nr).to(DEV)])
        got = _x64(ys[inst])[np.ix_(mr, nr)]
        if kind == "w8a8":
            ref = orc.linear_w8a8(x_h, w_h, bn, 256)
            P.check_y(got, ref["y"], "mixed instance %d (W8A8)" % inst)
        else:
            ref = orc.linear_w4a4(x_h, w_h, bn, 256)
            P.check_y(got, ref["y"], "mixed instance %d (W4A4)" % inst, strict_frac=2e-2)
            wq4, ws4 = cr.prepare_weight(w, 256, 4)
            assert torch.equal(ys[inst], cr.linear_w4a4(x, wq4, ws4, b))


# ------------------------------------------------------------------ W4A8 (decode, M <= 16)

def _w4a8_case(cr, x, w, b, what, g=256):
    xd, wd = x.to(DEV), w.to(DEV)
    bd = None if b is None else b.to(DEV)
    N = w.shape[0]
    wq, ws = cr.prepare_weight(wd, g, 4)
    wp = cr.pack_weight_w4a8(wq, ws, g)
    y = cr.linear_w4a8(xd, wp, N, bd, group=g)
    xq, xs = cr.quantize_act(xd, g, 8)
    y2 = cr.linear_w4a8(None, wp, N, bd, group=g, xq=xq, x_scale=xs)
    torch.cuda.synchronize()
    bn = None if b is None else b.numpy()
    ref = orc.linear_w4a8(_x64(x), _x64(w), bn, g)
    P.check_codes(_np(xq), ref["qx"], "qx")
    P.check_scales_f32(_np(xs), ref["sx"], "sx")
    P.check_scales_f16(_np(ws).T, ref["sw"], "sw16")
    P.check_codes(orc.unpack_i4(_np(wq)), ref["cw"], "int4 weight codes")
    # exact integer group sums on the GPU's own codes: only fp32 rounding of the scaled sums differs
    yown = orc.linear_w4a8_codes(_np(xq), _np(xs), orc.unpack_i4(_np(wq)), _np(ws).T, bn, g)
    P.check_y(_x64(y), yown, what + " (own codes)", strict_frac=1e-4)
    P.check_y(_x64(y), ref["y"], what + " (oracle codes)", strict_frac=2e-2)
    assert torch.equal(y, y2), "pre-quantized path differs from the fused path"
    return y


W4A8_CASES = [
    # M, N, K: one group (no split), ragged row tiles, several splits, the longest K
    (5, 64, 256), (1, 200, 512), (16, 520, 768), (12, 1000, 5120), (13, 1024, 5376), (7, 136, 25600),
    (12, 64, 131072), (3, 8, 512),
]


@pytest.mark.parametrize("M,N,K", W4A8_CASES)
def test_linear_w4a8_parity(cr, M, N, K):
    P.say("linear_w4a8 M=%d N=%d K=%d" % (M, N, K))
    x, w, b = workloads.ragged_case(M, K, N, seed=7)
    _w4a8_case(cr, x, w, b, "w4a8 y")


# 128-channel scale groups (the dynamic group): one half block (K = 128), K % 256 == 128 (a
# zero upper half in the last block), K % 256 == 0, ragged rows, several wavefront splits
W4A8_G128_CASES = [(5, 64, 128), (3, 200, 384), (16, 520, 2688), (12, 1000, 5120), (7, 136, 25600 + 128),
                   # N >= 4096: workgroups of two 16-row blocks, with and without the zero upper half
                   (12, 8192, 2688), (12, 5120, 5120 + 128)]


@pytest.mark.parametrize("M,N,K", W4A8_G128_CASES)
def test_linear_w4a8_group128_parity(cr, M, N, K):
    P.say("linear_w4a8 g=128 M=%d N=%d K=%d" % (M, N, K))
    x, w, b = workloads.ragged_case(M, K, N, seed=8)
    _w4a8_case(cr, x, w, b, "w4a8 g128 y", g=128)


@pytest.mark.parametrize("K,N", workloads.DECODE_SHAPES)
def test_linear_w4a8_decode_shapes(cr, K, N):
    P.say("w4a8 decode M=12 K=%d N=%d" % (K, N))
    x, w = workloads.decode_inputs(K, N)
    _w4a8_case(cr, x, w, None, "w4a8 decode y")


def _unpack_w4a8_layout(buf: np.ndarray, N: int, K: int, g: int = 256):
    """CPU reading of the W4A8 block layout as the header and kernel source describe it:
    per 64-row tile t and 256-channel block j a block of BS bytes at (t*G + j)*BS (BS = 8320 for
    group 256, 8448 for group 128); piece (b, i) at 1024*(2b+i), lane l = (r, q) at 16*l holds
    K-steps 2i, 2i+1 of row 16b+r as dwords (dA, dB); dA byte u = channel 64kk+16q+u (high
    nibble) | channel 64kk+16q+4+u (low nibble), dB the same for +8, +12; scale set s (one for
    group 256; for group 128 s = 0 the block's lower, s = 1 its upper 128 channels) at
    8192 + 128s + 32q + 8b + 2v for row 16b+4q+v.  Returns the codes over all blocks' channels
    (G*256, past K included) and the scales [rows, K/g]."""
    G = -(-K // 256)
    T = -(-N // 64)
    nsc = 2 if g == 128 else 1
    BS = 8192 + 128 * nsc
    blocks = buf[: T * G * BS].reshape(T, G, BS)
    codes = np.zeros((T * 64, G * 256), np.int8)
    scales = np.zeros((T * 64, G * nsc), np.uint16)
    def s4(x):
        return ((x.astype(np.int16) ^ 8) - 8).astype(np.int8)
    for b in range(4):
        for i in range(2):
            piece = blocks[:, :, 1024 * (2 * b + i): 1024 * (2 * b + i + 1)].reshape(T, G, 4, 16, 16)  # q, r, bytes
            for h in range(2):
                kk = 2 * i + h
                for part in range(2):                     # dA (s 0..7), dB (s 8..15)
                    by = piece[:, :, :, :, 8 * h + 4 * part: 8 * h + 4 * part + 4]    # [T, G, q, r, u]
                    for u in range(4):
                        hi, lo = s4(by[..., u] >> 4), s4(by[..., u] & 15)
                        for q in range(4):
                            k_hi = 64 * kk + 16 * q + 8 * part + u
                            for j in range(G):
                                rows = np.arange(T)[:, None] * 64 + 16 * b + np.arange(16)[None, :]
                                codes[rows, 256 * j + k_hi] = hi[:, j, q, :]
                                codes[rows, 256 * j + k_hi + 4] = lo[:, j, q, :]
    sc = blocks[:, :, 8192:].reshape(T, G, nsc, 4, 4, 4, 2)   # set, q, b, v, 2 bytes
    sv = sc[..., 0].astype(np.uint16) | (sc[..., 1].astype(np.uint16) << 8)
    for st in range(nsc):
        for q in range(4):
            for b in range(4):
                for v in range(4):
                    scales[np.arange(T) * 64 + 16 * b + 4 * q + v, st::nsc] = sv[:, :, st, q, b, v]
    return codes, scales[:, : K // g]


@pytest.mark.parametrize("N,K,g", [(64, 256, 256), (200, 512, 256), (1024, 5120, 256), (64, 384, 128),
                                   (200, 2688, 128), (72, 1024, 128)])
def test_pack_w4a8_layout(cr, N, K, g):
    """The packed buffer holds exactly the prepared codes and scales, in the documented order,
    with zero rows past N (and, for group 128 with K % 256 == 128, zero channels and scales in the
    last block's upper half)."""
    w = workloads.gaussian_weights(N, K, cfg=96).to(DEV)
    wq, ws = cr.prepare_weight(w, g, 4)
    wp = cr.pack_weight_w4a8(wq, ws, g)
    torch.cuda.synchronize()
    assert wp.numel() == cr.packed_bytes_w4a8(N, K, g)
    codes, scales = _unpack_w4a8_layout(_np(wp), N, K, g)
    assert np.array_equal(codes[:N, :K], orc.unpack_i4(_np(wq)))
    assert not codes[:, K:].any() and not codes[N:].any() and not scales[N:].any()
    assert np.array_equal(scales[:N], _np(ws).view(np.uint16).T)
    if g == 128 and K % 256:
        last = _np(wp)[: -(-N // 64) * -(-K // 256) * 8448].reshape(-1, -(-K // 256), 8448)[:, -1]
        assert not last[:, 8192 + 128:].any()             # the empty half's scale set


def test_linear_w4a8_repeat_and_limits(cr):
    K, N = 5120, 1024
    w = workloads.gaussian_weights(N, K, cfg=97).to(DEV)
    wq, ws = cr.prepare_weight(w, 256, 4)
    wp = cr.pack_weight_w4a8(wq, ws)
    y = cr.linear_w4a8(torch.empty(0, K, dtype=torch.bfloat16, device=DEV), wp, N)
    assert y.shape == (0, N)
    # consecutive calls with different token counts on the same weights
    for M in (12, 16, 3):
        x = workloads.heavy_tailed_acts(M, K, cfg=97, layer=M).to(DEV)
        y = cr.linear_w4a8(x, wp, N)
        torch.cuda.synchronize()
        ref = orc.linear_w4a8(_x64(x), _x64(w), None, 256)
        P.check_y(_x64(y), ref["y"], "w4a8 repeat M=%d" % M, strict_frac=2e-2)
    with pytest.raises(cr.ConvRotError, match="M <= 16"):
        cr.linear_w4a8(torch.zeros(17, K, dtype=torch.bfloat16, device=DEV), wp, N)
    # pre-quantized tokens need no workspace at all
    x = workloads.heavy_tailed_acts(12, K, cfg=97, layer=5).to(DEV)
    xq, xs = cr.quantize_act(x, 256, 8)
    y = torch.empty((12, N), dtype=torch.bfloat16, device=DEV)
    st = torch.cuda.current_stream().cuda_stream
    cr._call("convrot_linear_w4a8", None, 0, xq.data_ptr(), xs.data_ptr(), 12, N, K, 256, wp.data_ptr(),
             wp.numel(), None, y.data_ptr(), None, 0, st)
    torch.cuda.synchronize()
    assert torch.equal(y, cr.linear_w4a8(x, wp, N))


# ------------------------------------------------------------------ streams and graph replay

def _replay_matches(fn, out, ref, replays=3):
    """Capture fn() on a side stream, replay it several times with eager work and
    synchronisations in between, and check every replay against the eager result."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.synchronize()
    for i in range(replays):
        out.zero_()
        torch.randn(1024, device=DEV).sum()            # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "replay %d differs from the eager result" % i


def test_decode_linears_run_on_the_callers_stream_and_replay(cr):
    """Every launch goes to the stream the caller passes: the captured graph holds the kernels
    (a launch on another stream would leave it empty and the output untouched)."""
    K, N, M = 5120, 1024, 12
    w = workloads.gaussian_weights(N, K, cfg=95).to(DEV)
    x = workloads.heavy_tailed_acts(M, K, cfg=95, layer=0).to(DEV)
    xq, xs = cr.quantize_act(x, 256, 8)
    wq8, ws8 = cr.prepare_weight(w, 256, 8)
    wq4, ws4 = cr.prepare_weight(w, 256, 4)
    wp = cr.pack_weight_w4a8(wq4, ws4)
    torch.cuda.synchronize()
    y8 = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    y4 = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    ref8 = cr.linear(None, wq8, ws8, xq=xq, x_scale=xs).clone()
    ref4 = cr.linear_w4a8(None, wp, N, xq=xq, x_scale=xs).clone()
    torch.cuda.synchronize()
    _replay_matches(lambda: cr.linear(None, wq8, ws8, xq=xq, x_scale=xs, out=y8), y8, ref8)
    _replay_matches(lambda: cr.linear_w4a8(None, wp, N, xq=xq, x_scale=xs, out=y4), y4, ref4)


def test_split_k_gemm_runs_on_the_callers_stream_and_replays(cr):
    """The split-K tail's two kernels (K-slices writing partial sums, then their reduction) both go
    to the caller's stream, so a captured graph holds them, and every replay rewrites the partial
    slots it reads (no state carried between calls)."""
    M, N, K = 64, 8192, 5120
    assert cr.workspace_bytes(M, N, K, 8) > _r256(M * K) + _r256(4 * M)     # a split is planned
    w = workloads.gaussian_weights(N, K, cfg=94).to(DEV)
    x = workloads.heavy_tailed_acts(M, K, cfg=94, layer=0).to(DEV)
    b = torch.randn(N, generator=torch.Generator().manual_seed(94)).to(DEV)
    xq, xs = cr.quantize_act(x, 256, 8)
    wq, ws = cr.prepare_weight(w, 256, 8)
    ref = cr.linear(None, wq, ws, b, xq=xq, x_scale=xs).clone()
    whole = cr.linear(None, wq, ws, b, xq=xq, x_scale=xs, split_k=False)
    torch.cuda.synchronize()
    assert torch.equal(ref, whole)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    _replay_matches(lambda: cr.linear(None, wq, ws, b, xq=xq, x_scale=xs, out=y), y, ref)
    # rotate+quantize, the K-slices and the reduction in one graph
    _replay_matches(lambda: cr.linear(x, wq, ws, b, out=y), y, ref)


def test_w4a4_linears_run_on_the_callers_stream_and_replay(cr):
    """The W4A4 linear's kernels (rotate+quantize into FP6 tiles, the weight re-encode when the
    weights are not pre-encoded, the GEMM) all go to the caller's stream and replay equal to eager,
    at both scale groups."""
    for M, N, K, g in ((100, 264, 768, 256), (33, 520, 384, 128)):
        x, w, b = workloads.ragged_case(M, K, N, seed=13)
        xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
        wq, ws = cr.prepare_weight(wd, g, 4)
        wp = cr.pack_weight_w4a4(wq)
        ref = cr.linear_w4a4(xd, wq, ws, bd, group=g).clone()
        refp = cr.linear_w4a4_packed(xd, wp, ws, bd, group=g).clone()
        torch.cuda.synchronize()
        assert torch.equal(ref, refp)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        _replay_matches(lambda: cr.linear_w4a4(xd, wq, ws, bd, group=g, out=y), y, ref)
        _replay_matches(lambda: cr.linear_w4a4_packed(xd, wp, ws, bd, group=g, out=y), y, ref)


def test_linears_on_two_streams_at_once_match_sequential(cr):
    """The library keeps no per-call state outside the caller's buffers (the no-allocation entry
    point excepted): INT8 and W4A4 linears issued on two streams at the same time, each with its
    own workspace, give the results of running them one after the other."""
    M, N, K = 300, 2048, 1024
    x1, w, b = workloads.ragged_case(M, K, N, seed=21)
    x2, _, _ = workloads.ragged_case(M, K, N, seed=22)
    x1, x2, wd, bd = x1.to(DEV), x2.to(DEV), w.to(DEV), b.to(DEV)
    wq8, ws8 = cr.prepare_weight(wd, 256, 8)
    wq4, ws4 = cr.prepare_weight(wd, 256, 4)
    wp = cr.pack_weight_w4a4(wq4)
    ref = [cr.linear(x1, wq8, ws8, bd).clone(), cr.linear_w4a4_packed(x2, wp, ws4, bd).clone(),
           cr.linear(x2, wq8, ws8, bd).clone(), cr.linear_w4a4_packed(x1, wp, ws4, bd).clone()]
    torch.cuda.synchronize()
    outs = [torch.empty((M, N), dtype=torch.bfloat16, device=DEV) for _ in range(4)]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        with torch.cuda.stream(s1):
            cr.linear(x1, wq8, ws8, bd, out=outs[0])
            cr.linear_w4a4_packed(x1, wp, ws4, bd, out=outs[3])
        with torch.cuda.stream(s2):
            cr.linear_w4a4_packed(x2, wp, ws4, bd, out=outs[1])
            cr.linear(x2, wq8, ws8, bd, out=outs[2])
    torch.cuda.synchronize()
    for i in range(4):
        assert torch.equal(outs[i], ref[i]), "output %d differs from the sequential run" % i


# ------------------------------------------------------------------ randomized legal shapes

def _random_cases(n: int, seed: int):
    """Seeded random shapes within each entry point's documented limits: INT8 at any power-of-two
    group 1..256 and M across the GEMV/GEMM switch (ragged N), W4A4 and W4A8 at groups 128/256,
    bf16 or fp32 x, with or without bias; sizes bounded so the oracle stays fast."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        path = ["w8a8", "w8a8", "w4a4", "w4a8"][int(rng.integers(0, 4))]
        dtype = "bf16" if rng.random() < 0.7 else "f32"
        if path == "w8a8":
            g = int(2 ** rng.integers(0, 9))
            K = max(g, 64) * int(rng.integers(1, max(2, 4096 // max(g, 64))))
            M = int(rng.integers(1, 17)) if rng.random() < 0.5 else int(rng.integers(17, 600))
            N = int(rng.integers(1, 1300))
        elif path == "w4a4":
            g = int(rng.choice([128, 256]))
            K = g * int(rng.integers(max(1, 256 // g), 4096 // g))
            M, N = int(rng.integers(1, 400)), 8 * int(rng.integers(1, 160))
        else:
            g = int(rng.choice([128, 256]))
            K = g * int(rng.integers(1, 8192 // g))
            M, N = int(rng.integers(1, 17)), 8 * int(rng.integers(1, 600))
        while M * N * K > 1.2e8:
            N = max(8, (N // 2) // 8 * 8)
            M = max(1, M // 2)
        cases.append((i, path, M, N, K, g, dtype, bool(rng.random() < 0.7)))
    return cases


@pytest.mark.parametrize("case", _random_cases(48, 2024), ids=lambda c: "%d-%s-%dx%dx%d-g%d-%s%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], "-bias" if c[7] else ""))
def test_random_legal_shapes(cr, case):
    i, path, M, N, K, g, dtype, with_bias = case
    P.say("random case %d: %s M=%d N=%d K=%d g=%d %s bias=%s" % (case[:7] + (with_bias,)))
    x, w, b = workloads.ragged_case(M, K, N, seed=4000 + i, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
    if path == "w8a8":
        _linear_case(cr, x, w, b if with_bias else None, g)
    elif path == "w4a4":
        _w4a4_case(cr, x, w, b, g)
    else:
        _w4a8_case(cr, x, w, b if with_bias else None, "w4a8", g)


def _structured_cases(n: int, seed: int):
    """INT8 linears on structured activations: small integers (exact half-integer quotients are
    common), a row of tiny magnitude (scale below 2^-100), a zero row; bf16 or fp32 x."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        kind = ["int", "tinyrow", "zerorow"][i % 3]
        g = int(2 ** rng.integers(0, 9))
        K = max(g, 64) * int(rng.integers(1, max(2, 4096 // max(g, 64))))
        M = int(rng.integers(1, 17)) if rng.random() < 0.5 else int(rng.integers(17, 400))
        N = int(rng.integers(1, 1100))
        while M * N * K > 1.0e8:
            N = max(1, N // 2)
            M = max(1, M // 2)
        cases.append((i, kind, M, N, K, g, "bf16" if rng.random() < 0.6 else "f32"))
    return cases


@pytest.mark.parametrize("case", _structured_cases(18, 77), ids=lambda c: "%d-%s-%dx%dx%d-g%d-%s" % c)
def test_linear_structured_inputs(cr, case):
    i, kind, M, N, K, g, dtype = case
    P.say("structured case %d: %s M=%d N=%d K=%d g=%d %s" % case)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x, w, b = workloads.ragged_case(M, K, N, seed=5000 + i, dtype=dt)
    rng = np.random.default_rng(6000 + i)
    if kind == "int":
        x = torch.from_numpy(rng.integers(-3, 4, size=(M, K)).astype(np.float32)).to(dt)
    elif kind == "tinyrow":
        x = x.float()
        x[int(rng.integers(0, M))] *= 2.0 ** -112
        x = x.to(dt)
    else:
        x = x.clone()
        x[int(rng.integers(0, M))] = 0
    _linear_case(cr, x, w, b, g)
