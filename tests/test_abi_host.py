"""Host-side checks of the C-ABI library (no GPU needed, no kernel launched).

* every function declared in include/convrot.h is exported by libconvrot.so and has a ctypes
  signature in the binding;
* status names and the workspace-size query;
* every precondition violation returns its status code (and a message) before anything touches
  the device: the arguments below always break a rule the library checks first, and pointers are
  fake but never dereferenced because the call is rejected on the host.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "convrot.h")

cr = pytest.importorskip("int4_quantized_linear_amd.convrot")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(convrot_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(cr.LIB_PATH):
        pytest.fail("libconvrot.so is not built; run python -m int4_quantized_linear_amd.build")
    return cr.load()


def test_header_declares_the_boundary():
    fns = header_functions()
    for name in ("convrot_prepare_weight", "convrot_quantize_act", "convrot_linear", "convrot_linear_w4a4",
                 "convrot_pack_weight_w4a4", "convrot_packed_bytes_w4a4", "convrot_linear_w4a4_packed",
                 "convrot_linear_w4a8", "convrot_pack_weight_w4a8", "convrot_packed_bytes_w4a8",
                 "convrot_pack_weight_w4a8_group", "convrot_packed_bytes_w4a8_group",
                 "convrot_workspace_bytes", "convrot_workspace_bytes_w4a8",
                 "convrot_gemm_i8_i32", "convrot_gemm_i4_i32", "convrot_dynamic_group", "convrot_last_error",
                 "convrot_linear_noalloc",
                 "convrot_status_string"):
        assert name in fns
    assert set(fns) == set(cr.SIGNATURES), "binding signatures and header disagree"


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", cr.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for name in header_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_exports_are_c_linkage_only(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", cr.LIB_PATH], capture_output=True, text=True, check=True).stdout
    ours = sorted({ln.split()[-1] for ln in out.splitlines() if " T " in ln and "convrot" in ln})
    assert ours == header_functions(), ours


def test_status_strings(lib):
    for code, name in cr.STATUS.items():
        assert lib.convrot_status_string(code).decode() == name
    assert lib.convrot_status_string(99).decode() == "CONVROT_ERR_UNKNOWN"


def test_workspace_bytes(lib):
    ws = lib.convrot_workspace_bytes
    assert ws(-1, 8, 256, 8) == 0 and ws(4, -1, 256, 8) == 0 and ws(4, 8, 0, 8) == 0 and ws(4, 8, 256, 5) == 0
    for M, N, K in [(4096, 16128, 5376), (17, 256, 512), (12, 8192, 5120), (12, 5120, 25600), (1, 64, 64)]:
        b8 = ws(M, N, K, 8)
        assert b8 % 256 == 0 and b8 >= M * K + 4 * M, (M, N, K)
    for M, K in [(4096, 5376), (3, 512), (300, 2688)]:
        b4 = ws(M, 1024, K, 4)
        # room for 128-channel scale groups too (the query has no group argument)
        assert b4 % 256 == 0 and b4 >= M * K // 2 + 2 * M * (K // 128)


def _r256(n):
    return (n + 255) // 256 * 256


def test_workspace_bytes_split_k_tail(lib):
    # On a host without a GPU the grid capacity falls back to MI355X's 256 CUs.
    ws = lib.convrot_workspace_bytes
    base = lambda M, K: _r256(M * K) + _r256(4 * M)
    # under-filled grids whose tail tiles are split: room for the int32 partial slots (256 KiB
    # each, tail tiles x slices), past the quantized x
    for M, N, K in [(64, 8192, 5120), (17, 520, 1024), (300, 1000, 4096), (2048, 1024, 5120), (200, 5120, 25600)]:
        extra = ws(M, N, K, 8) - base(M, K)
        assert extra > 0 and extra % (256 * 256 * 4) == 0, (M, N, K, extra)
    # no split: whole rounds but the last nearly full (the prefill shape), a tail that keeps ~3/4
    # of the CUs busy (160 tiles; the kernel is power-bound there), a short tail after a whole
    # round (q|k|v: the partial sums' round trip costs what the tail saves), N % 8 != 0 (the
    # element-store epilogue has no partial-sum path), and the decode GEMV (M <= 16)
    for M, N, K in [(4096, 16128, 5376), (2048, 5120, 25600), (2048, 5120, 8192), (2048, 10240, 5120),
                    (130, 1001, 2048), (12, 8192, 5120)]:
        assert ws(M, N, K, 8) == base(M, K), (M, N, K)


def test_workspace_bytes_w4a8(lib):
    ws = lib.convrot_workspace_bytes_w4a8
    assert ws(17, 256, 512) == 0 and ws(-1, 256, 512) == 0 and ws(4, -1, 512) == 0
    assert ws(4, 256, 320) == 0 and ws(4, 256, 0) == 0 and ws(4, 256, 131072 + 256) == 0
    for M, N, K in [(12, 5120, 5120), (12, 25600, 5120), (12, 5120, 25600), (1, 64, 256), (16, 7, 768), (0, 64, 256)]:
        b = ws(M, N, K)
        # the INT8 activation codes and scales fit besides whatever the kernel needs
        assert b % 256 == 0 and b >= M * K + 4 * M and (b > 0 or M == 0), (M, N, K)


def test_dynamic_group_matches_the_oracle(lib):
    from oracle import oracle as orc
    for K in list(range(1, 1100)) + [2688, 5120, 5376, 25600, 131072]:
        for mg in (256, 128, 1):
            assert lib.convrot_dynamic_group(K, mg) == orc.dynamic_group(K, mg), (K, mg)
    assert lib.convrot_dynamic_group(0, 256) == 0 and lib.convrot_dynamic_group(-5, 256) == 0
    assert lib.convrot_dynamic_group(512, 96) == 0 and lib.convrot_dynamic_group(512, 512) == 0
    assert cr.dynamic_group(2688) == 128
    with pytest.raises(cr.ConvRotError):
        cr.dynamic_group(512, 3)


def test_packed_bytes_w4a8_group(lib):
    pb = lib.convrot_packed_bytes_w4a8_group
    assert pb(64, 512, 64) == 0 and pb(64, 384, 256) == 0 and pb(64, 320, 128) == 0 and pb(-1, 512, 128) == 0
    for N, K in [(64, 256), (1000, 5376)]:
        assert pb(N, K, 256) == lib.convrot_packed_bytes_w4a8(N, K)
    # group 128: 256-channel blocks (the last one half empty when K % 256 == 128), each with two
    # scale sets of 128 bytes
    for N, K in [(64, 128), (64, 384), (200, 2688), (1024, 5120)]:
        assert pb(N, K, 128) == -(-N // 64) * -(-K // 256) * (8192 + 256), (N, K)


def test_packed_bytes_w4a8(lib):
    pb = lib.convrot_packed_bytes_w4a8
    assert pb(-1, 512) == 0 and pb(64, 320) == 0 and pb(64, 0) == 0 and pb(64, 131072 + 256) == 0
    assert pb(0, 512) == 0
    # 64-row tiles x 256-channel groups, each 8 KiB of codes + 128 bytes of scales
    for N, K in [(64, 256), (1, 256), (1024, 5120), (1000, 5376), (5120, 25600)]:
        assert pb(N, K) == -(-N // 64) * (K // 256) * (8192 + 128), (N, K)


def test_packed_bytes_w4a4(lib):
    pb = lib.convrot_packed_bytes_w4a4
    assert pb(-1, 512) == 0 and pb(64, 320) == 0 and pb(64, 0) == 0 and pb(64, 131072 + 256) == 0
    assert pb(0, 512) == 0 and pb(64, 192) == 0
    # 32-row blocks x 64-channel K-steps of 1536 bytes (0.75 bytes per code, rows padded to 32)
    for N, K in [(32, 256), (1, 256), (10752, 5376), (1000, 5120), (8, 131072), (64, 2688), (40, 128)]:
        assert pb(N, K) == -(-N // 32) * (K // 64) * 1536, (N, K)


def test_packed_w4a4_linear_needs_no_weight_workspace(lib):
    if _gpu_present():
        pytest.skip("host-only check (fake device pointers)")
    M, N, K = 64, 1024, 512
    small = lib.convrot_workspace_bytes(M, 0, K, 4)
    assert 0 < small < lib.convrot_workspace_bytes(M, N, K, 4)
    # the per-call path needs room for the weights' FP6 tiles ...
    rc = lib.convrot_linear_w4a4(*w4_args(M=M, N=N, K=K, wsb=small))
    assert rc == ERR["CONVROT_ERR_WORKSPACE"], lib.convrot_last_error().decode()
    # ... the pre-encoded one passes every argument check with the smaller workspace and stops
    # only at the missing device (hipGetDevice fails on a host without one)
    rc = lib.convrot_linear_w4a4_packed(*w4_args(M=M, N=N, K=K, wsb=small))
    assert rc == ERR["CONVROT_ERR_HIP"], lib.convrot_last_error().decode()
    assert "hipGetDevice" in lib.convrot_last_error().decode()
    rc = lib.convrot_linear_w4a4_packed(*w4_args(M=M, N=N, K=K, wsb=small - 1))
    assert rc == ERR["CONVROT_ERR_WORKSPACE"], lib.convrot_last_error().decode()


A = 0x100000          # fake 256-byte aligned device addresses (never dereferenced)
B = 0x200000
C = 0x300000
D = 0x400000
E = 0x500000
MIS = 0x100002        # misaligned


def q_args(x=A, dtype=1, R=4, K=512, group=256, bits=8, q=B, s=C):
    return (x, dtype, R, K, group, bits, q, s, None)


def lin_args(x=A, dt=1, xq=None, xs=None, M=32, N=256, K=512, group=256, wq=B, sw=C, bias=None, y=D, ws=E,
             wsb=1 << 30):
    return (x, dt, xq, xs, M, N, K, group, wq, sw, bias, y, ws, wsb, None)


def w48_args(x=A, dt=1, xq=None, xs=None, M=12, N=256, K=512, group=256, wp=B, wpb=None, bias=None, y=D, ws=E,
             wsb=1 << 30):
    # wpb: the packed weight size the call states; by default the right one for (N, K, group)
    if wpb is None:
        wpb = cr.load().convrot_packed_bytes_w4a8_group(N, K, group)
    return (x, dt, xq, xs, M, N, K, group, wp, wpb, bias, y, ws, wsb, None)


def w4_args(x=A, dt=1, xq=None, xs=None, M=32, N=256, K=512, group=256, wq=B, sw=C, bias=None, y=D, ws=E,
            wsb=1 << 30):
    return (x, dt, xq, xs, M, N, K, group, wq, sw, bias, y, ws, wsb, None)


ERR = {name: code for code, name in cr.STATUS.items()}


def _gpu_present() -> bool:
    import torch
    return torch.cuda.is_available()


CASES = [
    # quantize / prepare
    ("convrot_quantize_act", q_args(x=None), "CONVROT_ERR_NULL"),
    ("convrot_quantize_act", q_args(s=None), "CONVROT_ERR_NULL"),
    ("convrot_quantize_act", q_args(dtype=7), "CONVROT_ERR_DTYPE"),
    ("convrot_quantize_act", q_args(bits=6), "CONVROT_ERR_BITS"),
    ("convrot_quantize_act", q_args(K=500), "CONVROT_ERR_SHAPE"),
    ("convrot_quantize_act", q_args(K=0), "CONVROT_ERR_SHAPE"),
    ("convrot_quantize_act", q_args(K=131072 + 64), "CONVROT_ERR_SHAPE"),
    ("convrot_quantize_act", q_args(R=-1), "CONVROT_ERR_SHAPE"),
    ("convrot_quantize_act", q_args(R=1 << 31), "CONVROT_ERR_SHAPE"),
    ("convrot_quantize_act", q_args(group=3), "CONVROT_ERR_GROUP"),
    ("convrot_quantize_act", q_args(group=512), "CONVROT_ERR_GROUP"),
    ("convrot_quantize_act", q_args(K=192, group=128), "CONVROT_ERR_SHAPE"),
    ("convrot_quantize_act", q_args(bits=4, group=64), "CONVROT_ERR_GROUP"),
    ("convrot_quantize_act", q_args(bits=4, K=320, group=64), "CONVROT_ERR_GROUP"),
    ("convrot_quantize_act", q_args(x=MIS), "CONVROT_ERR_ALIGN"),
    ("convrot_quantize_act", q_args(q=MIS), "CONVROT_ERR_ALIGN"),
    ("convrot_quantize_act", q_args(s=C + 2), "CONVROT_ERR_ALIGN"),
    ("convrot_prepare_weight", q_args(q=None), "CONVROT_ERR_NULL"),
    ("convrot_prepare_weight", q_args(dtype=2), "CONVROT_ERR_DTYPE"),
    ("convrot_prepare_weight", q_args(group=0), "CONVROT_ERR_GROUP"),
    # INT8 linear
    ("convrot_linear", lin_args(K=100), "CONVROT_ERR_SHAPE"),
    ("convrot_linear", lin_args(group=100), "CONVROT_ERR_GROUP"),
    ("convrot_linear", lin_args(wq=None), "CONVROT_ERR_NULL"),
    ("convrot_linear", lin_args(y=None), "CONVROT_ERR_NULL"),
    ("convrot_linear", lin_args(x=None, xq=A), "CONVROT_ERR_NULL"),
    ("convrot_linear", lin_args(dt=5), "CONVROT_ERR_DTYPE"),
    ("convrot_linear", lin_args(y=MIS), "CONVROT_ERR_ALIGN"),
    ("convrot_linear", lin_args(bias=E + 1), "CONVROT_ERR_ALIGN"),
    ("convrot_linear", lin_args(x=None, xq=A, xs=C + 2), "CONVROT_ERR_ALIGN"),
    ("convrot_linear", lin_args(ws=None), "CONVROT_ERR_WORKSPACE"),
    ("convrot_linear", lin_args(wsb=16), "CONVROT_ERR_WORKSPACE"),
    ("convrot_linear", lin_args(ws=E + 16), "CONVROT_ERR_WORKSPACE"),
    # the tiled GEMM's N limit (2^24); the decode GEMV (M <= 16) takes a larger N
    ("convrot_linear", lin_args(N=1 << 24), "CONVROT_ERR_SHAPE"),
    ("convrot_linear", lin_args(M=16, N=1 << 24, wq=None), "CONVROT_ERR_NULL"),
    # the no-allocation linear: the same checks, and activations too large for its fixed scratch
    ("convrot_linear_noalloc", lin_args(K=100)[:12] + (None,), "CONVROT_ERR_SHAPE"),
    ("convrot_linear_noalloc", lin_args(wq=None)[:12] + (None,), "CONVROT_ERR_NULL"),
    ("convrot_linear_noalloc", lin_args(M=8192, K=8192)[:12] + (None,), "CONVROT_ERR_WORKSPACE"),
    # W4A4 linear
    ("convrot_linear_w4a4", w4_args(group=64), "CONVROT_ERR_GROUP"),
    ("convrot_linear_w4a4", w4_args(K=384), "CONVROT_ERR_SHAPE"),         # group 256 must divide K
    ("convrot_linear_w4a4", w4_args(K=128, group=128), "CONVROT_ERR_SHAPE"),   # K >= 256
    ("convrot_linear_w4a4", w4_args(K=320, group=64), "CONVROT_ERR_GROUP"),
    ("convrot_linear_w4a4", w4_args(N=252), "CONVROT_ERR_SHAPE"),
    ("convrot_linear_w4a4", w4_args(M=1, N=1 << 24), "CONVROT_ERR_SHAPE"),
    ("convrot_linear_w4a4", w4_args(sw=None), "CONVROT_ERR_NULL"),
    ("convrot_linear_w4a4", w4_args(x=None, xs=C), "CONVROT_ERR_NULL"),
    ("convrot_linear_w4a4", w4_args(dt=9), "CONVROT_ERR_DTYPE"),
    ("convrot_linear_w4a4", w4_args(sw=C + 2), "CONVROT_ERR_ALIGN"),
    ("convrot_linear_w4a4", w4_args(ws=None), "CONVROT_ERR_WORKSPACE"),
    # the FP6 tiles live in the workspace even for pre-quantized activations
    ("convrot_linear_w4a4", w4_args(x=None, xq=A, xs=C, ws=None, wsb=0), "CONVROT_ERR_WORKSPACE"),
    # W4A4 with pre-encoded weights, and the one-time re-encode
    ("convrot_linear_w4a4_packed", w4_args(group=64), "CONVROT_ERR_GROUP"),
    ("convrot_linear_w4a4_packed", w4_args(N=252), "CONVROT_ERR_SHAPE"),
    ("convrot_linear_w4a4_packed", w4_args(N=1 << 24), "CONVROT_ERR_SHAPE"),
    ("convrot_linear_w4a4_packed", w4_args(wq=None), "CONVROT_ERR_NULL"),
    ("convrot_linear_w4a4_packed", w4_args(sw=None), "CONVROT_ERR_NULL"),
    ("convrot_linear_w4a4_packed", w4_args(wq=B + 8), "CONVROT_ERR_ALIGN"),
    ("convrot_linear_w4a4_packed", w4_args(x=None, xq=A, xs=C, ws=None, wsb=0), "CONVROT_ERR_WORKSPACE"),
    ("convrot_pack_weight_w4a4", (A, 64, 320, B, None), "CONVROT_ERR_SHAPE"),
    ("convrot_pack_weight_w4a4", (A, 64, 100, B, None), "CONVROT_ERR_SHAPE"),
    ("convrot_pack_weight_w4a4", (A, -1, 512, B, None), "CONVROT_ERR_SHAPE"),
    ("convrot_pack_weight_w4a4", (None, 64, 512, B, None), "CONVROT_ERR_NULL"),
    ("convrot_pack_weight_w4a4", (A, 64, 512, None, None), "CONVROT_ERR_NULL"),
    ("convrot_pack_weight_w4a4", (A + 8, 64, 512, B, None), "CONVROT_ERR_ALIGN"),
    ("convrot_pack_weight_w4a4", (A, 64, 512, B + 8, None), "CONVROT_ERR_ALIGN"),
    # W4A8 decode linear and its weight re-layout
    ("convrot_linear_w4a8", w48_args(M=17), "CONVROT_ERR_SHAPE"),
    ("convrot_linear_w4a8", w48_args(K=100), "CONVROT_ERR_SHAPE"),
    ("convrot_linear_w4a8", w48_args(group=512), "CONVROT_ERR_GROUP"),
    ("convrot_linear_w4a8", w48_args(K=384), "CONVROT_ERR_SHAPE"),           # group 256 must divide K
    ("convrot_linear_w4a8", w48_args(K=320, group=64), "CONVROT_ERR_GROUP"),
    ("convrot_linear_w4a8", w48_args(wp=None), "CONVROT_ERR_NULL"),
    ("convrot_linear_w4a8", w48_args(x=None, xq=A), "CONVROT_ERR_NULL"),
    ("convrot_linear_w4a8", w48_args(dt=4), "CONVROT_ERR_DTYPE"),
    ("convrot_linear_w4a8", w48_args(N=252), "CONVROT_ERR_SHAPE"),
    ("convrot_linear_w4a8", w48_args(wp=B + 8), "CONVROT_ERR_ALIGN"),
    ("convrot_linear_w4a8", w48_args(x=None, xq=A, xs=C + 2), "CONVROT_ERR_ALIGN"),
    ("convrot_linear_w4a8", w48_args(y=MIS), "CONVROT_ERR_ALIGN"),
    ("convrot_linear_w4a8", w48_args(ws=None), "CONVROT_ERR_WORKSPACE"),
    ("convrot_linear_w4a8", w48_args(wsb=256), "CONVROT_ERR_WORKSPACE"),
    ("convrot_linear_w4a8", w48_args(ws=E + 64), "CONVROT_ERR_WORKSPACE"),
    # weights packed with the other scale group (or any other size): rejected, never read
    ("convrot_linear_w4a8", w48_args(K=512, group=128, wpb=2 * 4 * 8320), "CONVROT_ERR_SHAPE"),
    ("convrot_linear_w4a8", w48_args(K=512, group=256, wpb=2 * 4 * 8448), "CONVROT_ERR_SHAPE"),
    ("convrot_linear_w4a8", w48_args(wpb=0), "CONVROT_ERR_SHAPE"),
    ("convrot_pack_weight_w4a8", (A, C, 64, 320, B, None), "CONVROT_ERR_SHAPE"),
    ("convrot_pack_weight_w4a8", (A, C, 64, 100, B, None), "CONVROT_ERR_SHAPE"),
    ("convrot_pack_weight_w4a8", (A, C, -1, 512, B, None), "CONVROT_ERR_SHAPE"),
    ("convrot_pack_weight_w4a8", (None, C, 64, 512, B, None), "CONVROT_ERR_NULL"),
    ("convrot_pack_weight_w4a8", (A, C, 64, 512, None, None), "CONVROT_ERR_NULL"),
    ("convrot_pack_weight_w4a8", (A, C + 1, 64, 512, B, None), "CONVROT_ERR_ALIGN"),
    ("convrot_pack_weight_w4a8", (A, C, 64, 512, B + 8, None), "CONVROT_ERR_ALIGN"),
    ("convrot_pack_weight_w4a8_group", (A, C, 64, 512, 64, B, None), "CONVROT_ERR_GROUP"),
    ("convrot_pack_weight_w4a8_group", (A, C, 64, 384, 256, B, None), "CONVROT_ERR_SHAPE"),
    ("convrot_pack_weight_w4a8_group", (None, C, 64, 384, 128, B, None), "CONVROT_ERR_NULL"),
    ("convrot_pack_weight_w4a8_group", (A, C + 1, 64, 384, 128, B, None), "CONVROT_ERR_ALIGN"),
    # integer cores
    ("convrot_gemm_i8_i32", (A, B, 32, 256, 96, C, None, 0, None), "CONVROT_ERR_SHAPE"),
    ("convrot_gemm_i8_i32", (A, B, 32, 1 << 24, 512, C, None, 0, None), "CONVROT_ERR_SHAPE"),
    ("convrot_gemm_i8_i32", (None, B, 16, 1 << 24, 512, C, None, 0, None), "CONVROT_ERR_NULL"),
    ("convrot_gemm_i8_i32", (None, B, 32, 256, 512, C, None, 0, None), "CONVROT_ERR_NULL"),
    ("convrot_gemm_i8_i32", (A, B, 32, 256, 512, MIS, None, 0, None), "CONVROT_ERR_ALIGN"),
    ("convrot_gemm_i4_i32", (A, B, 32, 256, 320, C, E, 1 << 30, None), "CONVROT_ERR_SHAPE"),
    ("convrot_gemm_i4_i32", (A, B, 32, 250, 512, C, E, 1 << 30, None), "CONVROT_ERR_SHAPE"),
    ("convrot_gemm_i4_i32", (A, B, 32, 1 << 24, 512, C, E, 1 << 30, None), "CONVROT_ERR_SHAPE"),
    ("convrot_gemm_i4_i32", (A, None, 32, 256, 512, C, E, 1 << 30, None), "CONVROT_ERR_NULL"),
    ("convrot_gemm_i4_i32", (A, B + 4, 32, 256, 512, C, E, 1 << 30, None), "CONVROT_ERR_ALIGN"),
    ("convrot_gemm_i4_i32", (A, B, 32, 256, 512, C, None, 0, None), "CONVROT_ERR_WORKSPACE"),
    ("convrot_gemm_i4_i32", (A, B, 32, 256, 512, C, E, 4096, None), "CONVROT_ERR_WORKSPACE"),
]


@pytest.mark.parametrize("name,args,status", CASES, ids=["%s-%d-%s" % (c[0][8:], i, c[2][12:]) for i, c in enumerate(CASES)])
def test_precondition_errors(lib, name, args, status):
    # The fake pointers are safe only because every case is rejected on the host.  Where a device
    # is present, a case that a tuning change made valid would launch on them: run these only on
    # hosts without a GPU.
    if _gpu_present():
        pytest.skip("host-only check (fake device pointers)")
    rc = getattr(lib, name)(*args)
    assert rc == ERR[status], (cr.STATUS.get(rc, rc), lib.convrot_last_error().decode())
    assert name in lib.convrot_last_error().decode()


def test_empty_inputs_are_noops(lib):
    # M == 0 or N == 0: OK without any pointer and without touching a device
    assert lib.convrot_quantize_act(None, 1, 0, 512, 256, 8, None, None, None) == 0
    assert lib.convrot_linear(None, 1, None, None, 0, 256, 512, 256, None, None, None, None, None, 0, None) == 0
    assert lib.convrot_linear(None, 1, None, None, 16, 0, 512, 256, None, None, None, None, None, 0, None) == 0
    assert lib.convrot_linear_w4a4(None, 1, None, None, 0, 256, 512, 256, None, None, None, None, None, 0, None) == 0
    assert lib.convrot_linear_w4a8(None, 1, None, None, 0, 256, 512, 256, None, 0, None, None, None, 0, None) == 0
    assert lib.convrot_linear_w4a8(None, 1, None, None, 5, 0, 512, 256, None, 0, None, None, None, 0, None) == 0
    assert lib.convrot_pack_weight_w4a8(None, None, 0, 512, None, None) == 0
    assert lib.convrot_pack_weight_w4a4(None, 0, 512, None, None) == 0
    assert lib.convrot_linear_w4a4_packed(None, 1, None, None, 0, 256, 512, 256, None, None, None, None, None, 0,
                                          None) == 0
    assert lib.convrot_gemm_i8_i32(None, None, 0, 256, 512, None, None, 0, None) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    # the Python layer never falls back to another implementation
    monkeypatch.setattr(cr, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(cr, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        cr.load()
