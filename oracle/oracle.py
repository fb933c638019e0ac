"""Python face of the CPU oracle for the ConvRot quantized linear layer.

TEST INFRASTRUCTURE ONLY: the test-suite, the package smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product path (the HIP library and its Python
binding) never imports this module, and this module never imports the product path.

The arithmetic lives in ``convrot_oracle.c`` (plain C, fp64, scalar loops); this file
marshals numpy arrays into it and composes the steps in the order the pages give them:
rotate by the grouped Hadamard, quantize (INT8 per row / INT4 per group), integer GEMM,
dequantize ("minimax-h3-nvfp4-convrot核心原理", sections 四 and 五).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "convrot_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

ORACLE_OK, ORACLE_ERR_ARG, ORACLE_ERR_RANGE = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (IEEE semantics: no fast-math, no FMA contraction)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        sig = {
            "oracle_num_threads": ([], I),
            "oracle_hadamard_entry": ([I, I], I),
            "oracle_rotate": ([P, I64, I64, I, P], I),
            "oracle_quantize_rows_i8": ([P, I64, I64, P, P], I),
            "oracle_f16_from_double": ([ctypes.c_double], ctypes.c_uint16),
            "oracle_f16_to_double": ([ctypes.c_uint16], ctypes.c_double),
            "oracle_quantize_groups_i4": ([P, I64, I64, I, P, P], I),
            "oracle_pack_i4": ([P, I64, I64, P], I),
            "oracle_unpack_i4": ([P, I64, I64, P], I),
            "oracle_gemm_i32": ([P, P, I64, I64, I64, P], I),
            "oracle_gemm_i32_pairs": ([P, P, I64, P, P, I64, P], I),
            "oracle_dequant": ([P, P, P, P, I64, I64, P], I),
            "oracle_linear_i4": ([P, P, P, P, P, I64, I64, I64, I, P], I),
            "oracle_linear_w4a8": ([P, P, P, P, P, I64, I64, I64, I, P], I),
        }
        for name, (args, res) in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
        return lib


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str):
    if rc != ORACLE_OK:
        raise OracleError("%s failed with code %d" % (what, rc))


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a) -> int | None:
    return None if a is None else a.ctypes.data


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def dynamic_group(K: int, max_group: int = 256) -> int:
    """Rotation group chosen per layer by the converter's dynamic mode: the largest group size
    compatible with the layer, capped by the configured group size ("minimax-h3-nvfp4-convrot
    核心原理", section 四, detail 3: --dynamic-convrot picks each layer's largest compatible group,
    with --convrot-group-size 256).  Reading: compatible = a power of two (a Sylvester Hadamard
    block) that divides in_features K.  Walks down from max_group, halving, as the definition
    reads."""
    if K <= 0 or max_group < 1 or max_group & (max_group - 1):
        raise ValueError("K must be positive and max_group a power of two")
    g = max_group
    while K % g:
        g //= 2
    return g


def hadamard_entry(i: int, j: int) -> int:
    return int(_load().oracle_hadamard_entry(i, j))


def rotate(x: np.ndarray, g: int) -> np.ndarray:
    """x . blockdiag(H_g/sqrt(g)) along the last axis, fp64."""
    x = _c(x, np.float64)
    rows, K = x.reshape(-1, x.shape[-1]).shape
    y = np.empty_like(x)
    _check(_load().oracle_rotate(_p(x), rows, K, g, _p(y)), "rotate")
    return y


def quantize_rows_i8(y: np.ndarray):
    """Per-row symmetric INT8 of rotated values -> (codes int8 [R,K], scale fp32 [R])."""
    y = _c(y, np.float64)
    R, K = y.shape
    q = np.empty((R, K), np.int8)
    s = np.empty((R,), np.float32)
    _check(_load().oracle_quantize_rows_i8(_p(y), R, K, _p(s), _p(q)), "quantize_rows_i8")
    return q, s


def quantize_groups_i4(y: np.ndarray, g: int):
    """Per-(row, group) symmetric INT4 -> (codes int8 [R,K], scale fp16 [R,K/g])."""
    y = _c(y, np.float64)
    R, K = y.shape
    c = np.empty((R, K), np.int8)
    s = np.empty((R, K // g), np.uint16)
    _check(_load().oracle_quantize_groups_i4(_p(y), R, K, g, _p(s), _p(c)), "quantize_groups_i4")
    return c, s.view(np.float16)


def f16_from_double(v: float) -> int:
    return int(_load().oracle_f16_from_double(float(v)))


def f16_to_double(h: int) -> float:
    return float(_load().oracle_f16_to_double(int(h)))


def pack_i4(codes: np.ndarray) -> np.ndarray:
    codes = _c(codes, np.int8)
    R, K = codes.shape
    out = np.empty((R, K // 2), np.uint8)
    _check(_load().oracle_pack_i4(_p(codes), R, K, _p(out)), "pack_i4")
    return out


def unpack_i4(packed: np.ndarray) -> np.ndarray:
    packed = _c(packed, np.uint8)
    R, Kh = packed.shape
    out = np.empty((R, 2 * Kh), np.int8)
    _check(_load().oracle_unpack_i4(_p(packed), R, 2 * Kh, _p(out)), "unpack_i4")
    return out


def gemm_i32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """acc = a @ b.T with int64 accumulation, returned as int32 (refuses overflow)."""
    a = _c(a, np.int8)
    b = _c(b, np.int8)
    M, K = a.shape
    N, K2 = b.shape
    assert K == K2
    acc = np.empty((M, N), np.int32)
    _check(_load().oracle_gemm_i32(_p(a), _p(b), M, N, K, _p(acc)), "gemm_i32")
    return acc


def gemm_i32_pairs(a: np.ndarray, b: np.ndarray, ms: np.ndarray, ns: np.ndarray) -> np.ndarray:
    a = _c(a, np.int8)
    b = _c(b, np.int8)
    ms = _c(ms, np.int64)
    ns = _c(ns, np.int64)
    assert a.shape[1] == b.shape[1] and ms.shape == ns.shape
    out = np.empty(ms.shape, np.int32)
    _check(_load().oracle_gemm_i32_pairs(_p(a), _p(b), a.shape[1], _p(ms), _p(ns), ms.size, _p(out)),
           "gemm_i32_pairs")
    return out


def dequant(acc: np.ndarray, sx: np.ndarray, sw: np.ndarray, bias: np.ndarray | None) -> np.ndarray:
    acc = _c(acc, np.int32)
    sx = _c(sx, np.float32)
    sw = _c(sw, np.float32)
    bias = None if bias is None else _c(bias, np.float32)
    M, N = acc.shape
    y = np.empty((M, N), np.float64)
    _check(_load().oracle_dequant(_p(acc), _p(sx), _p(sw), _p(bias), M, N, _p(y)), "dequant")
    return y


def linear_i4(cx, sx, cw, sw, bias, g: int) -> np.ndarray:
    cx = _c(cx, np.int8)
    cw = _c(cw, np.int8)
    sx = _c(np.asarray(sx, np.float16).view(np.uint16), np.uint16)
    sw = _c(np.asarray(sw, np.float16).view(np.uint16), np.uint16)
    bias = None if bias is None else _c(bias, np.float32)
    M, K = cx.shape
    N = cw.shape[0]
    y = np.empty((M, N), np.float64)
    _check(_load().oracle_linear_i4(_p(cx), _p(sx), _p(cw), _p(sw), _p(bias), M, N, K, g, _p(y)), "linear_i4")
    return y


def linear_w4a8_codes(qx, sx, cw, sw, bias, g: int) -> np.ndarray:
    """y = sx[m] * sum_j sw[n,j] * (int dot product of group j) + bias[n]; sw is [N, K/g] fp16."""
    qx = _c(qx, np.int8)
    cw = _c(cw, np.int8)
    sx = _c(sx, np.float32)
    sw = _c(np.asarray(sw, np.float16).view(np.uint16), np.uint16)
    bias = None if bias is None else _c(bias, np.float32)
    M, K = qx.shape
    N = cw.shape[0]
    y = np.empty((M, N), np.float64)
    _check(_load().oracle_linear_w4a8(_p(qx), _p(sx), _p(cw), _p(sw), _p(bias), M, N, K, g, _p(y)), "linear_w4a8")
    return y


# ---------------------------------------------------------------------------------------------
# The method end to end, step by step in the pages' order.
# ---------------------------------------------------------------------------------------------

def prepare_weight_i8(w: np.ndarray, g: int):
    """Offline: rotate each weight row by the grouped Hadamard, then row-wise INT8 -> (q, s)."""
    return quantize_rows_i8(rotate(w, g))


def quantize_act_i8(x: np.ndarray, g: int):
    """Online: rotate each token by the same R, then per-token INT8 -> (q, s)."""
    return quantize_rows_i8(rotate(x, g))


def prepare_i4(v: np.ndarray, g: int):
    """Rotate, then per-group INT4 -> (codes int8, scales fp16, packed uint8)."""
    c, s = quantize_groups_i4(rotate(v, g), g)
    return c, s, pack_i4(c)


def linear_w8a8(x: np.ndarray, w: np.ndarray, bias: np.ndarray | None, g: int) -> dict:
    """ConvRot INT8 linear: y = dequant(gemm(q(xR), q(wR)))."""
    qw, sw = prepare_weight_i8(w, g)
    qx, sx = quantize_act_i8(x, g)
    acc = gemm_i32(qx, qw)
    y = dequant(acc, sx, sw, bias)
    return dict(qx=qx, sx=sx, qw=qw, sw=sw, acc=acc, y=y)


def linear_w4a4(x: np.ndarray, w: np.ndarray, bias: np.ndarray | None, g: int) -> dict:
    """ConvRot W4A4 linear: both operands rotated, INT4 per group, group-wise int dot products."""
    cw, sw, pw = prepare_i4(w, g)
    cx, sx, px = prepare_i4(x, g)
    y = linear_i4(cx, sx, cw, sw, bias, g)
    return dict(cx=cx, sx=sx, px=px, cw=cw, sw=sw, pw=pw, y=y)


def linear_w4a8(x: np.ndarray, w: np.ndarray, bias: np.ndarray | None, g: int) -> dict:
    """ConvRot W4A8 linear: weights rotated and INT4 per group, tokens rotated and INT8 per token."""
    cw, sw, pw = prepare_i4(w, g)
    qx, sx = quantize_act_i8(x, g)
    y = linear_w4a8_codes(qx, sx, cw, sw, bias, g)
    return dict(qx=qx, sx=sx, cw=cw, sw=sw, pw=pw, y=y)
