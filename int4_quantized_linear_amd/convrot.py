"""Python binding of libconvrot (ctypes).  Argument marshalling only: every step of the ConvRot
linear runs in the library's HIP kernels; torch provides device memory and the current stream.

Raises ``ConvRotError`` when the library rejects a call and ``ImportError``-style
``RuntimeError`` when the built library is missing -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libconvrot.so")

CONVROT_DTYPE_F32, CONVROT_DTYPE_BF16 = 0, 1
STATUS = {0: "CONVROT_OK", 1: "CONVROT_ERR_NULL", 2: "CONVROT_ERR_SHAPE", 3: "CONVROT_ERR_GROUP",
          4: "CONVROT_ERR_ALIGN", 5: "CONVROT_ERR_DTYPE", 6: "CONVROT_ERR_BITS", 7: "CONVROT_ERR_WORKSPACE",
          8: "CONVROT_ERR_HIP", 9: "CONVROT_ERR_DEVICE"}

# name -> (argtypes, restype); mirrors include/convrot.h
P, I64, I, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "convrot_prepare_weight": ([P, I, I64, I64, I, I, P, P, P], I),
    "convrot_quantize_act": ([P, I, I64, I64, I, I, P, P, P], I),
    "convrot_workspace_bytes": ([I64, I64, I64, I], SZ),
    "convrot_linear": ([P, I, P, P, I64, I64, I64, I, P, P, P, P, P, SZ, P], I),
    "convrot_linear_noalloc": ([P, I, P, P, I64, I64, I64, I, P, P, P, P, P], I),
    "convrot_linear_w4a4": ([P, I, P, P, I64, I64, I64, I, P, P, P, P, P, SZ, P], I),
    "convrot_pack_weight_w4a4": ([P, I64, I64, P, P], I),
    "convrot_packed_bytes_w4a4": ([I64, I64], SZ),
    "convrot_linear_w4a4_packed": ([P, I, P, P, I64, I64, I64, I, P, P, P, P, P, SZ, P], I),
    "convrot_linear_w4a8": ([P, I, P, P, I64, I64, I64, I, P, SZ, P, P, P, SZ, P], I),
    "convrot_pack_weight_w4a8": ([P, P, I64, I64, P, P], I),
    "convrot_packed_bytes_w4a8": ([I64, I64], SZ),
    "convrot_pack_weight_w4a8_group": ([P, P, I64, I64, I, P, P], I),
    "convrot_packed_bytes_w4a8_group": ([I64, I64, I], SZ),
    "convrot_workspace_bytes_w4a8": ([I64, I64, I64], SZ),
    "convrot_gemm_i8_i32": ([P, P, I64, I64, I64, P, P, SZ, P], I),
    "convrot_gemm_i4_i32": ([P, P, I64, I64, I64, P, P, SZ, P], I),
    "convrot_dynamic_group": ([I64, I], I),
    "convrot_last_error": ([], ctypes.c_char_p),
    "convrot_status_string": ([I], ctypes.c_char_p),
}

_lock = threading.Lock()
_lib = None


class ConvRotError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def load() -> ctypes.CDLL:
    """Load the in-tree libconvrot.so (built by ``python -m int4_quantized_linear_amd.build``)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("libconvrot.so is not built (%s); run python -m int4_quantized_linear_amd.build"
                                   % LIB_PATH)
            lib = ctypes.CDLL(LIB_PATH)
            for name, (args, res) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.argtypes = args
                fn.restype = res
            _lib = lib
        return _lib


def _call(name: str, *args) -> int:
    lib = load()
    rc = getattr(lib, name)(*args)
    if rc != 0:
        raise ConvRotError(rc, lib.convrot_last_error().decode() or STATUS.get(rc, str(rc)))
    return rc


def _ptr(t: torch.Tensor | None):
    return None if t is None else t.data_ptr()


def _stream(dev: torch.device):
    return torch.cuda.current_stream(dev).cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return CONVROT_DTYPE_BF16
    if t.dtype == torch.float32:
        return CONVROT_DTYPE_F32
    raise TypeError("ConvRot inputs are bf16 or fp32, got %s" % t.dtype)


def _check_dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("ConvRot tensors must be on a GPU device")
            if not t.is_contiguous():
                raise ValueError("ConvRot tensors must be contiguous")


def dynamic_group(K: int, max_group: int = 256) -> int:
    """Largest power-of-two rotation group <= max_group dividing K (dynamic ConvRot mode)."""
    g = int(load().convrot_dynamic_group(K, max_group))
    if g == 0:
        raise ConvRotError(3, "CONVROT_ERR_GROUP: invalid K=%d or max_group=%d" % (K, max_group))
    return g


def workspace_bytes(M: int, N: int, K: int, bits: int = 8) -> int:
    return int(load().convrot_workspace_bytes(M, N, K, bits))


def _workspace(M: int, N: int, K: int, bits: int, dev: torch.device) -> torch.Tensor:
    return torch.empty(max(workspace_bytes(M, N, K, bits), 256), dtype=torch.uint8, device=dev)


def _quant(name: str, v: torch.Tensor, group: int, bits: int):
    _check_dev(v)
    R, K = v.shape
    if bits == 8:
        q = torch.empty((R, K), dtype=torch.int8, device=v.device)
        s = torch.empty((R,), dtype=torch.float32, device=v.device)
    else:
        q = torch.empty((R, K // 2), dtype=torch.uint8, device=v.device)
        # one fp16 scale per (group, row); an invalid group is rejected by the library before any write
        ngroups = K // group if group > 0 and K % group == 0 else 1
        s = torch.empty((ngroups, R), dtype=torch.float16, device=v.device)
    _call(name, _ptr(v), _dtype_code(v), R, K, group, bits, _ptr(q), _ptr(s), _stream(v.device))
    return q, s


def prepare_weight(w: torch.Tensor, group: int = 256, bits: int = 8):
    """Rotate + quantize a weight [N, K] -> (wq, w_scale).  bits 8: int8 [N,K], fp32 [N];
    bits 4: uint8 [N,K/2] packed, fp16 [K/group, N] (group 256 or 128)."""
    return _quant("convrot_prepare_weight", w, group, bits)


def quantize_act(x: torch.Tensor, group: int = 256, bits: int = 8):
    """Rotate + quantize activations [M, K] per token -> (xq, x_scale) (layouts as prepare_weight)."""
    return _quant("convrot_quantize_act", x, group, bits)


def linear(x: torch.Tensor | None, wq: torch.Tensor, w_scale: torch.Tensor, bias: torch.Tensor | None = None,
           group: int = 256, xq: torch.Tensor | None = None, x_scale: torch.Tensor | None = None,
           out: torch.Tensor | None = None, split_k: bool = True) -> torch.Tensor:
    """INT8 ConvRot linear: y = bf16((q(xR) . q(wR)^T) * sx * sw + bias).  Pass x (bf16/fp32 [M,K])
    or a pre-quantized (xq, x_scale) pair.  The workspace passed has room for the GEMM's split-K
    tail; split_k=False (pre-quantized x only) passes none, so the GEMM runs without it."""
    _check_dev(x, wq, w_scale, bias, xq, x_scale, out)
    N, K = wq.shape
    M = x.shape[0] if x is not None else xq.shape[0]
    dev = wq.device
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if split_k:
        ws = _workspace(M, N, K, 8, dev)
    elif x is None:
        ws = None
    else:
        raise ValueError("split_k=False needs a pre-quantized (xq, x_scale) pair")
    _call("convrot_linear", _ptr(x), _dtype_code(x) if x is not None else 0, _ptr(xq), _ptr(x_scale), M, N, K, group,
          _ptr(wq), _ptr(w_scale), _ptr(bias), _ptr(y), _ptr(ws), ws.numel() if ws is not None else 0, _stream(dev))
    return y


def linear_noalloc(x: torch.Tensor | None, wq: torch.Tensor, w_scale: torch.Tensor, bias: torch.Tensor | None = None,
                   group: int = 256, xq: torch.Tensor | None = None, x_scale: torch.Tensor | None = None,
                   out: torch.Tensor | None = None) -> torch.Tensor:
    """linear() through convrot_linear_noalloc: the library's fixed per-GPU scratch instead of a
    workspace (the output is allocated here unless ``out`` is given)."""
    _check_dev(x, wq, w_scale, bias, xq, x_scale, out)
    N, K = wq.shape
    M = x.shape[0] if x is not None else xq.shape[0]
    dev = wq.device
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    _call("convrot_linear_noalloc", _ptr(x), _dtype_code(x) if x is not None else 0, _ptr(xq), _ptr(x_scale), M, N, K,
          group, _ptr(wq), _ptr(w_scale), _ptr(bias), _ptr(y), _stream(dev))
    return y


def linear_w4a4(x: torch.Tensor | None, wq: torch.Tensor, w_scale: torch.Tensor, bias: torch.Tensor | None = None,
                group: int = 256, xq: torch.Tensor | None = None, x_scale: torch.Tensor | None = None,
                out: torch.Tensor | None = None) -> torch.Tensor:
    """W4A4 ConvRot linear with packed int4 operands and fp16 group scales."""
    _check_dev(x, wq, w_scale, bias, xq, x_scale, out)
    N, Kh = wq.shape
    K = 2 * Kh
    M = x.shape[0] if x is not None else xq.shape[0]
    dev = wq.device
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = _workspace(M, N, K, 4, dev)
    _call("convrot_linear_w4a4", _ptr(x), _dtype_code(x) if x is not None else 0, _ptr(xq), _ptr(x_scale), M, N, K,
          group, _ptr(wq), _ptr(w_scale), _ptr(bias), _ptr(y), _ptr(ws), ws.numel(), _stream(dev))
    return y


def packed_bytes_w4a4(N: int, K: int) -> int:
    return int(load().convrot_packed_bytes_w4a4(N, K))


def pack_weight_w4a4(wq: torch.Tensor) -> torch.Tensor:
    """Re-encode INT4 weights (prepare_weight(bits=4): wq uint8 [N, K/2]) once as FP6 codes in
    matrix-core order (a flat uint8 buffer) for linear_w4a4_packed; the scales are unchanged."""
    _check_dev(wq)
    N, Kh = wq.shape
    K = 2 * Kh
    out = torch.empty(max(packed_bytes_w4a4(N, K), 16), dtype=torch.uint8, device=wq.device)
    _call("convrot_pack_weight_w4a4", _ptr(wq), N, K, _ptr(out), _stream(wq.device))
    return out


def linear_w4a4_packed(x: torch.Tensor | None, w_packed: torch.Tensor, w_scale: torch.Tensor,
                       bias: torch.Tensor | None = None, group: int = 256, xq: torch.Tensor | None = None,
                       x_scale: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """linear_w4a4 with weights from pack_weight_w4a4 (N = w_scale.shape[1]); same result."""
    _check_dev(x, w_packed, w_scale, bias, xq, x_scale, out)
    N = w_scale.shape[1]
    M, K = x.shape if x is not None else (xq.shape[0], 2 * xq.shape[1])
    dev = w_packed.device
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = _workspace(M, 0, K, 4, dev)
    _call("convrot_linear_w4a4_packed", _ptr(x), _dtype_code(x) if x is not None else 0, _ptr(xq), _ptr(x_scale), M,
          N, K, group, _ptr(w_packed), _ptr(w_scale), _ptr(bias), _ptr(y), _ptr(ws), ws.numel(), _stream(dev))
    return y


def workspace_bytes_w4a8(M: int, N: int, K: int) -> int:
    return int(load().convrot_workspace_bytes_w4a8(M, N, K))


def packed_bytes_w4a8(N: int, K: int, group: int = 256) -> int:
    return int(load().convrot_packed_bytes_w4a8_group(N, K, group))


def pack_weight_w4a8(wq: torch.Tensor, w_scale: torch.Tensor, group: int = 256) -> torch.Tensor:
    """Re-lay out INT4 weights (prepare_weight(bits=4): wq uint8 [N, K/2], w_scale fp16
    [K/group, N], group 256 or 128) into the W4A8 decode kernel's block layout (a flat uint8
    buffer); linear_w4a8 must then be called with the same group."""
    _check_dev(wq, w_scale)
    N, Kh = wq.shape
    K = 2 * Kh
    out = torch.empty(max(packed_bytes_w4a8(N, K, group), 16), dtype=torch.uint8, device=wq.device)
    if group == 256:
        _call("convrot_pack_weight_w4a8", _ptr(wq), _ptr(w_scale), N, K, _ptr(out), _stream(wq.device))
    else:
        _call("convrot_pack_weight_w4a8_group", _ptr(wq), _ptr(w_scale), N, K, group, _ptr(out), _stream(wq.device))
    return out


def linear_w4a8(x: torch.Tensor | None, w_packed: torch.Tensor, N: int, bias: torch.Tensor | None = None,
                group: int = 256, xq: torch.Tensor | None = None, x_scale: torch.Tensor | None = None,
                out: torch.Tensor | None = None) -> torch.Tensor:
    """W4A8 ConvRot linear (at most 16 tokens): INT4 weights in the W4A8 block layout
    (pack_weight_w4a8) with N output channels, against int8 tokens (quantize_act(bits=8), or x
    quantized here)."""
    _check_dev(x, w_packed, bias, xq, x_scale, out)
    M, K = x.shape if x is not None else xq.shape
    dev = w_packed.device
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    # the workspace only holds the quantized tokens when x is given
    ws = None if x is None else torch.empty(max(workspace_bytes_w4a8(M, N, K), 256), dtype=torch.uint8, device=dev)
    # the library checks the packed size against this group's layout (the two groups' sizes differ)
    _call("convrot_linear_w4a8", _ptr(x), _dtype_code(x) if x is not None else 0, _ptr(xq), _ptr(x_scale), M, N, K,
          group, _ptr(w_packed), w_packed.numel() * w_packed.element_size(), _ptr(bias), _ptr(y), _ptr(ws),
          0 if ws is None else ws.numel(), _stream(dev))
    return y


def gemm_i8_i32(xq: torch.Tensor, wq: torch.Tensor) -> torch.Tensor:
    """Unscaled integer core: int32 [M, N] = xq . wq^T (same dispatch as linear)."""
    _check_dev(xq, wq)
    M, K = xq.shape
    N = wq.shape[0]
    acc = torch.empty((M, N), dtype=torch.int32, device=xq.device)
    ws = _workspace(M, N, K, 8, xq.device)
    _call("convrot_gemm_i8_i32", _ptr(xq), _ptr(wq), M, N, K, _ptr(acc), _ptr(ws), ws.numel(), _stream(xq.device))
    return acc


def gemm_i4_i32(xq: torch.Tensor, wq: torch.Tensor) -> torch.Tensor:
    """Unscaled W4A4 integer core over packed codes: int32 [M, N] = sum_k cx * cw."""
    _check_dev(xq, wq)
    M, Kh = xq.shape
    N = wq.shape[0]
    acc = torch.empty((M, N), dtype=torch.int32, device=xq.device)
    ws = _workspace(M, N, 2 * Kh, 4, xq.device)
    _call("convrot_gemm_i4_i32", _ptr(xq), _ptr(wq), M, N, 2 * Kh, _ptr(acc), _ptr(ws), ws.numel(), _stream(xq.device))
    return acc
