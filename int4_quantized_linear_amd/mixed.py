"""Mixed W4A4 / W8A8 schedule of ConvRot linears (argument marshalling and dispatch only).

The nvfp4-convrot page's per-layer precision profile (section 五, "INT4 W4A4 ConvRot") runs most
layers as W4A4 ConvRot and promotes about a fifth of them (48 layers) to INT8 ConvRot, because
the 4-bit path alone loses too much quality.  ``MixedSchedule`` holds one weight per layer
instance, all resident in device memory: INT4 weights re-encoded once for the FP6 matrix core
(``convrot_pack_weight_w4a4``) for the W4A4 instances, row-wise INT8 weights for the promoted
ones.  ``run`` enqueues the instances in order on the current stream, each one a full ConvRot
linear from bf16 activations (rotate + quantize, then the GEMM with its dequant epilogue) through
the C-ABI; no arithmetic happens here.
"""
from __future__ import annotations

import torch

from . import convrot as cr


class MixedSchedule:
    """``count`` linears of one shape (M tokens, K in, N out); the instances in ``promoted`` run
    W8A8 (INT8 ConvRot), the others W4A4 with pre-encoded weights.  ``weight(i)`` returns the
    bf16/fp32 [N, K] weight of instance i on the device (prepared here, then dropped)."""

    def __init__(self, M: int, K: int, N: int, count: int, promoted, weight, bias=None, group: int = 256):
        self.M, self.K, self.N, self.count, self.group = M, K, N, count, group
        self.promoted = frozenset(int(i) for i in promoted)
        if not all(0 <= i < count for i in self.promoted):
            raise ValueError("promoted instances must lie in [0, count)")
        self.bias = bias
        self.inst = []
        for i in range(count):
            w = weight(i)
            if w.shape != (N, K):
                raise ValueError("instance %d: weight shape %s, expected (%d, %d)" % (i, tuple(w.shape), N, K))
            if i in self.promoted:
                wq, ws = cr.prepare_weight(w, group, 8)
                self.inst.append(("w8a8", wq, ws))
            else:
                wq4, ws4 = cr.prepare_weight(w, group, 4)
                wp = cr.pack_weight_w4a4(wq4)
                del wq4
                self.inst.append(("w4a4", wp, ws4))
            del w
        dev = self.inst[0][1].device if self.inst else torch.device("cuda")
        # one scratch buffer for every instance: stream order serialises them
        need = max(cr.workspace_bytes(M, N, K, 8), cr.workspace_bytes(M, 0, K, 4))
        self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)

    def kinds(self):
        return [k for k, _, _ in self.inst]

    def weight_bytes(self) -> int:
        return sum(a.numel() * a.element_size() + b.numel() * b.element_size() for _, a, b in self.inst)

    def run(self, xs, ys):
        """Enqueue every instance in order: instance i reads xs[i % len(xs)] (bf16/fp32 [M, K])
        and writes ys[i % len(ys)] (bf16 [M, N])."""
        cr._check_dev(*xs, *ys)
        dev = self.ws.device
        st = torch.cuda.current_stream(dev).cuda_stream
        M, K, N, g = self.M, self.K, self.N, self.group
        bias = self.bias.data_ptr() if self.bias is not None else None
        for i, (kind, w, s) in enumerate(self.inst):
            x, y = xs[i % len(xs)], ys[i % len(ys)]
            dt = cr._dtype_code(x)
            if kind == "w8a8":
                cr._call("convrot_linear", x.data_ptr(), dt, None, None, M, N, K, g, w.data_ptr(), s.data_ptr(),
                         bias, y.data_ptr(), self.ws.data_ptr(), self.ws.numel(), st)
            else:
                cr._call("convrot_linear_w4a4_packed", x.data_ptr(), dt, None, None, M, N, K, g, w.data_ptr(),
                         s.data_ptr(), bias, y.data_ptr(), self.ws.data_ptr(), self.ws.numel(), st)
