"""Seeded synthetic inputs for the ConvRot linear workloads.

This module only draws random numbers and casts them; it holds none of the method's
arithmetic (no rotation, no quantization, no GEMM).  Both the HIP path's tests/benchmark and
the CPU oracle's tests take their inputs from here.

The shapes stand in for the matrices the pages run through ConvRot linears:
  * the Qwen3-VL-32B text encoder used as the MiniMax-H3 conditioning encoder runs at 12 tokens
    with hidden size 5120 ("Qwen3-VL-32B-...-INT8-ConvRot部署优化", section 运行时验证指标:
    output (1, 12, 5120)), i.e. every linear there is a 12-row GEMV;
  * MiniMax-H3 attn.qkv_proj layers have in_features 5376, divisible by the group of 256
    ("minimax-h3-nvfp4-convrot核心原理", section 四, detail 3).
The remaining dimensions (8192/1024/25600 projections, 16128 = 3 x 5376 outputs, 10752) and all
value distributions are the workload definitions this library is measured on; nothing here
comes from a dataset or trained weights.

Generators: numpy PCG64.  A workload's stream is ``SeedSequence([cfg, layer, role])`` with
role 0 = activations, 1 = outlier channel pick, 2 = weights, 3 = bias, 4 = mixed-layer pick,
except the tiny case, which uses ``default_rng(0)`` and draws X, outlier channels, W in order.
"N(0, 0.02)" is a standard deviation of 0.02.  Outlier channels are chosen without replacement
and scaled before the cast to the stored dtype (bf16 casts round to nearest even via torch).
"""
from __future__ import annotations

import numpy as np
import torch

GROUP = 256

# Decode-shaped (M = 12) matrices: (K, N).
DECODE_SHAPES = [(5120, 8192), (5120, 1024), (5120, 25600), (25600, 5120)]
DECODE_M = 12

PREFILL = dict(M=4096, K=5376, N=16128)
W4A4_SHAPE = dict(M=4096, K=5376, N=10752)

# Qwen3-32B-shaped decoder layer: name -> (K, N); activations shared as noted.
STACK_M = 2048
STACK_LAYERS = 64
STACK_MATRICES = [("q", 5120, 8192), ("k", 5120, 1024), ("v", 5120, 1024), ("o", 8192, 5120),
                  ("gate", 5120, 25600), ("up", 5120, 25600), ("down", 25600, 5120)]
# Which activation each matrix consumes (q/k/v share attn-in, gate/up share mlp-in).
STACK_INPUT_OF = {"q": "attn_in", "k": "attn_in", "v": "attn_in", "o": "o_in",
                  "gate": "mlp_in", "up": "mlp_in", "down": "down_in"}
STACK_INPUTS = [("attn_in", 5120), ("o_in", 8192), ("mlp_in", 5120), ("down_in", 25600)]

CFG_TINY, CFG_DECODE, CFG_PREFILL, CFG_STACK, CFG_W4A4 = 1, 2, 3, 4, 5
ROLE_X, ROLE_OUTLIER, ROLE_W, ROLE_BIAS, ROLE_MIX = 0, 1, 2, 3, 4


def rng_for(cfg: int, layer: int, role: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg, layer, role])))


def to_bf16(a: np.ndarray) -> torch.Tensor:
    """Round an fp32/fp64 array to bf16 (nearest even) as a CPU tensor."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def _outliers(a: np.ndarray, rng: np.random.Generator, count: int, factor: float) -> np.ndarray:
    ch = rng.choice(a.shape[1], count, replace=False)
    a[:, ch] *= factor
    return ch


def tiny_inputs():
    """4 x 512 fp32 N(0,1) with 5 channels x20; W 256 x 512 fp32 N(0, 0.02); seed 0."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal((4, 512))
    _outliers(x, rng, 5, 20.0)
    w = rng.normal(0.0, 0.02, (256, 512))
    return torch.from_numpy(x.astype(np.float32)), torch.from_numpy(w.astype(np.float32))


def heavy_tailed_acts(M: int, K: int, cfg: int, layer: int, frac: float = 0.01, factor: float = 30.0,
                      key: int = 0) -> torch.Tensor:
    """Student-t (nu = 4) activations, round(frac*K) channels scaled by `factor`, bf16."""
    rng = rng_for(cfg, layer * 16 + key, ROLE_X)
    x = rng.standard_t(4.0, size=(M, K)).astype(np.float32)
    _outliers(x, rng_for(cfg, layer * 16 + key, ROLE_OUTLIER), int(round(frac * K)), factor)
    return to_bf16(x)


def gaussian_acts(M: int, K: int, cfg: int, layer: int = 0, frac: float = 0.005, factor: float = 50.0
                  ) -> torch.Tensor:
    """N(0, 1) activations, round(frac*K) channels scaled by `factor`, bf16."""
    x = rng_for(cfg, layer, ROLE_X).standard_normal((M, K), dtype=np.float32)
    _outliers(x, rng_for(cfg, layer, ROLE_OUTLIER), int(round(frac * K)), factor)
    return to_bf16(x)


def gaussian_weights(N: int, K: int, cfg: int, layer: int = 0, key: int = 0, std: float = 0.02) -> torch.Tensor:
    w = rng_for(cfg, layer * 16 + key, ROLE_W).standard_normal((N, K), dtype=np.float32)
    w *= np.float32(std)
    return to_bf16(w)


def bias_vector(N: int, cfg: int, layer: int = 0, key: int = 0) -> torch.Tensor:
    return torch.from_numpy(rng_for(cfg, layer * 16 + key, ROLE_BIAS).standard_normal(N, dtype=np.float32))


def decode_inputs(K: int, N: int):
    """M = 12 decode case: X bf16 Student-t(4) with 1% channels x30; W bf16 N(0, 0.02)."""
    key = DECODE_SHAPES.index((K, N)) if (K, N) in DECODE_SHAPES else (K * 7 + N) % 1000
    x = heavy_tailed_acts(DECODE_M, K, CFG_DECODE, 0, key=key)
    w = gaussian_weights(N, K, CFG_DECODE, 0, key=key)
    return x, w


def prefill_inputs(M: int = PREFILL["M"], K: int = PREFILL["K"], N: int = PREFILL["N"], cfg: int = CFG_PREFILL):
    """Prefill case: X bf16 N(0,1) with 0.5% channels x50; W bf16 N(0, 0.02); bias fp32 N(0,1)."""
    x = gaussian_acts(M, K, cfg)
    w = gaussian_weights(N, K, cfg)
    b = bias_vector(N, cfg)
    return x, w, b


def mixed_profile_layers(total: int = 240, promoted: int = 48) -> np.ndarray:
    """Seeded pick of the layer instances that run W8A8 in the mixed W4A4/W8A8 profile."""
    return np.sort(rng_for(CFG_W4A4, 0, ROLE_MIX).choice(total, promoted, replace=False))


def ragged_case(M: int, K: int, N: int, seed: int, dtype=torch.bfloat16, outlier_frac: float = 0.01,
                factor: float = 30.0):
    """Generic seeded case for parity tests at arbitrary (possibly ragged) sizes."""
    rng = rng_for(100 + seed, M * 131 + N, ROLE_X)
    x = rng.standard_t(4.0, size=(M, K)).astype(np.float32)
    if K >= 100:
        _outliers(x, rng_for(100 + seed, M * 131 + N, ROLE_OUTLIER), max(1, int(round(outlier_frac * K))), factor)
    w = rng_for(100 + seed, M * 131 + N, ROLE_W).normal(0.0, 0.02, (N, K)).astype(np.float32)
    b = rng_for(100 + seed, M * 131 + N, ROLE_BIAS).standard_normal(N).astype(np.float32)
    if dtype == torch.bfloat16:
        return to_bf16(x), to_bf16(w), torch.from_numpy(b)
    return torch.from_numpy(x), torch.from_numpy(w), torch.from_numpy(b)


def _device_generator(cfg: int, layer: int, role: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence([cfg, layer, role]).generate_state(1, dtype=np.uint64)[0] >> 1))
    return g


def stack_weight(layer: int, idx: int, N: int, K: int, device, std: float = 0.02) -> torch.Tensor:
    """Layer-stack weight drawn on the device (31 GB of them would take minutes on the host):
    bf16 N(0, std), seeded per (layer, matrix)."""
    g = _device_generator(CFG_STACK, layer * 16 + idx, ROLE_W, device)
    return (torch.randn(N, K, generator=g, device=device, dtype=torch.float32) * std).to(torch.bfloat16)


def stack_acts(layer: int, key: int, M: int, K: int, device, frac: float = 0.01, factor: float = 30.0
               ) -> torch.Tensor:
    """Layer-stack activation drawn on the device: Student-t (nu = 4) as Z / sqrt(V / 4) with V the
    sum of 4 squared standard normals, round(frac*K) channels scaled by `factor`, bf16; a fresh
    seed per (layer, input)."""
    g = _device_generator(CFG_STACK, layer * 16 + key, ROLE_X, device)
    z = torch.randn(M, K, generator=g, device=device, dtype=torch.float32)
    v = torch.zeros(M, K, device=device, dtype=torch.float32)
    for _ in range(4):
        v += torch.randn(M, K, generator=g, device=device, dtype=torch.float32).square_()
    x = z / torch.sqrt(v * 0.25)
    go = _device_generator(CFG_STACK, layer * 16 + key, ROLE_OUTLIER, device)
    ch = torch.randperm(K, generator=go, device=device)[: int(round(frac * K))]
    x[:, ch] *= factor
    return x.to(torch.bfloat16)


# Mixed W4A4 / W8A8 profile: MIXED_COUNT instances of the W4A4 shape, MIXED_PROMOTED of them
# (mixed_profile_layers) running W8A8.
MIXED_COUNT, MIXED_PROMOTED = 240, 48


def mixed_weight(inst: int, N: int, K: int, device, std: float = 0.02) -> torch.Tensor:
    """Weight of one instance of the mixed profile, drawn on the device (240 of them would take
    minutes on the host): bf16 N(0, std), seeded per instance."""
    g = _device_generator(CFG_W4A4, 1000 + inst, ROLE_W, device)
    return (torch.randn(N, K, generator=g, device=device, dtype=torch.float32) * std).to(torch.bfloat16)


def mixed_acts(key: int, M: int, K: int, device, frac: float = 0.005, factor: float = 50.0) -> torch.Tensor:
    """Activation of the mixed profile drawn on the device: N(0, 1) with round(frac*K) channels
    scaled by `factor` (the prefill distribution), bf16, seeded per key."""
    g = _device_generator(CFG_W4A4, 1000 + key, ROLE_X, device)
    x = torch.randn(M, K, generator=g, device=device, dtype=torch.float32)
    go = _device_generator(CFG_W4A4, 1000 + key, ROLE_OUTLIER, device)
    ch = torch.randperm(K, generator=go, device=device)[: int(round(frac * K))]
    x[:, ch] *= factor
    return x.to(torch.bfloat16)
