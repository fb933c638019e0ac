"""convrot_linear_noalloc (the library's fixed per-GPU scratch, no allocation) against
convrot_linear (caller's workspace): the same kernels, so the outputs must be equal bit for bit,
on two calls in a row (the second smaller, so stale contents of the shared scratch from the first
call must not leak into it), through the C-ABI."""
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


# (M, N, K, g): the tiled GEMM with a split-K tail whose partial sums fit the scratch, then a
# smaller decode-sized call (the weight-streaming GEMV), then a GEMM call with pre-quantized x
CASES = [(300, 1000, 4096, 256), (12, 520, 1024, 256), (130, 264, 2688, 128)]


def test_noalloc_linear_equals_linear(cr):
    for i, (M, N, K, g) in enumerate(CASES):
        P.say("linear_noalloc M=%d N=%d K=%d g=%d" % (M, N, K, g))
        x, w, b = workloads.ragged_case(M, K, N, seed=40 + i)
        xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
        wq, ws = cr.prepare_weight(wd, g, 8)
        ref = cr.linear(xd, wq, ws, bd, group=g)
        got = cr.linear_noalloc(xd, wq, ws, bd, group=g)
        xq, xs = cr.quantize_act(xd, g, 8)
        got_q = cr.linear_noalloc(None, wq, ws, bd, group=g, xq=xq, x_scale=xs)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), "noalloc differs from convrot_linear"
        assert torch.equal(got_q, ref), "noalloc with pre-quantized x differs from convrot_linear"
        # and against the oracle on the same inputs (rule d)
        yref = orc.linear_w8a8(P.to_np64(x), P.to_np64(w), b.numpy(), g)["y"]
        P.check_y(P.to_np64(got), yref, "noalloc y")


def test_noalloc_rejects_activations_past_the_scratch(cr):
    # 8192 x 8192 INT8 activations (64 MiB) do not fit the 32 MiB scratch: rejected on the host
    # before anything is enqueued
    K, N = 8192, 64
    w = torch.zeros((N, K), dtype=torch.bfloat16, device=DEV)
    wq, ws = cr.prepare_weight(w, 256, 8)
    x = torch.zeros((8192, K), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(cr.ConvRotError, match="WORKSPACE"):
        cr.linear_noalloc(x, wq, ws)
    torch.cuda.synchronize()
