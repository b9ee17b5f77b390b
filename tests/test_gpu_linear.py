"""GPU: the MFMA GEMM itself through dora_linear (y = x W^T, the forward's
base-product kernel and plan) against the plain fp64 product, on shapes
that exercise every tile configuration's tails: M, N and K not multiples
of the tile or of the 64-wide K stage, single partial tiles, few tiles
(split-K chosen), and K past the pipelined kernel's one-stage boundary."""
import numpy as np
import pytest
import torch

from dora_adapter_amd import dora as D
from gpu_util import check_close, np64, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,d_in,d_out", [
    (1, 8, 8), (7, 72, 40), (33, 264, 520), (257, 1032, 776), (64, 4104, 512),
    (512, 8192, 384), (1000, 136, 2056), (300, 64, 4096),
])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_linear_matches_fp64_product(T, d_in, d_out, dtype):
    say("linear", T, d_in, d_out, dtype)
    g = torch.Generator().manual_seed(T * 7 + d_in)
    x = torch.randn(T, d_in, generator=g).to(dtype)
    W = (torch.randn(d_out, d_in, generator=g) * d_in ** -0.5).to(dtype)
    y = D.dora_linear(x.cuda(), W.cuda())
    torch.cuda.synchronize()
    ref = np64(x) @ np64(W).T
    # one rounding of an fp32 sum (bf16 output) or fp32 accumulation (fp32)
    tol = 2e-2 if dtype == torch.bfloat16 else 1e-5
    check_close(y, ref, dtype, f"x W^T {T}x{d_in}x{d_out}", tol=tol)


def test_linear_empty_tokens():
    say("linear T=0")
    x = torch.empty(0, 128, dtype=torch.bfloat16, device="cuda")
    W = torch.randn(64, 128, device="cuda").bfloat16()
    y = D.dora_linear(x, W)
    torch.cuda.synchronize()
    assert y.shape == (0, 64)
