"""GPU: the single rounding to bf16 is round-to-nearest-even, ties included,
bit for bit against torch's fp32 -> bf16 conversion, through every epilogue
that rounds a result: the one-tile and persistent GEMM stores (dora_linear),
the fused forward's scaled store (B = 0 and m = n, so g - 1 = 0 exactly) and
the standalone compose.

The inputs are built so that each output is an exact fp32 sum a + b of two
bf16 values with a in [1, 2) and b = +-2^-8, +-2^-8 (1 + 2^-9) or +-2^-9:
exactly half an ulp of a (a tie, resolved to the even mantissa), just above
half an ulp, or a quarter of one."""
import pytest
import torch

from dora_adapter_amd import dora as D
from gpu_util import say

pytestmark = pytest.mark.gpu


def _pairs(n, seed):
    """a in [1, 2) with random 7-bit mantissas (bf16), b from the cases above."""
    g = torch.Generator().manual_seed(seed)
    mant = torch.randint(0, 128, (n,), generator=g)
    a = (1.0 + mant.double() / 128.0).float()
    choices = torch.tensor([2.0 ** -8, -(2.0 ** -8), 2.0 ** -8 * (1 + 2.0 ** -9),
                            -(2.0 ** -8) * (1 + 2.0 ** -9), 2.0 ** -9, -(2.0 ** -9)])
    b = choices[torch.randint(0, len(choices), (n,), generator=g)].float()
    return a, b


def _expected(a, b):
    return (a + b).to(torch.bfloat16)  # a + b is exact in fp32


@pytest.mark.parametrize("T,N,K,cfg", [
    (300, 1024, 136, "4"),    # 256 x 256 tiles, persistent (three K stages)
    (300, 1024, 64, "4"),     # one K stage: the one-tile launch
    (100, 200, 8, None),      # the planner's choice for a small product
])
def test_gemm_store_rounds_to_nearest_even(T, N, K, cfg, monkeypatch):
    say("rne linear", T, N, K, cfg)
    if cfg is None:
        monkeypatch.delenv("DORA_TILE_CFG", raising=False)
    else:
        monkeypatch.setenv("DORA_TILE_CFG", cfg)
    a, b = _pairs(N, seed=N + K)
    b_bf = b.to(torch.bfloat16)
    # the 2^-8 (1 + 2^-9) offsets are not bf16: split them into two bf16 terms
    b_rest = (b - b_bf.float()).to(torch.bfloat16)
    assert torch.equal(b_bf.float() + b_rest.float(), b)
    W = torch.zeros(N, K, dtype=torch.bfloat16)
    W[:, 0], W[:, 1], W[:, 2] = a.to(torch.bfloat16), b_bf, b_rest
    x = torch.zeros(T, K, dtype=torch.bfloat16)
    x[:, :3] = 1.0
    y = D.dora_linear(x.cuda(), W.cuda())
    torch.cuda.synchronize()
    want = _expected(a, b).expand(T, N)
    assert torch.equal(y.cpu(), want)


@pytest.mark.parametrize("cfg", ["4", None])
def test_fused_forward_store_rounds_to_nearest_even(cfg, monkeypatch):
    say("rne forward", cfg)
    if cfg is None:
        monkeypatch.delenv("DORA_TILE_CFG", raising=False)
    else:
        monkeypatch.setenv("DORA_TILE_CFG", cfg)
    T, N, K, r = 300, 1024, 136, 8
    a, b = _pairs(N, seed=3)
    b_bf = b.to(torch.bfloat16)
    b_rest = (b - b_bf.float()).to(torch.bfloat16)
    W = torch.zeros(N, K, dtype=torch.bfloat16)
    W[:, 0], W[:, 1], W[:, 2] = a.to(torch.bfloat16), b_bf, b_rest
    x = torch.zeros(T, K, dtype=torch.bfloat16)
    x[:, :3] = 1.0
    A = torch.randn(r, K).bfloat16()
    B = torch.zeros(N, r, dtype=torch.bfloat16)
    Wg = W.cuda()
    n = D.dora_factored_norm(Wg, A.cuda(), B.cuda(), 1.0)
    y, _, _ = D.dora_forward(x.cuda(), Wg, A.cuda(), B.cuda(), n.clone(), 1.0, n_in=n)
    torch.cuda.synchronize()
    assert torch.equal(y.cpu(), _expected(a, b).expand(T, N))


def test_compose_rounds_to_nearest_even():
    say("rne compose")
    T, N = 64, 4096
    a, b = _pairs(T * N, seed=5)
    base = a.view(T, N).to(torch.bfloat16)
    b_bf = b.view(T, N).to(torch.bfloat16)
    # compose forms base + g s lora with one rounding: lora carries b (bf16
    # cases only: the split offsets need two terms)
    exact = (base.float() + b_bf.float())
    m = torch.rand(N) + 1.0
    y = D.dora_compose(base.cuda(), b_bf.cuda(), m.cuda(), m.cuda(), 1.0)
    torch.cuda.synchronize()
    assert torch.equal(y.cpu(), exact.to(torch.bfloat16))
