"""GPU parity: dora_factored_norm vs the oracle's dense row norms of
W + s*B*A (and the base / cross / Gram terms), on shapes spanning several
tiles with ragged tails, at the full module shapes on sampled rows, on rows
near cancellation, and for the B = 0 invariant and determinism."""
import numpy as np
import pytest
import torch

from dora_adapter_amd import dora as D
from dora_adapter_amd import synth
from gpu_util import check_norm, gpu, np64, say, sample_ids
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _terms_ok(out, ref, s, dtype, what):
    n, base, cross, gram = (np64(t) for t in out)
    check_norm(n, ref["n"], dtype, what)
    scale = ref["n"] ** 2 + ref["base"]
    tol = 1e-6 if dtype == torch.float32 else 2e-4
    for name, got in (("base", base), ("cross", cross), ("gram", gram)):
        err = np.abs(got - ref[name]) / scale
        assert err.max() <= tol, f"{what} {name}: max err {err.max():.2e} of n^2 scale"


@pytest.mark.parametrize("d_out,d_in,r,dtype,s", [
    (64, 128, 8, torch.float32, 2.0),       # the tiny fp32 module
    (70, 100, 5, torch.float32, 0.75),      # fp32, no multiple-of-8 widths
    (264, 520, 24, torch.bfloat16, 1.0),
    (600, 1032, 40, torch.bfloat16, 2.0),
    (1000, 2048, 384, torch.bfloat16, 1.0),  # full rank-384 tile set, ragged d_out
    (520, 4096, 64, torch.bfloat16, 2.0),
    # small ranks on the 128 x 128 row-dot tiles, split over K with G's split
    # tiles in U's launch: a full tile width, a ragged one, a ragged d_out
    (2048, 3072, 128, torch.bfloat16, 1.0),
    (1288, 2056, 96, torch.bfloat16, 0.5),
])
def test_norm_matches_oracle(d_out, d_in, r, dtype, s):
    say("norm", d_out, d_in, r, dtype)
    mod = synth.custom(d_out, d_in, r, 1, "f32" if dtype == torch.float32 else "bf16", s,
                       sigma_B=0.05, seed=d_out)
    W, A, B = mod["W"], mod["A"], mod["B"]
    out = D.dora_factored_norm(gpu(W), gpu(A), gpu(B), s, terms=True)
    torch.cuda.synchronize()
    _terms_ok(out, O.norm(W, A, B, s), s, dtype, f"norm {d_out}x{d_in} r{r}")


@pytest.mark.parametrize("shape", [synth.SQUARE_R64, synth.SQUARE_R384, synth.TRAIN_R384,
                                   synth.MLP_UP, synth.MLP_DOWN], ids=lambda s: s.name)
def test_norm_full_size_sampled_rows(shape):
    say("norm full size", shape.name)
    mod = synth.make_module(shape, seed=0, T=1, with_dy=False)
    W, A, B, s = mod["W"], mod["A"], mod["B"], mod["s"]
    n = D.dora_factored_norm(gpu(W), gpu(A), gpu(B), s)
    torch.cuda.synchronize()
    rows = sample_ids(1, 48, shape.d_out)
    ref = O.norm(W, A, B, s, rows=rows)
    check_norm(np64(n)[rows], ref["n"], torch.bfloat16, f"{shape.name} sampled rows")


@pytest.mark.parametrize("d_out,d_in,r", [
    (12000, 2056, 384),   # whole-rank row-block tiles: ragged last block, K tail of 8
    (40000, 1032, 200),   # rank below the tile width (ragged columns), K tail of 8
    (5120, 27648, 384),   # few row blocks, long K: split over K
])
def test_norm_row_block_tiles(d_out, d_in, r):
    """Shapes large enough that the planner takes the 128 x 384 row-block
    tiles of the W A^T product (row sums and row dots formed from registers),
    with ragged rows, columns and K, and split K; rows sampled, the last tile
    included; a second call must agree bit for bit."""
    say("norm row-block tiles", d_out, d_in, r)
    mod = synth.custom(d_out, d_in, r, 1, "bf16", 1.0, sigma_B=0.05, seed=r)
    W, A, B = gpu(mod["W"]), gpu(mod["A"]), gpu(mod["B"])
    out = D.dora_factored_norm(W, A, B, 1.0, terms=True)
    again = D.dora_factored_norm(W, A, B, 1.0, terms=True)
    torch.cuda.synchronize()
    for a, b in zip(out, again):
        assert torch.equal(a, b), "factored norm not deterministic"
    W, A, B = mod["W"], mod["A"], mod["B"]
    rows = sorted(set(sample_ids(3, 40, d_out) + list(range(d_out - 130, d_out))))
    ref = O.norm(W, A, B, 1.0, rows=rows)
    got = {k: np64(v)[rows] for k, v in zip(("n", "base", "cross", "gram"), out)}
    check_norm(got["n"], ref["n"], torch.bfloat16, f"norm {d_out}x{d_in} r{r}")
    scale = ref["n"] ** 2 + ref["base"]
    for name in ("base", "cross", "gram"):
        err = np.abs(got[name] - ref[name]) / scale
        assert err.max() <= 2e-4, f"{name}: max err {err.max():.2e} of n^2 scale"


def test_norm_near_cancellation():
    """Rows with W_i close to -s B_i A: ||W_i + s B_i A|| is 0.1 or 0.01 of
    ||W_i||.  The factored sum subtracts nearly equal terms there; the error
    is reported separately from the ordinary tolerance."""
    say("norm near cancellation")
    d_out, d_in, r, s = 256, 1024, 64, 1.0
    mod = synth.custom(d_out, d_in, r, 1, "bf16", s, sigma_B=0.3, seed=9)
    W, A, B = mod["W"].clone(), mod["A"], mod["B"]
    ba = (B.double() @ A.double())
    g = torch.Generator().manual_seed(4)
    for i, frac in ((3, 0.1), (17, 0.1), (100, 0.01), (200, 0.01)):
        target = -s * ba[i]
        noise = torch.randn(d_in, generator=g).double()
        noise *= frac * target.norm() / noise.norm()
        W[i] = (target + noise).bfloat16()
    out = D.dora_factored_norm(gpu(W), gpu(A), gpu(B), s, terms=True)
    torch.cuda.synchronize()
    ref = O.norm(W, A, B, s)
    n = np64(out[0])
    rel = np.abs(n - ref["n"]) / ref["n"]
    ordinary = [i for i in range(d_out) if i not in (3, 17, 100, 200)]
    assert rel[ordinary].max() <= 1e-3
    assert rel[[3, 17]].max() <= 1e-3, f"n/||W|| = 0.1 rows: {rel[[3, 17]]}"
    assert rel[[100, 200]].max() <= 3e-2, f"n/||W|| = 0.01 rows: {rel[[100, 200]]}"
    print("near-cancellation rel err:", {i: float(rel[i]) for i in (3, 17, 100, 200)})


def test_norm_b_zero_and_determinism():
    say("norm B=0 / determinism")
    mod = synth.custom(512, 1024, 64, 1, "bf16", 1.0, seed=12)
    W, A, B = gpu(mod["W"]), gpu(mod["A"]), gpu(mod["B"])
    n0, base0, cross0, gram0 = D.dora_factored_norm(W, A, torch.zeros_like(B), 1.0, terms=True)
    n1 = D.dora_factored_norm(W, A, B, 1.0)
    n2 = D.dora_factored_norm(W, A, B, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(n1, n2), "factored norm is not bitwise deterministic"
    assert torch.all(cross0 == 0) and torch.all(gram0 == 0)
    assert torch.allclose(n0.double(), torch.sqrt(base0.double()), rtol=1e-7, atol=0)
    ref = np.linalg.norm(mod["W"].double().numpy(), axis=1)
    check_norm(n0, ref, torch.bfloat16, "B=0 norm")
