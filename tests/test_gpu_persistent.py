"""GPU: the persistent 256 x 256 product (one workgroup per CU walking its
tiles as one stream of K stages, the epilogue staged per wave) against the
one-tile-per-workgroup launch of the same tile configuration, bit for bit
(the same MFMA sums in the same order, one rounding), and against the
oracle, on shapes that reach its edge cases: fewer tiles than XCDs, a tile
count that is not a multiple of 8 (workgroups with different tile counts),
ragged M and N (masked stores), a K tail, an odd number of K stages (the
stage slots alternate differently from one tile to the next), two K
segments, the column scale of the fused forward, the MN-major second
operand of dx, and many tiles per workgroup at the training shape."""
import pytest
import torch

from dora_adapter_amd import dora as D
from dora_adapter_amd import synth
from gpu_util import check_close, check_norm, gpu, np64, say
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _kernels(fn):
    """Names of the kernels fn launches (profiler device trace)."""
    from torch.profiler import ProfilerActivity, profile
    fn()
    torch.cuda.synchronize()
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        fn()
        torch.cuda.synchronize()
    return [e.name for e in prof.events() if e.device_type.name == "CUDA"]


def _both(fn, monkeypatch):
    """fn() with the persistent kernel allowed, then with it turned off."""
    monkeypatch.setenv("DORA_TILE_CFG", "4")
    monkeypatch.delenv("DORA_PERSISTENT", raising=False)
    a = fn()
    torch.cuda.synchronize()
    used = any("persistent" in k for k in _kernels(fn))
    monkeypatch.setenv("DORA_PERSISTENT", "0")
    b = fn()
    torch.cuda.synchronize()
    assert not any("persistent" in k for k in _kernels(fn))
    return a, b, used


@pytest.mark.parametrize("T,d_in,d_out,persistent", [
    (200, 960, 512, True),      # 2 tiles (fewer than the 8 XCDs), K tail
    (2000, 520, 3000, True),    # 96 tiles, M and N ragged, K tail
    (1030, 136, 2056, True),    # 3 K stages: slot parity alternates per tile
    (4096, 72, 8192, True),     # 2 K stages (the least), 2 tiles per workgroup
    (300, 64, 512, False),      # one K stage: the one-tile launch serves it
])
def test_linear_persistent_is_the_tiled_product(T, d_in, d_out, persistent, monkeypatch):
    say("persistent linear", T, d_in, d_out)
    g = torch.Generator().manual_seed(T + d_in)
    x = torch.randn(T, d_in, generator=g).bfloat16()
    W = (torch.randn(d_out, d_in, generator=g) * d_in ** -0.5).bfloat16()
    xg, Wg = x.cuda(), W.cuda()
    a, b, used = _both(lambda: D.dora_linear(xg, Wg), monkeypatch)
    assert used == persistent
    assert torch.equal(a, b)
    check_close(a, np64(x) @ np64(W).T, torch.bfloat16, f"x W^T {T}x{d_in}x{d_out}")


@pytest.mark.parametrize("T,d_out,d_in,r,s", [
    (300, 264, 520, 24, 1.0),      # 4 tiles, both K segments ragged; dx too
    (777, 1000, 896, 40, 2.0),     # 16 tiles, N ragged, scale s != 1
    (2100, 4096, 136, 72, 0.5),    # 5 K stages over two segments (odd)
    (1500, 600, 1024, 16, 0.75),   # dx: 24 tiles over K = 600 + 16
])
def test_forward_and_backward_persistent(T, d_out, d_in, r, s, monkeypatch):
    say("persistent forward/backward", T, d_out, d_in, r)
    mod = synth.custom(d_out, d_in, r, T, "bf16", s, sigma_B=0.02, seed=T, with_dy=True)
    t = {k: gpu(mod[k]) for k in ("x", "W", "A", "B", "m", "dy")}

    def step():
        y, n, P = D.dora_forward(t["x"], t["W"], t["A"], t["B"], t["m"], s)
        gr = D.dora_backward(t["dy"], t["x"], t["W"], t["A"], t["B"], t["m"], n, s, P, y)
        return [y, n, P, gr["dx"], gr["dA"], gr["dB"], gr["dm"]]

    a, b, used = _both(step, monkeypatch)
    assert used
    for name, u, v in zip(("y", "n", "P", "dx", "dA", "dB", "dm"), a, b):
        assert torch.equal(u, v), name
    ref_y, ref_n = O.forward(mod["x"], mod["W"], mod["A"], mod["B"], mod["m"], s)
    check_norm(a[1], ref_n, torch.bfloat16)
    check_close(a[0], ref_y, torch.bfloat16, f"y {T}x{d_out}")


def test_training_shape_persistent_matches_tiled(monkeypatch):
    """8192 tokens, 8192 -> 28672, r 384: 14 tiles per workgroup, the fused
    forward product and dx both persistent."""
    say("persistent training shape")
    mod = synth.make_module(synth.TRAIN_R384, seed=1, with_dy=True)
    t = {k: gpu(mod[k]) for k in ("x", "W", "A", "B", "m", "dy")}
    s = mod["s"]
    del mod

    def step():
        y, n, P = D.dora_forward(t["x"], t["W"], t["A"], t["B"], t["m"], s)
        gr = D.dora_backward(t["dy"], t["x"], t["W"], t["A"], t["B"], t["m"], n, s, P, y)
        return [y, gr["dx"]]

    monkeypatch.delenv("DORA_TILE_CFG", raising=False)
    monkeypatch.delenv("DORA_PERSISTENT", raising=False)
    a = step()
    names = _kernels(step)
    assert sum("persistent" in k for k in names) == 2
    monkeypatch.setenv("DORA_PERSISTENT", "0")
    b = step()
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]), "y"
    assert torch.equal(a[1], b[1]), "dx"
