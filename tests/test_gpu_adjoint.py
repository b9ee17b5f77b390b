"""GPU: the backward is the adjoint of the forward (norm held constant).

With n given (dora_forward's n_in), the forward is linear in x, in m, in A
for fixed B and in B for fixed A (DoRA summary, Method: y = (m / n)(x (W +
s B A)^T)), so for random directions v

    <dy, J_x v>  = <dx, v>      J_x v   = forward(x := v)
    <dy, J_A vA> = <dA, vA>     J_A vA  = forward(W := 0, A := vA)
    <dy, J_B vB> = <dB, vB>     J_B vB  = forward(W := 0, B := vB)
    <dy, J_m vm> = <dm, vm>     J_m vm  = forward(m := vm)

each side formed from the library's own outputs (promoted to fp64).  No
oracle is involved: this pins the backward against the forward through an
identity that holds for any correct pair, in both element types.  The
directions are taken along the gradients, so that a mistake in either
changes the two sides by the order of the terms."""
import numpy as np
import pytest
import torch

from dora_adapter_amd import dora as D
from dora_adapter_amd import synth
from gpu_util import gpu, say

pytestmark = pytest.mark.gpu


def _dot(a, b):
    return float(np.sum(a.double().cpu().numpy() * b.double().cpu().numpy()))


def _norm(a):
    return float(np.linalg.norm(a.double().cpu().numpy()))


@pytest.mark.parametrize("dtype,T,d_out,d_in,r,s,tol", [
    ("bf16", 300, 264, 520, 24, 1.5, 1e-2),
    ("bf16", 1030, 1000, 2056, 64, 0.5, 1e-2),
    ("f32", 33, 70, 100, 5, 1.25, 1e-5),
])
def test_backward_is_the_adjoint_of_the_forward(dtype, T, d_out, d_in, r, s, tol):
    say("adjoint", dtype, T, d_out, d_in, r)
    mod = synth.custom(d_out, d_in, r, T, dtype, s, sigma_B=0.05, seed=T + r, with_dy=True)
    t = {k: gpu(mod[k]) for k in ("x", "W", "A", "B", "m", "dy")}
    x, W, A, B, m, dy = (t[k] for k in ("x", "W", "A", "B", "m", "dy"))
    n = D.dora_factored_norm(W, A, B, s)
    y, _, P = D.dora_forward(x, W, A, B, m, s, n_in=n)
    g = D.dora_backward(dy, x, W, A, B, m, n, s, P, y)
    torch.cuda.synchronize()

    # directions along the gradients (plus noise), so that both inner products
    # are of the order of the norms: a wrong sign, factor or operand then
    # moves them by that order, far beyond the rounding allowance below
    gen = torch.Generator().manual_seed(7 + T)

    def along(grad):
        gc = grad.float().cpu()
        rms = float(gc.pow(2).mean().sqrt())
        v = gc + 0.1 * rms * torch.randn(gc.shape, generator=gen)
        return v.to(grad.dtype).to(grad.device)

    vx, vA, vB, vm = along(g["dx"]), along(g["dA"]), along(g["dB"]), along(g["dm"])
    zero_W = torch.zeros_like(W)

    cases = [
        ("x", D.dora_forward(vx, W, A, B, m, s, n_in=n)[0], g["dx"], vx),
        ("A", D.dora_forward(x, zero_W, vA, B, m, s, n_in=n)[0], g["dA"], vA),
        ("B", D.dora_forward(x, zero_W, A, vB, m, s, n_in=n)[0], g["dB"], vB),
        ("m", D.dora_forward(x, W, A, B, vm, s, n_in=n)[0], g["dm"], vm),
    ]
    torch.cuda.synchronize()
    for name, Jv, grad, v in cases:
        lhs, rhs = _dot(dy, Jv), _dot(grad, v)
        # both sides are inner products of rounded tensors: compare against the
        # scale of the terms, not of the (possibly cancelling) sums.  Each side
        # carries a few roundings to the element type (the output, P or dh, Q),
        # each within u |term| (u = 2^-8 for bf16), so a few u of the
        # Cauchy-Schwarz scale bounds the difference; a wrong sign, factor or
        # operand is off by the scale itself
        scale = max(_norm(dy) * _norm(Jv), _norm(grad) * _norm(v))
        say(f"  {name}: <dy, Jv> {lhs:.6g}, <grad, v> {rhs:.6g}, |diff| / scale "
            f"{abs(lhs - rhs) / scale:.2e}")
        assert abs(lhs - rhs) <= tol * scale, (name, lhs, rhs, scale)
