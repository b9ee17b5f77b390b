"""GPU parity of every bf16 tile configuration through every call.

The planners pick one tile shape per product by a time model, so a shape
that no default plan reaches at the tested sizes would go unchecked.
DORA_TILE_CFG=<index> restricts the planners to one configuration wherever
it can serve the product (others fall back to the model's pick); each
configuration here runs the forward (with the norm's U kept), the detached
backward, the backward through the norm (reusing U), the merge, the grouped
forward of sibling modules and the grouped norm, against the oracle.  The
shapes have ragged M, N and K tails and include one with a long K on the
token side and one with a long K on the input side, where the planners split
K and the partial-sum path runs."""
import os

import pytest
import torch

from dora_adapter_amd import dora as D
from dora_adapter_amd import synth
from gpu_util import check_close, check_norm, gpu, np64, say
from oracle import oracle as O

pytestmark = pytest.mark.gpu

N_CFGS = 10  # register-staged 0-3, direct-to-LDS 4-9

SHAPES = [
    # T, d_out, d_in, r, s
    (200, 1000, 1024, 40, 2.0),
    (64, 520, 4008, 40, 0.5),    # long K over d_in: x A^T, W A^T split
    (2056, 264, 520, 24, 1.0),   # long K over tokens: dh^T P, Q^T x split
]

_refs = {}


def _reference(shape):
    """Oracle results for one shape, computed once for all configurations."""
    if shape not in _refs:
        T, d_out, d_in, r, s = shape
        mod = synth.custom(d_out, d_in, r, T, "bf16", s, sigma_B=0.02, seed=T + d_out,
                           with_dy=True)
        args = (mod["x"], mod["W"], mod["A"], mod["B"], mod["m"])
        n = O.norm(mod["W"], mod["A"], mod["B"], s)["n"]
        ref = {"mod": mod, "n": n, "y": O.forward(*args, s)[0],
               "det": O.backward_full(mod["dy"], *args, n, s),
               "thru": O.backward_through_norm(mod["dy"], *args, s),
               "merge": O.merge(mod["W"], mod["A"], mod["B"], mod["m"], s),
               # the definitions of the kept V A^T and of P
               "U": (np64(mod["W"]) + s * np64(mod["B"]) @ np64(mod["A"])) @ np64(mod["A"]).T,
               "P": np64(mod["x"]) @ np64(mod["A"]).T}
        # a sibling module: B halved (exact in bf16)
        ref["B2"] = (mod["B"].float() * 0.5).to(torch.bfloat16)
        ref["y2"], ref["n2"] = O.forward(mod["x"], mod["W"], mod["A"], ref["B2"], mod["m"], s)
        _refs[shape] = ref
    return _refs[shape]


@pytest.fixture
def tile_cfg(request):
    prev = os.environ.get("DORA_TILE_CFG")
    os.environ["DORA_TILE_CFG"] = str(request.param)
    yield request.param
    if prev is None:
        del os.environ["DORA_TILE_CFG"]
    else:
        os.environ["DORA_TILE_CFG"] = prev


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s[:4])))
@pytest.mark.parametrize("tile_cfg", range(N_CFGS), indirect=True)
def test_every_call_on_tile_config(tile_cfg, shape):
    T, d_out, d_in, r, s = shape
    say("tile config", tile_cfg, "shape", shape)
    ref = _reference(shape)
    mod = ref["mod"]
    t = {k: gpu(mod[k]) for k in ("x", "W", "A", "B", "m", "dy")}
    bf = torch.bfloat16
    tag = f"cfg {tile_cfg} {T}x{d_out}x{d_in} r{r}"

    U = torch.empty(d_out, r, dtype=torch.float32, device=t["x"].device)
    y, n, P = D.dora_forward(t["x"], t["W"], t["A"], t["B"], t["m"], s, U_out=U)
    torch.cuda.synchronize()
    check_norm(n, ref["n"], bf, f"n {tag}")
    check_close(y, ref["y"], bf, f"y {tag}")
    check_close(U, ref["U"], torch.float32, f"V A^T {tag}", tol=1e-4)

    det = D.dora_backward(t["dy"], t["x"], t["W"], t["A"], t["B"], t["m"], n, s, P, y)
    thru = D.dora_backward(t["dy"], t["x"], t["W"], t["A"], t["B"], t["m"], n, s, P, y,
                           through_norm=True, U=U)
    torch.cuda.synchronize()
    for k in ("dx", "dA", "dB", "dm"):
        check_close(det[k], ref["det"][k], bf, f"{k} detached {tag}")
        check_close(thru[k], ref["thru"][k], bf, f"{k} through norm {tag}")

    Wm = D.dora_merge(t["W"], t["A"], t["B"], t["m"], s)
    torch.cuda.synchronize()
    check_close(Wm, ref["merge"], bf, f"merge {tag}")

    # two sibling modules on the same x: grouped forward and grouped norm
    mods = [(t["W"], t["A"], t["B"], t["m"], s), (t["W"], t["A"], gpu(ref["B2"]), t["m"], s)]
    ys, ns, Ps = D.dora_forward_grouped(t["x"], mods)
    ng = D.dora_factored_norm_grouped(mods)
    torch.cuda.synchronize()
    for k, (yr, nr) in enumerate(((ref["y"], ref["n"]), (ref["y2"], ref["n2"]))):
        check_close(ys[k], yr, bf, f"grouped y{k} {tag}")
        check_norm(ns[k], nr, bf, f"grouped n{k} {tag}")
        check_norm(ng[k], nr, bf, f"grouped norm {k} {tag}")
    check_close(P, ref["P"], bf, f"P {tag}")
    check_close(Ps[0], ref["P"], bf, f"grouped P {tag}")
