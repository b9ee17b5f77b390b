"""Pins that tie the fp64 oracle to facts outside itself.

Each pin returns None when it holds and raises AssertionError otherwise, so
the same checks serve as individual tests (tests/test_oracle.py) and as the
battery that every planted mistake in a copy of the oracle must trip
(tests/test_oracle_mutants.py).

What pins what:
* the hand-worked module in tests/golden/hand_module.txt (values derived by
  hand from the definitions: norm, its three terms, y and every gradient);
* the factored identity ||W_i + sB_iA||^2 = base + 2s*cross + s^2*gram, with
  the right-hand side computed along an independent route (numpy U = W A^T
  and G = A A^T), as the Scaling-DoRA abstract states the decomposition;
* special cases with closed forms: B = 0 or s = 0 is the textbook row norm,
  W = 0 with r = 1 is |s B_i| * ||A||, and an exactly orthogonal adapter gives
  ||W_i||^2 + s^2 ||B_i||^2;
* invariants of y = (m/n)(x V^T): B = 0 with m = n returns x W^T bit for bit,
  power-of-two scaling of W and B leaves y unchanged bit for bit, and y is
  linear in m and in x;
* the backward against torch autograd (a library differentiator, fp64, n
  detached) and against central finite differences of the oracle forward
  with n frozen (exact up to rounding, since L is linear in each input).
"""
import ast
import math
import os

import numpy as np
import torch

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------- fixtures
def _eval(expr):
    """Evaluate a fixture expression: numbers, + - * /, unary -, sqrt(), lists."""
    def ev(node):
        if isinstance(node, ast.Expression):
            return ev(node.body)
        if isinstance(node, ast.Constant) and isinstance(node.value, (int, float)):
            return float(node.value)
        if isinstance(node, ast.List):
            return [ev(e) for e in node.elts]
        if isinstance(node, ast.UnaryOp) and isinstance(node.op, ast.USub):
            return -ev(node.operand)
        if isinstance(node, ast.BinOp):
            a, b = ev(node.left), ev(node.right)
            ops = {ast.Add: lambda: a + b, ast.Sub: lambda: a - b,
                   ast.Mult: lambda: a * b, ast.Div: lambda: a / b}
            return ops[type(node.op)]()
        if (isinstance(node, ast.Call) and isinstance(node.func, ast.Name)
                and node.func.id == "sqrt" and len(node.args) == 1):
            return math.sqrt(ev(node.args[0]))
        raise ValueError(f"fixture: unsupported expression {ast.dump(node)}")
    return ev(ast.parse(expr, mode="eval"))


def load_golden(name="hand_module.txt"):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, expr = line.split("=", 1)
            vals[key.strip()] = np.asarray(_eval(expr.strip()), dtype=np.float64)
    return vals


def _close(a, b, rtol, atol=0.0, what=""):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.abs(a - b)
    lim = atol + rtol * np.abs(b)
    assert np.all(err <= lim), f"{what}: max err {err.max():.3e} (rtol {rtol})"


def _t32(a):
    return torch.tensor(np.asarray(a, np.float64), dtype=torch.float32)


def _rand_module(seed, d_out, d_in, r, T, dtype=torch.float32, sb=0.3):
    g = torch.Generator().manual_seed(seed)
    W = (torch.randn(d_out, d_in, generator=g) * d_in ** -0.5).to(dtype)
    A = (torch.randn(r, d_in, generator=g) * d_in ** -0.5).to(dtype)
    B = (torch.randn(d_out, r, generator=g) * sb).to(dtype)
    m = (torch.rand(d_out, generator=g) + 0.5).float()
    x = torch.randn(T, d_in, generator=g).to(dtype)
    dy = torch.randn(T, d_out, generator=g).to(dtype)
    return W, A, B, m, x, dy


def _np64(t):
    return t.double().numpy()


# ------------------------------------------------------------------- pins
def pin_hand_norm():
    g = load_golden()
    W, A, B = _t32(g["W"]), _t32(g["A"]), _t32(g["B"])
    for s, key in ((2.0, "s2"), (0.5, "s05")):
        out = O.norm(W, A, B, s)
        for term in ("n", "base", "cross", "gram"):
            _close(out[term], g[f"{key}.{term}"], 1e-15, 1e-15, f"hand {key}.{term}")


def pin_hand_forward():
    g = load_golden()
    W, A, B, x = _t32(g["W"]), _t32(g["A"]), _t32(g["B"]), _t32(g["x"])
    for s, key in ((2.0, "s2"), (0.5, "s05")):
        y, n = O.forward(x, W, A, B, g["m"], s)
        _close(n, g[f"{key}.n"], 1e-15, 0, f"hand {key}.n (forward)")
        _close(y, g[f"{key}.y"], 1e-14, 1e-14, f"hand {key}.y")


def pin_hand_backward():
    g = load_golden()
    W, A, B, x, dy = (_t32(g[k]) for k in ("W", "A", "B", "x", "dy"))
    full = O.backward_full(dy, x, W, A, B, g["m"], g["s2.n"], 2.0)
    for k in ("dx", "dA", "dB", "dm"):
        _close(full[k], g[f"s2.{k}"], 1e-14, 1e-14, f"hand full {k}")
    T, d_in, d_out, r = 2, 3, 2, 1
    smp = O.backward_sampled(
        dy, x, W, A, B, g["m"], g["s2.n"], 2.0,
        dx_idx=[(t, j) for t in range(T) for j in range(d_in)],
        dA_idx=[(k, j) for k in range(r) for j in range(d_in)],
        dB_idx=[(i, k) for i in range(d_out) for k in range(r)],
        dm_idx=list(range(d_out)))
    _close(smp["dx"], g["s2.dx"].reshape(-1), 1e-14, 1e-14, "hand sampled dx")
    _close(smp["dA"], g["s2.dA"].reshape(-1), 1e-14, 1e-14, "hand sampled dA")
    _close(smp["dB"], g["s2.dB"].reshape(-1), 1e-14, 1e-14, "hand sampled dB")
    _close(smp["dm"], g["s2.dm"], 1e-14, 1e-14, "hand sampled dm")


def pin_factored_identity():
    """Dense oracle norm vs base + 2s*cross + s^2*gram along another route."""
    for dtype in (torch.float32, torch.bfloat16):
        for s in (0.75, 2.0):
            W, A, B, *_ = _rand_module(3, 37, 53, 5, 1, dtype)
            w, a, b = _np64(W), _np64(A), _np64(B)
            U = w @ a.T                # [d_out, r]
            G = a @ a.T                # [r, r]
            base = (w * w).sum(1)
            cross = (b * U).sum(1)
            gram = ((b @ G) * b).sum(1)
            out = O.norm(W, A, B, s)
            _close(out["n"] ** 2, base + 2 * s * cross + s * s * gram, 1e-12, 0, "identity n^2")
            _close(out["base"], base, 1e-13, 0, "identity base")
            _close(out["cross"], cross, 1e-12, 1e-15, "identity cross")
            _close(out["gram"], gram, 1e-12, 0, "identity gram")
            rows = [36, 0, 17]
            sub = O.norm(W, A, B, s, rows=rows)
            _close(sub["n"], out["n"][rows], 0, 0, "row subset")


def pin_textbook_b0():
    W, A, B, *_ = _rand_module(4, 29, 41, 6, 1)
    ref = np.linalg.norm(_np64(W), axis=1)
    _close(O.norm(W, A, torch.zeros_like(B), 1.5)["n"], ref, 1e-14, 0, "B=0")
    _close(O.norm(W, A, B, 0.0)["n"], ref, 1e-14, 0, "s=0")


def pin_rank1():
    g = torch.Generator().manual_seed(5)
    A = torch.randn(1, 23, generator=g)
    B = torch.randn(11, 1, generator=g)
    s = 1.25
    ref = np.abs(s * _np64(B)[:, 0]) * np.linalg.norm(_np64(A))
    _close(O.norm(torch.zeros(11, 23), A, B, s)["n"], ref, 1e-14, 0, "rank-1")


def pin_orthogonal():
    """A = selected rows of the identity (A A^T = I exactly) and W zero on
    those columns (W A^T = 0 exactly): n_i^2 = ||W_i||^2 + s^2 ||B_i||^2."""
    g = torch.Generator().manual_seed(6)
    d_out, d_in, r, s = 13, 19, 4, 0.625
    cols = torch.randperm(d_in, generator=g)[:r]
    A = torch.zeros(r, d_in)
    A[torch.arange(r), cols] = 1.0
    W = torch.randn(d_out, d_in, generator=g)
    W[:, cols] = 0.0
    B = torch.randn(d_out, r, generator=g)
    ref = np.sqrt((_np64(W) ** 2).sum(1) + s * s * (_np64(B) ** 2).sum(1))
    _close(O.norm(W, A, B, s)["n"], ref, 1e-14, 0, "orthogonal")


def pin_forward_b0_exact():
    """B = 0 with m = n gives g = 1 exactly and y = x W^T bit for bit
    (small integers, so x W^T is exact in fp64)."""
    g = torch.Generator().manual_seed(7)
    W = torch.randint(-4, 5, (9, 14), generator=g).float()
    A = torch.randint(-4, 5, (3, 14), generator=g).float()
    x = torch.randint(-4, 5, (6, 14), generator=g).float()
    B = torch.zeros(9, 3)
    n = O.norm(W, A, B, 1.0)["n"]
    y, _ = O.forward(x, W, A, B, n, 1.0)
    assert np.array_equal(y, _np64(x) @ _np64(W).T), "B=0, m=n: y != x W^T"


def pin_forward_lora_reduction():
    """m = n gives plain LoRA: y = x W^T + s (x A^T) B^T."""
    W, A, B, m, x, _ = _rand_module(8, 21, 30, 4, 7)
    s = 1.5
    n = O.norm(W, A, B, s)["n"]
    y, _ = O.forward(x, W, A, B, n, s)
    xx, w, a, b = _np64(x), _np64(W), _np64(A), _np64(B)
    _close(y, xx @ w.T + s * (xx @ a.T) @ b.T, 1e-12, 1e-13, "LoRA reduction")


def pin_forward_scale_invariance():
    """y(2^k W, 2^k B) == y(W, B) bit for bit (direction is scale-free)."""
    W, A, B, m, x, _ = _rand_module(9, 17, 24, 3, 5)
    y0, n0 = O.forward(x, W, A, B, m, 0.75)
    y1, n1 = O.forward(x, W * 8, A, B * 8, m, 0.75)
    assert np.array_equal(y0, y1), "scale invariance (bitwise)"
    assert np.array_equal(n1, 8 * n0), "norm scales with W and B"


def pin_forward_linearity():
    W, A, B, m, x, _ = _rand_module(10, 15, 22, 3, 6)
    y0, _ = O.forward(x, W, A, B, m, 1.0)
    y2, _ = O.forward(x, W, A, B, 2 * m, 1.0)
    assert np.array_equal(y2, 2 * y0), "linearity in m"
    g = torch.Generator().manual_seed(11)
    # integer-valued tokens so that x1 + x2 is exact in fp32
    x = torch.randint(-8, 9, x.shape, generator=g).float()
    x2 = torch.randint(-8, 9, x.shape, generator=g).float()
    y0, _ = O.forward(x, W, A, B, m, 1.0)
    ya, _ = O.forward(x2, W, A, B, m, 1.0)
    yb, _ = O.forward(x + x2, W, A, B, m, 1.0)
    _close(yb, y0 + ya, 1e-12, 1e-12, "linearity in x")


def pin_forward_subsets():
    W, A, B, m, x, _ = _rand_module(12, 19, 26, 4, 9)
    yf, nf = O.forward(x, W, A, B, m, 1.25)
    toks, rows = [8, 0, 3], [18, 5, 0, 7]
    ys, ns = O.forward(x, W, A, B, m, 1.25, toks=toks, rows=rows)
    assert np.array_equal(ys, yf[np.ix_(toks, rows)]), "forward subsets"
    assert np.array_equal(ns, nf[rows])


def _autograd(W, A, B, m, x, dy, s, detach=True):
    w, a, b = (t.double().clone().requires_grad_(True) for t in (W, A, B))
    mm = m.double().clone().requires_grad_(True)
    xx = x.double().clone().requires_grad_(True)
    V = w + s * (b @ a)
    n = torch.linalg.vector_norm(V, dim=1)
    if detach:
        n = n.detach()
    y = (mm / n)[None, :] * (xx @ V.T)
    (y * dy.double()).sum().backward()
    return {"dx": xx.grad.numpy(), "dA": a.grad.numpy(), "dB": b.grad.numpy(),
            "dm": mm.grad.numpy(), "n": torch.linalg.vector_norm(V, dim=1).detach().numpy()}


def pin_backward_autograd():
    """Oracle gradients vs torch autograd (fp64 CPU) with the norm detached;
    dx and dm must also equal the gradients without the detach."""
    for dtype in (torch.float32, torch.bfloat16):
        W, A, B, m, x, dy = _rand_module(13, 23, 31, 5, 11, dtype)
        s = 1.75
        ref = _autograd(W, A, B, m, x, dy, s, detach=True)
        full = O.backward_full(dy, x, W, A, B, m, ref["n"], s)
        for k in ("dx", "dA", "dB", "dm"):
            _close(full[k], ref[k], 1e-11, 1e-13, f"autograd {k}")
        nd = _autograd(W, A, B, m, x, dy, s, detach=False)
        _close(full["dx"], nd["dx"], 1e-11, 1e-13, "dx without detach")
        _close(full["dm"], nd["dm"], 1e-11, 1e-13, "dm without detach")
        ix = {"dx_idx": [(0, 0), (10, 30), (4, 7)], "dA_idx": [(0, 0), (4, 30), (2, 9)],
              "dB_idx": [(0, 0), (22, 4), (9, 1)], "dm_idx": [0, 22, 13]}
        smp = O.backward_sampled(dy, x, W, A, B, m, ref["n"], s, **ix)
        _close(smp["dx"], [full["dx"][t, j] for t, j in ix["dx_idx"]], 1e-12, 1e-14, "smp dx")
        _close(smp["dA"], [full["dA"][k, j] for k, j in ix["dA_idx"]], 1e-12, 1e-14, "smp dA")
        _close(smp["dB"], [full["dB"][i, k] for i, k in ix["dB_idx"]], 1e-12, 1e-14, "smp dB")
        _close(smp["dm"], [full["dm"][i] for i in ix["dm_idx"]], 1e-12, 1e-14, "smp dm")


def pin_backward_finite_differences():
    """Central differences of L = sum(dy * y) through oracle.forward with n
    frozen.  L is linear in each of x, A, B and m, so the difference quotient
    equals the derivative up to rounding."""
    W, A, B, m, x, dy = _rand_module(14, 9, 12, 3, 5)
    s = 1.25
    n = O.norm(W, A, B, s)["n"]
    full = O.backward_full(dy, x, W, A, B, m, n, s)
    dyy = _np64(dy)

    def L(x_, A_, B_, m_):
        y, _ = O.forward(x_, W, A_, B_, m_, s, n_in=n)
        return float((y * dyy).sum())

    h = 2.0 ** -6
    for (name, idx) in (("dx", (2, 5)), ("dA", (1, 7)), ("dB", (4, 2)), ("dm", (6,))):
        base = [x, A, B, m]
        pos = ["dx", "dA", "dB", "dm"].index(name)
        plus, minus = [t.clone() for t in base], [t.clone() for t in base]
        plus[pos][idx] += h
        minus[pos][idx] -= h
        # the fp32 perturbation may round: divide by the step actually taken
        step = float(plus[pos][idx]) - float(minus[pos][idx])
        fd = (L(*plus) - L(*minus)) / step
        _close([fd], [full[name][idx]], 1e-9, 1e-12, f"finite difference {name}")


def pin_compose_reductions():
    """compose with m = n is base + s*lora exactly; with exact integer base
    and lora it reproduces the forward's y."""
    g = torch.Generator().manual_seed(15)
    base = torch.randn(5, 12, generator=g).bfloat16()
    lora = torch.randn(5, 12, generator=g).bfloat16()
    n = np.linspace(0.5, 2.0, 12)
    y = O.compose(base, lora, n, n, 2.0)
    assert np.array_equal(y, _np64(base) + 2.0 * _np64(lora)), "compose m=n"
    # integer module: base = x W^T and lora = (x A^T) B^T are exact in fp32
    W = torch.randint(-3, 4, (12, 10), generator=g).float()
    A = torch.randint(-3, 4, (2, 10), generator=g).float()
    B = torch.randint(-3, 4, (12, 2), generator=g).float()
    x = torch.randint(-3, 4, (5, 10), generator=g).float()
    m = torch.rand(12, generator=g).float() + 0.5
    s = 0.5
    yf, nf = O.forward(x, W, A, B, m, s)
    bse = torch.tensor(_np64(x) @ _np64(W).T, dtype=torch.float32)
    lra = torch.tensor((_np64(x) @ _np64(A).T) @ _np64(B).T, dtype=torch.float32)
    yc = O.compose(bse, lra, m, nf, s)
    _close(yc, yf, 1e-15, 1e-15, "compose vs forward")


def pin_hand_merge():
    g = load_golden()
    W, A, B = _t32(g["W"]), _t32(g["A"]), _t32(g["B"])
    for s, key in ((2.0, "s2"), (0.5, "s05")):
        _close(O.merge(W, A, B, g["m"], s), g[f"{key}.merge"], 1e-15, 1e-15, f"hand {key}.merge")


def pin_merge_properties():
    """The merged rows have norm m_i and the direction of V_i = W_i + s B_i A
    (V along numpy's route); x W'^T reproduces the oracle forward; rows and
    a given n select and fix as in the forward."""
    for dtype in (torch.float32, torch.bfloat16):
        W, A, B, m, x, _ = _rand_module(16, 19, 27, 4, 6, dtype)
        s = 1.25
        Wm = O.merge(W, A, B, m, s)
        _close(np.linalg.norm(Wm, axis=1), _np64(m), 1e-14, 0, "merged row norms = m")
        V = _np64(W) + s * _np64(B) @ _np64(A)
        unit = V / np.linalg.norm(V, axis=1, keepdims=True)
        _close(Wm / np.linalg.norm(Wm, axis=1, keepdims=True), unit, 1e-13, 1e-15,
               "merged direction")
        y, _ = O.forward(x, W, A, B, m, s)
        _close(_np64(x) @ Wm.T, y, 1e-12, 1e-13, "x W'^T = forward")
        rows = [18, 0, 7]
        assert np.array_equal(O.merge(W, A, B, m, s, rows=rows), Wm[rows]), "merge rows"
        n = O.norm(W, A, B, s)["n"]
        assert np.array_equal(O.merge(W, A, B, m, s, n_in=2 * n), Wm / 2), "merge with n_in"


def pin_hand_backward_through_norm():
    g = load_golden()
    W, A, B, x, dy = (_t32(g[k]) for k in ("W", "A", "B", "x", "dy"))
    out = O.backward_through_norm(dy, x, W, A, B, g["m"], 2.0)
    _close(out["dA"], g["s2.thru.dA"], 1e-14, 1e-14, "hand through-norm dA")
    _close(out["dB"], g["s2.thru.dB"], 1e-14, 1e-14, "hand through-norm dB")
    _close(out["dx"], g["s2.dx"], 1e-14, 1e-14, "hand through-norm dx")
    _close(out["dm"], g["s2.dm"], 1e-14, 1e-14, "hand through-norm dm")


def pin_backward_through_norm_autograd():
    """Through-norm gradients vs torch autograd (fp64 CPU) without detach."""
    for dtype in (torch.float32, torch.bfloat16):
        W, A, B, m, x, dy = _rand_module(17, 21, 29, 5, 9, dtype)
        s = 1.5
        ref = _autograd(W, A, B, m, x, dy, s, detach=False)
        out = O.backward_through_norm(dy, x, W, A, B, m, s)
        for k in ("dx", "dA", "dB", "dm"):
            _close(out[k], ref[k], 1e-11, 1e-13, f"through-norm autograd {k}")


def pin_backward_through_norm_finite_differences():
    """Central differences of L = sum(dy * y) through oracle.forward with n
    recomputed from the perturbed A or B (L is no longer linear in them, so
    the quotient matches the derivative to O(h^2))."""
    W, A, B, m, x, dy = _rand_module(18, 8, 11, 3, 4)
    s = 0.75
    out = O.backward_through_norm(dy, x, W, A, B, m, s)
    dyy = _np64(dy)

    def L(A_, B_):
        y, _ = O.forward(x, W, A_, B_, m, s)
        return float((y * dyy).sum())

    h = 2.0 ** -12
    for name, idx in (("dA", (1, 6)), ("dA", (2, 0)), ("dB", (5, 1)), ("dB", (0, 2))):
        pos = 0 if name == "dA" else 1
        plus, minus = [A.clone(), B.clone()], [A.clone(), B.clone()]
        plus[pos][idx] += h
        minus[pos][idx] -= h
        step = float(plus[pos][idx]) - float(minus[pos][idx])
        fd = (L(*plus) - L(*minus)) / step
        _close([fd], [out[name][idx]], 1e-6, 1e-10, f"through-norm finite difference {name}")


ALL_PINS = [pin_hand_norm, pin_hand_forward, pin_hand_backward, pin_factored_identity,
            pin_textbook_b0, pin_rank1, pin_orthogonal, pin_forward_b0_exact,
            pin_forward_lora_reduction, pin_forward_scale_invariance, pin_forward_linearity,
            pin_forward_subsets, pin_backward_autograd, pin_backward_finite_differences,
            pin_compose_reductions, pin_hand_merge, pin_merge_properties,
            pin_hand_backward_through_norm, pin_backward_through_norm_autograd,
            pin_backward_through_norm_finite_differences]
