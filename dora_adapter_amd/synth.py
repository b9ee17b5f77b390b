"""Seeded synthetic DoRA modules.

This module only draws random inputs; it holds none of the DoRA arithmetic
(no norm of W + sBA, no composition, no gradient).  The GPU tests, the smoke
check and the benchmark use it, and so do the oracle's tests, so both sides
see identical inputs.

Recipe (one ``torch.Generator('cpu')`` per module, seed 0 unless a test says
otherwise; draw order W, A, B, m-noise, x, dy; fp32 normals are scaled and
then rounded to the compute dtype with round-to-nearest-even):

* W ~ N(0, 1/d_in) and A ~ N(0, 1/d_in): 1/d_in is a variance
  (std = d_in**-0.5), the usual Linear init that keeps x W^T at unit scale.
* B ~ N(0, sigma_B) with sigma_B a standard deviation (0.01 or 0.02).
* m_i = ||W_i|| * (1 + sigma_m * z_i), z ~ N(0, 1), sigma_m = 0.01, with
  ||W_i|| taken in fp64 over the already-rounded W and m stored as fp32.  This
  is the magnitude initialisation from the pretrained row norm that the DoRA
  summary pages describe ("Method"), jittered so that m / ||W + sBA|| sits in
  the near-unity regime the Scaling-DoRA abstract names.
* x ~ N(0, 1), dy ~ N(0, 1).
"""
from dataclasses import dataclass, field

import torch

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class ModuleShape:
    name: str
    d_out: int
    d_in: int
    r: int
    T: int
    dtype: str = "bf16"
    s: float = 1.0
    sigma_B: float = 0.02
    sigma_m: float = 0.01
    backward: bool = False
    notes: str = field(default="", compare=False)


# The workloads: a tiny fp32 module, two square bf16 modules, an MLP up/down
# pair and a training-shaped module, with the sizes the Scaling-DoRA abstract
# works at (d_in = 8192, r = 384, bf16) and typical MLP widths.
TINY_F32 = ModuleShape("tiny_f32_64x128_r8_t16", 64, 128, 8, 16, "f32", 2.0, 0.01, 0.01)
SQUARE_R64 = ModuleShape("square_4096_r64_t4096", 4096, 4096, 64, 4096, "bf16", 128 / 64, 0.01)
SQUARE_R384 = ModuleShape("square_8192_r384_t8192", 8192, 8192, 384, 8192, "bf16", 1.0, 0.02)
MLP_UP = ModuleShape("mlp_up_5120to27648_r384_t16384", 27648, 5120, 384, 16384, "bf16", 1.0, 0.02)
MLP_DOWN = ModuleShape("mlp_down_27648to5120_r384_t16384", 5120, 27648, 384, 16384, "bf16", 1.0, 0.02)
TRAIN_R384 = ModuleShape("train_8192to28672_r384_t8192", 28672, 8192, 384, 8192, "bf16", 1.0,
                         0.02, 0.01, backward=True)


def _normal(gen, shape, std, dtype):
    return (torch.randn(*shape, generator=gen, dtype=torch.float32, device=gen.device) *
            std).to(dtype)


def draw_weights(gen, d_out, d_in, r, dtype, sigma_B, sigma_m):
    """W, A, B and m for one module, drawn in that order from ``gen``."""
    W = _normal(gen, (d_out, d_in), d_in ** -0.5, dtype)
    A = _normal(gen, (r, d_in), d_in ** -0.5, dtype)
    B = _normal(gen, (d_out, r), sigma_B, dtype)
    z = torch.randn(d_out, generator=gen, dtype=torch.float32, device=gen.device).double()
    row = torch.linalg.vector_norm(W.double(), dim=1)
    m = (row * (1.0 + sigma_m * z)).float()
    return W, A, B, m


def make_module(shape: ModuleShape, seed: int = 0, T: int = None, with_dy: bool = None):
    """Draw one module's tensors on the CPU.

    Returns a dict with W, A, B, m, x (and dy when ``with_dy``), s (Python
    float), dtype (torch dtype) and the shape.  ``T`` overrides the token count.
    """
    dt = _DT[shape.dtype]
    T = shape.T if T is None else T
    with_dy = shape.backward if with_dy is None else with_dy
    gen = torch.Generator("cpu").manual_seed(seed)
    W, A, B, m = draw_weights(gen, shape.d_out, shape.d_in, shape.r, dt,
                              shape.sigma_B, shape.sigma_m)
    x = _normal(gen, (T, shape.d_in), 1.0, dt)
    out = {"W": W, "A": A, "B": B, "m": m, "x": x, "s": float(shape.s), "dtype": dt,
           "shape": shape, "T": T}
    if with_dy:
        out["dy"] = _normal(gen, (T, shape.d_out), 1.0, dt)
    return out


def make_mlp_pair(up: ModuleShape = MLP_UP, down: ModuleShape = MLP_DOWN, seed: int = 0,
                  T: int = None):
    """Up then down module from one generator (up's tensors, down's, then x)."""
    dt = _DT[up.dtype]
    T = up.T if T is None else T
    gen = torch.Generator("cpu").manual_seed(seed)
    wu = draw_weights(gen, up.d_out, up.d_in, up.r, dt, up.sigma_B, up.sigma_m)
    wd = draw_weights(gen, down.d_out, down.d_in, down.r, dt, down.sigma_B, down.sigma_m)
    x = _normal(gen, (T, up.d_in), 1.0, dt)
    mk = lambda w, sh: {"W": w[0], "A": w[1], "B": w[2], "m": w[3], "s": float(sh.s),
                        "dtype": dt, "shape": sh}
    return mk(wu, up), mk(wd, down), x


def custom(d_out, d_in, r, T, dtype="bf16", s=1.0, sigma_B=0.02, sigma_m=0.01, seed=0,
           with_dy=False):
    """A module of arbitrary shape with the same recipe."""
    sh = ModuleShape(f"custom_{d_out}x{d_in}_r{r}_t{T}_{dtype}", d_out, d_in, r, T, dtype, s,
                     sigma_B, sigma_m, backward=with_dy)
    return make_module(sh, seed=seed)


def sample_indices(seed, n, *bounds):
    """n seeded index tuples, uniform in [0, b) per bound, always including
    the first and the last index of every dimension (tile edges and tails)."""
    gen = torch.Generator("cpu").manual_seed(10_000 + seed)
    cols = [torch.randint(0, b, (n,), generator=gen) for b in bounds]
    out = torch.stack(cols, dim=1)
    edges = torch.tensor([[0] * len(bounds), [b - 1 for b in bounds]])
    return torch.cat([edges, out], dim=0).tolist()


# The seven adapted projections of one decoder layer as (name, d_out, d_in):
# query, key, value, output, gate, up, down.  Default widths are those of an
# 8B-class decoder with grouped-query attention (hidden 4096, key/value 1024,
# MLP 14336), the scale of the smallest models the Scaling-DoRA abstract
# measures.
def decoder_layer_shapes(hidden=4096, kv=1024, inter=14336):
    return [("q", hidden, hidden), ("k", kv, hidden), ("v", kv, hidden), ("o", hidden, hidden),
            ("gate", inter, hidden), ("up", inter, hidden), ("down", hidden, inter)]


def make_group(shapes, r, dtype="bf16", s=1.0, sigma_B=0.02, sigma_m=0.01, seed=0,
               device="cpu"):
    """Modules of the given (name, d_out, d_in) shapes from one generator on
    `device`, in list order; each a dict with W, A, B, m, s, name."""
    dt = _DT[dtype]
    gen = torch.Generator(device).manual_seed(seed)
    out = []
    for name, d_out, d_in in shapes:
        W, A, B, m = draw_weights(gen, d_out, d_in, r, dt, sigma_B, sigma_m)
        out.append({"W": W, "A": A, "B": B, "m": m, "s": float(s), "name": name})
    return out
