"""CPU test: plausible mistakes planted in a copy of the oracle must each trip
at least one pin.  This shows the pins would catch a dropped term, a wrong
sign, a transposed operand or a misplaced factor anywhere in the oracle.

Each mutant is a textual edit of oracle/dora_oracle.c, compiled with gcc into
a temporary directory; the committed oracle is never modified.
"""
import os
import tempfile

import pytest

import oracle_pins as P
from oracle import build as OB
from oracle import oracle as O

MUTANTS = {
    "lora_sign": ("v[j] = elem(W, dt, i * d_in + j) + s * ba[j];",
                  "v[j] = elem(W, dt, i * d_in + j) - s * ba[j];"),
    "lora_no_scale": ("v[j] = elem(W, dt, i * d_in + j) + s * ba[j];",
                      "v[j] = elem(W, dt, i * d_in + j) + ba[j];"),
    "A_transposed": ("ba[j] += b * elem(A, dt, k * d_in + j);",
                     "ba[j] += b * elem(A, dt, (j % r) * d_in + k);"),
    "norm_no_sqrt": ("n = sqrt(vv);", "n = vv;"),
    "g_inverted": ("double g = m[i] / n;", "double g = n / m[i];"),
    "cross_term_wrong": ("wb += w * ba[j];", "wb += w * v[j];"),
    "gram_term_wrong": ("bb += ba[j] * ba[j];", "bb += ba[j] * v[j];"),
    "compose_g_on_base_only": ("y[t * d_out + i] = (m[i] / n[i]) * (b + s * l);",
                               "y[t * d_out + i] = (m[i] / n[i]) * b + s * l;"),
    "dm_over_m": ("dm[i] = acc / n[i];", "dm[i] = acc / m[i];"),
    "dh_no_norm": ("dh[t * d_out + i] = elem(dy, dt, t * d_out + i) * (m[i] / n[i]);",
                   "dh[t * d_out + i] = elem(dy, dt, t * d_out + i) * m[i];"),
    "dx_base_only": ("acc += dh[t * d_out + i] * V[i * d_in + j];",
                     "acc += dh[t * d_out + i] * elem(W, dt, i * d_in + j);"),
    "dB_no_scale": ("dB[i * r + k] = s * acc;", "dB[i * r + k] = acc;"),
    "dA_double_scale": ("dA[k * d_in + j] = s * acc;", "dA[k * d_in + j] = s * s * acc;"),
    "P_wrong_operand": ("p += elem(x, dt, t * d_in + j) * elem(A, dt, k * d_in + j);",
                        "p += elem(x, dt, t * d_in + j) * elem(W, dt, k * d_in + j);"),
    "sampled_dx_no_g": ("acc += elem(dy, dt, t * d_out + i) * (m[i] / n[i]) * vij;",
                        "acc += elem(dy, dt, t * d_out + i) * vij;"),
    "sampled_dm_over_m": ("dm[q] = acc / n[i];", "dm[q] = acc / m[i];"),
    "merge_g_inverted": ("Wm[q * d_in + j] = (m[i] / ni) * v[j];",
                         "Wm[q * d_in + j] = (ni / m[i]) * v[j];"),
    "merge_base_only": ("Wm[q * d_in + j] = (m[i] / ni) * v[j];",
                        "Wm[q * d_in + j] = (m[i] / ni) * elem(W, dt, i * d_in + j);"),
    "merge_norm_squared": ("ni = sqrt(ni);", "ni = ni;"),
    "thru_cn_sign": ("dV[i * d_in + j] = acc - cn[i] * V[i * d_in + j];",
                     "dV[i * d_in + j] = acc + cn[i] * V[i * d_in + j];"),
    "thru_cn_power": ("cn[i] = m[i] / (nn[i] * nn[i] * nn[i]) * dyh;",
                      "cn[i] = m[i] / (nn[i] * nn[i]) * dyh;"),
    "thru_dB_no_scale": ("dB[i * r + k] = acc * s;", "dB[i * r + k] = acc;"),
    "thru_dA_double_scale": ("dA[k * d_in + j] = acc * s;", "dA[k * d_in + j] = acc * s * s;"),
    "thru_dA_uses_W": ("acc += elem(B, dt, i * r + k) * dV[i * d_in + j];",
                       "acc += elem(B, dt, i * r + k) * elem(W, dt, i * d_in + j);"),
}


def _run_pins():
    tripped = []
    for pin in P.ALL_PINS:
        try:
            pin()
        except AssertionError:
            tripped.append(pin.__name__)
    return tripped


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    old, new = MUTANTS[name]
    src = open(OB.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/present"
    with tempfile.TemporaryDirectory() as td:
        path = os.path.join(td, "mutant.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        lib = OB.build(src=path, out=os.path.join(td, f"lib_{name}.so"))
        prev = O.set_library(lib)
        try:
            tripped = _run_pins()
        finally:
            O.restore_library(prev)
    assert tripped, f"no pin catches the planted mistake {name}"
