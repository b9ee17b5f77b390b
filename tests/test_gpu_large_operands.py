"""GPU parity at the size limit of the pipelined GEMM's 32-bit offsets.

An activation x of 135168 tokens x 8192 (2.06 GiB of bf16) is past the
2 GiB - 4 KiB operand range of the direct-to-LDS kernel, so every product
that reads x (x A^T, the fused [x | sP][W | B]^T, dA = Q^T x) takes the
register-staged kernel, while the others keep the pipelined one.  Forward
and norm-detached backward are checked on sampled entries against the
oracle; x and dy come from a seeded generator on the device (drawing 1.1e9
normals on the host would take longer than the check)."""
import numpy as np
import pytest
import torch

from dora_adapter_amd import dora as D
from dora_adapter_amd import synth
from gpu_util import check_close, check_norm, gpu, say, sample_ids, sample_pairs
from oracle import oracle as O

pytestmark = pytest.mark.gpu

T, D_IN, D_OUT, R, S = 135168, 8192, 256, 16, 2.0


def test_forward_backward_past_2gib_operand():
    assert T * D_IN * 2 > (1 << 31)
    say("forward/backward with a 2.06 GiB activation", T, D_IN, D_OUT, R)
    mod = synth.custom(D_OUT, D_IN, R, 0, "bf16", S, sigma_B=0.02, seed=77)
    gen = torch.Generator("cuda").manual_seed(78)
    x = torch.randn(T, D_IN, generator=gen, device="cuda").bfloat16()
    dy = torch.randn(T, D_OUT, generator=gen, device="cuda").bfloat16()
    W, A, B, m = (gpu(mod[k]) for k in ("W", "A", "B", "m"))
    y, n, P = D.dora_forward(x, W, A, B, m, S)
    g = D.dora_backward(dy, x, W, A, B, m, n, S, P, y)
    torch.cuda.synchronize()
    n_ref = O.norm(mod["W"], mod["A"], mod["B"], S)["n"]
    check_norm(n, n_ref, torch.bfloat16, "n")
    toks = sample_ids(1, 24, T) + [0, T - 1]
    rows = sample_ids(2, 32, D_OUT)
    ti, ri = torch.tensor(toks, device="cuda"), torch.tensor(rows, device="cuda")
    x_s = x[ti].cpu()
    ref_y, _ = O.forward(x_s, mod["W"], mod["A"], mod["B"], mod["m"], S, rows=rows)
    check_close(y[ti][:, ri], ref_y, torch.bfloat16, "y sampled")
    del y, P
    # gradients on sampled entries (dA and dB sum over all tokens)
    xc, dyc = x.cpu(), dy.cpu()
    ix = {"dx_idx": sample_pairs(3, 16, T, D_IN), "dA_idx": sample_pairs(4, 12, R, D_IN),
          "dB_idx": sample_pairs(5, 12, D_OUT, R), "dm_idx": sample_ids(6, 12, D_OUT)}
    ref = O.backward_sampled(dyc, xc, mod["W"], mod["A"], mod["B"], mod["m"], n_ref, S, **ix)
    got = {"dx": [g["dx"][t, j].item() for t, j in ix["dx_idx"]],
           "dA": [g["dA"][k, j].item() for k, j in ix["dA_idx"]],
           "dB": [g["dB"][i, k].item() for i, k in ix["dB_idx"]],
           "dm": [g["dm"][i].item() for i in ix["dm_idx"]]}
    for k in got:
        check_close(np.asarray(got[k]), ref[k], torch.bfloat16, f"{k} sampled")
