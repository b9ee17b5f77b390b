"""dora_forward_noalloc: dora_forward on the library's fixed device scratch
(for callers that cannot allocate).  Through the C ABI: two calls in a row,
the second on a smaller module, each compared with dora_forward on the same
inputs (the same plan and kernels, so bit for bit) and with the oracle; the
size limit is enforced on the host before the device is touched."""
import pytest
import torch

from dora_adapter_amd import dora as D
from dora_adapter_amd import synth
from gpu_util import check_close, check_norm, gpu, np64, say
from oracle import oracle as O

BF16 = D.DORA_BF16


def test_oversized_module_is_rejected_on_the_host():
    L = D.lib()
    T, d_in, d_out, r = 1 << 20, 8192, 28672, 384
    assert L.dora_forward_workspace(T, d_in, d_out, r, BF16) > (96 << 20)
    fake = 1 << 40
    rc = L.dora_forward_noalloc(fake, fake + (1 << 36), fake + (2 << 36), fake + (3 << 36),
                                fake + (4 << 36), 1.0, T, d_in, d_out, r, BF16,
                                fake + (5 << 36), fake + (6 << 36), None, None, None, None)
    assert rc == 5, D.STATUS.get(rc)  # DORA_E_WORKSPACE
    assert b"scratch" in L.dora_last_error()


def test_invalid_arguments_are_reported_as_by_dora_forward():
    L = D.lib()
    fake = 1 << 40
    rc = L.dora_forward_noalloc(fake, fake, fake, fake, fake, 1.0, 16, 128, 64, 8, 7,
                                fake, fake, None, None, None, None)
    assert rc == 3  # DORA_E_DTYPE
    rc = L.dora_forward_noalloc(fake, fake, fake, fake, fake, 1.0, 16, 0, 64, 8, BF16,
                                fake, fake, None, None, None, None)
    assert rc == 2  # DORA_E_SHAPE


@pytest.mark.gpu
def test_noalloc_matches_dora_forward_on_two_calls():
    cases = [(2048, 3000, 1024, 64, 0.5, 41),   # the larger module first
             (129, 520, 264, 24, 1.0, 42)]      # then a smaller one on the same scratch
    for T, d_out, d_in, r, s, seed in cases:
        say("forward noalloc", T, d_out, d_in, r, s)
        mod = synth.custom(d_out, d_in, r, T, "bf16", s, sigma_B=0.02, seed=seed)
        t = {k: gpu(mod[k]) for k in ("x", "W", "A", "B", "m")}
        y0, n0, P0 = D.dora_forward(t["x"], t["W"], t["A"], t["B"], t["m"], s)
        y1, n1, P1 = D.dora_forward_noalloc(t["x"], t["W"], t["A"], t["B"], t["m"], s)
        torch.cuda.synchronize()
        assert D.lib().dora_last_error() == b""
        assert torch.equal(n0, n1), "n differs from dora_forward"
        assert torch.equal(P0, P1), "P differs from dora_forward"
        assert torch.equal(y0, y1), f"{int((y0 != y1).sum())} elements of y differ"
        ref_y, ref_n = O.forward(mod["x"], mod["W"], mod["A"], mod["B"], mod["m"], s)
        check_norm(n1, ref_n, torch.bfloat16, "noalloc n")
        check_close(y1, ref_y, torch.bfloat16, "noalloc y")
        check_close(P1, np64(mod["x"]) @ np64(mod["A"]).T, torch.bfloat16, "noalloc P")
        # the cached-norm form on the same scratch
        y2, _, _ = D.dora_forward_noalloc(t["x"], t["W"], t["A"], t["B"], t["m"], s, n_in=n1)
        torch.cuda.synchronize()
        assert torch.equal(y0, y2), "cached-norm y differs"
