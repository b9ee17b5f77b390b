"""GPU parity: grouped launches over many modules.

dora_factored_norm_grouped against the oracle's dense row norms (every row)
and against the single-module dora_factored_norm, on a decoder layer's seven
projections at reduced widths, on 23 modules (two chunks of up to 16, mixed
ranks and ragged widths), on fp32 modules (module-by-module path), and at
the 8B-class decoder widths on sampled rows.  dora_forward_grouped on
sibling modules sharing one input against the oracle forward and the
single-module dora_forward, with cached norms for some modules."""
import numpy as np
import pytest
import torch

from dora_adapter_amd import dora as D
from dora_adapter_amd import synth
from gpu_util import check_close, check_norm, gpu, np64, say, sample_ids
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _gpu_mods(group):
    return [(gpu(g["W"]), gpu(g["A"]), gpu(g["B"]), gpu(g["m"]), g["s"]) for g in group]


def _check_norms(group, mods, ns, dtype, what):
    for k, g in enumerate(group):
        ref = O.norm(g["W"], g["A"], g["B"], g["s"])["n"]
        check_norm(ns[k], ref, dtype, f"{what} module {k} ({g['name']})")
        one = D.dora_factored_norm(*mods[k][:3], mods[k][4])
        torch.cuda.synchronize()
        rel = (np64(ns[k]) - np64(one)) / np64(one)
        assert np.abs(rel).max() <= 4e-6, f"{what} module {k}: grouped vs single {rel.max():.2e}"


def test_grouped_norm_decoder_layer():
    say("grouped norm, decoder layer 512/128/1792 r64")
    group = synth.make_group(synth.decoder_layer_shapes(512, 128, 1792), 64, seed=1)
    mods = _gpu_mods(group)
    ns = D.dora_factored_norm_grouped(mods)
    torch.cuda.synchronize()
    _check_norms(group, mods, ns, torch.bfloat16, "layer")


def test_grouped_norm_two_chunks_mixed():
    """23 modules: more than one chunk of 16, ranks 8..384, ragged widths."""
    say("grouped norm, 23 mixed modules")
    shapes = [(f"m{k}", 8 * (9 + 37 * k % 97), 8 * (16 + 53 * k % 61)) for k in range(23)]
    group = []
    for k, sh in enumerate(shapes):
        r = [8, 24, 64, 136, 384][k % 5]
        group += synth.make_group([sh], r, s=[1.0, 2.0, 0.5][k % 3], seed=100 + k)
    mods = _gpu_mods(group)
    ns = D.dora_factored_norm_grouped(mods)
    again = D.dora_factored_norm_grouped(mods)
    torch.cuda.synchronize()
    for a, b in zip(ns, again):
        assert torch.equal(a, b), "grouped norm not deterministic"
    _check_norms(group, mods, ns, torch.bfloat16, "mixed")


def test_grouped_norm_fp32_modules():
    say("grouped norm, fp32")
    group = synth.make_group([("a", 64, 128), ("b", 70, 100), ("c", 33, 64)], 5, dtype="f32",
                             s=2.0, seed=7)
    mods = _gpu_mods(group)
    ns = D.dora_factored_norm_grouped(mods)
    torch.cuda.synchronize()
    _check_norms(group, mods, ns, torch.float32, "fp32")


def test_grouped_norm_decoder_8b_sampled_rows():
    """Two decoder layers at 8B-class widths (14 modules, r = 384) in one
    chunk; sampled rows of each module against the oracle."""
    say("grouped norm, 8B-class decoder x2, r384")
    shapes = synth.decoder_layer_shapes() * 2
    group = synth.make_group(shapes, 384, seed=3)
    mods = _gpu_mods(group)
    ns = D.dora_factored_norm_grouped(mods)
    torch.cuda.synchronize()
    for k, g in enumerate(group):
        rows = sample_ids(20 + k, 8, g["W"].shape[0])
        ref = O.norm(g["W"], g["A"], g["B"], g["s"], rows=rows)["n"]
        check_norm(ns[k][torch.tensor(rows, device=ns[k].device)], ref, torch.bfloat16,
                   f"8B module {k} ({g['name']})")


def _siblings(seed, s_list, T, d_in=512, outs=(512, 128, 128), r=64):
    shapes = [(f"p{k}", d_out, d_in) for k, d_out in enumerate(outs)]
    group = []
    for k, sh in enumerate(shapes):
        group += synth.make_group([sh], r, s=s_list[k], seed=seed + k)
    x = synth.custom(8, d_in, 8, T, seed=seed + 99)["x"]
    return group, x


@pytest.mark.parametrize("T", [300, 1])
def test_grouped_forward_siblings(T):
    """Query/key/value-like siblings on one x (s = 1, 2, 0.5)."""
    say("grouped forward siblings", T)
    group, x = _siblings(40, [1.0, 2.0, 0.5], T)
    mods = _gpu_mods(group)
    xg = gpu(x)
    ys, ns, Ps = D.dora_forward_grouped(xg, mods)
    torch.cuda.synchronize()
    for k, g in enumerate(group):
        ref_y, ref_n = O.forward(x, g["W"], g["A"], g["B"], g["m"], g["s"])
        check_norm(ns[k], ref_n, torch.bfloat16, f"n {k}")
        check_close(ys[k], ref_y, torch.bfloat16, f"y {k}")
        y1, n1, P1 = D.dora_forward(xg, *mods[k][:4], g["s"])
        torch.cuda.synchronize()
        check_close(ys[k], np64(y1), torch.bfloat16, f"y {k} vs single")
        check_close(Ps[k], np64(P1), torch.bfloat16, f"P {k} vs single")


def test_grouped_forward_cached_norms_and_chunks():
    """18 siblings (two chunks), norms cached for every third module (one of
    them in place: n_in is n_out), P kept for none."""
    say("grouped forward, 18 siblings, cached norms")
    outs = tuple(8 * (8 + 5 * k) for k in range(18))
    group, x = _siblings(60, [1.0, 0.5, 2.0] * 6, 64, d_in=256, outs=outs, r=16)
    mods = _gpu_mods(group)
    xg = gpu(x)
    cached = [D.dora_factored_norm(*m[:3], m[4]) if k % 3 == 0 else None
              for k, m in enumerate(mods)]
    ns = [torch.empty(m[0].shape[0], dtype=torch.float32, device=xg.device) for m in mods]
    ns[3] = cached[3]  # in place
    ys, ns, _ = D.dora_forward_grouped(xg, mods, n_in=cached, want_P=False, ns=ns)
    torch.cuda.synchronize()
    for k, g in enumerate(group):
        if cached[k] is not None:
            assert torch.equal(ns[k], cached[k]), f"cached n {k} not passed through"
        ref_y, ref_n = O.forward(x, g["W"], g["A"], g["B"], g["m"], g["s"])
        check_norm(ns[k], ref_n, torch.bfloat16, f"n {k}")
        check_close(ys[k], ref_y, torch.bfloat16, f"y {k}")


def test_grouped_forward_empty_tokens():
    say("grouped forward T=0")
    group, x = _siblings(80, [1.0, 1.0, 1.0], 0)
    mods = _gpu_mods(group)
    ys, ns, Ps = D.dora_forward_grouped(gpu(x), mods)
    torch.cuda.synchronize()
    for k, g in enumerate(group):
        assert ys[k].shape == (0, g["W"].shape[0])
        check_norm(ns[k], O.norm(g["W"], g["A"], g["B"], g["s"])["n"], torch.bfloat16, f"n {k}")
