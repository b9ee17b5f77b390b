"""CPU tests of the C ABI: the library loads, exports every symbol that
include/dora.h declares, sizes its workspaces without any d_out*d_in term,
and rejects bad arguments on the host before anything is enqueued.

No call here reaches a kernel launch: every validation case breaks exactly
one rule, and the pointers are fake addresses that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

from dora_adapter_amd import dora as D

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dora.h")

OK, E_NULL, E_SHAPE, E_DTYPE, E_ALIGN, E_WS, E_ALIAS = 0, 1, 2, 3, 4, 5, 6
F32, BF16 = 0, 1
FAKE = 1 << 40  # a 256-byte aligned address that is never dereferenced


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dora_[a-z_]+)\s*\(", text)))


def test_header_matches_binding_exports():
    assert header_functions() == sorted(D.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = D.lib()
    for name in header_functions():
        assert hasattr(L, name), f"libdora.so does not export {name}"


def test_strerror_and_last_error():
    L = D.lib()
    for code in range(8):
        assert L.dora_strerror(code)
    assert L.dora_strerror(99) == b"unknown status"
    assert isinstance(L.dora_last_error(), bytes)


def test_workspace_has_no_dense_term():
    """No workspace grows with d_out*d_in.  The norm workspace is bounded by
    O(r^2) split partials of G plus O(d_out) per-row partials, whatever d_in
    is (a dense [d_out, d_in] bf16 buffer at d_in = 262144 would be 4 GiB);
    the forward workspace grows with T*d_out (activations), not with d_in."""
    L = D.lib()
    r = 384
    for d_out in (8192, 28672):
        bound = 33 * r * r * 4 + 2 * r * r * 2 + 256 * d_out * 4
        for d_in in (8192, 65536, 262144):
            ws = L.dora_norm_workspace(d_out, d_in, r, BF16)
            assert 0 < ws <= bound, (d_out, d_in, ws, bound)
            assert ws < d_out * d_in * 2 / 8
    f1 = L.dora_forward_workspace(2048, 8192, 8192, r, BF16)
    f2 = L.dora_forward_workspace(2048, 65536, 8192, r, BF16)
    f3 = L.dora_forward_workspace(4096, 8192, 8192, r, BF16)
    # d_in x8 only moves split-K counts (capped at 32) of the O(T*r + r^2) partials
    assert f2 - f1 <= 33 * (2048 * r + r * r) * 4
    # the forward keeps no [T, d_out] intermediate: base and adapter products
    # share one fp32 accumulator whose epilogue writes y
    for T in (2048, 4096, 8192):
        assert L.dora_forward_workspace(T, 8192, 28672, r, BF16) < T * 28672 * 2 / 2
    # per extra token: P, s P and at most 32 split partials of P, all O(r)
    assert f3 - f1 <= 2048 * (33 * r * 4 + 2 * r * 2) + 4096
    assert L.dora_backward_workspace(2048, 8192, 8192, r, BF16) > 0


def test_workspace_queries_reject_bad_shapes():
    L = D.lib()
    assert L.dora_norm_workspace(64, 100, 8, BF16) > 0       # bf16: any width too
    assert L.dora_forward_workspace(7, 1003, 1001, 37, BF16) > 0
    assert L.dora_norm_workspace(64, 128, 0, BF16) == 0      # r = 0
    assert L.dora_forward_workspace(-1, 128, 64, 8, F32) == 0
    assert L.dora_forward_workspace(16, 128, 64, 8, 7) == 0  # dtype
    assert L.dora_norm_workspace(64, 100, 8, F32) > 0        # fp32: any width


def test_library_source_never_allocates():
    """The library's only scratch is the caller's workspace."""
    csrc = os.path.join(ROOT, "dora_adapter_amd", "csrc")
    for f in os.listdir(csrc):
        text = open(os.path.join(csrc, f)).read()
        for bad in ("hipMalloc", "hipFree", "malloc(", "new ", "hipHostMalloc"):
            assert bad not in text, f"{f} calls {bad}"


def _p(addr):
    return ctypes.c_void_p(addr)


def compose(base=FAKE, lora=FAKE + (1 << 30), m=FAKE + (2 << 30), n=FAKE + (3 << 30), s=1.0,
            T=16, d_out=64, dt=BF16, y=FAKE + (4 << 30)):
    return D.lib().dora_compose(_p(base), _p(lora), _p(m), _p(n), s, T, d_out, dt, _p(y), None)


@pytest.mark.parametrize("kw,code", [
    ({"base": 0}, E_NULL), ({"y": 0}, E_NULL), ({"m": 0}, E_NULL),
    ({"dt": 5}, E_DTYPE), ({"d_out": -60}, E_SHAPE), ({"T": -3}, E_SHAPE),
    ({"lora": FAKE + 8}, E_ALIGN), ({"y": FAKE + 4}, E_ALIGN),
    ({"y": FAKE + 16}, E_ALIAS),                      # partial overlap with base
    ({"y": FAKE + (1 << 30) + 64}, E_ALIAS),         # overlaps lora
])
def test_compose_validation(kw, code):
    assert compose(**kw) == code
    assert D.lib().dora_last_error()


@pytest.mark.parametrize("dt", [F32, BF16])
def test_compose_any_width_passes_shape_check(dt):
    # any d_out is accepted (ragged rows take the element-by-element path);
    # break only the alignment so nothing launches.
    assert compose(d_out=60, dt=dt, m=FAKE + (2 << 30) + 4) == E_ALIGN


def _norm(W=FAKE, A=FAKE + (1 << 32), B=FAKE + (2 << 32), n=FAKE + (3 << 32), d_out=64,
          d_in=128, r=8, dt=BF16, ws=FAKE + (4 << 32), ws_bytes=None, base=0, U=0):
    L = D.lib()
    if ws_bytes is None:
        ws_bytes = max(L.dora_norm_workspace(d_out, d_in, r, BF16), 1)
    return L.dora_factored_norm(_p(W), _p(A), _p(B), 1.0, d_out, d_in, r, dt, _p(n), _p(base),
                                None, None, _p(U), _p(ws), ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    ({"W": 0}, E_NULL), ({"n": 0}, E_NULL), ({"dt": 2}, E_DTYPE), ({"r": 0}, E_SHAPE),
    ({"d_in": -100}, E_SHAPE), ({"d_out": 0}, E_SHAPE), ({"B": FAKE + (2 << 32) + 2}, E_ALIGN),
    ({"ws": 0}, E_WS), ({"ws_bytes": 16}, E_WS),
    ({"base": FAKE + (3 << 32) + 128}, E_ALIAS),       # base overlaps n
    ({"n": FAKE + 256}, E_ALIAS),                      # n inside W
    ({"U": FAKE + (2 << 32) + 64}, E_ALIAS),           # U_out inside B
    ({"U": FAKE + (5 << 32) + 4}, E_ALIGN),
])
def test_norm_validation(kw, code):
    assert _norm(**kw) == code


def _fwd(x=FAKE, W=FAKE + (1 << 32), A=FAKE + (2 << 32), B=FAKE + (3 << 32),
         m=FAKE + (4 << 32), T=16, d_in=128, d_out=64, r=8, dt=BF16, y=FAKE + (5 << 32),
         n_out=FAKE + (6 << 32), P=0, n_in=0, ws=FAKE + (7 << 32), ws_bytes=None, U=0):
    L = D.lib()
    if ws_bytes is None:
        ws_bytes = max(L.dora_forward_workspace(T, d_in, d_out, r, BF16), 1)
    return L.dora_forward(_p(x), _p(W), _p(A), _p(B), _p(m), 1.0, T, d_in, d_out, r, dt, _p(y),
                          _p(n_out), _p(P), _p(n_in), _p(U), _p(ws), ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    ({"x": 0}, E_NULL), ({"n_out": 0}, E_NULL), ({"dt": -1}, E_DTYPE), ({"r": -12}, E_SHAPE),
    ({"m": FAKE + (4 << 32) + 4}, E_ALIGN), ({"ws_bytes": 1}, E_WS),
    ({"y": FAKE + 1024}, E_ALIAS),                     # y inside x
    ({"P": FAKE + (5 << 32) + 512}, E_ALIAS),          # P_out inside y
    ({"ws": FAKE + (2 << 32)}, E_ALIAS),               # workspace over A
    ({"U": FAKE + (8 << 32), "n_in": FAKE + (9 << 32)}, E_NULL),  # U_out with a cached norm
    ({"U": FAKE + (5 << 32) + 256}, E_ALIAS),          # U_out inside y
])
def test_forward_validation(kw, code):
    assert _fwd(**kw) == code


@pytest.mark.parametrize("name", ["dora_backward", "dora_backward_through_norm"])
def test_backward_validation(name):
    L = D.lib()
    T, d_in, d_out, r = 16, 128, 64, 8
    need = getattr(L, name + "_workspace")(T, d_in, d_out, r, BF16)
    fn = getattr(L, name)
    base = [FAKE + (k << 32) for k in range(16)]

    def call(**kw):
        a = dict(dy=base[0], x=base[1], W=base[2], A=base[3], B=base[4], m=base[5], n=base[6],
                 P=base[7], y=base[8], dx=base[9], dA=base[10], dB=base[11], dm=base[12],
                 ws=base[13], ws_bytes=need, T=T)
        a.update(kw)
        extra = (_p(a.get("U", 0)),) if name.endswith("through_norm") else ()
        return fn(_p(a["dy"]), _p(a["x"]), _p(a["W"]), _p(a["A"]), _p(a["B"]), _p(a["m"]),
                  _p(a["n"]), 1.0, _p(a["P"]), _p(a["y"]), *extra, a["T"], d_in, d_out, r, BF16,
                  _p(a["dx"]), _p(a["dA"]), _p(a["dB"]), _p(a["dm"]), _p(a["ws"]), a["ws_bytes"],
                  None)

    assert call(dy=0) == E_NULL
    assert call(dm=0) == E_NULL
    assert call(dA=base[10] + 2) == E_ALIGN
    assert call(ws_bytes=need - 1) == E_WS
    assert call(dx=base[0]) == E_ALIAS                  # dx over dy
    assert call(dB=base[10] + 64) == E_ALIAS            # dB inside dA
    assert call(T=-1) == E_SHAPE
    assert call(ws=base[2] + 64) == E_ALIAS             # workspace inside W
    if name.endswith("through_norm"):
        assert call(U=base[10] + 256) == E_ALIAS        # U inside dA
        assert call(U=base[14] + 4) == E_ALIGN


def test_through_norm_workspace_has_no_dense_term():
    """The backward through the norm adds only [d_out, r] and [r, d_in] fp32
    slots and [r, r] Gram terms to the detached backward's workspace: no
    [d_out, d_in] buffer (V or B A is never formed)."""
    L = D.lib()
    r = 384
    for T, d_out, d_in in ((2048, 8192, 8192), (8192, 28672, 8192), (2048, 8192, 65536)):
        det = L.dora_backward_workspace(T, d_in, d_out, r, BF16)
        thru = L.dora_backward_through_norm_workspace(T, d_in, d_out, r, BF16)
        extra = thru - det
        assert 0 < extra <= 66 * (d_out * r + r * d_in) * 4 + 70 * r * r * 4 + d_out * (4 + 2 * r)
    # where a dense bf16 [d_out, d_in] buffer would be 1 GiB, the extra is a fraction of it
    assert (L.dora_backward_through_norm_workspace(2048, 65536, 8192, r, BF16) -
            L.dora_backward_workspace(2048, 65536, 8192, r, BF16)) < 8192 * 65536 * 2 / 2


def _merge(W=FAKE, A=FAKE + (1 << 32), B=FAKE + (2 << 32), m=FAKE + (3 << 32), n_in=0,
           out=FAKE + (4 << 32), d_out=64, d_in=128, r=8, dt=BF16, ws=FAKE + (5 << 32),
           ws_bytes=None):
    L = D.lib()
    if ws_bytes is None:
        ws_bytes = max(L.dora_merge_workspace(d_out, d_in, r, BF16), 1)
    return L.dora_merge(_p(W), _p(A), _p(B), _p(m), 1.0, d_out, d_in, r, dt, _p(n_in), _p(out),
                        _p(ws), ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    ({"W": 0}, E_NULL), ({"out": 0}, E_NULL), ({"m": 0}, E_NULL), ({"dt": 3}, E_DTYPE),
    ({"r": 0}, E_SHAPE), ({"d_in": 0}, E_SHAPE), ({"A": FAKE + (1 << 32) + 8}, E_ALIGN),
    ({"ws": 0}, E_WS), ({"ws_bytes": 8}, E_WS),
    ({"out": FAKE + 256}, E_ALIAS),                   # W_out partially overlaps W
    ({"out": FAKE + (2 << 32)}, E_ALIAS),             # W_out over B
    ({"ws": FAKE + 4096}, E_ALIAS),                   # workspace inside W
])
def test_merge_validation(kw, code):
    assert _merge(**kw) == code
    assert D.lib().dora_last_error()


def test_merge_workspace_has_no_dense_term():
    """The merge keeps no [d_out, d_in] buffer besides its output: its
    workspace is the norm's plus one fp32 vector of row norms."""
    L = D.lib()
    for d_out, d_in in ((8192, 8192), (28672, 8192), (8192, 262144)):
        ws = L.dora_merge_workspace(d_out, d_in, 384, BF16)
        assert 0 < ws <= L.dora_norm_workspace(d_out, d_in, 384, BF16) + d_out * 4 + 256


def _mods(shapes, base=FAKE):
    """Module descriptors with fake, disjoint, aligned addresses."""
    arr = (D.DoraModule * max(len(shapes), 1))()
    for k, (d_out, d_in, r) in enumerate(shapes):
        a = base + (k << 36)
        arr[k] = D.DoraModule(a, a + (1 << 34), a + (2 << 34), a + (3 << 34), 1.0, d_out, d_in, r)
    return arr


def _vp(addrs):
    arr = (ctypes.c_void_p * max(len(addrs), 1))(*addrs)
    return ctypes.cast(arr, ctypes.c_void_p), arr


def test_grouped_norm_validation():
    L = D.lib()
    shapes = [(64, 128, 8), (264, 520, 24), (128, 128, 16)]
    mods = _mods(shapes)
    need = L.dora_factored_norm_grouped_workspace(mods, 3, BF16)
    assert need > 0
    outs = [FAKE + (60 << 36) + (k << 20) for k in range(3)]
    n, keep = _vp(outs)
    ws = FAKE + (61 << 36)

    def call(m=mods, count=3, nn=n, w=ws, wb=need, dt=BF16):
        return L.dora_factored_norm_grouped(m, count, dt, nn, _p(w), wb, None)

    assert call(count=0) == OK                       # nothing to do, nothing launched
    assert call(count=-1) == E_SHAPE
    assert call(m=None) == E_NULL
    assert call(nn=None) == E_NULL
    assert call(wb=need - 1) == E_WS
    assert call(dt=5) == E_DTYPE
    bad = _mods([(64, 128, 8), (264, 520, 24), (128, 100, 0)])  # module 2: r = 0
    assert call(m=bad) == E_SHAPE
    assert b"module 2" in L.dora_last_error()
    same, keep2 = _vp([outs[0], outs[0] + 64, outs[2]])         # n[0] and n[1] overlap
    assert call(nn=same) == E_ALIAS
    into_w, keep3 = _vp([outs[0], FAKE + (1 << 36) + 256, outs[2]])  # n[1] inside W of module 1
    assert call(nn=into_w) == E_ALIAS
    assert call(w=FAKE + 4096) == E_ALIAS            # workspace inside module 0's W


def test_grouped_workspaces_have_no_dense_term():
    """The grouped norm keeps per-module O(d_out + r^2) partials only, and
    the chunks of 16 reuse one region: a model's worth of modules needs no
    more than one chunk's partials."""
    L = D.lib()
    r = 384
    layer = [(4096, 4096, r), (1024, 4096, r), (1024, 4096, r), (4096, 4096, r),
             (14336, 4096, r), (14336, 4096, r), (4096, 14336, r)]
    one = L.dora_factored_norm_grouped_workspace(_mods(layer), 7, BF16)
    many = L.dora_factored_norm_grouped_workspace(_mods(layer * 32), 224, BF16)
    bound = 16 * (33 * r * r * 4 + 2 * r * r * 2 + 33 * 2 * 14336 * 4) + 16 * 5 * 256
    assert 0 < one <= bound and 0 < many <= bound     # 224 modules reuse one chunk's region
    # no d_in term: the same modules with 16x wider inputs change split counts only
    wide = L.dora_factored_norm_grouped_workspace(
        _mods([(d_out, 16 * d_in, r) for d_out, d_in, _ in layer]), 7, BF16)
    assert wide <= 16 * (33 * r * r * 4 + 2 * r * r * 2 + 33 * 2 * 14336 * 4) + 16 * 5 * 256


def test_grouped_forward_validation():
    L = D.lib()
    T, d_in = 16, 128
    shapes = [(64, d_in, 8), (128, d_in, 16)]
    mods = _mods(shapes)
    need = L.dora_forward_grouped_workspace(mods, 2, T, BF16, None, None)
    assert need > 0
    x = FAKE + (50 << 36)
    ys, k1 = _vp([FAKE + (51 << 36), FAKE + (51 << 36) + (1 << 24)])
    ns, k2 = _vp([FAKE + (52 << 36), FAKE + (52 << 36) + (1 << 20)])
    ws = FAKE + (53 << 36)

    def call(m=mods, count=2, xx=x, dinn=d_in, y=ys, n=ns, P=None, nin=None, wb=need, TT=T):
        return L.dora_forward_grouped(_p(xx), TT, dinn, m, count, BF16, y, n, P, nin, _p(ws), wb,
                                      None)

    assert call(count=0) == OK
    assert call(dinn=256) == E_SHAPE                 # modules' d_in differ from x's
    assert b"module 0" in L.dora_last_error()
    assert call(xx=0) == E_NULL
    assert call(y=None) == E_NULL
    assert call(wb=need - 1) == E_WS
    assert call(TT=-2) == E_SHAPE
    clash, k3 = _vp([FAKE + (51 << 36), FAKE + (51 << 36) + 64])  # y[0] and y[1] overlap
    assert call(y=clash) == E_ALIAS
    over_x, k4 = _vp([x, FAKE + (51 << 36) + (1 << 24)])       # y[0] over x
    assert call(y=over_x) == E_ALIAS
    # a cached norm changes the workspace (that module's norm partials are not needed)
    cached, k5 = _vp([FAKE + (54 << 36), 0])
    assert L.dora_forward_grouped_workspace(mods, 2, T, BF16, cached, None) <= need
