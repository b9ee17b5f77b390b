"""Thin ctypes binding of libdora.so (include/dora.h), same names as the C ABI.

Argument marshalling only: tensors are passed as device pointers, outputs and
the workspace are allocated with torch (device memory plumbing), and every
step of the computation runs in the library's HIP kernels.  There is no CPU
or PyTorch fallback: if the library is missing or cannot be loaded, every
call raises.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdora.so")

DORA_F32, DORA_BF16 = 0, 1
STATUS = {0: "DORA_OK", 1: "DORA_E_NULL", 2: "DORA_E_SHAPE", 3: "DORA_E_DTYPE",
          4: "DORA_E_ALIGN", 5: "DORA_E_WORKSPACE", 6: "DORA_E_ALIAS", 7: "DORA_E_HIP"}

# Every symbol include/dora.h declares.
EXPORTS = ("dora_strerror", "dora_last_error", "dora_norm_workspace", "dora_forward_workspace",
           "dora_backward_workspace", "dora_factored_norm", "dora_compose", "dora_forward",
           "dora_backward", "dora_linear_workspace", "dora_linear", "dora_merge_workspace",
           "dora_merge", "dora_backward_through_norm_workspace", "dora_backward_through_norm",
           "dora_factored_norm_grouped_workspace", "dora_factored_norm_grouped",
           "dora_forward_grouped_workspace", "dora_forward_grouped", "dora_forward_noalloc")

_lib = None


class DoraModule(ctypes.Structure):
    """struct dora_module of include/dora.h."""
    _fields_ = [("W", ctypes.c_void_p), ("A", ctypes.c_void_p), ("B", ctypes.c_void_p),
                ("m", ctypes.c_void_p), ("s", ctypes.c_float), ("d_out", ctypes.c_int64),
                ("d_in", ctypes.c_int64), ("r", ctypes.c_int64)]


class DoraError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def lib():
    """Load libdora.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} not built; run python -m dora_adapter_amd.build first")
        L = ctypes.CDLL(LIB_PATH)
        p, i64, sz, f = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
        c_int = ctypes.c_int
        L.dora_strerror.restype = ctypes.c_char_p
        L.dora_strerror.argtypes = [c_int]
        L.dora_last_error.restype = ctypes.c_char_p
        L.dora_last_error.argtypes = []
        L.dora_norm_workspace.restype = sz
        L.dora_norm_workspace.argtypes = [i64, i64, i64, c_int]
        L.dora_forward_workspace.restype = sz
        L.dora_forward_workspace.argtypes = [i64, i64, i64, i64, c_int]
        L.dora_backward_workspace.restype = sz
        L.dora_backward_workspace.argtypes = [i64, i64, i64, i64, c_int]
        L.dora_factored_norm.restype = c_int
        L.dora_factored_norm.argtypes = [p, p, p, f, i64, i64, i64, c_int, p, p, p, p, p, p, sz,
                                         p]
        L.dora_compose.restype = c_int
        L.dora_compose.argtypes = [p, p, p, p, f, i64, i64, c_int, p, p]
        L.dora_forward.restype = c_int
        L.dora_forward.argtypes = [p, p, p, p, p, f, i64, i64, i64, i64, c_int, p, p, p, p, p,
                                   p, sz, p]
        L.dora_backward.restype = c_int
        L.dora_backward.argtypes = [p, p, p, p, p, p, p, f, p, p, i64, i64, i64, i64, c_int, p,
                                    p, p, p, p, sz, p]
        L.dora_backward_through_norm_workspace.restype = sz
        L.dora_backward_through_norm_workspace.argtypes = [i64, i64, i64, i64, c_int]
        L.dora_backward_through_norm.restype = c_int
        L.dora_backward_through_norm.argtypes = [p, p, p, p, p, p, p, f, p, p, p, i64, i64, i64,
                                                 i64, c_int, p, p, p, p, p, sz, p]
        mp = ctypes.POINTER(DoraModule)
        L.dora_factored_norm_grouped_workspace.restype = sz
        L.dora_factored_norm_grouped_workspace.argtypes = [mp, c_int, c_int]
        L.dora_factored_norm_grouped.restype = c_int
        L.dora_factored_norm_grouped.argtypes = [mp, c_int, c_int, p, p, sz, p]
        L.dora_forward_grouped_workspace.restype = sz
        L.dora_forward_grouped_workspace.argtypes = [mp, c_int, i64, c_int, p, p]
        L.dora_forward_grouped.restype = c_int
        L.dora_forward_grouped.argtypes = [p, i64, i64, mp, c_int, c_int, p, p, p, p, p, sz, p]
        L.dora_linear_workspace.restype = sz
        L.dora_linear_workspace.argtypes = [i64, i64, i64, c_int]
        L.dora_linear.restype = c_int
        L.dora_linear.argtypes = [p, p, i64, i64, i64, c_int, p, p, sz, p]
        L.dora_forward_noalloc.restype = c_int
        L.dora_forward_noalloc.argtypes = [p, p, p, p, p, f, i64, i64, i64, i64, c_int, p, p, p,
                                           p, p, p]
        L.dora_merge_workspace.restype = sz
        L.dora_merge_workspace.argtypes = [i64, i64, i64, c_int]
        L.dora_merge.restype = c_int
        L.dora_merge.argtypes = [p, p, p, p, f, i64, i64, i64, c_int, p, p, p, sz, p]
        _lib = L
    return _lib


def _dt(t):
    if t.dtype == torch.bfloat16:
        return DORA_BF16
    if t.dtype == torch.float32:
        return DORA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(rc):
    if rc != 0:
        raise DoraError(rc, lib().dora_last_error().decode())


def _dev(t):
    if not t.is_cuda:
        raise ValueError("libdora needs device tensors")
    return t.device


def _ws(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def dora_norm_workspace(d_out, d_in, r, dtype):
    return lib().dora_norm_workspace(d_out, d_in, r, dtype)


def dora_forward_workspace(T, d_in, d_out, r, dtype):
    return lib().dora_forward_workspace(T, d_in, d_out, r, dtype)


def dora_backward_workspace(T, d_in, d_out, r, dtype):
    return lib().dora_backward_workspace(T, d_in, d_out, r, dtype)


def dora_backward_through_norm_workspace(T, d_in, d_out, r, dtype):
    return lib().dora_backward_through_norm_workspace(T, d_in, d_out, r, dtype)


def dora_backward_through_norm(dy, x, W, A, B, m, n, s, P, y, U=None, ws=None, out=None):
    """Backward with the gradient flowing through the row norm (U: the
    forward's kept V A^T = W A^T + s B A A^T, optional)."""
    return dora_backward(dy, x, W, A, B, m, n, s, P, y, ws=ws, out=out, through_norm=True, U=U)


def dora_factored_norm(W, A, B, s, terms=False, ws=None, n=None, U_out=None):
    """Row norms of W + s*B*A (fp32 [d_out]); with terms=True also returns
    (base, cross, gram).  U_out (fp32 [d_out, r]) receives
    V A^T = W A^T + s B A A^T."""
    dev = _dev(W)
    d_out, d_in = W.shape
    r = A.shape[0]
    dt = _dt(W)
    n = torch.empty(d_out, dtype=torch.float32, device=dev) if n is None else n
    extra = [torch.empty(d_out, dtype=torch.float32, device=dev) for _ in range(3)] if terms \
        else [None, None, None]
    need = lib().dora_norm_workspace(d_out, d_in, r, dt)
    ws = _ws(need, dev) if ws is None else ws
    _check(lib().dora_factored_norm(_ptr(W), _ptr(A), _ptr(B), float(s), d_out, d_in, r, dt,
                                    _ptr(n), *[_ptr(e) for e in extra], _ptr(U_out), _ptr(ws),
                                    ws.numel(), _stream(dev)))
    return (n, *extra) if terms else n


def dora_compose(base, lora, m, n, s, y=None):
    """y = (m/n) (.) (base + s*lora) in the stable single-pass form; y may be base."""
    dev = _dev(base)
    T, d_out = base.shape
    y = torch.empty_like(base) if y is None else y
    _check(lib().dora_compose(_ptr(base), _ptr(lora), _ptr(m), _ptr(n), float(s), T, d_out,
                              _dt(base), _ptr(y), _stream(dev)))
    return y


def dora_forward(x, W, A, B, m, s, n_in=None, want_P=True, ws=None, y=None, n_out=None,
                 P_out=None, U_out=None):
    """Module forward.  Returns (y, n, P) (P is None when want_P is False).
    U_out (fp32 [d_out, r]) receives the norm's V A^T = W A^T + s B A A^T for
    the backward through the norm."""
    dev = _dev(x)
    T, d_in = x.shape
    d_out = W.shape[0]
    r = A.shape[0]
    dt = _dt(x)
    y = torch.empty(T, d_out, dtype=x.dtype, device=dev) if y is None else y
    n_out = torch.empty(d_out, dtype=torch.float32, device=dev) if n_out is None else n_out
    if want_P and P_out is None:
        P_out = torch.empty(T, r, dtype=x.dtype, device=dev)
    need = lib().dora_forward_workspace(T, d_in, d_out, r, dt)
    ws = _ws(need, dev) if ws is None else ws
    _check(lib().dora_forward(_ptr(x), _ptr(W), _ptr(A), _ptr(B), _ptr(m), float(s), T, d_in,
                              d_out, r, dt, _ptr(y), _ptr(n_out), _ptr(P_out if want_P else None),
                              _ptr(n_in), _ptr(U_out), _ptr(ws), ws.numel(), _stream(dev)))
    return y, n_out, (P_out if want_P else None)


def dora_forward_noalloc(x, W, A, B, m, s, n_in=None, want_P=True, y=None, n_out=None,
                         P_out=None, U_out=None):
    """dora_forward on the library's fixed scratch (no workspace argument;
    the library allocates nothing).  Outputs as dora_forward."""
    dev = _dev(x)
    T, d_in = x.shape
    d_out = W.shape[0]
    r = A.shape[0]
    y = torch.empty(T, d_out, dtype=x.dtype, device=dev) if y is None else y
    n_out = torch.empty(d_out, dtype=torch.float32, device=dev) if n_out is None else n_out
    if want_P and P_out is None:
        P_out = torch.empty(T, r, dtype=x.dtype, device=dev)
    _check(lib().dora_forward_noalloc(_ptr(x), _ptr(W), _ptr(A), _ptr(B), _ptr(m), float(s), T,
                                      d_in, d_out, r, _dt(x), _ptr(y), _ptr(n_out),
                                      _ptr(P_out if want_P else None), _ptr(n_in), _ptr(U_out),
                                      _stream(dev)))
    return y, n_out, (P_out if want_P else None)


def dora_backward(dy, x, W, A, B, m, n, s, P, y, ws=None, out=None, through_norm=False, U=None):
    """Backward; returns dict(dx, dA, dB, dm).  The norm is detached unless
    through_norm is set (then dA and dB include the path through n)."""
    dev = _dev(W)
    T, d_in = x.shape
    d_out = W.shape[0]
    r = A.shape[0]
    dt = _dt(W)
    if out is None:
        out = {"dx": torch.empty(T, d_in, dtype=W.dtype, device=dev),
               "dA": torch.empty(r, d_in, dtype=W.dtype, device=dev),
               "dB": torch.empty(d_out, r, dtype=W.dtype, device=dev),
               "dm": torch.empty(d_out, dtype=torch.float32, device=dev)}
    L = lib()
    size, call = ((L.dora_backward_through_norm_workspace, L.dora_backward_through_norm)
                  if through_norm else (L.dora_backward_workspace, L.dora_backward))
    need = size(T, d_in, d_out, r, dt)
    ws = _ws(need, dev) if ws is None else ws
    extra = (_ptr(U),) if through_norm else ()
    if U is not None and not through_norm:
        raise ValueError("U is used by the backward through the norm only")
    _check(call(_ptr(dy), _ptr(x), _ptr(W), _ptr(A), _ptr(B), _ptr(m), _ptr(n), float(s),
                _ptr(P), _ptr(y), *extra, T, d_in, d_out, r, dt, _ptr(out["dx"]),
                _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dm"]), _ptr(ws), ws.numel(),
                _stream(dev)))
    return out


def dora_linear_workspace(T, d_in, d_out, dtype):
    return lib().dora_linear_workspace(T, d_in, d_out, dtype)


def dora_linear(x, W, y=None, ws=None):
    """y = x W^T on the forward's base-product kernel (merged-weight inference)."""
    dev = _dev(x)
    T, d_in = x.shape
    d_out = W.shape[0]
    dt = _dt(x)
    y = torch.empty(T, d_out, dtype=x.dtype, device=dev) if y is None else y
    need = lib().dora_linear_workspace(T, d_in, d_out, dt)
    if ws is None and need > 0:
        ws = _ws(need, dev)
    _check(lib().dora_linear(_ptr(x), _ptr(W), T, d_in, d_out, dt, _ptr(y), _ptr(ws),
                             0 if ws is None else ws.numel(), _stream(dev)))
    return y


def dora_merge_workspace(d_out, d_in, r, dtype):
    return lib().dora_merge_workspace(d_out, d_in, r, dtype)


def dora_merge(W, A, B, m, s, n_in=None, out=None, ws=None):
    """Merged weight W' = (m/n) (W + s B A) by rows (n factored unless n_in
    is given); out may be W itself."""
    dev = _dev(W)
    d_out, d_in = W.shape
    r = A.shape[0]
    dt = _dt(W)
    out = torch.empty_like(W) if out is None else out
    need = lib().dora_merge_workspace(d_out, d_in, r, dt)
    ws = _ws(need, dev) if ws is None else ws
    _check(lib().dora_merge(_ptr(W), _ptr(A), _ptr(B), _ptr(m), float(s), d_out, d_in, r, dt,
                            _ptr(n_in), _ptr(out), _ptr(ws), ws.numel(), _stream(dev)))
    return out


def _modules(mods):
    """(W, A, B, m, s) tuples -> a ctypes array of DoraModule."""
    arr = (DoraModule * max(len(mods), 1))()
    for k, (W, A, B, m, s) in enumerate(mods):
        arr[k] = DoraModule(W.data_ptr(), A.data_ptr(), B.data_ptr(),
                            None if m is None else m.data_ptr(), float(s), W.shape[0],
                            W.shape[1], A.shape[0])
    return arr


def _ptrs(ts):
    """Host array of device pointers (None entries stay NULL); None -> NULL."""
    if ts is None:
        return None
    arr = (ctypes.c_void_p * max(len(ts), 1))()
    for k, t in enumerate(ts):
        arr[k] = None if t is None else t.data_ptr()
    return arr


def dora_factored_norm_grouped_workspace(mods, dtype):
    return lib().dora_factored_norm_grouped_workspace(_modules(mods), len(mods), dtype)


def dora_forward_grouped_workspace(mods, T, dtype, n_in=None, P_out=None):
    return lib().dora_forward_grouped_workspace(_modules(mods), len(mods), T, dtype,
                                                _ptrs(n_in), _ptrs(P_out))


def dora_factored_norm_grouped(mods, ns=None, ws=None):
    """Row norms of W + sBA for every (W, A, B, m, s) in mods (m unused), in
    grouped launches.  Returns the list of fp32 norms."""
    if not mods:
        return []
    dev = _dev(mods[0][0])
    dt = _dt(mods[0][0])
    arr = _modules(mods)
    ns = [torch.empty(W.shape[0], dtype=torch.float32, device=dev) for W, *_ in mods] \
        if ns is None else ns
    need = lib().dora_factored_norm_grouped_workspace(arr, len(mods), dt)
    ws = _ws(need, dev) if ws is None else ws
    keep = _ptrs(ns)
    _check(lib().dora_factored_norm_grouped(arr, len(mods), dt, ctypes.cast(keep, ctypes.c_void_p),
                                            _ptr(ws), ws.numel(), _stream(dev)))
    return ns


def dora_forward_grouped(x, mods, n_in=None, want_P=True, ws=None, ys=None, ns=None, Ps=None):
    """dora_forward for sibling modules sharing x.  mods: (W, A, B, m, s)
    tuples; n_in: optional list of cached norms (entries may be None).
    Returns (ys, ns, Ps)."""
    if not mods:
        return [], [], []
    dev = _dev(x)
    T, d_in = x.shape
    dt = _dt(x)
    arr = _modules(mods)
    ys = [torch.empty(T, W.shape[0], dtype=x.dtype, device=dev) for W, *_ in mods] \
        if ys is None else ys
    ns = [torch.empty(W.shape[0], dtype=torch.float32, device=dev) for W, *_ in mods] \
        if ns is None else ns
    if want_P and Ps is None:
        Ps = [torch.empty(T, A.shape[0], dtype=x.dtype, device=dev) for _, A, *_ in mods]
    if not want_P:
        Ps = None
    py, pn, pP, pnin = _ptrs(ys), _ptrs(ns), _ptrs(Ps), _ptrs(n_in)
    vp = lambda a: None if a is None else ctypes.cast(a, ctypes.c_void_p)  # noqa: E731
    need = lib().dora_forward_grouped_workspace(arr, len(mods), T, dt, vp(pnin), vp(pP))
    ws = _ws(need, dev) if ws is None else ws
    _check(lib().dora_forward_grouped(_ptr(x), T, d_in, arr, len(mods), dt, vp(py), vp(pn),
                                      vp(pP), vp(pnin), _ptr(ws), ws.numel(), _stream(dev)))
    return ys, ns, Ps
