"""ctypes wrapper around the fp64 CPU oracle (oracle/dora_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  Nothing in the HIP product path
imports this module.

Inputs are torch CPU tensors (fp32 or bf16) or numpy arrays; bf16 data is
handed to C as raw 16-bit patterns and promoted exactly there.  m, n and s
are promoted exactly from their fp32 values to double here, so the oracle
sees the very numbers the GPU path receives.  Outputs are numpy float64.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

F32, BF16 = 0, 1

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_d = ctypes.c_double


def load(path=None):
    """Load liboracle.so (building it first only if it does not exist)."""
    global _LIB
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _LIB is None:
        lib = os.path.join(HERE, "liboracle.so")
        if not os.path.exists(lib):
            from . import build as _build  # noqa: F401  (package-relative import)
            _build.build()
        _LIB = _declare(ctypes.CDLL(lib))
    return _LIB


def _declare(lib):
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_norm.argtypes = [_p, _p, _p, ctypes.c_int, _d, _i64, _i64, _i64,
                                _p, _i64, _p, _p, _p, _p]
    lib.oracle_forward.argtypes = [_p, _p, _p, _p, _p, ctypes.c_int, _d,
                                   _i64, _i64, _i64, _i64, _p, _i64, _p, _i64,
                                   _p, _p, _p]
    lib.oracle_compose.argtypes = [_p, _p, _p, _p, ctypes.c_int, _d, _i64, _i64, _p]
    lib.oracle_backward_full.argtypes = [_p, _p, _p, _p, _p, _p, _p, ctypes.c_int,
                                         _d, _i64, _i64, _i64, _i64, _p, _p, _p, _p]
    lib.oracle_backward_sampled.argtypes = [_p, _p, _p, _p, _p, _p, _p, ctypes.c_int,
                                            _d, _i64, _i64, _i64, _i64,
                                            _p, _i64, _p, _p, _i64, _p,
                                            _p, _i64, _p, _p, _i64, _p]
    lib.oracle_merge.argtypes = [_p, _p, _p, _p, ctypes.c_int, _d, _i64, _i64, _i64,
                                 _p, _i64, _p, _p]
    lib.oracle_backward_through_norm.argtypes = [_p, _p, _p, _p, _p, _p, ctypes.c_int, _d,
                                                 _i64, _i64, _i64, _i64, _p, _p, _p, _p]
    for f in ("oracle_norm", "oracle_forward", "oracle_compose", "oracle_merge",
              "oracle_backward_full", "oracle_backward_sampled",
              "oracle_backward_through_norm"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


def _raw(t):
    """(contiguous numpy array, dtype code) for a CPU tensor or numpy array."""
    try:
        import torch
        if isinstance(t, torch.Tensor):
            t = t.detach().cpu().contiguous()
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view(np.uint16), BF16
            if t.dtype == torch.float32:
                return t.numpy(), F32
            raise TypeError(f"oracle: unsupported dtype {t.dtype}")
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(t)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    raise TypeError(f"oracle: unsupported dtype {a.dtype}")


def _f64(v):
    """fp32 vector -> exact float64 copy (double inputs pass through)."""
    try:
        import torch
        if isinstance(v, torch.Tensor):
            v = v.detach().cpu()
            if v.dtype != torch.float64:
                v = v.float()
            v = v.double().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(v, dtype=np.float64))


def _s(s):
    """The scale as the GPU sees it: rounded to fp32, then exactly widened."""
    return float(np.float32(s))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _idx(lst):
    if lst is None:
        return None
    return np.ascontiguousarray(np.asarray(lst, dtype=np.int64).reshape(-1))


def _same_dtype(*codes):
    if len(set(codes)) != 1:
        raise TypeError("oracle: all matrix inputs must share one dtype")
    return codes[0]


def num_threads():
    return int(load().oracle_num_threads())


def norm(W, A, B, s, rows=None):
    """Dense row norms of W + s*B*A and the base/cross/gram terms (fp64)."""
    (w, dw), (a, da), (b, db) = _raw(W), _raw(A), _raw(B)
    dt = _same_dtype(dw, da, db)
    d_out, d_in = w.shape
    r = a.shape[0]
    rw = _idx(rows)
    nr = d_out if rw is None else rw.size
    out = {k: np.zeros(nr) for k in ("n", "base", "cross", "gram")}
    rc = load().oracle_norm(_ptr(w), _ptr(a), _ptr(b), dt, _s(s), d_out, d_in, r,
                            _ptr(rw), nr, _ptr(out["n"]), _ptr(out["base"]),
                            _ptr(out["cross"]), _ptr(out["gram"]))
    if rc:
        raise MemoryError("oracle_norm failed")
    return out


def forward(x, W, A, B, m, s, toks=None, rows=None, n_in=None):
    """y[t, i] = (m_i/n_i) * sum_j x[t,j] V[i,j] for listed tokens/rows.

    Returns (y [ntok, nrow] float64, n [nrow] float64)."""
    (xx, dx_), (w, dw), (a, da), (b, db) = _raw(x), _raw(W), _raw(A), _raw(B)
    dt = _same_dtype(dx_, dw, da, db)
    T, d_in = xx.shape
    d_out = w.shape[0]
    r = a.shape[0]
    mm = _f64(m)
    tk, rw = _idx(toks), _idx(rows)
    nt = T if tk is None else tk.size
    nr = d_out if rw is None else rw.size
    nin = None if n_in is None else _f64(n_in)
    y = np.zeros((nt, nr))
    nout = np.zeros(nr)
    rc = load().oracle_forward(_ptr(xx), _ptr(w), _ptr(a), _ptr(b), _ptr(mm), dt, _s(s),
                               T, d_in, d_out, r, _ptr(tk), nt, _ptr(rw), nr,
                               _ptr(nin), _ptr(y), _ptr(nout))
    if rc:
        raise MemoryError("oracle_forward failed")
    return y, nout


def compose(base, lora, m, n, s):
    """Plain y = (m/n) * (base + s*lora), [T, d_out] float64."""
    (bb, d1), (ll, d2) = _raw(base), _raw(lora)
    dt = _same_dtype(d1, d2)
    T, d_out = bb.shape
    y = np.zeros((T, d_out))
    load().oracle_compose(_ptr(bb), _ptr(ll), _ptr(_f64(m)), _ptr(_f64(n)), dt, _s(s),
                          T, d_out, _ptr(y))
    return y


def merge(W, A, B, m, s, rows=None, n_in=None):
    """Merged weight W'[i] = (m_i/n_i) (W + s B A)[i] for the listed rows
    (all by default), [nrow, d_in] float64; n from the dense rows unless
    n_in is given."""
    (w, dw), (a, da), (b, db) = _raw(W), _raw(A), _raw(B)
    dt = _same_dtype(dw, da, db)
    d_out, d_in = w.shape
    r = a.shape[0]
    rw = _idx(rows)
    nr = d_out if rw is None else rw.size
    nin = None if n_in is None else _f64(n_in)
    out = np.zeros((nr, d_in))
    rc = load().oracle_merge(_ptr(w), _ptr(a), _ptr(b), _ptr(_f64(m)), dt, _s(s), d_out, d_in,
                             r, _ptr(rw), nr, _ptr(nin), _ptr(out))
    if rc:
        raise MemoryError("oracle_merge failed")
    return out


def backward_full(dy, x, W, A, B, m, n, s):
    """All gradients with n held constant; dict of float64 arrays."""
    (g, d0), (xx, d1), (w, d2), (a, d3), (b, d4) = (_raw(dy), _raw(x), _raw(W),
                                                    _raw(A), _raw(B))
    dt = _same_dtype(d0, d1, d2, d3, d4)
    T, d_in = xx.shape
    d_out, r = b.shape
    out = {"dx": np.zeros((T, d_in)), "dA": np.zeros((r, d_in)),
           "dB": np.zeros((d_out, r)), "dm": np.zeros(d_out)}
    rc = load().oracle_backward_full(_ptr(g), _ptr(xx), _ptr(w), _ptr(a), _ptr(b),
                                     _ptr(_f64(m)), _ptr(_f64(n)), dt, _s(s),
                                     T, d_in, d_out, r, _ptr(out["dx"]), _ptr(out["dA"]),
                                     _ptr(out["dB"]), _ptr(out["dm"]))
    if rc:
        raise MemoryError("oracle_backward_full failed")
    return out


def backward_through_norm(dy, x, W, A, B, m, s):
    """All gradients with the gradient flowing through n (no stop-gradient);
    n is the dense row norm.  Dict of float64 arrays."""
    (g, d0), (xx, d1), (w, d2), (a, d3), (b, d4) = (_raw(dy), _raw(x), _raw(W), _raw(A),
                                                    _raw(B))
    dt = _same_dtype(d0, d1, d2, d3, d4)
    T, d_in = xx.shape
    d_out, r = w.shape[0], a.shape[0]
    out = {"dx": np.zeros((T, d_in)), "dA": np.zeros((r, d_in)), "dB": np.zeros((d_out, r)),
           "dm": np.zeros(d_out)}
    rc = load().oracle_backward_through_norm(_ptr(g), _ptr(xx), _ptr(w), _ptr(a), _ptr(b),
                                             _ptr(_f64(m)), dt, _s(s), T, d_in, d_out, r,
                                             _ptr(out["dx"]), _ptr(out["dA"]), _ptr(out["dB"]),
                                             _ptr(out["dm"]))
    if rc:
        raise MemoryError("oracle_backward_through_norm failed")
    return out


def backward_sampled(dy, x, W, A, B, m, n, s, dx_idx=(), dA_idx=(), dB_idx=(), dm_idx=()):
    """Selected gradient entries with n held constant.

    dx_idx: (t, j) pairs; dA_idx: (k, j); dB_idx: (i, k); dm_idx: i."""
    (g, d0), (xx, d1), (w, d2), (a, d3), (b, d4) = (_raw(dy), _raw(x), _raw(W),
                                                    _raw(A), _raw(B))
    dt = _same_dtype(d0, d1, d2, d3, d4)
    T, d_in = xx.shape
    d_out, r = b.shape
    ix = {k: np.ascontiguousarray(np.asarray(v, dtype=np.int64).reshape(-1))
          for k, v in (("dx", dx_idx), ("dA", dA_idx), ("dB", dB_idx), ("dm", dm_idx))}
    cnt = {"dx": ix["dx"].size // 2, "dA": ix["dA"].size // 2,
           "dB": ix["dB"].size // 2, "dm": ix["dm"].size}
    out = {k: np.zeros(max(c, 1)) for k, c in cnt.items()}
    rc = load().oracle_backward_sampled(
        _ptr(g), _ptr(xx), _ptr(w), _ptr(a), _ptr(b), _ptr(_f64(m)), _ptr(_f64(n)),
        dt, _s(s), T, d_in, d_out, r,
        _ptr(ix["dx"]), cnt["dx"], _ptr(out["dx"]),
        _ptr(ix["dA"]), cnt["dA"], _ptr(out["dA"]),
        _ptr(ix["dB"]), cnt["dB"], _ptr(out["dB"]),
        _ptr(ix["dm"]), cnt["dm"], _ptr(out["dm"]))
    if rc:
        raise MemoryError("oracle_backward_sampled failed")
    return {k: out[k][:cnt[k]] for k in out}


def set_library(path):
    """Point this wrapper at another build of the oracle (used by the test
    that plants mistakes in a copy of the oracle source); returns the
    previous handle so the caller can restore it with ``restore_library``."""
    global _LIB
    prev = _LIB
    _LIB = _declare(ctypes.CDLL(path))
    return prev


def restore_library(prev):
    global _LIB
    _LIB = prev
