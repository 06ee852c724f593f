"""fp64 CPU oracle for the SSD scan -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and it shares no code
with them: it is a plain fp64 implementation written from the pages
("Structured State Space Duality" concept page; "Diagonal Equivalence in State
Space Models" abstract; "Semiseparable Matrix Transformations" definition).

Three independent forms of the same map, and its gradients, all in fp64:

* :func:`recurrence` -- O1, the selective recurrence stepped token by token
  (C, OpenMP); :func:`recurrence_packed` runs it per sequence of a packed batch;
* :func:`quadratic`  -- O2, the materialised lower-triangular matrix M with
  explicit decay products (C), and :func:`quadratic_np`, a numpy twin of O2
  for tiny inputs;
* :func:`chunked`    -- O3, the chunked algorithm with every intermediate
  dumped (chunk-local cumulative step, C B^T blocks, chunk states, entering
  states, diagonal-block and off-diagonal outputs);
* :func:`recurrence_bwd` -- O4, the gradients of O1 (the backward pass) by
  reverse-mode differentiation of the recurrence written out by hand (C, OpenMP).

Inputs are numpy arrays in the layouts x [b,T,H,P], dt [b,T,H],
A [H] or [H,N], B/C [b,T,G,N], D [H], h0 [b,H,P,N]; they are converted to
float64 exactly.  Parity pins for every function live in the CPU test suite.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP, strict IEEE: no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
             "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        i64, dp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.oracle_recurrence.argtypes = [i64] * 6 + [ci] + [dp] * 9 + [ci]
        lib.oracle_quadratic.argtypes = [i64] * 6 + [ci] + [dp] * 10 + [ci]
        lib.oracle_chunked.argtypes = [i64] * 6 + [ci, i64] + [dp] * 15 + [ci]
        lib.oracle_recurrence_bwd.argtypes = [i64] * 6 + [ci] + [dp] * 16 + [ci]
        for f in (lib.oracle_recurrence, lib.oracle_quadratic, lib.oracle_chunked, lib.oracle_recurrence_bwd):
            f.restype = ci
        _lib = lib
    return _lib


def _f64(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dims(x, dt, A, B, diag):
    b, T, H, P = x.shape
    _, _, G, N = B.shape
    assert dt.shape == (b, T, H)
    assert A.shape == ((H, N) if diag else (H,))
    assert H % G == 0
    return b, T, H, P, N, G


def _prep(x, dt, A, B, C, D, h0, diag):
    x, dt, A, B, C, D, h0 = (_f64(v) for v in (x, dt, A, B, C, D, h0))
    dims = _dims(x, dt, A, B, diag)
    b, T, H, P, N, G = dims
    assert C.shape == B.shape
    assert D is None or D.shape == (H,)
    assert h0 is None or h0.shape == (b, H, P, N)
    return (x, dt, A, B, C, D, h0), dims


def default_threads() -> int:
    return len(os.sched_getaffinity(0))


def recurrence(x, dt, A, B, C, D=None, h0=None, diag=False, nthreads=None):
    """O1: step h_t = a_t h_{t-1} + x_t B_t^T, y_t = h_t C_t + D x_t. Returns (y, hT)."""
    (x, dt, A, B, C, D, h0), (b, T, H, P, N, G) = _prep(x, dt, A, B, C, D, h0, diag)
    y = np.empty((b, T, H, P))
    hT = np.empty((b, H, P, N))
    rc = _load().oracle_recurrence(b, T, H, P, N, G, int(diag), _ptr(x), _ptr(dt), _ptr(A),
                                   _ptr(B), _ptr(C), _ptr(D), _ptr(h0), _ptr(y), _ptr(hT),
                                   nthreads or default_threads())
    if rc:
        raise ValueError("oracle_recurrence: bad dimensions")
    return y, hT


def recurrence_packed(x, dt, A, B, C, cu_seqlens, D=None, h0=None, diag=False, nthreads=None):
    """O1 over packed variable-length sequences.  x [T,H,P], dt [T,H], B/C [T,G,N] hold
    the sequences back to back, sequence s on tokens [cu[s], cu[s+1]); h0 [nseq,H,P,N]
    (None: zero).  Each sequence is its own map with its own state, which the chunked
    algorithm passes only between the chunks of one sequence ("Structured State Space
    Duality" concept page, section "The chunked algorithm takes both"), so each slice
    runs through :func:`recurrence` alone; an empty sequence keeps its initial state.
    Returns (y [T,H,P], hT [nseq,H,P,N])."""
    x = np.asarray(x)
    cu = [int(v) for v in np.asarray(cu_seqlens)]
    T, H, P = x.shape
    N = np.asarray(B).shape[2]
    nseq = len(cu) - 1
    if cu[0] != 0 or cu[-1] != T or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must be nondecreasing from 0 to T")
    y = np.zeros((T, H, P))
    hT = np.zeros((nseq, H, P, N))
    for s in range(nseq):
        a, b = cu[s], cu[s + 1]
        h0s = None if h0 is None else np.asarray(h0)[s:s + 1]
        if a == b:
            if h0s is not None:
                hT[s] = h0s[0]
            continue
        ys, hs = recurrence(x[None, a:b], np.asarray(dt)[None, a:b], A, np.asarray(B)[None, a:b],
                            np.asarray(C)[None, a:b], D, h0s, diag=diag, nthreads=nthreads)
        y[a:b] = ys[0]
        hT[s] = hs[0]
    return y, hT


def recurrence_bwd(x, dt, A, B, C, D=None, h0=None, dy=None, dhT=None, diag=False, nthreads=None):
    """O4: gradients of O1 for the output gradients dy [b,T,H,P] and dhT [b,H,P,N]
    (None: zero).  Returns a dict with dx [b,T,H,P], ddt [b,T,H], dA [H] or [H,N],
    dB and dC [b,T,G,N], dD [H] and dh0 [b,H,P,N], all float64.  dD and dh0 are the
    gradients for D and h0 whether or not those were given (a missing D or h0 is zero)."""
    (x, dt, A, B, C, D, h0), (b, T, H, P, N, G) = _prep(x, dt, A, B, C, D, h0, diag)
    dy = _f64(dy) if dy is not None else np.zeros((b, T, H, P))
    dhT = _f64(dhT)
    assert dy.shape == (b, T, H, P)
    assert dhT is None or dhT.shape == (b, H, P, N)
    out = dict(dx=np.empty((b, T, H, P)), ddt=np.empty((b, T, H)), dA=np.empty((H, N) if diag else (H,)),
               dB=np.empty((b, T, G, N)), dC=np.empty((b, T, G, N)), dD=np.empty((H,)),
               dh0=np.empty((b, H, P, N)))
    rc = _load().oracle_recurrence_bwd(b, T, H, P, N, G, int(diag), _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                                       _ptr(C), _ptr(D), _ptr(h0), _ptr(dy), _ptr(dhT), _ptr(out["dx"]),
                                       _ptr(out["ddt"]), _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]),
                                       _ptr(out["dD"]), _ptr(out["dh0"]), nthreads or default_threads())
    if rc:
        raise ValueError("oracle_recurrence_bwd: bad dimensions or out of memory")
    return out


def quadratic(x, dt, A, B, C, D=None, h0=None, diag=False, return_M=False, nthreads=None):
    """O2: materialised M with explicit decay products. Returns (y, hT[, M[b,H,T,T]])."""
    (x, dt, A, B, C, D, h0), (b, T, H, P, N, G) = _prep(x, dt, A, B, C, D, h0, diag)
    y = np.empty((b, T, H, P))
    hT = np.empty((b, H, P, N))
    M = np.empty((b, H, T, T)) if return_M else None
    rc = _load().oracle_quadratic(b, T, H, P, N, G, int(diag), _ptr(x), _ptr(dt), _ptr(A),
                                  _ptr(B), _ptr(C), _ptr(D), _ptr(h0), _ptr(y), _ptr(hT),
                                  _ptr(M), nthreads or default_threads())
    if rc:
        raise ValueError("oracle_quadratic: bad dimensions")
    return (y, hT, M) if return_M else (y, hT)


def chunked(x, dt, A, B, C, D=None, h0=None, Q=64, diag=False, dumps=False, nthreads=None):
    """O3: the chunked algorithm. Returns (y, hT) or (y, hT, dict of stage dumps)."""
    (x, dt, A, B, C, D, h0), (b, T, H, P, N, G) = _prep(x, dt, A, B, C, D, h0, diag)
    nc = (T + Q - 1) // Q
    y = np.empty((b, T, H, P))
    hT = np.empty((b, H, P, N))
    d = {}
    if dumps:
        d = dict(cdt=np.empty((b, H, nc, Q)),
                 S=np.empty((b, H, nc, P, N)), Hc=np.empty((b, H, nc, P, N)),
                 ydiag=np.empty((b, T, H, P)), yoff=np.empty((b, T, H, P)))
        if not diag:
            d["G"] = np.empty((b, nc, G, Q, Q))
    rc = _load().oracle_chunked(b, T, H, P, N, G, int(diag), Q, _ptr(x), _ptr(dt), _ptr(A),
                                _ptr(B), _ptr(C), _ptr(D), _ptr(h0), _ptr(y), _ptr(hT),
                                _ptr(d.get("cdt")), _ptr(d.get("G")), _ptr(d.get("S")),
                                _ptr(d.get("Hc")), _ptr(d.get("ydiag")), _ptr(d.get("yoff")),
                                nthreads or default_threads())
    if rc:
        raise ValueError("oracle_chunked: bad dimensions")
    return (y, hT, d) if dumps else (y, hT)


def quadratic_np(x, dt, A, B, C, D=None, h0=None, diag=False):
    """Numpy twin of O2 for tiny inputs (pure-Python loops over (b, h, i, j)).

    M_ij = sum_n C_in B_jn prod_{k=j+1..i} a_{k,n}; y = M x + (prod_{k<=i} a_k) h0 C_i
    + D x_i; hT = (prod a) h0 + sum_j (prod_{k>j} a_k) x_j B_j^T, every product by
    np.prod over the explicit decays.
    """
    (x, dt, A, B, C, D, h0), (b, T, H, P, N, G) = _prep(x, dt, A, B, C, D, h0, diag)
    y = np.zeros((b, T, H, P))
    hT = np.zeros((b, H, P, N))
    for bi in range(b):
        for h in range(H):
            g = h * G // H
            Ah = A[h] if diag else np.full(N, A[h])
            a = np.exp(dt[bi, :, h][:, None] * Ah[None, :])          # [T, N]
            Cb, Bb = C[bi, :, g, :], B[bi, :, g, :]                  # [T, N]
            M = np.zeros((T, T))
            for i in range(T):
                for j in range(i + 1):
                    M[i, j] = np.sum(Cb[i] * Bb[j] * np.prod(a[j + 1:i + 1], axis=0))
            xs = x[bi, :, h, :]                                      # [T, P]
            yy = M @ xs
            if h0 is not None:
                for i in range(T):
                    yy[i] += h0[bi, h] @ (np.prod(a[:i + 1], axis=0) * Cb[i])
            if D is not None:
                yy += D[h] * xs
            y[bi, :, h, :] = yy
            st = np.zeros((P, N))
            if h0 is not None:
                st += np.prod(a, axis=0)[None, :] * h0[bi, h]
            for j in range(T):
                st += np.outer(xs[j], np.prod(a[j + 1:], axis=0) * Bb[j])
            hT[bi, h] = st
    return y, hT
