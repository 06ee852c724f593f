"""Seeded synthetic inputs for the SSD scan (numpy only).

This module holds the input distributions and nothing of the scan's arithmetic;
both the HIP path's tests/benchmark and the fp64 oracle consume its arrays.

Distributions (per workload, ``numpy.random.Generator(PCG64(seed))``, draws in
this fixed order: x, z, d_h, A, B, C, D, h0):

* x ~ N(0, 1);
* dt = clip(softplus(0.5 z + b_h), lo, hi), z ~ N(0, 1), where per head
  d_h = exp(U[ln lo, ln hi]) and b_h = softplus^-1(d_h) = d_h + ln(1 - e^-d_h);
* A = -exp(U[0, ln 16]) per head (scalar decay) or per (head, state) (diagonal);
* B, C ~ N(0, 1) / sqrt(N);  D ~ N(0, 1);  h0 ~ N(0, 0.1^2) when drawn, else 0.

x, B and C of a bf16 workload are rounded to bfloat16 (round to nearest even)
here, once; both sides then see the identical rounded values.  dt, A, D and h0
are float32.
"""
from __future__ import annotations

import numpy as np

from .configs import Workload


def bf16_round_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even; NaN kept quiet."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _softplus(v):
    return np.logaddexp(0.0, v)


def make_inputs(w: Workload, seed: int | None = None, diag_equal_A: bool = False) -> dict:
    """Draw one workload's inputs.

    Returns a dict with float32 arrays ``x, dt, A, B, C, D, h0`` (x/B/C already
    rounded to bf16 values for bf16 workloads; ``h0`` is None when not drawn) and,
    for bf16 workloads, the bit patterns ``x_bits, B_bits, C_bits`` (uint16).
    With ``diag_equal_A`` the diagonal workload's A repeats A[h, 0] across n.
    """
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    b, T, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    x = rng.standard_normal((b, T, H, P), dtype=np.float32)
    z = rng.standard_normal((b, T, H), dtype=np.float32)
    d_h = np.exp(rng.uniform(np.log(w.dt_lo), np.log(w.dt_hi), size=H))
    bias = d_h + np.log(-np.expm1(-d_h))
    dt = np.clip(_softplus(0.5 * z.astype(np.float64) + bias[None, None, :]), w.dt_lo, w.dt_hi)
    dt = dt.astype(np.float32)
    if w.diag:
        A = -np.exp(rng.uniform(0.0, np.log(16.0), size=(H, N)))
        if diag_equal_A:
            A = np.repeat(A[:, :1], N, axis=1)
    else:
        A = -np.exp(rng.uniform(0.0, np.log(16.0), size=H))
    A = A.astype(np.float32)
    scale = np.float32(1.0 / np.sqrt(N))
    B = rng.standard_normal((b, T, G, N), dtype=np.float32) * scale
    C = rng.standard_normal((b, T, G, N), dtype=np.float32) * scale
    D = rng.standard_normal(H, dtype=np.float32)
    h0 = (rng.standard_normal((b, H, P, N), dtype=np.float32) * np.float32(0.1)) if w.h0 else None
    out = dict(x=x, dt=dt, A=A, B=B, C=C, D=D, h0=h0)
    if w.dtype == "bf16":
        for k in ("x", "B", "C"):
            bits = bf16_round_bits(out[k])
            out[k + "_bits"] = bits
            out[k] = bf16_bits_to_f32(bits)
    elif w.dtype != "f32":
        raise ValueError(f"unknown dtype {w.dtype}")
    return out


def make_small(b, T, H, P, N, G, seed, *, diag=False, dtype="f32", dt_lo=1e-3, dt_hi=0.1,
               h0=True, D=True) -> dict:
    """Inputs for an ad-hoc small shape (tests): same distributions as the workloads."""
    w = Workload("adhoc", b, T, H, P, N, G, 64, dtype, dt_lo, dt_hi, diag=diag, h0=h0, seed=seed)
    d = make_inputs(w)
    if not D:
        d["D"] = None
    return d


def make_packed(lengths, H, P, N, G, seed, *, dtype="bf16", dt_lo=1e-3, dt_hi=0.1, h0=True) -> dict:
    """Inputs for packed variable-length sequences (tests, bench): the sequences of
    `lengths` back to back on one token axis, with the workloads' distributions.
    Returns x [T,H,P], dt [T,H], B/C [T,G,N] (float32 arrays, bf16-rounded for bf16),
    A [H], D [H], h0 [nseq,H,P,N] (N(0, 0.1), or None) and cu_seqlens (int32, nseq + 1)."""
    lengths = [int(v) for v in lengths]
    T = sum(lengths)
    d = make_small(1, max(T, 1), H, P, N, G, seed, dtype=dtype, dt_lo=dt_lo, dt_hi=dt_hi, h0=False)
    out = {k: (v[0, :T] if k in ("x", "dt", "B", "C") else v) for k, v in d.items()
           if k in ("x", "dt", "B", "C", "A", "D")}
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    out["h0"] = (rng.standard_normal((len(lengths), H, P, N)) * 0.1).astype(np.float32) if h0 else None
    out["cu_seqlens"] = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return out


def make_grads(b, T, H, P, N, seed, *, dtype="f32", dhT=True) -> dict:
    """Output gradients for a backward pass over inputs of shape (b, T, H, P, N): the
    gradient of a loss with respect to y, dy ~ N(0, 1) [b,T,H,P] (rounded to bfloat16
    for a bf16 problem, like x), and with respect to the final state, dhT ~ N(0, 0.1^2)
    [b,H,P,N] float32 (None when not drawn).  Its own generator stream (seed + 104729),
    drawn in the order dy, dhT."""
    rng = np.random.Generator(np.random.PCG64(seed + 104729))
    dy = rng.standard_normal((b, T, H, P), dtype=np.float32)
    g = rng.standard_normal((b, H, P, N), dtype=np.float32) * np.float32(0.1)
    out = dict(dy=dy, dhT=g if dhT else None)
    if dtype == "bf16":
        bits = bf16_round_bits(dy)
        out["dy_bits"] = bits
        out["dy"] = bf16_bits_to_f32(bits)
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype}")
    return out
