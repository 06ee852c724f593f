"""Algorithmic work of one SSD forward (and backward): matrix-core flops and minimal HBM bytes.

Flops use the causal convention: a Q x Q block product counts only the L(L+1)/2
entries on or below the diagonal (L = tokens in the chunk); C B^T counts once per
(batch, group, chunk) for the scalar decay and once per (batch, head, chunk) for the
diagonal decay (it is formed per head there); the chunk-state and state-output
contractions count 2 L P N each.  Exponentials, masks, the state scan and the skip
term are not counted.

Bytes are per kernel of the split schedule, each operand that kernel must touch
counted once (es = bytes of the x/B/C dtype):
  k_cumsum  dt read + cdt write
  k_cb      B + C read + C B^T blocks (64 x 64, on/below the diagonal) write
  k_state   x + B + cdt read + chunk states (es) write
  k_scan    chunk states (es) + chunk-end cdt + h0 read, entering states (es) + hT write
  k_out     x + C + cdt + C B^T blocks + entering states read, y write
  k_bt      B read + per-chunk transposed B write, C read + per-chunk C write (fused)
  k_fused   x + C + transposed B + cdt + C B^T blocks + h0 read, y + hT write
The path minimum is x + y + B + C + dt + h0 + hT, each touched once.
"""
from __future__ import annotations


def _chunks(T, Q):
    full, rem = divmod(T, Q)
    return [Q] * full + ([rem] if rem else [])


def flops(b, T, H, P, N, G, Q, diag=False) -> dict:
    tri = sum(L * (L + 1) // 2 for L in _chunks(T, Q))
    tok = T
    out = {
        "diag_block": b * H * tri * 2 * P,
        "cb": b * (H if diag else G) * tri * 2 * N,
        "chunk_state": b * H * tok * 2 * P * N,
        "state_output": b * H * tok * 2 * P * N,
    }
    out["total"] = sum(out.values())
    return out


def kernel_bytes(b, T, H, P, N, G, Q, es, diag=False, h0=True) -> dict:
    nc = -(-T // Q)
    nb = Q // 64
    x = b * T * H * P * es
    bc = b * T * G * N * es
    dt = b * T * H * 4
    cdt = b * H * nc * Q * 4
    cbb = 0 if diag else b * nc * G * (nb * (nb + 1) // 2) * 64 * 64 * es
    stx = b * H * nc * P * N * es
    hstate = b * H * P * N * 4
    return {
        "k_cumsum": dt + cdt,
        "k_cb": 0 if diag else 2 * bc + cbb,
        "k_state": x + bc + cdt + stx,
        "k_scan": stx + b * H * nc * 4 + (hstate if h0 else 0) + stx + hstate,
        "k_out": x + bc * (2 if diag else 1) + cdt + cbb + stx + x,
        "k_bt": 0 if diag else 4 * bc,
        "k_fused": 2 * x + 2 * bc + cdt + cbb + (2 if h0 else 1) * hstate,
    }


def gtab_bytes(b, T, H, G, N, Q, es) -> int:
    """The diagonal decay's table kernel: B and C rows of each (batch, head, chunk) block
    pair read once per head, the lower 64 x 64 blocks of the table written."""
    nc = -(-T // Q)
    nb = Q // 64
    return 2 * b * H * T * N * es + b * H * nc * (nb * (nb + 1) // 2) * 64 * 64 * es

def path_min_bytes(b, T, H, P, N, G, es, h0=True) -> int:
    return 2 * b * T * H * P * es + 2 * b * T * G * N * es + b * T * H * 4 + \
        (2 if h0 else 1) * b * H * P * N * 4


def bwd_path_min_bytes(b, T, H, P, N, G, es, h0=True, dhT=True) -> int:
    """Backward pass: x, dy, B, C, dt (h0, dhT when given) read once; dx, dB, dC, ddt and
    dh0 written once (dA, dD are H floats)."""
    x = b * T * H * P * es
    bc = b * T * G * N * es
    dt = b * T * H * 4
    st = b * H * P * N * 4
    return 3 * x + 4 * bc + 2 * dt + (st if h0 else 0) + (st if dhT else 0) + st


def bwd_kernel_bytes(b, T, H, P, N, G, Q, es, h0=True, dhT=True) -> dict:
    """Algorithmic bytes of each backward kernel (each operand it must touch, once)."""
    nc = -(-T // Q)
    nb = Q // 64
    x = b * T * H * P * es
    bc = b * T * G * N * es
    dt = b * T * H * 4
    cdt = b * H * nc * Q * 4
    cbb = b * nc * G * (nb * (nb + 1) // 2) * 64 * 64 * es
    st32 = b * H * nc * P * N * 4
    stx = b * H * nc * P * N * es
    hstate = b * H * P * N * 4
    ds = b * H * nc * Q * 4
    return {
        "k_cumsum": dt + cdt,
        "k_cb": 2 * bc + cbb,                      # each of the two launches (C B^T, B C^T)
        "k_bt": 2 * bc,                            # each of the two launches (B, C)
        "k_state": x + bc + cdt + st32,            # forward chunk states; the adjoint's reads dy, C
        "k_scan": st32 + b * H * nc * 4 + (hstate if h0 else 0) + stx + (hstate if dhT else 0),
        "k_scan_rev": st32 + b * H * nc * 4 + (hstate if dhT else 0) + stx + hstate,
        "k_bwd_x": 2 * x + 2 * bc + 2 * cbb + 2 * stx + cdt + x + ds,
        "k_bwd_bc": 2 * x + 2 * stx + cdt + 2 * bc + 2 * bc,
        "k_bwd_dt": ds + dt + (2 * hstate if dhT else 0) + dt,
    }


def fused_mfma_flops(b, T, H, N, Q) -> int:
    """Matrix-core flops the fused kernel issues (whole 16x16x32 bf16 steps, headdim 64):
    per chunk of one (batch, head), the output passes take sum_t (floor(t/2) + 1) C B^T
    fragments over the Q/16 row tiles t, each times 4 column tiles of x; the state term
    (Q/16) (N/32) 4 steps; the state update (Q/32) (N/16) 4 steps.  Ragged chunks issue
    whole tiles too."""
    nc = -(-T // Q)
    rt = Q // 16
    diag = sum(t // 2 + 1 for t in range(rt)) * 4
    state_term = rt * (N // 32) * 4
    state_update = (Q // 32) * (N // 16) * 4
    return b * H * nc * (diag + state_term + state_update) * 2 * 16 * 16 * 32


KERNEL_SOURCES = ("kernels.hpp", "device.hpp", "fused.hpp", "launch.hpp")


def kernel_source_hash() -> str:
    """Short digest of the kernel sources: a counter summary taken on other sources no
    longer describes the built kernels."""
    import hashlib
    import os
    h = hashlib.sha256()
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(here, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]
