"""GPU parity on seeded random shapes: forward (scalar and diagonal decay, both
schedules where they exist) and backward, against the fp64 oracle, with the bars of
the fixed-shape tests (per-slice max-norm relative error below 1e-4 for float32 and
2e-2 for bfloat16).

The shapes are drawn once from a fixed seed, over the whole supported set: batch 1-3,
seqlen 1 to three chunks and more (ragged tails included), 1-6 heads with every group
count that divides them, headdim 16-128, dstate 16-256, chunk 64/128/256.  Every forward
draw runs (the diagonal decay through its table of decay-weighted products where its
LDS tile of x rows and rescaled C and B rows would exceed 160 KiB).  A backward draw
outside the supported set must be refused with SSD_ERR_UNSUPPORTED and nothing else: the
scalar backward has no float32 headdim 128 at chunk 256 (the diagonal backward takes
every shape)."""
import numpy as np
import pytest
import torch

import ssd_chunked_scan_03_amd as ssd
from gpu_common import check, oracle_ref, run_gpu
from ssd_chunked_scan_03_amd.synth import make_grads, make_small
from test_gpu_bwd import check as check_bwd
from test_gpu_bwd import run_bwd

pytestmark = pytest.mark.gpu


def _draw(n, seed, diag_ok):
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(n):
        Q = int(rng.choice([64, 128, 256]))
        H = int(rng.integers(1, 7))
        G = int(rng.choice([g for g in range(1, H + 1) if H % g == 0]))
        out.append(dict(b=int(rng.integers(1, 4)), T=int(rng.integers(1, 3 * Q + 60)), H=H,
                        P=int(rng.choice([16, 32, 64, 128])), N=int(rng.choice([16, 32, 64, 128, 256])),
                        G=G, Q=Q, dtype=str(rng.choice(["f32", "bf16"])),
                        diag=bool(diag_ok and rng.random() < 0.4),
                        h0=bool(rng.random() < 0.7), D=bool(rng.random() < 0.7)))
    return out


FWD = _draw(24, 20261203, diag_ok=True)
BWD = _draw(12, 4051, diag_ok=False)
BWD_DIAG = [dict(c, diag=True) for c in _draw(10, 9176, diag_ok=False)]


def _diag_table(c):
    """The diagonal decay's output tile (x rows, rescaled C and B rows) exceeds 160 KiB:
    the table path runs."""
    es = 2 if c["dtype"] == "bf16" else 4
    Q, P, N = c["Q"], c["P"], c["N"]
    return c["diag"] and (Q * (P + 8) + 2 * Q * (N + 8)) * es + (2 * Q + N) * 4 > 160 * 1024


def _ident(c):
    return "b{b}T{T}H{H}P{P}N{N}G{G}Q{Q}-{dtype}-{d}".format(d="diag" if c["diag"] else "scalar", **c)


@pytest.mark.parametrize("c", FWD, ids=_ident)
def test_random_forward_matches_oracle(c):
    print(f"[random fwd] {_ident(c)} h0={c['h0']} D={c['D']}", flush=True)
    inp = make_small(c["b"], c["T"], c["H"], c["P"], c["N"], c["G"], seed=c["T"] + 7 * c["N"], diag=c["diag"],
                     dtype=c["dtype"], h0=c["h0"], D=c["D"])
    ref = oracle_ref(inp, c["diag"])
    check(run_gpu(inp, c["dtype"], c["Q"], c["diag"]), ref, c["dtype"], _ident(c))
    fused = c["dtype"] == "bf16" and not c["diag"] and c["P"] == 64 and c["N"] in (64, 128)
    for flags in (ssd.SCHEDULE_SPLIT, ssd.SCHEDULE_FUSED):
        if flags == ssd.SCHEDULE_FUSED and not fused:
            with pytest.raises(ssd.SSDError) as e:
                run_gpu(inp, c["dtype"], c["Q"], c["diag"], flags=flags)
            assert e.value.status == 3
            continue
        check(run_gpu(inp, c["dtype"], c["Q"], c["diag"], flags=flags), ref, c["dtype"], f"{_ident(c)} flags {flags}")


@pytest.mark.parametrize("c", BWD, ids=_ident)
def test_random_backward_matches_oracle(c):
    print(f"[random bwd] {_ident(c)} h0={c['h0']} D={c['D']}", flush=True)
    inp = make_small(c["b"], c["T"], c["H"], c["P"], c["N"], c["G"], seed=c["T"] + 11 * c["P"], dtype=c["dtype"])
    gr = make_grads(c["b"], c["T"], c["H"], c["P"], c["N"], seed=c["T"], dtype=c["dtype"])
    if c["dtype"] == "f32" and c["P"] == 128 and c["Q"] == 256:
        with pytest.raises(ssd.SSDError) as e:
            run_bwd(inp, gr, c["dtype"], c["Q"], use_D=c["D"], use_h0=c["h0"])
        assert e.value.status == 3
        return
    got, ref = run_bwd(inp, gr, c["dtype"], c["Q"], use_D=c["D"], use_h0=c["h0"])
    check_bwd(got, ref, c["dtype"], _ident(c))


@pytest.mark.parametrize("c", BWD_DIAG, ids=_ident)
def test_random_diag_backward_matches_oracle(c):
    from test_gpu_bwd_diag import check_diag
    print(f"[random bwd diag] {_ident(c)} h0={c['h0']} D={c['D']}", flush=True)
    inp = make_small(c["b"], c["T"], c["H"], c["P"], c["N"], c["G"], seed=c["T"] + 13 * c["N"], diag=True,
                     dtype=c["dtype"])
    gr = make_grads(c["b"], c["T"], c["H"], c["P"], c["N"], seed=c["T"] + 1, dtype=c["dtype"])
    got, ref = run_bwd(inp, gr, c["dtype"], c["Q"], use_D=c["D"], use_h0=c["h0"], diag=True)
    check_diag(got, ref, c["dtype"], _ident(c))


def test_random_draws_cover_the_support_set():
    """The draws reach every chunk, headdim, dstate and dtype, both decays, and refused
    as well as accepted forward problems (a host-only check of the lists above)."""
    for key, vals in (("Q", {64, 128, 256}), ("P", {16, 32, 64, 128}), ("N", {16, 32, 64, 128, 256}),
                      ("dtype", {"f32", "bf16"})):
        assert {c[key] for c in FWD} == vals, key
    assert {c["diag"] for c in FWD} == {False, True}
    assert any(_diag_table(c) for c in FWD) and any(c["diag"] and not _diag_table(c) for c in FWD)
    assert any(c["G"] > 1 for c in FWD + BWD) and any(c["T"] % c["Q"] for c in FWD + BWD)
    # the diagonal backward's draws reach every headdim and chunk, and dstate split into slices
    assert {c["P"] for c in BWD_DIAG} == {16, 32, 64, 128} and {c["Q"] for c in BWD_DIAG} == {64, 128, 256}
    assert any(c["P"] * c["N"] > 4096 or c["N"] > 64 for c in BWD_DIAG)
