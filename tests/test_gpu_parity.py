"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Metric: for y [b,T,H,P] and hT [b,H,P,N], the max over (b, h) slices of
||gpu - oracle||_inf / ||oracle||_inf; bar 1e-4 for float32 inputs, 2e-2 for
bfloat16 inputs with float32 accumulation.  Outputs and workspace are NaN-poisoned
before each call, so an element the kernels never write fails the comparison.
"""
import numpy as np
import pytest
import torch

import oracle
import ssd_chunked_scan_03_amd as ssd
from gpu_common import TOL, check, oracle_ref, run_gpu, upload
from helpers import max_rel_err, rel_h, rel_y
from ssd_chunked_scan_03_amd.configs import DIAG, LONG, LONG_CHUNKS, M2P7B, M780, TINY_F32
from ssd_chunked_scan_03_amd.synth import make_inputs, make_small

pytestmark = pytest.mark.gpu


def setup_module():
    print(f"[gpu parity] library {ssd.library_path()} version {ssd.version()}", flush=True)
    assert torch.cuda.is_available(), "GPU tests need a GPU"


SMALL = [  # b, T, H, P, N, G, Q, dtype, diag, h0, D
    (1, 64, 1, 16, 16, 1, 64, "f32", False, False, False),
    (2, 200, 4, 16, 32, 2, 64, "f32", False, True, True),
    (1, 333, 2, 32, 64, 1, 128, "f32", False, True, True),
    (2, 300, 4, 64, 128, 2, 128, "bf16", False, True, True),
    (1, 700, 3, 64, 128, 1, 256, "bf16", False, True, True),
    (1, 257, 2, 128, 64, 1, 256, "bf16", False, True, False),
    (1, 130, 8, 64, 256, 4, 64, "bf16", False, False, True),
    (2, 1, 2, 64, 128, 1, 256, "bf16", False, True, True),
    (1, 96, 2, 16, 16, 1, 64, "f32", True, True, True),
    (2, 300, 4, 64, 64, 2, 128, "f32", True, True, True),
    (1, 517, 2, 64, 64, 1, 128, "bf16", True, True, True),
    (1, 200, 2, 32, 128, 1, 64, "bf16", True, False, True),
    (1, 150, 2, 64, 32, 1, 256, "bf16", True, True, False),
    # diagonal decay through the table of decay-weighted products (LDS tile over 160 KiB)
    (1, 700, 3, 64, 128, 1, 256, "bf16", True, True, True),
    (2, 300, 4, 64, 256, 2, 256, "bf16", True, True, True),
    (1, 333, 2, 128, 256, 1, 128, "f32", True, True, False),
    (2, 129, 2, 16, 256, 2, 256, "f32", True, False, True),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "b{}T{}H{}P{}N{}G{}Q{}-{}-{}".format(
    *c[:8], "diag" if c[8] else "scalar"))
def test_small_shapes_match_oracle(case):
    b, T, H, P, N, G, Q, dtype, diag, h0, D = case
    print(f"[case] {case}", flush=True)
    inp = make_small(b, T, H, P, N, G, seed=1000 + T + P + N, diag=diag, dtype=dtype, h0=h0, D=D)
    check(run_gpu(inp, dtype, Q, diag), oracle_ref(inp, diag), dtype, str(case))


def frag_to_rows(t, R, Q):
    """A workspace table stored in matrix-core fragment order (include/ssd.h: the 16-row x
    32-column fragment (r / 16, col / 32) is 512 consecutive elements, lane 16 ((col % 32) / 8)
    + r % 16 holding 8 consecutive columns) back to rows of Q columns: [..., R * Q] -> [..., R, Q]."""
    r = np.arange(R)[:, None]
    col = np.arange(Q)[None, :]
    idx = ((r // 16) * (Q // 32) + col // 32) * 512 + ((col % 32) // 8) * 128 + (r % 16) * 8 + col % 8
    return t[..., idx]


@pytest.mark.parametrize("diag", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_stage_outputs_match_oracle_dumps(dtype, diag):
    """Each kernel's output in the workspace against the chunked oracle's stage dumps:
    cumulative step, C B^T blocks (lower part), chunk states, entering states."""
    b, T, H, P, N, G, Q = 2, 300, 4, 32, 64, 2, 128
    inp = make_small(b, T, H, P, N, G, seed=77, diag=diag, dtype=dtype)
    y, hT, ws, prob = run_gpu(inp, dtype, Q, diag, return_ws=True, flags=ssd.SCHEDULE_SPLIT)
    _, _, st = oracle.chunked(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"],
                              Q=Q, diag=diag, dumps=True)
    lay = ssd.workspace_layout(prob, diag)
    nc = (T + Q - 1) // Q
    td = torch.bfloat16 if dtype == "bf16" else torch.float32

    def view(off, nbytes, dt, shape):
        return ws[off:off + nbytes].view(dt).reshape(shape).float().cpu().numpy()
    cdt = view(lay["cdt_off"], lay["cdt_bytes"], torch.float32, (b, H, nc, Q))
    np.testing.assert_allclose(cdt, st["cdt"], rtol=2e-6, atol=1e-6)
    S = view(lay["states_off"], lay["states_bytes"], td, (b, H, nc, P, N))  # stored in the input type
    Hc = view(lay["hin_off"], lay["hin_bytes"], td, (b, H, nc, P, N))
    tol = TOL[dtype]
    assert max_rel_err(S, st["S"], (0, 1, 2)) < tol
    assert max_rel_err(Hc, st["Hc"], (0, 1, 2)) < tol
    if not diag:
        cb = frag_to_rows(view(lay["cb_off"], lay["cb_bytes"], td, (b, nc, G, Q * Q)), Q, Q)
        ref = st["G"]
        low = np.tril(np.ones((Q, Q), dtype=bool))
        for c in range(nc):
            valid = min(Q, T - c * Q)
            m = low.copy()
            m[valid:, :] = False
            m[:, valid:] = False
            got, want = cb[:, c][..., m], ref[:, c][..., m]
            assert np.abs(got - want).max() <= tol * np.abs(want).max()
        # above the diagonal, inside the 64 x 64 blocks on it, the table holds exact zeros
        up = np.triu(np.ones((64, 64), dtype=bool), 1)
        for blk in range(Q // 64):
            sl = slice(64 * blk, 64 * blk + 64)
            assert np.all(cb[..., sl, sl][..., up] == 0)
    check((y, hT), oracle_ref(inp, diag), dtype, "stage case end-to-end")


FUSED = [  # b, T, H, P, N, G, Q, h0, D   (bf16, scalar decay; fused schedule forced)
    (1, 64, 1, 64, 64, 1, 64, False, False),
    (2, 300, 4, 64, 128, 2, 128, True, True),
    (1, 700, 3, 64, 128, 1, 256, True, True),
    (2, 1000, 2, 64, 64, 1, 256, True, False),
    (1, 257, 8, 64, 128, 4, 64, False, True),
    (3, 512, 2, 64, 128, 2, 256, True, True),
    (1, 1, 2, 64, 128, 1, 256, True, True),
]


@pytest.mark.parametrize("case", FUSED, ids=lambda c: "b{}T{}H{}P{}N{}G{}Q{}".format(*c[:7]))
def test_fused_schedule_matches_oracle(case):
    """The fused per-(batch, head) kernel (state kept on chip across chunks)."""
    b, T, H, P, N, G, Q, h0, D = case
    print(f"[fused case] {case}", flush=True)
    inp = make_small(b, T, H, P, N, G, seed=2000 + T + N, dtype="bf16", h0=h0, D=D)
    check(run_gpu(inp, "bf16", Q, False, flags=ssd.SCHEDULE_FUSED), oracle_ref(inp, False), "bf16", str(case))


@pytest.mark.parametrize("decay", ["one", "zero", "strong", "mixed"])
def test_fused_schedule_decay_extremes(decay):
    """The fused kernel splits each diagonal block's decay into two factors when every
    32-token block of the chunk decays by at most 2^64, and takes direct exponentials
    otherwise.  a = 1 (A = 0), a = 0 (dt A = -1e7 per token), strong decays (A = -60:
    every chunk direct) and per-head mixtures (some chunks each way) against the oracle."""
    b, T, H, P, N, G, Q = 2, 700, 4, 64, 128, 2, 256
    inp = make_small(b, T, H, P, N, G, seed=61, dtype="bf16")
    A = {"one": [0.0] * H, "zero": [-1e7] * H, "strong": [-60.0] * H, "mixed": [-0.5, -14.0, -40.0, 0.0]}[decay]
    inp["A"] = np.asarray(A, dtype=np.float32)
    if decay == "mixed":
        inp["dt"][:, 300:500, :] = 0.1  # one stretch of fast decay in every head
    check(run_gpu(inp, "bf16", Q, False, flags=ssd.SCHEDULE_FUSED), oracle_ref(inp, False), "bf16", decay)


def test_fused_and_split_agree():
    """Both schedules on the same inputs agree within the bf16 bar (not bitwise: the
    fused kernel rounds the carried state to bf16 only as an MFMA operand)."""
    inp = make_small(2, 777, 4, 64, 128, 1, seed=31, dtype="bf16")
    yf, hf = run_gpu(inp, "bf16", 256, False, flags=ssd.SCHEDULE_FUSED)
    ys, hs = run_gpu(inp, "bf16", 256, False, flags=ssd.SCHEDULE_SPLIT)
    assert rel_y(yf, ys) < TOL["bf16"] and rel_h(hf, hs) < TOL["bf16"]


def test_fused_unsupported_is_reported():
    inp = make_small(1, 64, 2, 32, 64, 1, seed=1, dtype="bf16")
    with pytest.raises(ssd.SSDError) as e:
        run_gpu(inp, "bf16", 64, False, flags=ssd.SCHEDULE_FUSED)
    assert e.value.status == 3


@pytest.mark.parametrize("w", [TINY_F32, M780, DIAG], ids=lambda w: w.name)
def test_workload_full_parity(w):
    print(f"[workload] {w.name}", flush=True)
    inp = make_inputs(w)
    check(run_gpu(inp, w.dtype, w.chunk, w.diag), oracle_ref(inp, w.diag), w.dtype, w.name)


_FULL = {}


def full_reference(w, **kw):
    """Inputs and the oracle's (y, hT) for a whole workload, computed once per process (the
    oracle does not depend on the chunk size or the schedule, so every run of the
    workload is compared with the same reference)."""
    key = (w.name, w.seqlen, w.diag, tuple(sorted(kw.items())))
    if key not in _FULL:
        _FULL.clear()  # one whole workload's reference held at a time
        inp = make_inputs(w, **kw)
        _FULL[key] = (inp, oracle_ref(inp, w.diag))
    return _FULL[key]


def full_parity(w, chunk, flags=0, **kw):
    """The whole workload on the GPU against the oracle on the whole workload: y and hT
    compared on every (batch, head) slice, batch row by batch row to bound host memory."""
    inp, (yr, hr) = full_reference(w, **kw)
    y, hT = run_gpu(inp, w.dtype, chunk, w.diag, flags=flags)
    ey = max(rel_y(y[bi:bi + 1], yr[bi:bi + 1]) for bi in range(w.batch))
    eh = rel_h(hT, hr)
    print(f"[full parity] {w.name} Q={chunk} flags={flags:#x}: y {ey:.3e} hT {eh:.3e}", flush=True)
    assert ey < TOL[w.dtype] and eh < TOL[w.dtype], (w.name, chunk, flags, ey, eh)
    return y, hT


@pytest.mark.parametrize("schedule", ["default", "split"])
def test_headline_workload_full_parity(schedule):
    """Mamba-2 2.7B layer shape (b8 T4096 H80 P64 N128, Q256, nonzero h0) in full, every
    (batch, head) slice of y and hT, with the default schedule (fused: 640 (batch, head)
    chains) and with the split one."""
    w = M2P7B
    print(f"[workload] {w.name} {schedule}", flush=True)
    full_parity(w, w.chunk, ssd.SCHEDULE_SPLIT if schedule == "split" else 0)


@pytest.mark.parametrize("chunk", LONG_CHUNKS)
def test_long_workload_full_parity(chunk):
    """T = 65536, N = 256, 8 groups, in full at each chunk size of the sweep."""
    w = LONG
    print(f"[workload] {w.name} Q={chunk}", flush=True)
    full_parity(w, chunk)


def test_diag_equal_decays_match_scalar_kernel():
    """The diagonal-decay workload's shape in full (b4 T4096 H32 P64 N64 Q128) with
    A[h, n] = A[h, 0] for all n: the diagonal kernels reproduce the scalar-decay kernels'
    result, and both match the oracle's scalar-decay result on every slice."""
    w = DIAG
    inp = make_inputs(w, diag_equal_A=True)
    yd, hd = run_gpu(inp, w.dtype, w.chunk, True)
    s = dict(inp)
    s["A"] = np.ascontiguousarray(inp["A"][:, 0])
    ys, hs = run_gpu(s, w.dtype, w.chunk, False)
    e = (rel_y(yd, ys), rel_h(hd, hs))
    print(f"[diag equal A] diag vs scalar kernel: y {e[0]:.3e} hT {e[1]:.3e}", flush=True)
    assert e[0] < TOL["bf16"] and e[1] < TOL["bf16"]
    ref = oracle_ref(s, False)
    check((yd, hd), ref, "bf16", "diag-equal vs oracle scalar")
    check((ys, hs), ref, "bf16", "scalar kernel vs oracle scalar")


def test_diag_decay_at_the_layer_shape_full_parity():
    """The diagonal decay at the 2.7B layer shape (b8 T4096 H80 P64 N128 Q256, bf16,
    A[h, n] drawn per head and state dimension, nonzero h0): its output tile does not fit
    LDS, so it runs through the table of decay-weighted products; every (batch, head)
    slice of y and hT against the oracle."""
    w = M2P7B.with_(diag=True)
    print(f"[workload] {w.name} diagonal decay", flush=True)
    prob = ssd.make_problem(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk, ssd.SSD_BF16)
    assert ssd.workspace_layout(prob, True)["cb_bytes"] > 0  # the table path
    full_parity(w, w.chunk)


@pytest.mark.parametrize("diag", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decay_one_and_zero(dtype, diag):
    """a = 1 (A = 0): causal linear attention; a = 0 (dt * A <= -1e4, finite): per-token
    output (C_t . B_t) x_t + D x_t and hT = x_{T-1} B_{T-1}^T."""
    b, T, H, P, N, G, Q = 1, 300, 2, 32, 64, 1, 128
    for A_val in (0.0, -1e7):
        inp = make_small(b, T, H, P, N, G, seed=5, diag=diag, dtype=dtype)
        inp["A"] = np.full(inp["A"].shape, A_val, dtype=np.float32)
        check(run_gpu(inp, dtype, Q, diag), oracle_ref(inp, diag), dtype, f"A={A_val}")


def test_bitwise_deterministic():
    inp = make_small(2, 600, 4, 64, 128, 1, seed=9, dtype="bf16")
    r1 = run_gpu(inp, "bf16", 256, False)
    r2 = run_gpu(inp, "bf16", 256, False)
    assert np.array_equal(r1[0], r2[0]) and np.array_equal(r1[1], r2[1])
    inp = make_small(1, 300, 2, 64, 64, 1, seed=9, dtype="bf16", diag=True)
    r1 = run_gpu(inp, "bf16", 128, True)
    r2 = run_gpu(inp, "bf16", 128, True)
    assert np.array_equal(r1[0], r2[0]) and np.array_equal(r1[1], r2[1])


def test_empty_sequence_and_batch():
    inp = make_small(2, 5, 2, 16, 16, 1, seed=1)
    d = upload(inp, "f32")
    x0 = d["x"][:, :0].contiguous()
    B0, C0, dt0 = d["B"][:, :0].contiguous(), d["C"][:, :0].contiguous(), d["dt"][:, :0].contiguous()
    y, hT = ssd.scan_fwd(x0, dt0, d["A"], B0, C0, d["D"], d["h0"], chunk=64)
    torch.cuda.synchronize()
    assert y.shape == (2, 0, 2, 16)
    assert torch.equal(hT, d["h0"])
    y, hT = ssd.scan_fwd(x0, dt0, d["A"], B0, C0, d["D"], None, chunk=64)
    torch.cuda.synchronize()
    assert torch.count_nonzero(hT) == 0


def test_python_api_and_stream():
    """scan_fwd/diag_scan_fwd on a side stream, hT optional."""
    inp = make_small(1, 260, 2, 64, 128, 1, seed=3, dtype="bf16")
    d = upload(inp, "bf16")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y, hT = ssd.scan_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=128)
        y2, none = ssd.scan_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=128,
                                return_final_state=False)
    s.synchronize()
    assert none is None
    assert torch.equal(y, y2)
    check((y.float().cpu().numpy(), hT.cpu().numpy()), oracle_ref(inp, False), "bf16", "api")


SEGMENTED = [  # b, T, H, P, N, G, Q, dtype, diag -- few state elements, many chunks
    (1, 16384, 4, 64, 64, 1, 64, "bf16", False),      # 256 chunks: 32 segments of 8
    (1, 41 * 64 + 5, 4, 64, 64, 2, 64, "bf16", False),  # 42 chunks, ragged: 9 segments of 5 (last 2)
    (1, 8192, 2, 64, 64, 1, 64, "f32", True),         # diagonal decay: 32 segments of 4
    (2, 4096, 2, 32, 32, 1, 64, "f32", False),        # 64 chunks: 16 segments of 4
]


@pytest.mark.parametrize("case", SEGMENTED, ids=lambda c: "b{}T{}H{}P{}N{}G{}Q{}{}{}".format(*c[:8], "D" if c[8] else "S"))
def test_segmented_state_scan_matches_oracle(case):
    """The split schedule's state scan as a parallel scan over segments of chunks (few
    state elements, many chunks): end to end against the oracle, and every chunk's
    entering state against the chunked oracle's dumps."""
    b, T, H, P, N, G, Q, dtype, diag = case
    print(f"[segmented case] {case}", flush=True)
    inp = make_small(b, T, H, P, N, G, seed=91, diag=diag, dtype=dtype)
    y, hT, ws, prob = run_gpu(inp, dtype, Q, diag, return_ws=True, flags=ssd.SCHEDULE_SPLIT)
    lay = ssd.workspace_layout(prob, diag)
    assert lay["carry_bytes"] > 0, "this shape should run the state scan in segments"
    check((y, hT), oracle_ref(inp, diag), dtype, f"segmented {case}")
    nc = (T + Q - 1) // Q
    _, _, st = oracle.chunked(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"],
                              Q=Q, diag=diag, dumps=True)
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    Hc = ws[lay["hin_off"]:lay["hin_off"] + lay["hin_bytes"]].view(td).reshape(b, H, nc, P, N).float().cpu().numpy()
    assert max_rel_err(Hc, st["Hc"], (0, 1, 2)) < TOL[dtype]


@pytest.mark.parametrize("schedule,N,Q", [("fused", 128, 128), ("split", 128, 128), ("split", 256, 256),
                                          ("split", 256, 128)])
def test_prep_launch_matches_separate_stage_kernels(schedule, N, Q):
    """A whole forward runs its preparation (cumsum, C B^T, and B^T on the fused schedule)
    as one k_prep launch; a forward enqueued one kernel per stage runs the separate
    kernels (at dstate 256 k_prep takes a whole 64-row block row of C B^T per work-group,
    k_cb one tile).  Same arithmetic per element, so y and hT agree bit for bit."""
    from gpu_common import upload
    inp = make_small(2, 700, 8, 64, N, 2, seed=41, dtype="bf16")
    d = upload(inp, "bf16")
    b, T, H, P = d["x"].shape
    G, N = d["B"].shape[2], d["B"].shape[3]
    sf = ssd.SCHEDULE_FUSED if schedule == "fused" else ssd.SCHEDULE_SPLIT
    outs = []
    for staged in (False, True):
        base = ssd.make_problem(b, T, H, P, N, G, Q, ssd.SSD_BF16, sf)
        y = torch.full_like(d["x"], float("nan"))
        hT = torch.full((b, H, P, N), float("nan"), device="cuda")
        ws = torch.full((ssd.workspace_bytes(base),), 0xFF, dtype=torch.uint8, device="cuda")
        kernels = ssd.FUSED_KERNELS if schedule == "fused" else ssd.SPLIT_KERNELS
        masks = [ssd.STAGES[k] for k in kernels] if staged else [0]
        for m in masks:
            p = ssd.make_problem(b, T, H, P, N, G, Q, ssd.SSD_BF16, sf | m)
            ssd.scan_fwd_into(p, False, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], y, hT, ws)
        torch.cuda.synchronize()
        outs.append((y.float().cpu().numpy(), hT.cpu().numpy()))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])
