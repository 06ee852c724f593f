"""The C ABI on the CPU: the library loads, exports every function include/ssd.h
declares, and rejects bad arguments on the host before any HIP call (no GPU needed:
the fake device addresses below are never dereferenced)."""
import ctypes
import os
import re

import pytest

import ssd_chunked_scan_03_amd as ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "ssd.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = ssd._load()
    declared = header_functions()
    assert set(declared) == set(ssd.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    assert ssd.version() == 100
    for code in range(8):
        s = ssd.status_string(code)
        assert isinstance(s, str) and s
    assert ssd.status_string(0) == "ok"
    assert ssd.status_string(99) == "unknown status"


def prob(b=2, T=300, H=4, P=64, N=128, G=2, Q=128, dtype=ssd.SSD_BF16):
    return ssd.make_problem(b, T, H, P, N, G, Q, dtype)


def test_workspace_layout_arithmetic():
    """The workspace holds the regions of the schedule that runs: cdt and C B^T always
    (C B^T for the scalar decay only), B^T and C per chunk for the fused schedule, chunk
    states and entering states for the split one."""
    nc = 3
    for flags in (0, ssd.SCHEDULE_SPLIT, ssd.SCHEDULE_FUSED):
        p = ssd.make_problem(2, 300, 4, 64, 128, 2, 128, ssd.SSD_BF16, flags)
        for diag in (False, True):
            fused = flags == ssd.SCHEDULE_FUSED and not diag  # 8 (batch, head) chains: split by default
            if flags == ssd.SCHEDULE_FUSED and diag:
                continue  # no fused diagonal-decay kernel
            lay = ssd.workspace_layout(p, diag)
            assert lay["cdt_bytes"] == 2 * 4 * nc * 128 * 4
            assert lay["cb_bytes"] == (0 if diag else 2 * nc * 2 * 128 * 128 * 2)
            assert lay["states_bytes"] == (0 if fused else 2 * 4 * nc * 64 * 128 * 2)  # in the input type
            assert lay["hin_bytes"] == (0 if fused else 2 * 4 * nc * 64 * 128 * 2)
            assert lay["bt_bytes"] == (2 * (2 * nc * 2 * 128 * 128 * 2) if fused else 0)  # B^T, then C
            assert lay["carry_bytes"] == 0  # 2 x 4 x 64 x 128 / 4 threads is not "few", and nc < 8
            offs = [lay[k] for k in ("cdt_off", "cb_off", "states_off", "hin_off", "bt_off", "carry_off")]
            assert all(o % 256 == 0 for o in offs) and offs == sorted(offs)
            assert lay["total_bytes"] >= lay["bt_off"] + lay["bt_bytes"]
            assert ssd.workspace_bytes(p, diag) == lay["total_bytes"]
    assert ssd.workspace_bytes(prob(T=0)) == 0
    assert ssd.workspace_bytes(prob(b=0)) == 0


def test_workspace_follows_the_schedule_at_the_layer_shape():
    """The 2.7B layer shape (b8 T4096 H80 P64 N128 G1 Q256, bf16) runs the fused schedule
    by default: its workspace is cdt + C B^T + B^T and C per chunk (about 44 MB), none of
    the split schedule's 335 MB of chunk states and entering states."""
    b, T, H, P, N, G, Q = 8, 4096, 80, 64, 128, 1, 256
    nc = T // Q
    cdt, cb, bt = b * H * nc * Q * 4, b * nc * G * Q * Q * 2, 2 * b * nc * G * N * Q * 2
    fused = ssd.workspace_layout(ssd.make_problem(b, T, H, P, N, G, Q, ssd.SSD_BF16))
    assert (fused["cdt_bytes"], fused["cb_bytes"], fused["bt_bytes"]) == (cdt, cb, bt)
    assert fused["states_bytes"] == fused["hin_bytes"] == fused["carry_bytes"] == 0
    assert fused["total_bytes"] == cdt + cb + bt == 44_040_192
    split = ssd.workspace_layout(ssd.make_problem(b, T, H, P, N, G, Q, ssd.SSD_BF16, ssd.SCHEDULE_SPLIT))
    assert split["bt_bytes"] == 0
    assert split["states_bytes"] == b * H * nc * P * N * 2 and split["hin_bytes"] == b * H * nc * P * N * 2
    assert split["total_bytes"] == cdt + cb + split["states_bytes"] + split["hin_bytes"]


def test_segmented_state_scan_workspace():
    """Few state elements (b H P N / 4 = 4096 threads) and 256 chunks: the state scan runs
    in 32 segments of 8 chunks (enough segments for about 128 K threads, at least 4 chunks
    each, at most 64), with one entering state per segment and one summed cdt total per
    (head, segment) in the carry region."""
    p = ssd.make_problem(1, 16384, 4, 64, 64, 1, 64, ssd.SSD_BF16)
    lay = ssd.workspace_layout(p)
    assert lay["carry_bytes"] == 32 * 4 * (64 * 64 + 1) * 4
    assert lay["bt_bytes"] == 0 and lay["carry_off"] >= lay["hin_off"] + lay["hin_bytes"]
    assert lay["total_bytes"] >= lay["carry_off"] + lay["carry_bytes"]
    # segments need at least 4 chunks each: 40 chunks allow 10
    p = ssd.make_problem(1, 40 * 64, 4, 64, 64, 1, 64, ssd.SSD_BF16)
    assert ssd.workspace_layout(p)["carry_bytes"] == 10 * 4 * (64 * 64 + 1) * 4
    # 7 chunks: one sequential pass
    assert ssd.workspace_layout(ssd.make_problem(1, 7 * 64, 4, 64, 64, 1, 64, ssd.SSD_BF16))["carry_bytes"] == 0


@pytest.mark.parametrize("kw,status", [
    (dict(H=6, G=4), 2), (dict(H=0), 2), (dict(P=0), 2), (dict(b=-1), 2), (dict(Q=0), 2),
    (dict(Q=96), 3), (dict(Q=512), 3), (dict(P=48), 3), (dict(N=512), 3), (dict(P=256), 3),
    (dict(dtype=7), 3),
])
def test_workspace_bytes_rejects_bad_problems(kw, status):
    p = prob(**kw)
    assert ssd.workspace_bytes(p) == 0
    lay = ssd.WorkspaceLayout()
    assert ssd._load().ssd_get_workspace_layout(ctypes.byref(p), 0, ctypes.byref(lay)) == status


BASE = 1 << 40  # fake, never dereferenced device addresses


def fake_ptrs(p, diag=False):
    """Disjoint fake device addresses for every argument of problem p (never used)."""
    lay_bytes = max(ssd.workspace_bytes(p, diag), 1)
    b, T, H, P, N, G = p.batch, p.seqlen, p.nheads, p.headdim, p.dstate, p.ngroups
    es = 2 if p.dtype == ssd.SSD_BF16 else 4
    sizes = dict(x=b * T * H * P * es, dt=b * T * H * 4, A=H * N * 4, B=b * T * G * N * es,
                 C=b * T * G * N * es, D=H * 4, h0=b * H * P * N * 4, y=b * T * H * P * es,
                 hT=b * H * P * N * 4, ws=lay_bytes)
    ptrs, cur = {}, BASE
    for k, n in sizes.items():
        ptrs[k] = cur
        cur += (n + (1 << 20)) // 4096 * 4096 + 4096
    return ptrs, lay_bytes


def call(p, diag=False, **over):
    """Call the entry point with fake well-formed pointers, some overridden.  Every use
    below makes the call invalid on purpose, so the host rejects it before any launch."""
    ptrs, lay_bytes = fake_ptrs(p, diag)
    ptrs.update(over)
    ws_bytes = over.pop("ws_bytes", lay_bytes) if "ws_bytes" in over else lay_bytes
    fn = ssd._load().ssd_diag_scan_fwd if diag else ssd._load().ssd_scan_fwd
    v = lambda k: ctypes.c_void_p(ptrs[k]) if ptrs[k] else None
    return fn(ctypes.byref(p), v("x"), v("dt"), v("A"), v("B"), v("C"), v("D"), v("h0"), v("y"),
              v("hT"), v("ws"), ws_bytes, None), ptrs


@pytest.mark.parametrize("diag", [False, True])
def test_error_paths_return_before_any_launch(diag):
    p = prob()
    assert call(p, diag, x=0)[0] == ssd_status("SSD_ERR_NULL")
    assert call(p, diag, y=0)[0] == ssd_status("SSD_ERR_NULL")
    assert call(p, diag, A=0)[0] == ssd_status("SSD_ERR_NULL")
    assert call(p, diag, ws=0)[0] == ssd_status("SSD_ERR_WORKSPACE")
    assert call(p, diag, ws_bytes=100)[0] == ssd_status("SSD_ERR_WORKSPACE")
    assert call(p, diag, x=BASE + 8)[0] == ssd_status("SSD_ERR_ALIGN")
    assert call(p, diag, hT=BASE + 4)[0] == ssd_status("SSD_ERR_ALIGN")
    assert call(p, diag, dt=BASE + 2)[0] == ssd_status("SSD_ERR_ALIGN")
    assert call(p, diag, ws=BASE + 16)[0] == ssd_status("SSD_ERR_ALIGN")
    ptrs, _ = fake_ptrs(prob(), diag)
    assert call(p, diag, y=ptrs["x"])[0] == ssd_status("SSD_ERR_ALIAS")
    assert call(p, diag, hT=ptrs["ws"])[0] == ssd_status("SSD_ERR_ALIAS")
    assert call(p, diag, hT=ptrs["y"])[0] == ssd_status("SSD_ERR_ALIAS")
    assert call(p, diag, y=ptrs["B"] + 256)[0] == ssd_status("SSD_ERR_ALIAS")
    assert call(prob(H=6, G=4), diag)[0] == ssd_status("SSD_ERR_SHAPE")
    assert call(prob(Q=32), diag)[0] == ssd_status("SSD_ERR_UNSUPPORTED")
    assert call(prob(N=24), diag)[0] == ssd_status("SSD_ERR_UNSUPPORTED")
    assert ssd._load().ssd_scan_fwd(None, *([None] * 10), 0, None) == ssd_status("SSD_ERR_NULL")


def test_diag_table_path_workspace():
    """The diagonal-decay output kernel keeps a chunk's x rows and rescaled C and B rows in
    LDS where they fit 160 KiB; otherwise a table kernel writes each (batch, head, chunk)'s
    decay-weighted query-key block into the cb region, batch * nheads * nchunks * chunk^2
    elements, which the output kernel reads (host arithmetic only)."""
    for (P, N, Q, dt, es) in ((64, 128, 256, ssd.SSD_BF16, 2), (64, 256, 256, ssd.SSD_BF16, 2),
                              (128, 256, 128, ssd.SSD_F32, 4), (64, 64, 128, ssd.SSD_BF16, 2)):
        p = prob(b=2, T=600, H=4, P=P, N=N, G=2, Q=Q, dtype=dt)
        nc = -(-600 // Q)
        lay = ssd.workspace_layout(p, True)
        tab = ssd.diag_uses_table(Q, P, N, dt)
        assert tab == ((Q * (P + 8) + 2 * Q * (N + 8)) * es + (2 * Q + N) * 4 > 160 * 1024)
        assert lay["cb_bytes"] == (2 * 4 * nc * Q * Q * es if tab else 0), (P, N, Q)
        assert lay["states_bytes"] == 2 * 4 * nc * P * N * es
    assert ssd.diag_uses_table(256, 64, 128, ssd.SSD_BF16) and not ssd.diag_uses_table(128, 64, 64, ssd.SSD_BF16)


def test_grid_limits_refused_on_the_host():
    """Shapes whose preparation launch would exceed a grid dimension are refused before any
    HIP call: ceil(nheads / 16) + 28 ngroups <= 65535 (the backward's table tasks at chunk
    256), batch * ngroups <= 65535."""
    ok = ssd.make_problem(1, 256, 2300, 64, 64, 2300, 256, ssd.SSD_BF16)  # 144 + 64400 tasks
    assert ssd.workspace_bytes(ok) > 0 and ssd.bwd_workspace_bytes(ok) > 0
    big = ssd.make_problem(1, 256, 2341 * 4, 64, 64, 2341, 256, ssd.SSD_BF16)  # 586 + 65548
    assert ssd.workspace_bytes(big) == 0 and ssd.bwd_workspace_bytes(big) == 0
    assert ssd.workspace_bytes(ssd.make_problem(2, 256, 65536, 64, 64, 32768, 64, ssd.SSD_BF16)) == 0


def test_schedule_flags_validated():
    p = prob()
    p.flags = ssd.SCHEDULE_SPLIT | ssd.SCHEDULE_FUSED
    assert call(p)[0] == ssd_status("SSD_ERR_UNSUPPORTED")
    p.flags = 0x400
    assert call(p)[0] == ssd_status("SSD_ERR_UNSUPPORTED")
    p = prob(P=32)
    p.flags = ssd.SCHEDULE_FUSED   # no fused kernel for headdim 32: rejected before any launch
    assert call(p)[0] == ssd_status("SSD_ERR_UNSUPPORTED")
    p = prob(dtype=ssd.SSD_F32)
    p.flags = ssd.SCHEDULE_FUSED
    assert call(p)[0] == ssd_status("SSD_ERR_UNSUPPORTED")


def test_stage_mask_must_name_kernels_of_the_running_schedule():
    """The workspace holds only the running schedule's regions, so a stage mask naming a
    kernel of the other schedule is refused before any launch."""
    p = prob(b=8, H=80, N=128, G=1)                   # fused by default
    for m in (ssd.STAGE_STATE, ssd.STAGE_SCAN, ssd.STAGE_OUT, ssd.STAGE_CUMSUM | ssd.STAGE_STATE):
        p.flags = m
        assert call(p)[0] == ssd_status("SSD_ERR_UNSUPPORTED"), m
    q = prob()                                       # split by default
    for m in (ssd.STAGE_BT, ssd.STAGE_FUSED):
        q.flags = m
        assert call(q)[0] == ssd_status("SSD_ERR_UNSUPPORTED"), m
        q.flags = m | ssd.SCHEDULE_SPLIT
        assert call(q)[0] == ssd_status("SSD_ERR_UNSUPPORTED"), m


def test_schedule_choice():
    assert ssd.schedule_of(prob(b=8, H=80, N=128, G=1), False) == "fused"
    assert ssd.schedule_of(prob(b=2, H=48, N=128, G=1), False) == "split"
    assert ssd.schedule_of(prob(b=8, H=80, N=128, G=1), True) == "split"
    p = prob(b=8, H=80, N=128, G=1)
    p.flags = ssd.SCHEDULE_SPLIT
    assert ssd.schedule_of(p, False) == "split"
    p.flags = ssd.SCHEDULE_FUSED
    assert ssd.schedule_of(p, False) == "fused"
    assert ssd.schedule_of(p, True) == "unsupported"
    p = prob(b=8, H=80, N=256, G=1)
    p.flags = ssd.SCHEDULE_FUSED
    assert ssd.schedule_of(p, False) == "unsupported"


def test_empty_batch_is_a_no_op():
    assert call(prob(b=0))[0] == 0


def ssd_status(name):
    return {v: k for k, v in ssd.STATUS.items()}[name]


def call_step(p, diag=False, **over):
    """ssd_step / ssd_diag_step with fake well-formed pointers, some overridden (every use
    below is invalid on purpose, so the host rejects it before any launch)."""
    ptrs, _ = fake_ptrs(p, diag)
    ptrs["h"] = ptrs.pop("h0")
    ptrs.update(over)
    fn = ssd._load().ssd_diag_step if diag else ssd._load().ssd_step
    v = lambda k: ctypes.c_void_p(ptrs[k]) if ptrs[k] else None
    return fn(ctypes.byref(p), v("x"), v("dt"), v("A"), v("B"), v("C"), v("D"), v("h"), v("y"), None)


@pytest.mark.parametrize("diag", [False, True])
def test_step_error_paths(diag):
    p = prob(T=1)
    assert call_step(p, diag, x=0) == ssd_status("SSD_ERR_NULL")
    assert call_step(p, diag, h=0) == ssd_status("SSD_ERR_NULL")
    assert call_step(p, diag, h=BASE + 8) == ssd_status("SSD_ERR_ALIGN")
    assert call_step(p, diag, B=BASE + 2) == ssd_status("SSD_ERR_ALIGN")
    ptrs, _ = fake_ptrs(p, diag)
    assert call_step(p, diag, y=ptrs["x"]) == ssd_status("SSD_ERR_ALIAS")
    assert call_step(p, diag, h=ptrs["B"]) == ssd_status("SSD_ERR_ALIAS")
    assert call_step(p, diag, y=ptrs["h0"]) == ssd_status("SSD_ERR_ALIAS")
    assert call_step(prob(T=1, H=6, G=4), diag) == ssd_status("SSD_ERR_SHAPE")
    assert call_step(prob(T=1, N=24), diag) == ssd_status("SSD_ERR_UNSUPPORTED")
    q = prob(T=1)
    q.flags = ssd.STAGE_CUMSUM
    assert call_step(q, diag) == ssd_status("SSD_ERR_UNSUPPORTED")
    # the chunk size plays no part in the recurrence: any value is accepted
    assert call_step(prob(T=0, Q=7), diag) == 0
    assert call_step(prob(b=0, T=1), diag) == 0
    assert ssd._load().ssd_step(None, *([None] * 8), None) == ssd_status("SSD_ERR_NULL")


def _align(v, a=256):
    return (v + a - 1) // a * a


def test_varlen_workspace_bytes_and_support():
    """Packed sequences run on the fused schedule: bf16, headdim 64, dstate 64/128.
    Workspace = cdt [H][kcap][Q] f32 + C B^T [kcap][G][Q][Q] + B^T [kcap][G][N][Q] and C
    [kcap][G][Q][N] (bf16) + two int32 row maps of nseq + 1 entries, kcap = ceil(T/Q) + nseq."""
    for nseq, T, H, N, G, Q in [(3, 1000, 8, 128, 1, 256), (7, 33, 4, 64, 2, 64), (1, 4096, 80, 128, 1, 128)]:
        p = ssd.make_problem(nseq, T, H, 64, N, G, Q, ssd.SSD_BF16)
        kcap = -(-T // Q) + nseq
        want = (_align(H * kcap * Q * 4) + _align(kcap * G * Q * Q * 2) + _align(2 * kcap * G * N * Q * 2)
                + 2 * _align((nseq + 1) * 4))
        assert ssd.varlen_workspace_bytes(p) == want
    for kw in ({"dtype": ssd.SSD_F32}, {"P": 32}, {"N": 256}, {"N": 32}, {"Q": 32}):
        a = dict(b=3, T=1000, H=8, P=64, N=128, G=1, Q=256, dtype=ssd.SSD_BF16)
        a.update(kw)
        p = ssd.make_problem(a["b"], a["T"], a["H"], a["P"], a["N"], a["G"], a["Q"], a["dtype"])
        assert ssd.varlen_workspace_bytes(p) == 0, kw
    assert ssd.varlen_workspace_bytes(ssd.make_problem(3, 0, 8, 64, 128, 1, 256, ssd.SSD_BF16)) == 0


def test_varlen_error_paths_return_before_any_launch():
    nseq, T, H, P, N, G, Q = 3, 300, 4, 64, 128, 2, 128
    p = ssd.make_problem(nseq, T, H, P, N, G, Q, ssd.SSD_BF16)
    need = ssd.varlen_workspace_bytes(p)
    sizes = {"cu": (nseq + 1) * 4, "x": T * H * P * 2, "dt": T * H * 4, "A": H * 4, "B": T * G * N * 2,
             "C": T * G * N * 2, "D": H * 4, "h0": nseq * H * P * N * 4, "y": T * H * P * 2,
             "hT": nseq * H * P * N * 4, "ws": need}
    ptrs, off = {}, BASE
    for k, n in sizes.items():
        ptrs[k] = off
        off += _align(n) + 4096
    fn = ssd._load().ssd_scan_fwd_varlen

    def run(prob=p, ws_bytes=need, **over):
        q = dict(ptrs, **over)
        v = lambda k: ctypes.c_void_p(q[k]) if q[k] else None
        return fn(ctypes.byref(prob), v("cu"), v("x"), v("dt"), v("A"), v("B"), v("C"), v("D"), v("h0"),
                  v("y"), v("hT"), v("ws"), ws_bytes, None)

    assert run(cu=0) == ssd_status("SSD_ERR_NULL")
    assert run(x=0) == ssd_status("SSD_ERR_NULL")
    assert run(A=0) == ssd_status("SSD_ERR_NULL")
    assert run(ws=0) == ssd_status("SSD_ERR_WORKSPACE")
    assert run(ws_bytes=need - 1) == ssd_status("SSD_ERR_WORKSPACE")
    assert run(cu=BASE + 2) == ssd_status("SSD_ERR_ALIGN")
    assert run(x=ptrs["x"] + 8) == ssd_status("SSD_ERR_ALIGN")
    assert run(ws=ptrs["ws"] + 16) == ssd_status("SSD_ERR_ALIGN")
    assert run(y=ptrs["x"]) == ssd_status("SSD_ERR_ALIAS")
    assert run(hT=ptrs["h0"]) == ssd_status("SSD_ERR_ALIAS")
    assert run(cu=ptrs["ws"] + 256) == ssd_status("SSD_ERR_ALIAS")
    assert run(y=ptrs["cu"]) == ssd_status("SSD_ERR_ALIAS")
    split = ssd.make_problem(nseq, T, H, P, N, G, Q, ssd.SSD_BF16, flags=ssd.SCHEDULE_SPLIT)
    assert run(prob=split) == ssd_status("SSD_ERR_UNSUPPORTED")
    f32 = ssd.make_problem(nseq, T, H, P, N, G, Q, ssd.SSD_F32)
    assert run(prob=f32) == ssd_status("SSD_ERR_UNSUPPORTED")
    assert run(prob=ssd.make_problem(nseq, T, 6, P, N, 4, Q, ssd.SSD_BF16)) == ssd_status("SSD_ERR_SHAPE")
    assert fn(None, *([None] * 11), 0, None) == ssd_status("SSD_ERR_NULL")
    # no sequences: nothing to do
    assert run(prob=ssd.make_problem(0, T, H, P, N, G, Q, ssd.SSD_BF16)) == 0


# ---- backward pass (ssd_scan_bwd) ----

def bwd_fake_ptrs(p, diag=False):
    b, T, H, P, N, G = p.batch, p.seqlen, p.nheads, p.headdim, p.dstate, p.ngroups
    es = 2 if p.dtype == ssd.SSD_BF16 else 4
    lay_bytes = max(ssd.bwd_workspace_bytes(p, diag), 1)
    xs, bc, st = b * T * H * P * es, b * T * G * N * es, b * H * P * N * 4
    an = H * N * 4 if diag else H * 4
    sizes = dict(x=xs, dt=b * T * H * 4, A=an, B=bc, C=bc, D=H * 4, h0=st, dy=xs, dhT=st,
                 dx=xs, ddt=b * T * H * 4, dA=an, dB=bc, dC=bc, dD=H * 4, dh0=st, ws=lay_bytes)
    ptrs, cur = {}, BASE
    for k, n in sizes.items():
        ptrs[k] = cur
        cur += (n + (1 << 20)) // 4096 * 4096 + 4096
    return ptrs, lay_bytes


BWD_ARGS = ("x", "dt", "A", "B", "C", "D", "h0", "dy", "dhT", "dx", "ddt", "dA", "dB", "dC", "dD", "dh0")


def call_bwd(p, diag=False, **over):
    """ssd_scan_bwd / ssd_diag_scan_bwd with fake well-formed pointers, some overridden;
    every use below is invalid on purpose, so the host rejects it before any launch."""
    ptrs, lay_bytes = bwd_fake_ptrs(p, diag)
    ws_bytes = over.pop("ws_bytes", lay_bytes)
    ptrs.update(over)
    v = lambda k: ctypes.c_void_p(ptrs[k]) if ptrs[k] else None
    f = ssd._load().ssd_diag_scan_bwd if diag else ssd._load().ssd_scan_bwd
    return f(ctypes.byref(p), *(v(k) for k in BWD_ARGS), v("ws"), ws_bytes, None), ptrs


def test_bwd_workspace_arithmetic():
    p = prob()  # b2 T300 H4 P64 N128 G2 Q128 bf16: 3 chunks
    b, H, P, N, G, Q, nc = 2, 4, 64, 128, 2, 128, 3
    a = lambda n: (n + 255) // 256 * 256
    # cdt, C B^T both ways, B^T and C^T per chunk, B and C per chunk by token (bf16, headdim
    # 64), chunk states (few chains: no walks), H_c and R_c, hT, ds, dD / dA partials, kpart
    want = (a(b * H * nc * Q * 4) + 2 * a(b * nc * G * Q * Q * 2) + 2 * a(b * nc * G * N * Q * 2)
            + 2 * a(b * nc * G * N * Q * 2)
            + a(b * H * nc * P * N * 4) + 2 * a(b * H * nc * P * N * 2) + a(b * H * P * N * 4)
            + a(b * H * nc * Q * 4) + a(b * H * nc * 4) + a(b * H * nc * 4)
            + a(b * H * nc * 4 * ((P * N // 4 + 255) // 256) * 4))
    assert ssd.bwd_workspace_bytes(p) == want
    assert ssd.bwd_workspace_bytes(prob(T=0)) == 0
    assert ssd.bwd_workspace_bytes(prob(b=0)) == 0
    assert ssd.bwd_workspace_bytes(prob(Q=96)) == 0
    p.flags = ssd.SCHEDULE_SPLIT
    assert ssd.bwd_workspace_bytes(p) == 0


def test_bwd_workspace_without_chunk_states_when_the_walks_run():
    """With 512 or more (batch, head) chains at bfloat16, headdim 64 and dstate 64 / 128 the
    chunk walks carry both recurrences on chip: no float32 chunk-state region (335 MB at the
    2.7B layer shape); float32, other headdims and fewer chains keep it.  At bfloat16,
    headdim 64 and dstate 64 / 128 (k_bwd_xs) B and C are also copied per chunk by token."""
    a = lambda n: (n + 255) // 256 * 256

    def want(b, T, H, P, N, G, Q, es, states):
        nc = -(-T // Q)
        copies = es == 2 and P == 64 and N in (64, 128)
        return (a(b * H * nc * Q * 4) + 2 * a(b * nc * G * Q * Q * es) + 2 * a(b * nc * G * N * Q * es)
                + (2 * a(b * nc * G * N * Q * es) if copies else 0)
                + (a(b * H * nc * P * N * 4) if states else 0) + 2 * a(b * H * nc * P * N * es)
                + a(b * H * P * N * 4) + a(b * H * nc * Q * 4) + 2 * a(b * H * nc * 4)
                + a(b * H * nc * 4 * ((P * N // 4 + 255) // 256) * 4))

    layer = (8, 4096, 80, 64, 128, 1, 256)
    assert ssd.bwd_workspace_bytes(ssd.make_problem(*layer, ssd.SSD_BF16)) == want(*layer, 2, False)
    assert ssd.bwd_workspace_bytes(ssd.make_problem(*layer, ssd.SSD_F32)) == want(*layer, 4, True)
    for shape, walks in (((8, 300, 64, 64, 64, 4, 128), True), ((1, 100, 515, 64, 64, 5, 64), True),
                         ((8, 300, 63, 64, 64, 3, 128), False), ((8, 300, 64, 32, 64, 4, 128), False),
                         ((8, 300, 64, 64, 256, 4, 128), False)):
        assert ssd.bwd_workspace_bytes(ssd.make_problem(*shape, ssd.SSD_BF16)) == want(*shape, 2, not walks), shape


def test_bwd_error_paths_return_before_any_launch():
    p = prob()
    S = ssd_status
    for k in ("x", "dt", "B", "C", "dy", "dx", "ddt", "dB", "dC", "A", "dA"):
        assert call_bwd(p, **{k: 0})[0] == S("SSD_ERR_NULL"), k
    assert call_bwd(p, ws=0)[0] == S("SSD_ERR_WORKSPACE")
    assert call_bwd(p, ws_bytes=100)[0] == S("SSD_ERR_WORKSPACE")
    for k, off in (("dy", 8), ("dx", 8), ("dB", 8), ("dhT", 4), ("dh0", 4), ("ddt", 2), ("dA", 2), ("ws", 16)):
        assert call_bwd(p, **{k: BASE + off})[0] == S("SSD_ERR_ALIGN"), k
    ptrs, _ = bwd_fake_ptrs(p)
    for out, inp in (("dx", "x"), ("dx", "dy"), ("dB", "C"), ("dC", "ws"), ("dh0", "dhT"), ("dA", "A"),
                     ("ddt", "dt"), ("dD", "dA"), ("dx", "dB"), ("dh0", "h0")):
        assert call_bwd(p, **{out: ptrs[inp]})[0] == S("SSD_ERR_ALIAS"), (out, inp)
    assert call_bwd(prob(H=6, G=4))[0] == S("SSD_ERR_SHAPE")
    assert call_bwd(prob(Q=32))[0] == S("SSD_ERR_UNSUPPORTED")
    assert call_bwd(prob(N=24))[0] == S("SSD_ERR_UNSUPPORTED")
    p = prob()
    p.flags = ssd.STAGE_CUMSUM
    assert call_bwd(p)[0] == S("SSD_ERR_UNSUPPORTED")
    assert ssd._load().ssd_scan_bwd(None, *([None] * 17), 0, None) == S("SSD_ERR_NULL")


def test_bwd_empty_problem_aliasing_checked():
    ptrs, _ = bwd_fake_ptrs(prob(T=0))
    assert call_bwd(prob(T=0), dA=ptrs["A"])[0] == ssd_status("SSD_ERR_ALIAS")
    assert call_bwd(prob(T=0), dh0=ptrs["dhT"])[0] == ssd_status("SSD_ERR_ALIAS")


# ---- backward pass of the diagonal decay (ssd_diag_scan_bwd) ----

def test_diag_bwd_workspace_arithmetic():
    a = lambda n: (n + 255) // 256 * 256
    for (b, T, H, P, N, G, Q, nsl) in ((2, 300, 4, 64, 64, 2, 128, 1), (2, 300, 4, 64, 128, 2, 128, 2),
                                       (1, 70, 2, 128, 256, 1, 64, 8), (1, 70, 2, 16, 256, 1, 64, 4)):
        p = ssd.make_problem(b, T, H, P, N, G, Q, ssd.SSD_BF16)
        nc = -(-T // Q)
        bhc = b * H * nc
        want = (a(bhc * Q * 4) + a(bhc * P * N * 4) + 2 * a(bhc * P * N * 2) + a(b * H * P * N * 4)
                + 2 * a(bhc * Q * N * 4) + ((a(nsl * b * T * H * P * 4) + a(nsl * b * T * H * 4)) if nsl > 1 else 0)
                + a(bhc * 4) + a(bhc * N * 4))
        assert ssd.bwd_workspace_bytes(p, diag=True) == want, (P, N)
    assert ssd.bwd_workspace_bytes(prob(T=0), diag=True) == 0
    assert ssd.bwd_workspace_bytes(prob(Q=96), diag=True) == 0
    p = prob()
    p.flags = ssd.SCHEDULE_SPLIT
    assert ssd.bwd_workspace_bytes(p, diag=True) == 0


def test_diag_bwd_error_paths_return_before_any_launch():
    p = prob()
    S = ssd_status
    for k in ("x", "dt", "B", "C", "dy", "dx", "ddt", "dB", "dC", "A", "dA"):
        assert call_bwd(p, True, **{k: 0})[0] == S("SSD_ERR_NULL"), k
    assert call_bwd(p, True, ws_bytes=ssd.bwd_workspace_bytes(p, True) - 1)[0] == S("SSD_ERR_WORKSPACE")
    for k, off in (("dy", 8), ("dx", 8), ("dB", 8), ("dhT", 4), ("dh0", 4), ("ddt", 2), ("dA", 2), ("ws", 16)):
        assert call_bwd(p, True, **{k: BASE + off})[0] == S("SSD_ERR_ALIGN"), k
    ptrs, _ = bwd_fake_ptrs(p, True)
    # dA is [H, N]: an overlap past the first H floats of A is still an overlap
    assert call_bwd(p, True, dA=ptrs["A"] + 4 * p.nheads)[0] == S("SSD_ERR_ALIAS")
    assert call_bwd(p, True, dD=ptrs["dA"] + 4 * p.nheads)[0] == S("SSD_ERR_ALIAS")
    for out, inp in (("dx", "x"), ("dB", "C"), ("dC", "ws"), ("dh0", "dhT"), ("ddt", "dt")):
        assert call_bwd(p, True, **{out: ptrs[inp]})[0] == S("SSD_ERR_ALIAS"), (out, inp)
    assert call_bwd(prob(H=6, G=4), True)[0] == S("SSD_ERR_SHAPE")
    assert call_bwd(prob(Q=32), True)[0] == S("SSD_ERR_UNSUPPORTED")
    assert ssd._load().ssd_diag_scan_bwd(None, *([None] * 17), 0, None) == S("SSD_ERR_NULL")
    # an empty problem checks dA against A over [H, N] too
    ptrs0, _ = bwd_fake_ptrs(prob(T=0), True)
    assert call_bwd(prob(T=0), True, dA=ptrs0["A"] + 4 * p.nheads)[0] == S("SSD_ERR_ALIAS")


def call_noalloc(p, **over):
    """ssd_scan_fwd_noalloc with fake well-formed pointers, some overridden (every use
    below is invalid on purpose, so the host rejects it before any HIP call)."""
    ptrs, _ = fake_ptrs(p)
    ptrs.update(over)
    v = lambda k: ctypes.c_void_p(ptrs[k]) if ptrs[k] else None
    return ssd._load().ssd_scan_fwd_noalloc(ctypes.byref(p), v("x"), v("dt"), v("A"), v("B"), v("C"), v("D"),
                                            v("h0"), v("y"), v("hT"), None)


def test_noalloc_forward_checks_before_any_hip_call():
    """The forward without caller workspace checks its arguments like ssd_scan_fwd, and a
    problem whose workspace exceeds the 64 MiB per-GPU scratch array is refused."""
    p = prob()
    assert call_noalloc(p, x=0) == ssd_status("SSD_ERR_NULL")
    assert call_noalloc(p, A=0) == ssd_status("SSD_ERR_NULL")
    assert call_noalloc(p, x=BASE + 8) == ssd_status("SSD_ERR_ALIGN")
    ptrs, _ = fake_ptrs(p)
    assert call_noalloc(p, y=ptrs["x"]) == ssd_status("SSD_ERR_ALIAS")
    assert call_noalloc(prob(Q=32)) == ssd_status("SSD_ERR_UNSUPPORTED")
    assert call_noalloc(prob(b=0)) == 0
    # the 2.7B layer's split schedule needs 538 MB of workspace: more than the scratch holds
    big = ssd.make_problem(8, 4096, 80, 64, 128, 1, 256, ssd.SSD_BF16, ssd.SCHEDULE_SPLIT)
    assert ssd.workspace_bytes(big) > ssd.NOALLOC_SCRATCH_BYTES
    assert call_noalloc(big) == ssd_status("SSD_ERR_WORKSPACE")
    # its fused schedule fits
    assert ssd.workspace_bytes(ssd.make_problem(8, 4096, 80, 64, 128, 1, 256, ssd.SSD_BF16)) \
        <= ssd.NOALLOC_SCRATCH_BYTES
    assert ssd._load().ssd_scan_fwd_noalloc(None, *([None] * 9), None) == ssd_status("SSD_ERR_NULL")
