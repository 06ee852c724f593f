"""MI355X-native SSD chunked scan (the Mamba-2 core layer): forward and backward passes.

Thin Python binding over ``libssd.so`` (C ABI in ``include/ssd.h``): argument
marshalling only -- every step of the scan runs in the library's HIP kernels.
PyTorch supplies device memory and the stream.  If the library is missing or fails
to load, every call raises: there is no fallback path.

    y, hT = scan_fwd(x, dt, A, B, C, D=None, h0=None, chunk=256)
    y, hT = diag_scan_fwd(x, dt, A, B, C, D=None, h0=None, chunk=128)
    grads = scan_bwd(x, dt, A, B, C, dy, D=None, h0=None, dhT=None, chunk=256)

Layouts: x [b,T,H,P]; dt [b,T,H] f32; A [H] (scalar decay) or [H,N] (diagonal
decay) f32; B, C [b,T,G,N]; D [H] f32; h0 [b,H,P,N] f32.  x/B/C share one dtype,
bfloat16 or float32; y has that dtype, hT is float32.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["scan_fwd", "diag_scan_fwd", "scan_fwd_into", "scan_bwd", "scan_bwd_into", "bwd_workspace_bytes",
           "Problem", "workspace_bytes",
           "workspace_layout", "status_string", "version", "library_path", "SSDError"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libssd.so")
_lib = None

SSD_F32, SSD_BF16 = 0, 1
STATUS = {0: "SSD_OK", 1: "SSD_ERR_NULL", 2: "SSD_ERR_SHAPE", 3: "SSD_ERR_UNSUPPORTED",
          4: "SSD_ERR_WORKSPACE", 5: "SSD_ERR_ALIGN", 6: "SSD_ERR_ALIAS", 7: "SSD_ERR_HIP"}
EXPORTS = ("ssd_workspace_bytes", "ssd_get_workspace_layout", "ssd_scan_fwd", "ssd_scan_fwd_noalloc",
           "ssd_diag_scan_fwd",
           "ssd_varlen_workspace_bytes", "ssd_scan_fwd_varlen",
           "ssd_step", "ssd_diag_step", "ssd_bwd_workspace_bytes", "ssd_scan_bwd",
           "ssd_diag_bwd_workspace_bytes", "ssd_diag_scan_bwd",
           "ssd_status_string", "ssd_version")


class SSDError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status_string(status)})")


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("chunk", ctypes.c_int64), ("dtype", ctypes.c_int32), ("flags", ctypes.c_int32)]


class WorkspaceLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("cdt_off", "cdt_bytes", "cb_off", "cb_bytes", "states_off", "states_bytes",
                 "hin_off", "hin_bytes", "bt_off", "bt_bytes", "carry_off", "carry_bytes", "total_bytes")]


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"libssd.so not built ({_LIB_PATH}); run `python -m ssd_chunked_scan_03_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER(Problem)
    vp, fp, sz, ci = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.ssd_workspace_bytes.argtypes = [P, ci]
    lib.ssd_workspace_bytes.restype = sz
    lib.ssd_get_workspace_layout.argtypes = [P, ci, ctypes.POINTER(WorkspaceLayout)]
    lib.ssd_get_workspace_layout.restype = ci
    for f in (lib.ssd_scan_fwd, lib.ssd_diag_scan_fwd):
        f.argtypes = [P, vp, fp, fp, vp, vp, fp, fp, vp, fp, vp, sz, vp]
        f.restype = ci
    lib.ssd_scan_fwd_noalloc.argtypes = [P, vp, fp, fp, vp, vp, fp, fp, vp, fp, vp]
    lib.ssd_scan_fwd_noalloc.restype = ci
    lib.ssd_varlen_workspace_bytes.argtypes = [P]
    lib.ssd_varlen_workspace_bytes.restype = sz
    lib.ssd_scan_fwd_varlen.argtypes = [P, vp, vp, fp, fp, vp, vp, fp, fp, vp, fp, vp, sz, vp]
    lib.ssd_scan_fwd_varlen.restype = ci
    for f in (lib.ssd_step, lib.ssd_diag_step):
        f.argtypes = [P, vp, fp, fp, vp, vp, fp, fp, vp, vp]
        f.restype = ci
    for f in (lib.ssd_bwd_workspace_bytes, lib.ssd_diag_bwd_workspace_bytes):
        f.argtypes = [P]
        f.restype = sz
    for f in (lib.ssd_scan_bwd, lib.ssd_diag_scan_bwd):
        f.argtypes = [P, vp, fp, fp, vp, vp, fp, fp, vp, fp, vp, fp, fp, vp, vp, fp, fp, vp, sz, vp]
        f.restype = ci
    lib.ssd_status_string.argtypes = [ci]
    lib.ssd_status_string.restype = ctypes.c_char_p
    lib.ssd_version.argtypes = []
    lib.ssd_version.restype = ci
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return _load().ssd_status_string(int(status)).decode()


def version() -> int:
    return int(_load().ssd_version())


STAGE_CUMSUM, STAGE_CB, STAGE_STATE, STAGE_SCAN, STAGE_OUT = 0x01, 0x02, 0x04, 0x08, 0x10
STAGE_BT, STAGE_FUSED = 0x20, 0x40
SCHEDULE_SPLIT, SCHEDULE_FUSED = 0x100, 0x200
STAGES = {"k_cumsum": STAGE_CUMSUM, "k_cb": STAGE_CB, "k_state": STAGE_STATE, "k_scan": STAGE_SCAN,
          "k_out": STAGE_OUT, "k_bt": STAGE_BT, "k_fused": STAGE_FUSED}
SPLIT_KERNELS = ("k_cumsum", "k_cb", "k_state", "k_scan", "k_out")
FUSED_KERNELS = ("k_cumsum", "k_cb", "k_bt", "k_fused")


def diag_uses_table(chunk, headdim, dstate, dtype_code) -> bool:
    """Whether the diagonal decay's output kernel reads a per-(batch, head, chunk) table of
    decay-weighted query-key products (its LDS tile of x rows and rescaled C / B rows
    would not fit one CU's 160 KiB)."""
    es = 2 if dtype_code == SSD_BF16 else 4
    return (chunk * (headdim + 8) + 2 * chunk * (dstate + 8)) * es + (2 * chunk + dstate) * 4 > 160 * 1024


def schedule_kernels(schedule: str, diag: bool, prob: "Problem" = None):
    """(kernel name, stage mask) in the order a whole forward launches them.  A whole
    forward runs its preparation (cumsum, C B^T, and B^T on the fused schedule) as one
    launch, k_prep; a stage mask that holds all of those bits runs that same launch.
    The diagonal decay's table kernel, where it runs (see diag_uses_table), is the C B^T
    stage."""
    if schedule == "fused":
        return [("k_prep", STAGE_CUMSUM | STAGE_CB | STAGE_BT), ("k_fused", STAGE_FUSED)]
    first = [("k_cumsum", STAGE_CUMSUM)] if diag else [("k_prep", STAGE_CUMSUM | STAGE_CB)]
    if diag and prob is not None and diag_uses_table(prob.chunk, prob.headdim, prob.dstate, prob.dtype):
        first.append(("k_gtab", STAGE_CB))
    return first + [("k_state", STAGE_STATE), ("k_scan", STAGE_SCAN), ("k_out", STAGE_OUT)]


def fused_supported(dtype_code, diag, P, N) -> bool:
    """Whether the fused per-(batch, head) kernel exists for this problem."""
    return dtype_code == SSD_BF16 and not diag and P == 64 and N in (64, 128)


def schedule_of(prob: "Problem", diag: bool) -> str:
    """The schedule the library runs for flags without a stage mask."""
    if prob.flags & SCHEDULE_SPLIT:
        return "split"
    nc = (prob.seqlen + prob.chunk - 1) // prob.chunk
    lim = 1 << 31  # the fused kernel's per-batch-row tables use 32-bit offsets
    fits = (prob.seqlen * prob.nheads * prob.headdim * 2 < lim and prob.seqlen * prob.ngroups * prob.dstate * 2 < lim
            and nc * prob.ngroups * prob.chunk * max(prob.chunk, prob.dstate) * 2 < lim)
    ok = fused_supported(prob.dtype, diag, prob.headdim, prob.dstate) and fits
    if prob.flags & SCHEDULE_FUSED:
        return "fused" if ok else "unsupported"
    return "fused" if ok and prob.batch * prob.nheads >= 512 else "split"


def make_problem(b, T, H, P, N, G, chunk, dtype, flags=0) -> Problem:
    """flags = 0 runs the whole forward; a mask of STAGE_* bits runs only those kernels
    (diagnostics: earlier stages are read from a workspace a full call filled)."""
    return Problem(int(b), int(T), int(H), int(P), int(N), int(G), int(chunk), int(dtype), int(flags))


def workspace_bytes(prob: Problem, diag: bool = False) -> int:
    return int(_load().ssd_workspace_bytes(ctypes.byref(prob), int(bool(diag))))


def workspace_layout(prob: Problem, diag: bool = False) -> dict:
    lay = WorkspaceLayout()
    st = _load().ssd_get_workspace_layout(ctypes.byref(prob), int(bool(diag)), ctypes.byref(lay))
    if st:
        raise SSDError(st, "ssd_get_workspace_layout")
    return {n: int(getattr(lay, n)) for n, _ in WorkspaceLayout._fields_}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def scan_fwd_into(prob: Problem, diag: bool, x, dt, A, B, C, D, h0, y, hT, ws, stream=None) -> None:
    """Enqueue one forward into caller-provided outputs and workspace (no allocation)."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    lib = _load()
    fn = lib.ssd_diag_scan_fwd if diag else lib.ssd_scan_fwd
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = fn(ctypes.byref(prob), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0),
            _ptr(y), _ptr(hT), _ptr(ws), nbytes, ctypes.c_void_p(int(stream)))
    if st:
        raise SSDError(st, "ssd_diag_scan_fwd" if diag else "ssd_scan_fwd")


NOALLOC_SCRATCH_BYTES = 64 << 20


def scan_fwd_noalloc_into(prob: Problem, x, dt, A, B, C, D, h0, y, hT, stream=None) -> None:
    """Enqueue one scalar-decay forward into caller-provided outputs, with the library's
    per-GPU scratch array as workspace (no allocation anywhere; calls on one GPU must be
    ordered on one stream)."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    st = _load().ssd_scan_fwd_noalloc(ctypes.byref(prob), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                      _ptr(h0), _ptr(y), _ptr(hT), ctypes.c_void_p(int(stream)))
    if st:
        raise SSDError(st, "ssd_scan_fwd_noalloc")


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return SSD_BF16
    if t.dtype == torch.float32:
        return SSD_F32
    raise TypeError(f"x/B/C must be bfloat16 or float32, got {t.dtype}")


def _check_args(shapes, floats, same_dtype):
    """Host-side checks of a call's tensors before anything is enqueued: every expected
    shape (name -> (tensor or None, shape)), float32 where required, one shared dtype
    (bfloat16 or float32) for x-like tensors, and contiguous tensors on one GPU.  The C ABI
    sees only pointers and sizes, so a short or mistyped buffer would otherwise be read or
    written out of bounds by the kernels."""
    import torch
    for name, (t, shape) in shapes.items():
        if t is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    for name in floats:
        t = shapes[name][0]
        if t is not None and t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32, got {t.dtype}")
    first = shapes[same_dtype[0]][0]
    _dtype_code(first)
    for name in same_dtype[1:]:
        if shapes[name][0].dtype != first.dtype:
            raise TypeError(f"{', '.join(same_dtype)} must share one dtype")
    dev = None
    for name, (t, _) in shapes.items():
        if t is None:
            continue
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")


def _forward(diag, x, dt, A, B, C, D, h0, chunk, return_final_state, ws):
    import torch
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be [b, T, H, P] and B [b, T, G, N]")
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    _check_args({"x": (x, (b, T, H, P)), "dt": (dt, (b, T, H)), "A": (A, (H, N) if diag else (H,)),
                 "B": (B, (b, T, G, N)), "C": (C, (b, T, G, N)), "D": (D, (H,)), "h0": (h0, (b, H, P, N))},
                floats=("dt", "A", "D", "h0"), same_dtype=("x", "B", "C"))
    prob = make_problem(b, T, H, P, N, G, chunk, _dtype_code(x))
    y = torch.empty_like(x)
    hT = torch.empty((b, H, P, N), dtype=torch.float32, device=x.device) if return_final_state else None
    need = workspace_bytes(prob, diag)
    if ws is None or ws.numel() * ws.element_size() < need:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    scan_fwd_into(prob, diag, x, dt, A, B, C, D, h0, y, hT, ws)
    return y, hT


def scan_fwd(x, dt, A, B, C, D=None, h0=None, chunk=256, return_final_state=True, workspace=None):
    """Scalar-decay SSD forward (a_t = exp(dt_t A_h)). Returns (y, hT)."""
    return _forward(False, x, dt, A, B, C, D, h0, chunk, return_final_state, workspace)


def diag_scan_fwd(x, dt, A, B, C, D=None, h0=None, chunk=128, return_final_state=True, workspace=None):
    """Diagonal-decay SSD forward (a_{t,n} = exp(dt_t A_{h,n})). Returns (y, hT)."""
    return _forward(True, x, dt, A, B, C, D, h0, chunk, return_final_state, workspace)


def varlen_workspace_bytes(prob: Problem) -> int:
    return int(_load().ssd_varlen_workspace_bytes(ctypes.byref(prob)))


def scan_fwd_varlen_into(prob: Problem, cu_seqlens, x, dt, A, B, C, D, h0, y, hT, ws, stream=None) -> None:
    """Enqueue one packed variable-length forward (prob.batch sequences on one token axis
    of prob.seqlen tokens) into caller-provided outputs and workspace (no allocation)."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = _load().ssd_scan_fwd_varlen(ctypes.byref(prob), _ptr(cu_seqlens), _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                                     _ptr(C), _ptr(D), _ptr(h0), _ptr(y), _ptr(hT), _ptr(ws), nbytes,
                                     ctypes.c_void_p(int(stream)))
    if st:
        raise SSDError(st, "ssd_scan_fwd_varlen")


def scan_fwd_varlen(x, dt, A, B, C, cu_seqlens, D=None, h0=None, chunk=256, return_final_state=True,
                    workspace=None):
    """Scalar-decay SSD forward over packed sequences: x [T, H, P], dt [T, H], B/C [T, G, N]
    hold the sequences back to back, sequence s on tokens [cu_seqlens[s], cu_seqlens[s+1])
    (cu_seqlens: int32 GPU tensor of nseq + 1 offsets).  h0 / hT are [nseq, H, P, N].
    Returns (y, hT)."""
    import torch
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise TypeError("cu_seqlens must be a 1-D int32 tensor of nseq + 1 offsets")
    if x.dim() != 3 or B.dim() != 3:
        raise ValueError("x must be [T, H, P] and B [T, G, N]")
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    nseq = cu_seqlens.numel() - 1
    _check_args({"x": (x, (T, H, P)), "dt": (dt, (T, H)), "A": (A, (H,)), "B": (B, (T, G, N)),
                 "C": (C, (T, G, N)), "D": (D, (H,)), "h0": (h0, (nseq, H, P, N)),
                 "cu_seqlens": (cu_seqlens, (nseq + 1,))},
                floats=("dt", "A", "D", "h0"), same_dtype=("x", "B", "C"))
    prob = make_problem(nseq, T, H, P, N, G, chunk, _dtype_code(x))
    y = torch.empty_like(x)
    hT = torch.empty((nseq, H, P, N), dtype=torch.float32, device=x.device) if return_final_state else None
    need = varlen_workspace_bytes(prob)
    if need == 0 and nseq > 0 and T > 0:
        raise SSDError(3, "ssd_scan_fwd_varlen (problem not supported for packed sequences)")
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    scan_fwd_varlen_into(prob, cu_seqlens, x, dt, A, B, C, D, h0, y, hT, workspace)
    return y, hT


def step_into(prob: Problem, diag: bool, x, dt, A, B, C, D, h, y, stream=None) -> None:
    """Enqueue the token-by-token recurrence over prob.seqlen tokens: h (float32
    [b, H, P, N]) is updated in place, y receives the outputs.  No allocation."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    lib = _load()
    fn = lib.ssd_diag_step if diag else lib.ssd_step
    st = fn(ctypes.byref(prob), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h), _ptr(y),
            ctypes.c_void_p(int(stream)))
    if st:
        raise SSDError(st, "ssd_diag_step" if diag else "ssd_step")


def step(x, dt, A, B, C, h, D=None, diag=None):
    """Decode: run the recurrence over x's tokens on state h (updated in place).
    x [b, T, H, P] (bf16 or f32), dt [b, T, H] f32, A [H] or [H, N] f32, B/C [b, T, G, N],
    h [b, H, P, N] f32, D [H] f32 or None.  Returns y [b, T, H, P]."""
    import torch
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be [b, T, H, P] and B [b, T, G, N]")
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if diag is None:
        diag = A.dim() == 2
    if h is None:
        raise ValueError("h (the state, updated in place) is required")
    _check_args({"x": (x, (b, T, H, P)), "dt": (dt, (b, T, H)), "A": (A, (H, N) if diag else (H,)),
                 "B": (B, (b, T, G, N)), "C": (C, (b, T, G, N)), "D": (D, (H,)), "h": (h, (b, H, P, N))},
                floats=("dt", "A", "D", "h"), same_dtype=("x", "B", "C"))
    prob = make_problem(b, T, H, P, N, G, 64, _dtype_code(x))
    y = torch.empty_like(x)
    step_into(prob, diag, x, dt, A, B, C, D, h, y)
    return y


def bwd_workspace_bytes(prob: Problem, diag: bool = False) -> int:
    f = _load().ssd_diag_bwd_workspace_bytes if diag else _load().ssd_bwd_workspace_bytes
    return int(f(ctypes.byref(prob)))


def scan_bwd_into(prob: Problem, x, dt, A, B, C, D, h0, dy, dhT, dx, ddt, dA, dB, dC, dD, dh0, ws,
                  stream=None, diag: bool = False) -> None:
    """Enqueue one backward pass (diag: of the diagonal-decay forward, A and dA [H, N]) into
    caller-provided gradients and workspace (no allocation)."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(dA.device).cuda_stream
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    f, name = (_load().ssd_diag_scan_bwd, "ssd_diag_scan_bwd") if diag else (_load().ssd_scan_bwd, "ssd_scan_bwd")
    st = f(ctypes.byref(prob), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0), _ptr(dy), _ptr(dhT),
           _ptr(dx), _ptr(ddt), _ptr(dA), _ptr(dB), _ptr(dC), _ptr(dD), _ptr(dh0), _ptr(ws), nbytes,
           ctypes.c_void_p(int(stream)))
    if st:
        raise SSDError(st, name)


def _backward(diag, x, dt, A, B, C, dy, D, h0, dhT, chunk, workspace):
    import torch
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be [b, T, H, P] and B [b, T, G, N]")
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    _check_args({"x": (x, (b, T, H, P)), "dt": (dt, (b, T, H)), "A": (A, (H, N) if diag else (H,)),
                 "B": (B, (b, T, G, N)), "C": (C, (b, T, G, N)), "dy": (dy, (b, T, H, P)), "D": (D, (H,)),
                 "h0": (h0, (b, H, P, N)), "dhT": (dhT, (b, H, P, N))},
                floats=("dt", "A", "D", "h0", "dhT"), same_dtype=("x", "B", "C", "dy"))
    prob = make_problem(b, T, H, P, N, G, chunk, _dtype_code(x))
    dev = x.device
    out = dict(dx=torch.empty_like(x), ddt=torch.empty_like(dt), dA=torch.empty_like(A), dB=torch.empty_like(B),
               dC=torch.empty_like(C), dD=torch.empty((H,), dtype=torch.float32, device=dev),
               dh0=torch.empty((b, H, P, N), dtype=torch.float32, device=dev))
    need = bwd_workspace_bytes(prob, diag)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    scan_bwd_into(prob, x, dt, A, B, C, D, h0, dy, dhT, out["dx"], out["ddt"], out["dA"], out["dB"], out["dC"],
                  out["dD"], out["dh0"], workspace, diag=diag)
    return out


def scan_bwd(x, dt, A, B, C, dy, D=None, h0=None, dhT=None, chunk=256, workspace=None):
    """Backward pass of the scalar-decay forward: gradients of a loss with respect to every
    input, given dy (like x) and dhT ([b, H, P, N] float32, None = 0).  Returns a dict with
    dx (x's dtype), ddt (float32), dA (float32 [H]), dB and dC (B's dtype), dD (float32 [H])
    and dh0 (float32 [b, H, P, N])."""
    return _backward(False, x, dt, A, B, C, dy, D, h0, dhT, chunk, workspace)


def diag_scan_bwd(x, dt, A, B, C, dy, D=None, h0=None, dhT=None, chunk=128, workspace=None):
    """Backward pass of the diagonal-decay forward (A [H, N]): as scan_bwd, with dA
    float32 [H, N]."""
    return _backward(True, x, dt, A, B, C, dy, D, h0, dhT, chunk, workspace)
