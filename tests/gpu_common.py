"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path through
the C ABI, run the oracle on the same values, compare with the per-slice metric."""
import numpy as np
import torch

import oracle
import ssd_chunked_scan_03_amd as ssd
from helpers import rel_h, rel_y

TOL = {"f32": 1e-4, "bf16": 2e-2}


def torch_dtype(name):
    return torch.bfloat16 if name == "bf16" else torch.float32


def upload(inp, dtype):
    """numpy inputs -> cuda tensors (x/B/C hold bf16-exact values, so the cast is exact)."""
    td = torch_dtype(dtype)
    out = {}
    for k in ("x", "B", "C"):
        out[k] = torch.from_numpy(np.ascontiguousarray(inp[k])).to("cuda").to(td).contiguous()
    for k in ("dt", "A", "D", "h0"):
        v = inp.get(k)
        out[k] = None if v is None else torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to("cuda")
    return out


def run_gpu(inp, dtype, chunk, diag, poison=True, return_ws=False, flags=0):
    """One forward through the C ABI into NaN-poisoned outputs and workspace."""
    d = upload(inp, dtype)
    x, B = d["x"], d["B"]
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    prob = ssd.make_problem(b, T, H, P, N, G, chunk, ssd.SSD_BF16 if dtype == "bf16" else ssd.SSD_F32, flags)
    y = torch.empty_like(x)
    hT = torch.empty((b, H, P, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(ssd.workspace_bytes(prob, diag), 1), dtype=torch.uint8, device="cuda")
    if poison:
        y.fill_(float("nan"))
        hT.fill_(float("nan"))
        ws.fill_(0xFF)  # NaN bit patterns in every float/bf16 slot
    ssd.scan_fwd_into(prob, diag, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], y, hT, ws)
    torch.cuda.synchronize()
    out = (y.float().cpu().numpy(), hT.cpu().numpy())
    if return_ws:
        return out + (ws, prob)
    return out


def oracle_ref(inp, diag):
    return oracle.recurrence(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp.get("D"),
                             inp.get("h0"), diag=diag)


def check(got, ref, dtype, what=""):
    (y, hT), (yr, hr) = got, ref
    ey, eh = rel_y(y, yr), rel_h(hT, hr)
    tol = TOL[dtype]
    assert ey < tol and eh < tol, f"{what}: rel err y={ey:.3e} hT={eh:.3e} (tol {tol})"
    return ey, eh


def slice_inputs(inp, bi, h, H, G):
    """The inputs of one (batch, head) pair, as a b=1, H=1, G=1 problem."""
    g = h * G // H
    s = {"x": inp["x"][bi:bi + 1, :, h:h + 1], "dt": inp["dt"][bi:bi + 1, :, h:h + 1],
         "A": inp["A"][h:h + 1], "B": inp["B"][bi:bi + 1, :, g:g + 1], "C": inp["C"][bi:bi + 1, :, g:g + 1],
         "D": None if inp.get("D") is None else inp["D"][h:h + 1],
         "h0": None if inp.get("h0") is None else inp["h0"][bi:bi + 1, h:h + 1]}
    return s
