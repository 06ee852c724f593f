"""The Python binding checks every tensor's shape, dtype, device and layout before it
enqueues anything: the C ABI sees only pointers and sizes, so a short D or h0, a bf16
state or a transposed view would otherwise be read or written out of bounds on the
device.  On the CPU the shape and dtype checks come first (CPU tensors are then refused
as not on the GPU); the GPU test repeats the malformed cases with device tensors."""
import pytest
import torch

import ssd_chunked_scan_03_amd as ssd

b, T, H, P, N, G = 2, 10, 4, 16, 32, 2


def good(device="cpu", diag=False, dtype=torch.bfloat16):
    f32 = dict(dtype=torch.float32, device=device)
    return dict(x=torch.zeros(b, T, H, P, dtype=dtype, device=device), dt=torch.zeros(b, T, H, **f32),
                A=torch.zeros((H, N) if diag else (H,), **f32), B=torch.zeros(b, T, G, N, dtype=dtype, device=device),
                C=torch.zeros(b, T, G, N, dtype=dtype, device=device), D=torch.zeros(H, **f32),
                h0=torch.zeros(b, H, P, N, **f32), dy=torch.zeros(b, T, H, P, dtype=dtype, device=device),
                dhT=torch.zeros(b, H, P, N, **f32))


# (argument, replacement) pairs that must be refused before any launch
def bad_cases(device="cpu", diag=False):
    f32 = dict(dtype=torch.float32, device=device)
    return [
        ("D", torch.zeros(H - 1, **f32)),                       # short D
        ("D", torch.zeros(H, dtype=torch.float64, device=device)),
        ("h0", torch.zeros(b - 1, H, P, N, **f32)),             # too few batch rows
        ("h0", torch.zeros(b, H, P, N, dtype=torch.bfloat16, device=device)),
        ("dt", torch.zeros(b, T, H + 1, **f32)),
        ("dt", torch.zeros(b, T, H, dtype=torch.bfloat16, device=device)),
        ("A", torch.zeros((H,) if diag else (H, N), **f32)),     # the other decay's shape
        ("B", torch.zeros(b, T, G, N + 16, dtype=torch.bfloat16, device=device)),
        ("C", torch.zeros(b, T, G, N, dtype=torch.float32, device=device)),  # dtype unlike x
        ("C", torch.zeros(b, T, G, N, dtype=torch.bfloat16, device=device).transpose(0, 1).contiguous()
         .transpose(0, 1)),                                       # right shape, not contiguous
    ]


def call_forward(a, diag):
    f = ssd.diag_scan_fwd if diag else ssd.scan_fwd
    return f(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["h0"], chunk=64)


def call_step(a, diag):
    return ssd.step(a["x"], a["dt"], a["A"], a["B"], a["C"], a["h0"], D=a["D"], diag=diag)


def call_backward(a, diag):
    f = ssd.diag_scan_bwd if diag else ssd.scan_bwd
    return f(a["x"], a["dt"], a["A"], a["B"], a["C"], a["dy"], D=a["D"], h0=a["h0"], dhT=a["dhT"], chunk=64)


CALLS = {"forward": call_forward, "step": call_step, "backward": call_backward}


@pytest.mark.parametrize("call", list(CALLS))
@pytest.mark.parametrize("diag", [False, True])
def test_malformed_arguments_are_refused_on_the_host(call, diag):
    for name, repl in bad_cases(diag=diag):
        a = good(diag=diag)
        a["h0" if (call == "step" and name == "h0") else name] = repl
        with pytest.raises((ValueError, TypeError)) as e:
            CALLS[call](a, diag)
        assert "GPU tensor" not in str(e.value) or name == "C", (call, name, str(e.value))
    # well-formed CPU tensors pass every shape and dtype check and are then refused as not on the GPU
    with pytest.raises(ValueError, match="GPU tensor"):
        CALLS[call](good(diag=diag), diag)


def test_step_state_must_be_float32_of_full_size():
    a = good()
    for h in (torch.zeros(b, H, P, N, dtype=torch.bfloat16), torch.zeros(b, H, P, N // 2), torch.zeros(b * H * P * N)):
        with pytest.raises((ValueError, TypeError)):
            ssd.step(a["x"], a["dt"], a["A"], a["B"], a["C"], h, D=a["D"])
    with pytest.raises(ValueError):
        ssd.step(a["x"], a["dt"], a["A"], a["B"], a["C"], None, D=a["D"])


def test_varlen_arguments_are_refused_on_the_host():
    x = torch.zeros(T, H, P, dtype=torch.bfloat16)
    dt, A, D = torch.zeros(T, H), torch.zeros(H), torch.zeros(H)
    Bm = torch.zeros(T, G, N, dtype=torch.bfloat16)
    cu = torch.tensor([0, 4, T], dtype=torch.int32)
    with pytest.raises(ValueError, match="h0"):
        ssd.scan_fwd_varlen(x, dt, A, Bm, Bm, cu, D=D, h0=torch.zeros(3, H, P, N))  # 2 sequences, 3 states
    with pytest.raises(ValueError, match="D"):
        ssd.scan_fwd_varlen(x, dt, A, Bm, Bm, cu, D=torch.zeros(H + 1))
    with pytest.raises(TypeError):
        ssd.scan_fwd_varlen(x, dt, A, Bm, Bm, cu.to(torch.int64))
    with pytest.raises(ValueError, match="GPU tensor"):
        ssd.scan_fwd_varlen(x, dt, A, Bm, Bm, cu, D=D, h0=torch.zeros(2, H, P, N))


@pytest.mark.gpu
@pytest.mark.parametrize("call", list(CALLS))
def test_malformed_arguments_are_refused_before_launch_on_gpu(call):
    for diag in (False, True):
        for name, repl in bad_cases("cuda", diag):
            a = good("cuda", diag)
            a[name] = repl
            with pytest.raises((ValueError, TypeError)):
                CALLS[call](a, diag)
        # a tensor on the host among device tensors
        a = good("cuda", diag)
        a["D"] = a["D"].cpu()
        with pytest.raises(ValueError):
            CALLS[call](a, diag)
