"""Helpers for the GPU parity tests (device allocation and copies only)."""
import numpy as np
import torch

import w2a8_gemv_amd as w2a8

CANARY_I32 = -0x2A2A2A2B
GUARD = 64  # elements of guard band after every output


def dev():
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def packed_on_device(w: np.ndarray) -> torch.Tensor:
    return w2a8.pack_ternary(torch.from_numpy(np.ascontiguousarray(w))).to(dev())


def guarded(n: int, dtype) -> torch.Tensor:
    """Output buffer of n elements followed by a guard band of canaries."""
    t = torch.empty(n + GUARD, dtype=dtype, device=dev())
    if dtype == torch.int32:
        t.fill_(CANARY_I32)
    else:
        t.fill_(float("nan"))
    return t


def check_guard(t: torch.Tensor, n: int):
    tail = t[n:].cpu()
    if t.dtype == torch.int32:
        assert bool((tail == CANARY_I32).all()), "write past the end of the output"
    else:
        assert bool(torch.isnan(tail).all()), "write past the end of the output"


def gemv_dev(wp, x_dev, N, K, sa=None, sw=1.0, want_f32=False, stream=None, workspace=None):
    y = guarded(N, torch.int32)
    yf = guarded(N, torch.float32) if want_f32 else None
    w2a8.w2a8_gemv(wp, x_dev, N, K, y_i32=y[:N], s_a=sa, s_w=sw,
                   y_f32=None if yf is None else yf[:N], stream=stream, workspace=workspace)
    torch.cuda.synchronize()
    check_guard(y, N)
    if yf is not None:
        check_guard(yf, N)
        return y[:N].cpu().numpy(), yf[:N].cpu().numpy()
    return y[:N].cpu().numpy()
