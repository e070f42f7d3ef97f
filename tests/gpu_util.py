"""Helpers for the GPU parity tests (host <-> device copies and comparisons)."""
import numpy as np
import torch

from oracle import gemm as ogemm


def dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def x_dev(x_bits: np.ndarray) -> torch.Tensor:
    """bf16 bit patterns (uint16) -> device bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def y_host(Y: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return Y.float().cpu().numpy().astype(np.float64)


def assert_within_bound(y_gpu: np.ndarray, Y: np.ndarray, B: np.ndarray, out: str = "f32", what: str = ""):
    tol = ogemm.bound(B, Y, out)
    err = np.abs(y_gpu - Y)
    bad = ~(err <= tol)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside bound; first at {tuple(i)}: "
                             f"gpu={y_gpu[tuple(i)]!r} ref={Y[tuple(i)]!r} tol={tol[tuple(i)]!r}")
    return float((err / np.maximum(B, 1e-300)).max())
