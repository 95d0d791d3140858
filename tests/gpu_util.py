"""Helpers shared by the GPU parity tests: moving seeded host inputs to the
device and comparing device results with the oracle.  Nothing here does
any of the method's arithmetic."""
import sys

import numpy as np
import torch

TOL = 2e-3          # max |y - y_oracle| / ||y_oracle row||_2


def banner(msg: str):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray, bf16: bool | None = None) -> torch.Tensor:
    """Host array -> CUDA tensor.  uint16 arrays are bf16 bits."""
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to("cuda")


def dev_strided(a: np.ndarray) -> torch.Tensor:
    """Host 2-D array -> CUDA view whose row stride is padded to a multiple
    of 16 bytes plus one extra 16-byte chunk (exercises ld > cols)."""
    t = dev(a)
    rows, cols = t.shape
    per16 = 16 // t.element_size()
    ld = (cols + per16 - 1) // per16 * per16 + per16
    buf = torch.full((rows, ld), 1e30, dtype=t.dtype, device="cuda")   # poison: must never be read
    buf[:, :cols] = t
    return buf[:, :cols]


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().to("cpu")
    if t.dtype == torch.bfloat16:
        return (t.view(torch.int16).numpy().astype(np.uint16).astype(np.uint32) << 16).view(np.float32)
    return t.numpy()


def assert_bytes_equal(got: np.ndarray, want: np.ndarray, what: str):
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.nonzero(got != want)
    n = bad[0].size
    if n:
        idx = tuple(b[0] for b in bad)
        raise AssertionError(f"{what}: {n} mismatches, first at {idx}: got {got[idx]!r} want {want[idx]!r}")


def assert_scales_equal(got: np.ndarray, want: np.ndarray, what: str):
    assert_bytes_equal(got.view(np.uint32), want.view(np.uint32), what)
