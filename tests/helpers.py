"""Shared helpers for the GPU parity tests: moving stored bit patterns to the
device and back, guard-banded outputs, and the parity criterion
|d - ref| <= 1e-2 |ref| + 1e-2 (fp16 / bf16 outputs against the unrounded
fp64 oracle)."""
from __future__ import annotations

import numpy as np
import torch

RTOL = 1e-2
ATOL = 1e-2
SENTINEL = 0x7BAD  # a finite fp16 / bf16 pattern the kernels never produce from these inputs by chance

TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16}


def dev():
    return torch.device("cuda:0")


def to_dev(bits: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "f8e4m3":
        return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint8)).view(torch.float8_e4m3fn).to(dev())
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(TORCH_DT[dtype]).to(dev())


def bytes_to_dev(b: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(b)).to(dev())


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def check_close(got_bits: np.ndarray, ref: np.ndarray, dtype: str, what: str, rtol=RTOL, atol=ATOL):
    import oracle

    got = oracle.decode(got_bits, dtype)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    bad = ~(np.abs(got - ref) <= rtol * np.abs(ref) + atol)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = ", ".join(f"{tuple(i)}: got {got[tuple(i)]:.6g} want {ref[tuple(i)]:.6g}" for i in idx)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; {detail}")
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


class Guarded:
    """A [rows][ld] output inside a flat buffer with `pad` sentinel elements on
    each side; columns [cols, ld) are sentinels too."""

    def __init__(self, rows, cols, ld, dtype, pad=64):
        self.rows, self.cols, self.ld, self.pad = rows, cols, ld, pad
        n = rows * ld + 2 * pad
        self.flat = torch.full((n,), SENTINEL, dtype=torch.int16, device=dev()).view(TORCH_DT[dtype])
        self.view = self.flat[pad:pad + rows * ld].view(rows, ld)[:, :cols] if rows else \
            self.flat[pad:pad].view(0, ld)[:, :cols]

    def check_guards(self, what):
        h = self.flat.cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.all(h[:self.pad] == SENTINEL) and np.all(h[len(h) - self.pad:] == SENTINEL), f"{what}: guard band"
        body = h[self.pad:len(h) - self.pad].reshape(self.rows, self.ld)
        assert np.all(body[:, self.cols:] == SENTINEL), f"{what}: padding columns written"

    def bits(self):
        h = self.flat.cpu().view(torch.int16).numpy().view(np.uint16)
        return h[self.pad:len(h) - self.pad].reshape(self.rows, self.ld)[:, :self.cols]
