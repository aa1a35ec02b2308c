"""Helpers for the GPU parity tests: moving bit patterns to and from the device,
guard-banded outputs and the element-wise tolerance check."""
import sys

import numpy as np
import torch

from oracle import numerics as nm

# Per-element tolerance for floating-point outputs: |gpu - oracle| <= REL * (|oracle| + 1).
REL = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev16(bits: np.ndarray, dtype) -> torch.Tensor:
    """uint16 bit patterns -> device tensor of a 16-bit float dtype."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(dtype).cuda()


def dev32(words: np.ndarray) -> torch.Tensor:
    """uint32/int32 array -> device int32 tensor holding the same bits."""
    return torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).cuda()


def devf32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def dev8(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).cuda()


def host16(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class Guarded:
    """A contiguous output tensor with sentinel-filled guard bands on both sides."""
    PAD = 2048  # elements (4 KiB for 16-bit types), keeps 16-byte alignment

    def __init__(self, shape, dtype, fill_bits: int):
        n = int(np.prod(shape))
        self.n = n
        self.fill = fill_bits
        self.buf = torch.full((n + 2 * self.PAD,), 0, dtype=torch.int16, device="cuda")
        self.buf.fill_(np.int16(np.uint16(fill_bits).view(np.int16)))
        self.view = self.buf[self.PAD:self.PAD + n].view(dtype).view(*shape)

    def bands_intact(self) -> bool:
        h = host16(self.buf)
        return bool(np.all(h[:self.PAD] == self.fill) and np.all(h[self.PAD + self.n:] == self.fill))


def assert_close(gpu_vals: np.ndarray, ref_vals: np.ndarray, rel: float = REL, what: str = ""):
    """Element-wise |gpu - ref| <= rel*(|ref|+1); returns diagnostics (not gates)."""
    g = np.asarray(gpu_vals, dtype=np.float64)
    r = np.asarray(ref_vals, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    err = np.abs(g - r)
    bad = err > rel * (np.abs(r) + 1.0)
    nbad = int(bad.sum())
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    diag = dict(max_abs=float(err.max(initial=0.0)),
                rel_rms=float(np.sqrt(np.mean(err * err)) / rms) if rms > 0 else 0.0,
                max_over_rms=float(err.max(initial=0.0) / rms) if rms > 0 else 0.0,
                violations=nbad)
    if nbad:
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {nbad} elements out of tolerance, first {idx.tolist()}: "
                             f"gpu={g[tuple(idx[0])]}, ref={r[tuple(idx[0])]}; {diag}")
    return diag


def f16v(bits):
    return nm.decode_f16(bits)


def bf16v(bits):
    return nm.decode_bf16(bits)
