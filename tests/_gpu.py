"""Helpers for the GPU parity tests: host<->device copies, guard-banded output buffers."""
import numpy as np
import torch

DEV = torch.device("cuda:0")
SENTINEL = 0xA5


def to_dev(a: np.ndarray) -> torch.Tensor:
    """numpy uint16 (bf16 bits) / uint8 / float32 array -> device tensor with the same bytes."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bf16_view(rows, cols, ld, host_bits=None):
    """A [rows, cols] bf16 view with row stride ld inside a larger buffer (padding = random bits)."""
    buf = torch.randint(-32768, 32767, (rows, ld), dtype=torch.int16, device=DEV)
    v = buf[:, :cols]
    if host_bits is not None:
        v.copy_(torch.from_numpy(np.ascontiguousarray(host_bits).view(np.int16)))
    return v


class GuardedU8:
    """[rows, cols] uint8 output view with row stride ld, surrounded by sentinel bytes."""

    def __init__(self, rows, cols, ld, pad_rows=2):
        self.rows, self.cols, self.ld, self.pad = rows, cols, ld, pad_rows
        self.buf = torch.full((rows + 2 * pad_rows, ld), SENTINEL, dtype=torch.uint8, device=DEV)
        self.view = self.buf[pad_rows:pad_rows + rows, :cols]

    def check_untouched(self):
        b = self.buf.cpu().numpy()
        p = self.pad
        assert np.all(b[:p] == SENTINEL), "write before the first row"
        assert np.all(b[p + self.rows:] == SENTINEL), "write after the last row"
        assert np.all(b[p:p + self.rows, self.cols:] == SENTINEL), "write into row padding"

    def host(self):
        return self.view.cpu().numpy()


class GuardedF32:
    """Flat fp32 output of n elements shaped `shape`, NaN-prefilled, with NaN guard bands."""

    def __init__(self, shape, guard=64):
        self.n = int(np.prod(shape))
        self.guard = guard
        self.buf = torch.full((self.n + 2 * guard,), float("nan"), dtype=torch.float32, device=DEV)
        self.view = self.buf[guard:guard + self.n].view(*shape)

    def check_untouched(self):
        b = self.buf.cpu().numpy()
        assert np.all(np.isnan(b[:self.guard])), "scale write before the tensor"
        assert np.all(np.isnan(b[self.guard + self.n:])), "scale write past the tensor"

    def host(self):
        h = self.view.cpu().numpy()
        assert not np.any(np.isnan(h)), "scale element left unwritten"
        return h
