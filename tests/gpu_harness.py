"""Helpers for the GPU parity tests: canary-guarded device buffers and sampled reads.

Every output buffer is a byte tensor filled with a canary byte, with the fill written at
a chosen byte offset inside it, so each test also checks that no byte outside
[out, out + n) was written and that misaligned outputs work.
"""
import sys

import numpy as np
import torch

CANARY = 0xA5
PAD = 256


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class DevBuf:
    """n elements of itemsize bytes at byte offset `offset` of a canary-filled buffer."""

    def __init__(self, n, itemsize, offset=0, pad=PAD):
        self.n, self.itemsize, self.off = int(n), int(itemsize), int(offset)
        self.nbytes = self.n * self.itemsize
        self.buf = torch.full((PAD + self.off + self.nbytes + pad,), CANARY, dtype=torch.uint8, device="cuda")
        self.base = PAD + self.off

    @property
    def ptr(self):
        return self.buf.data_ptr() + self.base

    def host(self, dtype):
        """Whole output as a numpy array, after checking the canaries on both sides."""
        torch.cuda.synchronize()
        h = self.buf.cpu().numpy()
        assert (h[:self.base] == CANARY).all(), "bytes written before the output"
        assert (h[self.base + self.nbytes:] == CANARY).all(), "bytes written after the output"
        return h[self.base:self.base + self.nbytes].view(dtype)

    def sample(self, idx, dtype):
        """Elements at indices `idx` read on the device (for outputs too big to copy)."""
        torch.cuda.synchronize()
        idx_t = torch.as_tensor(idx, dtype=torch.int64, device="cuda")
        byte_idx = (idx_t[:, None] * self.itemsize + self.base + torch.arange(self.itemsize, device="cuda")[None, :])
        got = self.buf[byte_idx.reshape(-1)].cpu().numpy()
        edges = torch.cat([self.buf[:self.base], self.buf[self.base + self.nbytes:]]).cpu().numpy()
        assert (edges == CANARY).all(), "bytes written outside the output"
        return got.view(dtype)


def first_mismatch(got, want):
    g = got.view(np.uint8).reshape(got.size, -1)
    w = want.view(np.uint8).reshape(want.size, -1)
    bad = np.flatnonzero((g != w).any(axis=1))
    if bad.size == 0:
        return None
    k = int(bad[0])
    return f"{bad.size} mismatches; first at {k}: got {got[k]!r} want {want[k]!r}"


def assert_bits_equal(got, want, what=""):
    assert got.shape == want.shape, (got.shape, want.shape)
    if not np.array_equal(got.view(np.uint8), want.view(np.uint8)):
        raise AssertionError(f"{what}: {first_mismatch(got, want)}")
