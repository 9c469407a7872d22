"""Helpers for the GPU parity tests: device buffers with guard bands, bit views, sum tolerances.

Guard bands: every output region sits between 64 bytes of 0x7F (f32 3.3961514e38, finite) on each
side, and any padding columns of an output (ld > N) start out as the same bytes; after a call the
guard and padding bytes must be unchanged.
"""
import numpy as np
import torch

GUARD_FLOATS = 16                      # 64 bytes
LINE_GUARD_FLOATS = 32                 # 128 bytes: one cache line
SENTINEL_BITS = 0x7F7F7F7F
SENTINEL = np.array([SENTINEL_BITS], np.uint32).view(np.float32)[0]


def bits(a):
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def sentinel_buffer(n_floats, device):
    """A float32 device buffer of n_floats whose every byte is 0x7F."""
    return torch.full((max(n_floats, 1) * 4,), 0x7F, dtype=torch.uint8, device=device).view(torch.float32)


class Guarded:
    """One region of `n` floats inside a sentinel-filled device buffer, with `guard` guard floats
    before and after (GUARD_FLOATS = 64 bytes by default; LINE_GUARD_FLOATS = 128 bytes puts the
    region on a 128-byte line, since device allocations start on 256-byte boundaries) and an
    optional start offset (in floats) to break the alignment."""

    def __init__(self, n, device, offset=0, guard=GUARD_FLOATS):
        self.n = n
        self.off = guard + offset
        self.buf = sentinel_buffer(self.off + n + guard, device)
        assert self.buf.data_ptr() % 256 == 0

    @property
    def ptr(self):
        return self.buf.data_ptr() + 4 * self.off

    def payload(self):
        return self.buf[self.off:self.off + self.n]

    def upload(self, host):
        assert host.size == self.n
        self.payload().copy_(torch.from_numpy(host))

    def host(self):
        return self.buf.cpu().numpy()

    def guards_intact(self):
        b = bits(self.buf)
        return bool((b[:self.off] == SENTINEL_BITS).all() and
                    (b[self.off + self.n:] == SENTINEL_BITS).all())


def sentinel_host(n):
    return np.full(n, SENTINEL, np.float32)


def sum_tol(x_abs_sum):
    """Sums agree with the fp64 oracle within 1e-5 relative to sum |x| (plus a floor for exact 0)."""
    return 1e-5 * np.asarray(x_abs_sum) + 1e-30
