"""Helpers for the GPU parity tests: device buffers with canary guard bands,
tolerances, sampling."""
import numpy as np
import torch

GUARD = 64            # bytes of canary before and after every output buffer
CANARY = 0x5A


class Guarded:
    """A device output tensor embedded in a larger byte buffer whose margins
    hold a canary; check() fails if a kernel wrote outside the tensor."""

    def __init__(self, shape, dtype, fill=None):
        self.shape = tuple(shape)
        self.dtype = dtype
        n = int(np.prod(self.shape)) if len(self.shape) else 1
        nbytes = n * torch.tensor([], dtype=dtype).element_size()
        self.raw = torch.full((GUARD + nbytes + GUARD,), CANARY, dtype=torch.uint8, device="cuda")
        self.t = self.raw[GUARD:GUARD + nbytes].view(dtype).view(self.shape)
        if fill is not None:
            self.t.fill_(fill)

    def check(self):
        head = self.raw[:GUARD].cpu().numpy()
        tail = self.raw[-GUARD:].cpu().numpy()
        assert np.all(head == CANARY) and np.all(tail == CANARY), "write outside the output buffer"

    def np(self):
        self.check()
        return self.t.cpu().numpy()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def assert_close(y, ref, rtol):
    """|y - ref| <= rtol |ref| + rtol mean|ref| (relative error with a floor) on the
    finite entries; non-finite entries (an fp16 overflow) must be identical."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isnan(y), np.isnan(ref)), "NaN pattern differs"
    assert np.array_equal(y[~fin & ~np.isnan(ref)], ref[~fin & ~np.isnan(ref)]), "infinities differ"
    assert np.isfinite(y[fin]).all(), "non-finite output where the reference is finite"
    y, ref = y[fin], ref[fin]
    atol = rtol * float(np.mean(np.abs(ref))) if ref.size else 0.0
    bad = np.abs(y - ref) > rtol * np.abs(ref) + atol
    assert not bad.any(), (f"{bad.sum()} of {bad.size} outside tolerance; worst "
                           f"{np.max(np.abs(y - ref) / (np.abs(ref) + atol))}")


def assert_bits_equal(a, b, what):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    if a.dtype.kind == "f":
        a = a.view(np.uint16 if a.dtype == np.float16 else np.uint32)
        b = b.view(np.uint16 if b.dtype == np.float16 else np.uint32)
    neq = a != b
    assert not neq.any(), f"{what}: {neq.sum()} of {neq.size} differ, first at {np.argwhere(neq)[0]}"


def sample_positions(M, N, n, seed=0):
    rng = np.random.default_rng(seed)
    rows = rng.integers(0, M, n)
    cols = rng.integers(0, N, n)
    # always include the corners and the last row/column (ragged tile edges)
    rows = np.concatenate([rows, [0, 0, M - 1, M - 1]])
    cols = np.concatenate([cols, [0, N - 1, 0, N - 1]])
    return rows.astype(np.int64), cols.astype(np.int64)
