"""Helpers for the GPU parity tests: device selection, host copies and a
byte-exact comparison that names the first mismatching position."""
import numpy as np
import pytest
import torch


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def host(t):
    if t is None:
        return None
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.cpu().numpy()


def bits16(t):
    """bfloat16 tensor -> numpy uint16 bit patterns (host)."""
    return host(t).view(np.uint16)


def assert_same(name, got, want):
    got = np.ascontiguousarray(got).reshape(-1)
    want = np.ascontiguousarray(want).reshape(-1)
    assert got.shape == want.shape, f"{name}: shape {got.shape} vs {want.shape}"
    if got.dtype.kind == "f":
        gb, wb = got.view(np.uint32), want.view(np.uint32)
    else:
        gb, wb = got, want
    bad = np.nonzero(gb != wb)[0]
    if bad.size:
        i = bad[0]
        raise AssertionError(f"{name}: {bad.size} of {got.size} differ; first at {i}: "
                             f"got {got[i]!r} want {want[i]!r}")


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
