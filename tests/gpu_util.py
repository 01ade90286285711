"""Helpers for GPU parity tests: move seeded host matrices to the device and
read results back. No method arithmetic lives here."""
import sys

import numpy as np

import workloads as wl


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def to_device(m: wl.Matrix, device="cuda:0"):
    """Host Matrix -> torch tensor on the GPU, bit-identical storage."""
    torch = torch_mod()
    if m.dtype == wl.F32:
        return torch.from_numpy(np.ascontiguousarray(m.bits)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(m.bits).view(np.int16)).to(device)
    return t.view(torch.bfloat16)


def padded(t, ld):
    """Copy a 2-D tensor into a wider buffer (leading dimension ld), return the view."""
    torch = torch_mod()
    R, C = t.shape
    buf = torch.zeros((R, ld), dtype=t.dtype, device=t.device)
    buf[:, :C] = t
    return buf[:, :C]


def host(t):
    torch = torch_mod()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def f32_bits(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32)).view(np.uint32)


def assert_bits_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    if got.dtype == np.float32 or want.dtype == np.float32:
        g, w = f32_bits(got), f32_bits(want)
    else:
        g, w = got, want
    bad = np.argwhere(g != w)
    assert bad.size == 0, (f"{what}: {len(bad)} mismatches, first at {tuple(bad[0])}: "
                           f"got {got[tuple(bad[0])]!r} want {want[tuple(bad[0])]!r}")
