"""Shared helpers for the GPU parity tests: moving seeded numpy inputs onto the
GPU and back.  No method arithmetic lives here."""
import os
import sys

import numpy as np

os.environ.setdefault("ORACLE_THREADS", "16")


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_gpu(a):
    """numpy float32 -> cuda float32; numpy uint16 (bf16 bits) -> cuda bfloat16."""
    import torch

    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    if a.dtype == np.float32:
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_np(t):
    import torch

    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def assert_bits_equal(got, ref, what):
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if got.dtype.kind == "f":
        got = got.view(np.uint32 if got.itemsize == 4 else np.uint64)
        ref = ref.view(np.uint32 if ref.itemsize == 4 else np.uint64)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[:5].tolist()}"
