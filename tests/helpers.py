"""Test-side glue: moving seeded inputs between numpy (oracle side) and torch
GPU tensors (library side), and the parity tolerances."""
import numpy as np

from oracle.formats import bf16_to_f64

# Parity bars: bf16 outputs 2e-2 abs + 2e-2 rel elementwise, fp32 1e-4.
TOL = {"bf16": 2e-2, "fp32": 1e-4}


def to_dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_dev(arr):
    import torch
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def bf16_dev_to_f64(t):
    """bf16 GPU tensor -> float64 numpy (exact)."""
    import torch
    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return bf16_to_f64(bits)


def assert_close(got, ref, tol, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = np.abs(got - ref)
    bound = tol + tol * np.abs(ref)
    bad = err > bound
    if bad.any():
        idx = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {err.size} outside {tol} abs+rel; "
                             f"worst at {idx}: got {got[idx]} ref {ref[idx]}")


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def blocked32(x):
    """Token-major ``[..., cap, D]`` -> the draft main-segment V layout
    ``[..., cap/32, D, 32]`` (32-token blocks, channel-major inside)."""
    x = np.asarray(x)
    *lead, cap, D = x.shape
    assert cap % 32 == 0
    return np.ascontiguousarray(x.reshape(*lead, cap // 32, 32, D).swapaxes(-1, -2))
