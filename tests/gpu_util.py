"""Helpers shared by the GPU parity tests: device copies of the seeded workloads and the
error measures the tolerances are stated in."""
import os

import numpy as np

# (test, what, err, tol) of every checked bound, for the run's margin summary (conftest.py)
MARGINS = []


def torch_mod():
    import torch
    return torch


def dev(x, dtype="f32"):
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    elif dtype == "f32":
        t = t.to(torch.float32)
    return t.cuda()


def params(w):
    return dict(alpha=dev(w.alpha), beta=dev(w.beta), mu=dev(w.mu), s=dev(w.s))


def host(t):
    torch = torch_mod()
    return t.detach().to(torch.float64).cpu().numpy()


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0


def normwise_rel(a, ref):
    ref = np.asarray(ref, np.float64)
    return max_abs(a, ref) / max(float(np.max(np.abs(ref))), 1e-300)


def lse_rel(a, ref):
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(np.asarray(a, np.float64) - ref) / np.maximum(np.abs(ref), 1.0)))


# tolerances (fp32 path: normwise relative 1e-5; bf16 path: |O| 1e-2, lse 1e-3)
F32_REL = 1e-5
BF16_O_ABS = 1e-2
BF16_LSE_ABS = 1e-3


def within(err, tol, what):
    """Assert err <= tol with both numbers in the message; record the margin."""
    err, tol = float(err), float(tol)
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    MARGINS.append((test, what, err, tol))
    assert err <= tol, f"{what}: err {err:.3e} > tol {tol:.3e}"
    return err
