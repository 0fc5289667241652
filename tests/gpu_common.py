"""Helpers for the GPU parity tests: device upload of seeded numpy inputs and
the error metrics the tolerances are written in."""
import sys

import numpy as np
import torch

DEV = "cuda"
# Tolerances (relative L2): float32 workloads 1e-4, bfloat16 workloads 2e-2.
TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(dtype).contiguous()


def host(t):
    return t.detach().to("cpu").to(torch.float64).numpy() if t.is_floating_point() else t.detach().cpu().numpy()


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def bf16_values(a):
    """float32 values rounded to bfloat16 (torch's RNE), as float32 numpy."""
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()
