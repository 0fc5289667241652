"""Helpers for the GPU parity tests: device upload of seeded numpy inputs and
the error metrics the tolerances are written in."""
import os
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


def rel_l2_rows(got, ref):
    """Largest relative L2 error of any single row (first axis); a row whose
    reference is zero is measured in absolute terms."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if got.shape[0] == 0:
        return 0.0
    got = got.reshape(got.shape[0], -1)
    ref = ref.reshape(ref.shape[0], -1)
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    return float(np.max(num / np.where(den > 0, den, 1.0)))


def assert_rows_close(got, ref, tol, what=""):
    """Relative L2 within tol over the whole array and over every row: a few
    wrong rows cannot hide in the norm of many right ones."""
    whole, worst = rel_l2(got, ref), rel_l2_rows(got, ref)
    assert whole < tol and worst < tol, f"{what}: whole {whole:.3g}, worst row {worst:.3g}, tol {tol}"
    return whole, worst


def oracle_block_all_rows(O, om, l, h, idx, k_cache, v_cache, mod=None, branch=0, workers=None):
    """The oracle's block over every active row, computed in row chunks on a
    thread pool (BLAS single-threaded per chunk).

    The block is row-wise except that attention reads the whole cache.  The
    first chunk's call writes every active row's fresh K/V into k_cache /
    v_cache (in place, as one block_forward does); each later chunk then runs
    block_forward on its own rows against a private copy of that updated
    cache, rewriting only its own (already fresh) rows.  The result equals
    one call over all rows up to BLAS summation order."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    n = len(idx)
    workers = workers or max(1, min(16, os.cpu_count() or 1))
    chunks = [c for c in np.array_split(np.arange(n), 2 * workers) if c.size]
    first = O.block_forward(om, l, h, idx, k_cache, v_cache, rows=chunks[0], mod=mod, branch=branch)

    def run(ch):
        kc, vc = k_cache.copy(), v_cache.copy()
        return O.block_forward(om, l, h[ch], idx[ch], kc, vc, mod=mod, branch=branch)

    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        rest = list(ex.map(run, chunks[1:]))
    return np.concatenate([first] + rest)
