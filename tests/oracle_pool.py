"""Running the fp64 oracle on a process pool for the full-size GPU parity
tests.  Only oracle functions are called; the inputs are handed to forked
workers as numpy arrays set before the pool starts (copy-on-write, nothing
pickled), and each worker limits its BLAS to one thread."""
import multiprocessing as mp
import os

import numpy as np

SHARED = {}


def workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    # the GPU machine allows 16 processes on its card; forked workers inherit the
    # parent's device handle, so stay well below
    return max(1, min(12, n))


def _init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def run(fn, tasks, shared):
    """fn(task) for every task on forked workers that see `shared` (a dict of
    numpy arrays and tables) as oracle_pool.SHARED."""
    SHARED.clear()
    SHARED.update(shared)
    ctx = mp.get_context("fork")
    with ctx.Pool(processes=min(workers(), max(1, len(tasks))), initializer=_init) as pool:
        res = pool.map(fn, tasks, chunksize=1)
    SHARED.clear()
    return res


def to_f32(t):
    """Exact float32 copy of a torch CPU tensor (bf16 or fp32) as numpy."""
    import torch
    return t.detach().to("cpu").to(torch.float32).numpy()
