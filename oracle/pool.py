"""Run the oracle over many heads in worker processes (test infrastructure only).

The arithmetic is the oracle's own: each task is one call of
:func:`oracle.attention.attention_head` or :func:`oracle.attention.attention_backward` on one
head. This module only hands heads to a pool of worker processes (a fresh interpreter each,
started with ``spawn``, so no worker inherits a parent's GPU state) with one BLAS thread per
worker, and returns the results in task order.
"""

from __future__ import annotations

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

MAX_WORKERS = 16


def worker_count(limit: int = MAX_WORKERS) -> int:
    """Cores this process may run on (its affinity set), at most ``limit``."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - platforms without affinity
        n = os.cpu_count() or 1
    return max(1, min(limit, n))


def _one_blas_thread():
    try:
        from threadpoolctl import threadpool_limits

        threadpool_limits(1)
    except ImportError:  # pragma: no cover - threadpoolctl missing
        pass


def _forward_head(task):
    from .attention import attention_head

    q, k, v, scale, causal = task
    return attention_head(q, k, v, scale, causal)


def _backward_head(task):
    from .attention import attention_backward

    q, k, v, dout, scale, causal = task
    dq, dk, dv = attention_backward(q[None, None], k[None, None], v[None, None],
                                    dout[None, None], scale, causal)
    return dq[0, 0], dk[0, 0], dv[0, 0]


def _map(fn, tasks, workers):
    workers = worker_count() if workers is None else max(1, int(workers))
    ctx = mp.get_context("spawn")
    with ProcessPoolExecutor(max_workers=workers, mp_context=ctx,
                             initializer=_one_blas_thread) as ex:
        yield from ex.map(fn, tasks)


def attention_heads(heads, scale, causal, workers=None):
    """Yield (O, m, l) of :func:`attention_head` for each (q, k, v) of ``heads``, in order."""
    return _map(_forward_head, ((q, k, v, scale, causal) for q, k, v in heads), workers)


def attention_backward_heads(heads, scale, causal, workers=None):
    """Yield (dQ, dK, dV) of one head for each (q, k, v, dout) of ``heads``, in order: the
    gradients of that head alone (a shared key/value head's sum is the caller's)."""
    return _map(_backward_head, ((q, k, v, dout, scale, causal) for q, k, v, dout in heads),
                workers)
