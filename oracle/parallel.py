"""Row-parallel driver of the float64 oracle (test infrastructure only).

Every query row of the oracle's operations is computed from its own definition
(see ``hysparse_ref``), so disjoint sets of rows can be computed independently
and concurrently without changing any row's arithmetic. This module runs the
oracle's functions on chunks of rows in a pool of threads, each doing plain
single-threaded BLAS: numpy releases the interpreter lock inside its array
loops and BLAS calls, and one BLAS thread per worker avoids the oversubscription
that many BLAS threads per row cause on small row chunks.

Only the tests and the benchmark's CPU-baseline leg use it. Threads (not
processes) keep it safe to call from a process that has already initialised
a GPU: nothing is forked or executed.
"""
from __future__ import annotations

import os
from collections import deque
from concurrent.futures import ThreadPoolExecutor
from typing import Callable, Iterator, Optional, Sequence, Tuple

import numpy as np

from . import hysparse_ref as ref


def default_workers() -> int:
    """Worker threads: OMP_NUM_THREADS when set (the host's CPU share), else
    the visible CPU count."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def map_row_chunks(fn: Callable[[np.ndarray], object], rows: Sequence[int], chunk: int,
                   workers: Optional[int] = None) -> Iterator[Tuple[np.ndarray, object]]:
    """Yield (rows_of_chunk, fn(rows_of_chunk)) for consecutive chunks of
    ``rows``, in order, computed by ``workers`` threads with BLAS limited to
    one thread each. At most 2 * workers chunks are in flight, which bounds
    the memory held by finished results."""
    from threadpoolctl import threadpool_limits
    rows = np.asarray(rows, dtype=np.int64)
    chunks = [rows[i:i + chunk] for i in range(0, len(rows), chunk)]
    workers = workers or default_workers()
    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=workers) as ex:
        pending: deque = deque()
        it = iter(chunks)
        for c in it:
            pending.append((c, ex.submit(fn, c)))
            if len(pending) >= 2 * workers:
                break
        while pending:
            c, fut = pending.popleft()
            res = fut.result()
            nxt = next(it, None)
            if nxt is not None:
                pending.append((nxt, ex.submit(fn, nxt)))
            yield c, res


def metric_path_rows(q, kv64, sink, Dv: int, scale: float, top_k: int, rows: np.ndarray,
                     block_size: int = 64, kv_lens=None, doc_start=None, doc_end=None,
                     gather_idx=None):
    """The oracle's block scores, top-k and gather for the given rows of every
    batch entry: (out, lse, block_logit, idx, out_gather, lse_gather), each
    with the rows axis second. The gather uses ``gather_idx`` ([B, Sq, K],
    e.g. another implementation's selection) when given, else the oracle's own
    top-k."""
    kw = dict(block_size=block_size, kv_lens=kv_lens, doc_start=doc_start, doc_end=doc_end)
    B, Sq = q.shape[0], q.shape[1]
    out, lse, bl = ref.block_score(q, kv64, sink, Dv, scale, rows=rows, **kw)
    own = ref.own_blocks(B, Sq, kv64.shape[1], block_size, kv_lens, doc_start, doc_end, rows=rows)
    idx = ref.topk_blocks(bl, own, top_k)
    use = np.full((B, Sq, top_k), -1, dtype=np.int64)
    use[:, rows] = idx if gather_idx is None else np.asarray(gather_idx)[:, rows]
    og, lg = ref.sparse_gather(q, kv64, sink, Dv, scale, use, rows=rows, **kw)
    return out, lse, bl, idx, og, lg


def chunk_rows_for(Sq: int, H: int, L: int, target_entries: float = 2e7) -> int:
    """Rows per chunk so that one chunk's [rows, H, keys] score array holds about
    ``target_entries`` float64 values (the oracle's own chunking bound)."""
    return max(1, int(target_entries // (H * max(1, L))))

