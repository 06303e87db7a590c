"""Row-parallel runs of the oracle's column loop and replay (test helper, no GPU).

Rows of W are independent given U, the processing order and the dead
columns, so the oracle's loop over a whole large layer can be split by rows
across worker processes and concatenated.  The workers are spawned (fresh
interpreters that import only numpy and the oracle, never torch or the HIP
library), read U from a memory-mapped file, and run with one BLAS thread each.
"""
from __future__ import annotations

import dataclasses
import os
import tempfile
from concurrent.futures import ProcessPoolExecutor
import multiprocessing as mp

import numpy as np

import oracle

_U = None


def _init(path, shape, dtype):
    global _U
    from threadpoolctl import threadpool_limits

    threadpool_limits(1)
    _U = np.memmap(path, dtype=dtype, mode="r", shape=shape)


def _quantize(args):
    W, kw = args
    r = oracle.gptq_quantize(W, _U, **kw)
    return r.codes, r.scales, r.zeros, r.g_idx


def _replay(args):
    W, cq, sc, z, kw = args
    return oracle.replay_check(W, _U, codes_proc=cq, scales=sc, zeros=z, **kw)


@dataclasses.dataclass
class RowsResult:
    codes: np.ndarray
    scales: np.ndarray
    zeros: np.ndarray
    g_idx: np.ndarray


def workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


class RowPool:
    """A pool of spawned workers sharing one U (fp32 or fp64, [n, n])."""

    def __init__(self, U: np.ndarray, nproc: int | None = None):
        self.nproc = nproc or workers()
        fd, self.path = tempfile.mkstemp(suffix=".u", dir=os.environ.get("TMPDIR", "/tmp"))
        os.close(fd)
        U = np.ascontiguousarray(U)
        mm = np.memmap(self.path, dtype=U.dtype, mode="w+", shape=U.shape)
        mm[:] = U
        mm.flush()
        del mm
        ctx = mp.get_context("spawn")
        self.ex = ProcessPoolExecutor(self.nproc, mp_context=ctx, initializer=_init,
                                      initargs=(self.path, U.shape, U.dtype))

    def close(self):
        self.ex.shutdown()
        os.unlink(self.path)

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()

    def _split(self, m):
        return [c for c in np.array_split(np.arange(m), self.nproc) if len(c)]

    def quantize(self, W: np.ndarray, **kw) -> RowsResult:
        parts = list(self.ex.map(_quantize, [(W[c], kw) for c in self._split(W.shape[0])]))
        return RowsResult(codes=np.concatenate([p[0] for p in parts]),
                          scales=np.concatenate([p[1] for p in parts]),
                          zeros=np.concatenate([p[2] for p in parts]), g_idx=parts[0][3])

    def replay(self, W, codes_proc, scales, zeros, **kw) -> oracle.gptq.ReplayReport:
        chunks = self._split(W.shape[0])
        reps = list(self.ex.map(_replay, [(W[c], codes_proc[c], scales[c], zeros[c], kw)
                                          for c in chunks]))
        return oracle.gptq.ReplayReport(
            n_codes=sum(r.n_codes for r in reps), mismatches=sum(r.mismatches for r in reps),
            ties=sum(r.ties for r in reps), hard=sum(r.hard for r in reps),
            zero_mismatches=sum(r.zero_mismatches for r in reps),
            zero_ties=sum(r.zero_ties for r in reps), zero_hard=sum(r.zero_hard for r in reps),
            scale_max_rel=max(r.scale_max_rel for r in reps),
            row_err=np.concatenate([r.row_err for r in reps]))


def cascades(codes_a: np.ndarray, codes_b: np.ndarray, perm: np.ndarray):
    """Per diverging row (processing order): the first mismatch is its root; returns
    (rows with a root, total mismatches, mean and max mismatches per diverging row)."""
    bad = np.asarray(codes_a)[:, perm] != np.asarray(codes_b)[:, perm]
    per = bad.sum(axis=1)
    div = per[per > 0]
    return (int(div.size), int(bad.sum()), float(div.mean()) if div.size else 0.0,
            int(div.max()) if div.size else 0)
