"""Shared helpers for GPU-vs-oracle parity tests (test code only)."""

from __future__ import annotations

import numpy as np
import torch

from oracle import decode as od

# bf16 output vs the fp64 oracle: |out - ref| <= ATOL + RTOL * |ref| elementwise
# (the random-input tolerance used in the KDA² kernel article, §2.3).
ATOL = 1e-2
RTOL = 1e-2
# fp32 results before the bf16 cast: per (sequence, head[, partition]) row,
# max|x - ref| / max|ref| <= 1e-4; lse within 1e-4 * max(1, |ref|).
F32_REL = 1e-4


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().to("cpu").view(torch.int16).numpy().view(np.uint16)


def oracle_case(case, seqs=None):
    """fp64 oracle (o [S,Hq,D], lse [S,Hq]) on the case's logical K/V."""
    seqs = range(case.num_seqs) if seqs is None else seqs
    q = f64(case.q)
    o = np.zeros(q.shape)
    lse = np.zeros(q.shape[:2])
    for s in seqs:
        o[s], lse[s] = od.attention_decode(q[s], f64(case.keys(s)), f64(case.values(s)),
                                           case.scale)
    return o, lse


def oracle_case_parallel(case, seqs=None, workers=None):
    """oracle_case with the sequences spread over host threads (numpy releases
    the GIL in its loops; BLAS is held to one thread per worker)."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    seqs = list(range(case.num_seqs) if seqs is None else seqs)
    q = f64(case.q)
    o = np.zeros(q.shape)
    lse = np.zeros(q.shape[:2])
    if workers is None:
        try:
            workers = len(os.sched_getaffinity(0))
        except AttributeError:
            workers = os.cpu_count() or 1
        workers = max(1, min(16, workers, len(seqs)))

    def one(s):
        o[s], lse[s] = od.attention_decode(q[s], f64(case.keys(s)), f64(case.values(s)),
                                           case.scale)

    with threadpool_limits(limits=1), ThreadPoolExecutor(workers) as ex:
        list(ex.map(one, seqs))
    return o, lse


def assert_bf16_close(out: torch.Tensor, ref: np.ndarray, rows=None, what=""):
    got = f64(out)
    if rows is not None:
        got, ref = got[rows], ref[rows]
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = ATOL + RTOL * np.abs(ref)
    bad = err > bound
    assert not np.any(bad), (
        f"{what}: {int(bad.sum())} of {bad.size} elements outside atol={ATOL} rtol={RTOL}; "
        f"worst excess {float((err - bound).max()):.3e} at {np.unravel_index(np.argmax(err - bound), err.shape)}")


def assert_rows_rel(x: np.ndarray, ref: np.ndarray, tol=F32_REL, what=""):
    """Per-row relative error on the last axis."""
    x = np.asarray(x, dtype=np.float64)
    num = np.max(np.abs(x - ref), axis=-1)
    den = np.maximum(np.max(np.abs(ref), axis=-1), 1e-30)
    rel = num / den
    assert np.all(np.isfinite(x)), f"{what}: non-finite"
    assert np.all(rel <= tol), f"{what}: worst row rel err {rel.max():.3e} > {tol}"
    return float(rel.max())
