"""Row-chunk fan-out of oracle calls over host threads, for the full-size
parity tests.  The oracle is single-threaded NumPy whose array kernels
release the GIL, so chunks of rows run side by side on the host cores; each
chunk is one unchanged oracle call, and the results come back in row order."""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

import oracle


def n_threads() -> int:
    return max(1, min(8, os.cpu_count() or 1))


def mxfp4_quantize_rows(x_bits: np.ndarray, even: bool = False, chunk: int = 128):
    """oracle.mxfp4_quantize over every row of x_bits [T, H], chunk by chunk."""
    starts = range(0, x_bits.shape[0], chunk)
    with cf.ThreadPoolExecutor(n_threads()) as ex:
        parts = list(ex.map(lambda r0: oracle.mxfp4_quantize(x_bits[r0:r0 + chunk], even), starts))
    if not parts:
        h = x_bits.shape[1]
        return np.zeros((0, h // 2), np.uint8), np.zeros((0, h // 32), np.uint8)
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])
