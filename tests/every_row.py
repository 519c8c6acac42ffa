"""Every-row parity at full size: the oracle and the comparison run on blocks
of rows, several blocks at a time on the host's cores, so host memory stays
bounded (about 4 M elements per block) while every output element of a
full-size call is checked.

The oracle entry points (ctypes) and numpy's array operations release the
interpreter lock, so the blocks do run in parallel.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Callable, Dict, List, Tuple

# Elements per block of rows (a 32 MiB float64 array per block and output).
BLOCK_ELEMS = 1 << 22
# Worker threads; at most 16, the CPU share of a one-GPU host.
THREADS = max(1, min(16, os.cpu_count() or 1))


def blocks(N: int, D: int, align: int = 1) -> List[Tuple[int, int]]:
    """Consecutive [lo, hi) row blocks covering 0..N, each a multiple of
    ``align`` rows long (except the last) and about BLOCK_ELEMS elements."""
    rows = max(1, BLOCK_ELEMS // max(1, D))
    rows = max(align, rows // align * align)
    return [(lo, min(N, lo + rows)) for lo in range(0, N, rows)]


def merge(results: List[Dict[str, float]]) -> Dict[str, float]:
    """Worst error per key over the blocks; admitted counts are summed."""
    out: Dict[str, float] = {}
    for r in results:
        for k, v in r.items():
            if "admitted" in k:
                out[k] = out.get(k, 0) + int(v)
            else:
                out[k] = max(out.get(k, 0.0), float(v))
    return out


def run_blocks(N: int, D: int, fn: Callable[[slice], Dict[str, float]],
               align: int = 1) -> Dict[str, float]:
    """Call ``fn(slice(lo, hi))`` for every row block (in parallel) and merge
    the results; ``rows_checked`` counts the rows covered. An assertion
    raised in any block propagates."""
    bs = blocks(N, D, align)
    with ThreadPoolExecutor(THREADS) as ex:
        res = list(ex.map(lambda b: fn(slice(b[0], b[1])), bs))
    out = merge(res)
    out["rows_checked"] = sum(hi - lo for lo, hi in bs)
    return out
