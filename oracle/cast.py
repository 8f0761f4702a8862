"""Full-pool cast and gather-then-cast -- oracle (test infrastructure).

* ``cast_ref``: the pages' full-pool ``get_key_buffer(layer).to(q.dtype)``,
  every slot of a ``[num_slots, 576]`` FP8 pool to BF16
  ("The KV Cache Cast Bottleneck", *The Context* and *The Message*).
* ``gather_ref``: the pages' fallback, ``k_fp8[kv_indices]`` followed by a
  cast of the compact buffer, row r of the result holding pool row
  ``indices[r]`` ("The Gather-Then-Cast Pivot", *Reasoning Process* and
  *Assumptions*).

Both are unscaled dtype casts: the ``.to()`` calls the pages show carry no
scale factor.  The result is BF16 bit patterns (uint16).
"""
import numpy as np

from .e4m3 import cast_table_bf16

_TABLE = None


def _table() -> np.ndarray:
    global _TABLE
    if _TABLE is None:
        _TABLE = cast_table_bf16()
    return _TABLE


def cast_ref(pool: np.ndarray) -> np.ndarray:
    """uint16 array shaped like ``pool``: BF16 bits of each E4M3FN byte."""
    pool = np.asarray(pool)
    if pool.dtype != np.uint8:
        raise TypeError("pool must hold raw E4M3FN bytes (uint8)")
    return _table()[pool]


def gather_ref(pool: np.ndarray, indices: np.ndarray) -> np.ndarray:
    """uint16 [n, W]: row r is the BF16 cast of ``pool[indices[r]]``."""
    pool = np.asarray(pool)
    indices = np.asarray(indices)
    if pool.ndim != 2:
        raise ValueError("pool must be [num_slots, W]")
    if indices.ndim != 1:
        raise ValueError("indices must be 1-D")
    if indices.size and (indices.min() < 0 or indices.max() >= pool.shape[0]):
        raise IndexError("gather index outside the pool")
    return cast_ref(pool[indices.astype(np.int64)])
