"""CPU oracle for whole-block copies: copy-on-write and swapping.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``; never imported by the
product path and sharing no code with the GPU kernels.

What the pages say:

* Sequences forked from one prompt (parallel sampling, beam search) share
  the prompt's physical blocks, the way an operating system shares pages
  copy-on-write ("Deep Dive into vLLM", 2.2 "Advantages", item 2).  A shared
  block is copied when one of its owners must write into it.
* A sequence can be preempted and its KV moved to CPU memory (architvora,
  "Paged Attention", the closing list of advantages); bringing it back is
  the reverse move.

Both are whole-block copies: every KV head, every token slot, K and V, bit
for bit.  A copy maps a source block of one pool to a destination block of
another pool, or of the same pool.  Readings: a pair with a block id outside
its pool is skipped; destinations are distinct and no destination is also a
source in the same call (otherwise the result would depend on order).
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def ref_copy_blocks(src_k: np.ndarray, src_v: np.ndarray, dst_k: np.ndarray, dst_v: np.ndarray,
                    pairs: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Copies of the destination pools after copying block ``src`` to ``dst`` for every (src, dst) pair."""
    out_k = dst_k.copy()
    out_v = dst_v.copy()
    n_src, n_dst = src_k.shape[0], dst_k.shape[0]
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        if not (0 <= src < n_src and 0 <= dst < n_dst):
            continue
        out_k[dst] = src_k[src]
        out_v[dst] = src_v[src]
    return out_k, out_v


def check_pairs(pairs: np.ndarray) -> None:
    """The call's precondition: distinct destinations, none of them a source."""
    p = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    if np.unique(p[:, 1]).size != p.shape[0]:
        raise ValueError("duplicate destination block")
    if np.intersect1d(p[:, 0], p[:, 1]).size:
        raise ValueError("a destination block is also a source")
