"""CPU oracle for multi-token-query paged attention (chunked prefill), float64.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: imported by
``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg, never by the product path, and it shares no code with the GPU kernels.

What it computes, and where the pages define it:

* Prefill reads a whole prompt at once and caches the keys and values of all
  its tokens; it is parallel, compute-heavy work (runbyai section 1
  "Prefill and Decoding").
* A long prefill can stall decoding, so it is cut into chunks that share a
  per-step token budget with decode requests; newer schedulers no longer
  tell the two apart and only decide how many tokens each request processes
  in a step (architvora "Continuous Batching").

So a request s processes n_s >= 1 new tokens in a step.  Their keys and
values are already in the paged cache (written by the cache write of this
step), which then holds L_s tokens in all, the chunk being its last n_s.

Readings of points the pages leave open (each a documented reading):

* Query i of request s (0 <= i < n_s) sits at position p = L_s - n_s + i
  and attends to the tokens at positions 0..p of its own sequence: causal
  attention, aligned at the end of the context.  n_s = 1 is decode.
* The queries of all requests are packed row after row: request s owns rows
  ``query_start_loc[s] .. query_start_loc[s + 1] - 1`` of ``q`` and ``out``
  (``query_start_loc[0] = 0``, non-decreasing).
* Grouped-query mapping, pool layout, widening of bf16 as for decode.

The oracle follows the definition: walk the table to the contiguous K/V of
the sequence, then for every query token evaluate the softmax over its
causal prefix directly.
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence

import numpy as np

from .paged_attention import gather_contiguous, kv_head_of, q_dtype_of, softmax_attention, widen, widen_kv


def query_positions(context_len: int, num_queries: int) -> np.ndarray:
    """Positions of a request's query tokens: the last ``num_queries`` of its context."""
    return np.arange(context_len - num_queries, context_len, dtype=np.int64)


def ref_prefill_sequence(q_rows: np.ndarray, kc: np.ndarray, vc: np.ndarray, scale: float, num_kv_heads: int,
                         q_heads: Sequence[int], kv_heads_present: Sequence[int]) -> np.ndarray:
    """Causal attention of one request.

    ``q_rows`` float64 ``[n, Hq, D]``; ``kc``/``vc`` float64 ``[L, len(kv_heads_present), D]``.
    Returns float64 ``[n, len(q_heads), D]``.
    """
    n, Hq, D = q_rows.shape
    L = kc.shape[0]
    pos = query_positions(L, n)
    present = list(kv_heads_present)
    out = np.zeros((n, len(q_heads), D), dtype=np.float64)
    for i in range(n):
        p = int(pos[i])
        if p < 0:           # more queries than context: no key is visible
            continue
        for j, h in enumerate(q_heads):
            col = present.index(kv_head_of(h, Hq, num_kv_heads))
            out[i, j] = softmax_attention(q_rows[i, h], kc[:p + 1, col, :], vc[:p + 1, col, :], scale)
    return out


def ref_paged_attention_prefill(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, block_tables: np.ndarray,
                                context_lens: np.ndarray, query_start_loc: np.ndarray, scale: float, dtype: str,
                                seqs: Optional[Iterable[int]] = None,
                                q_heads: Optional[Sequence[int]] = None,
                                k_scale=None, v_scale=None) -> np.ndarray:
    """Multi-token-query paged attention, float64 ``[T, len(q_heads), D]``.

    Rows of requests not listed in ``seqs`` are left as NaN.  ``dtype``
    "fp8": E4M3 pools with per-KV-head scales, bf16 queries.
    """
    T, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    B = len(context_lens)
    seqs = list(range(B)) if seqs is None else list(seqs)
    q_heads = list(range(Hq)) if q_heads is None else list(q_heads)
    kv_needed = sorted({kv_head_of(h, Hq, Hkv) for h in q_heads})
    out = np.full((T, len(q_heads), D), np.nan, dtype=np.float64)
    for s in seqs:
        r0, r1 = int(query_start_loc[s]), int(query_start_loc[s + 1])
        L = int(context_lens[s])
        kc, vc = gather_contiguous(k_pool, v_pool, block_tables[s], L, heads=kv_needed)
        kw, vw = widen_kv(kc, vc, dtype, kv_needed, k_scale, v_scale)
        out[r0:r1] = ref_prefill_sequence(widen(q[r0:r1], q_dtype_of(dtype)), kw, vw, scale, Hkv, q_heads, kv_needed)
    return out

