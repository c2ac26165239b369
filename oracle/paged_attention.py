"""CPU oracle for paged-KV decode: the plain definition, in float64.

TEST INFRASTRUCTURE ONLY.  This module is imported by ``tests/``, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``;
the product path (``paged_kv_cache_372_amd``) never imports, calls or links
it, and it shares no code with the GPU kernels.

What it computes, and where the pages define it:

* Decode: one new query token per sequence attends over the keys and values
  of all earlier tokens, which are kept in the KV cache instead of being
  recomputed (runbyai section 1 "Prefill and Decoding" and section 2 "KV
  Cache"; architvora "KV cache problem").
* Paging: the cache is cut into fixed-size blocks; a per-sequence block table
  maps logically contiguous KV to scattered physical blocks (runbyai section
  3; ai-hpc "2.1 Algorithm Principle"; architvora "Paged Attention").  The
  GPU kernel "follows the block table to gather the blocks".

Because paging changes only *where* keys and values sit, the result is
exactly ordinary attention over the gathered, logically contiguous K/V.  The
oracle therefore (1) walks the table and materialises the contiguous K/V of a
sequence, then (2) evaluates softmax(scale * q K^T) V directly, in float64.

Readings of points the pages leave open (each a documented reading, not a
page fact):

* Query head h reads KV head ``h // (Hq / Hkv)`` (grouped-query attention
  with contiguous groups; Hq / Hkv = 1 is plain multi-head attention).
* Pool layout per (physical block, KV head): K ``[D/x, block_size, x]`` with
  ``x = 16 / element_size`` (the dims of one token are split into 16-byte
  chunks), V ``[D, block_size]`` (one row of block_size tokens per dim).
* A flat slot is ``block * block_size + offset``; a negative slot is skipped.
* ``context_lens[s]`` counts every token the new query attends to, the token
  written this step included.  ``context_lens[s] == 0`` yields zeros.
* bf16 data is carried as uint16 bit patterns and widened exactly.

Split-K (``partition_stats`` / ``merge_partitions``) is the log-sum-exp
identity that lets a long context be reduced in pieces: each piece keeps its
running max m, its sum of exponentials l and its unnormalised output o; the
pieces merge with weights exp(m_p - M).  It is not on the pages; it is the
mathematics of softmax, used to pin the GPU's split path.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np


# --------------------------------------------------------------------------
# element formats
# --------------------------------------------------------------------------

def bits_dtype(dtype: str):
    return {"f32": np.uint32, "bf16": np.uint16}[dtype]


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact conversion of f32 values or bf16 bit patterns to float64."""
    a = np.asarray(a)
    if dtype == "f32":
        return a.view(np.float32).astype(np.float64) if a.dtype == np.uint32 else a.astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        if a.dtype != np.uint16:
            raise TypeError("bf16 data must be uint16 bit patterns")
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def elem_bytes(dtype: str) -> int:
    return {"f32": 4, "bf16": 2}[dtype]


# --------------------------------------------------------------------------
# pool layout: one token's K row / V row of one KV head
# --------------------------------------------------------------------------

def read_k_row(k_pool: np.ndarray, block: int, head: int, offset: int) -> np.ndarray:
    """K row (D values, native bits) of the token at (block, offset) for ``head``.

    K tile layout: ``[D/x, block_size, x]``; dims ``c*x .. c*x+x-1`` of a token
    sit in chunk c at the token's offset.
    """
    return k_pool[block, head, :, offset, :].reshape(-1)


def read_v_row(v_pool: np.ndarray, block: int, head: int, offset: int) -> np.ndarray:
    """V row (D values) of the token at (block, offset); V tile layout ``[D, block_size]``."""
    return v_pool[block, head, :, offset]


def write_k_row(k_pool: np.ndarray, block: int, head: int, offset: int, row: np.ndarray) -> None:
    nchunk, x = k_pool.shape[2], k_pool.shape[4]
    k_pool[block, head, :, offset, :] = np.asarray(row).reshape(nchunk, x)


def write_v_row(v_pool: np.ndarray, block: int, head: int, offset: int, row: np.ndarray) -> None:
    v_pool[block, head, :, offset] = row


# --------------------------------------------------------------------------
# cache write
# --------------------------------------------------------------------------

def ref_reshape_and_cache(k_new: np.ndarray, v_new: np.ndarray, slot_mapping: np.ndarray,
                          k_pool: np.ndarray, v_pool: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Store token t's K/V rows (``[T, Hkv, D]``) at flat slot ``slot_mapping[t]``.

    This is "calculate and cache the KV of every token" (runbyai section 1)
    with the cache paged (runbyai section 3): the slot names the physical
    block and the offset inside it.  Returns new pools; the inputs are not
    modified.  Pure element copies, so the result is bit-exact.
    """
    k_out, v_out = k_pool.copy(), v_pool.copy()
    bs = k_pool.shape[3]
    nb, hkv = k_pool.shape[0], k_pool.shape[1]
    slots = np.asarray(slot_mapping, dtype=np.int64)
    live = slots[slots >= 0]
    if live.size and (live.max() >= nb * bs):
        raise ValueError("slot out of range")
    if np.unique(live).size != live.size:
        raise ValueError("duplicate slots make the write order-dependent")
    for t, slot in enumerate(slots):
        if slot < 0:
            continue
        block, offset = divmod(int(slot), bs)
        for h in range(hkv):
            write_k_row(k_out, block, h, offset, k_new[t, h])
            write_v_row(v_out, block, h, offset, v_new[t, h])
    return k_out, v_out


# --------------------------------------------------------------------------
# table walk
# --------------------------------------------------------------------------

def gather_contiguous(k_pool: np.ndarray, v_pool: np.ndarray, table_row: np.ndarray, context_len: int,
                      heads: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Follow one sequence's block table and return its logically contiguous K and V.

    Logical token ``pos`` lives in logical block ``pos // bs`` at offset
    ``pos % bs``; the table maps that logical block to a physical one.
    Returns native-bit arrays of shape ``[context_len, len(heads), D]``.
    """
    bs = k_pool.shape[3]
    if heads is None:
        heads = range(k_pool.shape[1])
    heads = np.asarray(list(heads), dtype=np.int64)
    D = k_pool.shape[2] * k_pool.shape[4]
    nblk = -(-context_len // bs)
    # physical block of each logical block j < nblk, and its tiles for the
    # listed heads: K [nblk, heads, D/x, bs, x], V [nblk, heads, D, bs]
    phys = np.asarray(table_row[:nblk], dtype=np.int64)
    k_tiles = k_pool[phys[:, None], heads[None, :]]
    v_tiles = v_pool[phys[:, None], heads[None, :]]
    # token t of logical block j is logical position j * bs + t; its K row
    # is the chunks at offset t, its V row the column t of the tile
    kc = np.transpose(k_tiles, (0, 3, 1, 2, 4)).reshape(nblk * bs, len(heads), D)[:context_len]
    vc = np.transpose(v_tiles, (0, 3, 1, 2)).reshape(nblk * bs, len(heads), D)[:context_len]
    return kc, vc


def kv_head_of(q_head: int, num_q_heads: int, num_kv_heads: int) -> int:
    """Grouped-query mapping: contiguous groups of Hq/Hkv query heads share a KV head."""
    return q_head // (num_q_heads // num_kv_heads)


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * k q) weighted sum of v, in float64.  q [D], k/v [L, D]."""
    if k.shape[0] == 0:
        return np.zeros(v.shape[1], dtype=np.float64)
    s = scale * (k @ q)
    w = np.exp(s - s.max())
    return (w @ v) / w.sum()


def ref_decode_sequence(q_s: np.ndarray, kc: np.ndarray, vc: np.ndarray, scale: float,
                        num_kv_heads: int, q_heads: Optional[Sequence[int]] = None,
                        kv_heads_present: Optional[Sequence[int]] = None) -> np.ndarray:
    """Decode output of one sequence for the listed query heads.

    ``q_s`` is float64 ``[Hq, D]``; ``kc``/``vc`` are float64 ``[L, n_heads, D]``
    holding the KV heads listed in ``kv_heads_present`` (all, by default).
    """
    Hq = q_s.shape[0]
    if q_heads is None:
        q_heads = range(Hq)
    present = list(range(num_kv_heads)) if kv_heads_present is None else list(kv_heads_present)
    out = np.empty((len(list(q_heads)), q_s.shape[1]), dtype=np.float64)
    rows = {}  # KV head -> its K and V rows as contiguous [L, D] arrays
    for i, h in enumerate(q_heads):
        kvh = kv_head_of(h, Hq, num_kv_heads)
        if kvh not in rows:
            j = present.index(kvh)
            rows[kvh] = (np.ascontiguousarray(kc[:, j, :]), np.ascontiguousarray(vc[:, j, :]))
        out[i] = softmax_attention(q_s[h], rows[kvh][0], rows[kvh][1], scale)
    return out


def widen_kv(kc: np.ndarray, vc: np.ndarray, dtype: str, heads: Sequence[int], k_scale=None, v_scale=None):
    """float64 K/V of gathered rows ``[L, len(heads), D]``.

    ``dtype`` "fp8": E4M3 codes times the per-KV-head scales (see
    ``oracle/fp8.py``); otherwise the stored values widened exactly.
    """
    if dtype != "fp8":
        return widen(kc, dtype), widen(vc, dtype)
    from .fp8 import e4m3_decode
    ks = np.asarray(k_scale, dtype=np.float64)[list(heads)].reshape(1, -1, 1)
    vs = np.asarray(v_scale, dtype=np.float64)[list(heads)].reshape(1, -1, 1)
    return e4m3_decode(kc) * ks, e4m3_decode(vc) * vs


def q_dtype_of(dtype: str) -> str:
    """Queries are not cached: with an fp8 cache they stay bf16."""
    return "bf16" if dtype == "fp8" else dtype


def ref_paged_attention_decode(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, block_tables: np.ndarray,
                               context_lens: np.ndarray, scale: float, dtype: str,
                               seqs: Optional[Iterable[int]] = None,
                               q_heads: Optional[Sequence[int]] = None,
                               k_scale=None, v_scale=None) -> np.ndarray:
    """Paged decode attention, float64 result ``[len(seqs), len(q_heads), D]``.

    For each sequence: walk its block table to get contiguous K/V (only the
    KV heads the requested query heads need), widen to float64 (for an fp8
    cache: decode and scale per KV head), then plain softmax attention per
    query head.
    """
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    seqs = list(range(B)) if seqs is None else list(seqs)
    q_heads = list(range(Hq)) if q_heads is None else list(q_heads)
    kv_needed = sorted({kv_head_of(h, Hq, Hkv) for h in q_heads})
    out = np.empty((len(seqs), len(q_heads), D), dtype=np.float64)
    for i, s in enumerate(seqs):
        L = int(context_lens[s])
        kc, vc = gather_contiguous(k_pool, v_pool, block_tables[s], L, heads=kv_needed)
        kw, vw = widen_kv(kc, vc, dtype, kv_needed, k_scale, v_scale)
        out[i] = ref_decode_sequence(widen(q[s], q_dtype_of(dtype)), kw, vw, scale, Hkv,
                                     q_heads=q_heads, kv_heads_present=kv_needed)
    return out


# --------------------------------------------------------------------------
# split-K: partial statistics and their merge
# --------------------------------------------------------------------------

def partition_stats(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                    partition_size: int) -> List[Tuple[float, float, np.ndarray]]:
    """Per partition of ``partition_size`` tokens: (m, l, o) with
    m = max score, l = sum exp(s - m), o = sum exp(s - m) v (unnormalised)."""
    L = k.shape[0]
    stats = []
    for lo in range(0, L, partition_size):
        s = scale * (k[lo:lo + partition_size] @ q)
        m = float(s.max())
        w = np.exp(s - m)
        stats.append((m, float(w.sum()), w @ v[lo:lo + partition_size]))
    return stats


def merge_partitions(stats: Sequence[Tuple[float, float, np.ndarray]], D: int) -> np.ndarray:
    """Log-sum-exp merge: out = sum_p e^(m_p-M) o_p / sum_p e^(m_p-M) l_p.

    Partitions with no tokens (m = -inf, l = 0) contribute nothing.
    """
    live = [(m, l, o) for (m, l, o) in stats if l > 0 and math.isfinite(m)]
    if not live:
        return np.zeros(D, dtype=np.float64)
    M = max(m for m, _, _ in live)
    num = np.zeros(D, dtype=np.float64)
    den = 0.0
    for m, l, o in live:
        w = math.exp(m - M)
        num += w * o
        den += w * l
    return num / den


def slot_of_position(table_row: np.ndarray, pos: int, block_size: int) -> int:
    """Flat slot of logical position ``pos``: physical block of ``pos // bs``, offset ``pos % bs``."""
    return int(table_row[pos // block_size]) * block_size + pos % block_size
