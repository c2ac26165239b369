"""CPU oracle for paged-KV attention (float64, NumPy): decode, the cache
write, multi-token-query (chunked prefill) attention, the fp8 (E4M3) cache and
whole-block copies (copy-on-write, swapping).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``.  The product package never
imports it, and it shares no code with the GPU kernels.
"""
from .paged_attention import (gather_contiguous, kv_head_of, merge_partitions, partition_stats,
                              read_k_row, read_v_row, ref_decode_sequence, ref_paged_attention_decode,
                              ref_reshape_and_cache, slot_of_position, softmax_attention, widen)
from .prefill import query_positions, ref_paged_attention_prefill
from .fp8 import dequantize_pool, e4m3_decode, e4m3_encode, ref_reshape_and_cache_fp8
from .block_copy import check_pairs, ref_copy_blocks

__all__ = ["gather_contiguous", "kv_head_of", "merge_partitions", "partition_stats", "read_k_row",
           "read_v_row", "ref_decode_sequence", "ref_paged_attention_decode", "ref_reshape_and_cache",
           "slot_of_position", "softmax_attention", "widen", "query_positions", "ref_paged_attention_prefill",
           "dequantize_pool", "e4m3_decode", "e4m3_encode", "ref_reshape_and_cache_fp8",
           "check_pairs", "ref_copy_blocks"]
