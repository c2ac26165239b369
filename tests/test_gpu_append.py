"""GPU parity of the fused decode step (pkv_paged_attention_decode_append):
the cache write of each sequence's new token folded into the decode launch.

Bars:
* the pools equal the oracle's cache write bit for bit (slot of position
  L - 1 of every sequence);
* the outputs are within the decode tolerance of the oracle;
* pools and outputs are bit-identical to the two-call path
  (reshape_and_cache, then paged_attention_decode) on the same inputs.
Workloads come from ``workloads`` (NaN-poisoned past every context), expected
values from ``oracle``.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import DeviceBatch, compare, oracle_decode_all, out_f64, say, to_host_bits
from paged_kv_cache_372_amd import ops
from paged_kv_cache_372_amd.blocks import tables_share_blocks

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ops.load_library()
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def fused(db, b, ps, max_ctx=None):
    shared = tables_share_blocks(b.block_tables, b.context_lens, b.block_size)
    ops.paged_attention_decode_append(db.q, db.k_new, db.v_new, db.k_cache, db.v_cache, db.bt, db.lens, b.scale,
                                      db.out, partition_size=ps,
                                      max_context_len=b.max_context_len if max_ctx is None else max_ctx,
                                      shared_blocks=shared)


def check(b, ps=None, slots=None, what=""):
    """Fused step vs the oracle and vs the two-call path.  ``slots``: the slots
    the oracle writes (default: the batch's, one per sequence at L - 1)."""
    ps = b.partition_size if ps is None else ps
    say(f"[append {b.name} seed={b.seed} B={b.num_seqs} Hq={b.num_q_heads} Hkv={b.num_kv_heads} "
        f"D={b.head_dim} ps={ps}] {what}")
    a = DeviceBatch(b)
    fused(a, b, ps)
    two = DeviceBatch(b)
    two.write()
    two.decode(ps)
    torch.cuda.synchronize()
    slots = b.slot_mapping if slots is None else slots
    kp, vp = oracle.ref_reshape_and_cache(b.k_new, b.v_new, slots, b.k_pool, b.v_pool)
    assert np.array_equal(to_host_bits(a.k_cache), kp), "K pool differs from the oracle"
    assert np.array_equal(to_host_bits(a.v_cache), vp), "V pool differs from the oracle"
    assert np.array_equal(to_host_bits(a.out), to_host_bits(two.out)), "output differs from the two-call path"
    got = out_f64(a.out)
    ref = oracle_decode_all(b.q, kp, vp, b.block_tables, b.context_lens, b.scale, b.dtype)
    compare(got, ref, b.dtype, f"{b.name} fused step, all {b.num_seqs} sequences")
    return a


@pytest.mark.parametrize("ps", [0, 16, 48, 512])
def test_llama3_small(ps):
    check(W.llama3_8b_decode(num_seqs=6), ps)


@pytest.mark.parametrize("seed", [W.DEFAULT_SEEDS["llama3_8b_decode"], 31])
def test_llama3_full_size(seed):
    b = W.llama3_8b_decode(seed)
    check(b, what="full size")


def test_shared_prefix_full_size():
    # the new tokens fall in private blocks past the shared prefix
    b = W.shared_prefix()
    check(b, what="full size")


@pytest.mark.parametrize("D,hq,hkv", [(64, 8, 8), (128, 64, 8), (128, 32, 16), (64, 16, 1)])
def test_many_short_sequences(D, hq, hkv):
    # lengths 1..70: most ranges hold several sequence ends, and some
    # sequences end in the first blocks of a range
    rng = np.random.default_rng([D, hq, hkv])
    lengths = rng.integers(1, 70, size=300, endpoint=True)
    nb = W.pool_blocks_for(lengths, 16)
    b = W.build_static("short_mix", 4100 + D + hq + hkv, "bf16", hq, hkv, D, lengths, num_blocks=nb)
    check(b)


@pytest.mark.parametrize("D", [128, 64])
def test_more_sequence_ends_than_lds_rows(D):
    # 3000 one-block sequences: each range holds about a dozen sequence
    # ends, more than a wave keeps in LDS, so the later ones go through the
    # store-before-walk path
    rng = np.random.default_rng(D)
    lengths = rng.integers(1, 16, size=3000, endpoint=True)
    nb = W.pool_blocks_for(lengths, 16)
    b = W.build_static("one_block_seqs", 4500 + D, "bf16", 8, 2, D, lengths, num_blocks=nb)
    check(b)


def test_empty_contexts_and_entries_outside_the_pool():
    rng = np.random.default_rng(7)
    lengths = rng.integers(1, 200, size=24, endpoint=True)
    nb = W.pool_blocks_for(lengths, 16)
    b = W.build_static("edge_mix", 4242, "bf16", 32, 8, 128, lengths, num_blocks=nb)
    slots = b.slot_mapping.copy()
    # empty contexts: nothing is stored, the output is zero
    for s in (0, 5, 23):
        b.context_lens[s] = 0
        slots[s] = -1
    # the last block of sequence 9 points outside the pool: nothing is stored
    s = 9
    L = int(b.context_lens[s])
    b.block_tables[s, (L - 1) // 16] = b.num_blocks + 3
    slots[s] = -1
    say("[append edge cases] empty contexts, table entry outside the pool")
    a = DeviceBatch(b)
    fused(a, b, 0)
    torch.cuda.synchronize()
    kp, vp = oracle.ref_reshape_and_cache(b.k_new, b.v_new, slots, b.k_pool, b.v_pool)
    assert np.array_equal(to_host_bits(a.k_cache), kp)
    assert np.array_equal(to_host_bits(a.v_cache), vp)
    got = out_f64(a.out)
    for s in (0, 5, 23):
        assert np.array_equal(got[s], np.zeros_like(got[s]))
    rest = [i for i in range(b.num_seqs) if i not in (0, 5, 9, 23)]
    ref = oracle.ref_paged_attention_decode(b.q, kp, vp, b.block_tables, b.context_lens, b.scale, b.dtype, seqs=rest)
    compare(got[rest], ref, b.dtype, "edge mix")


def test_more_sequences_than_one_launch():
    # > 4096 sequences run as two launches; k_new / v_new follow the split
    rng = np.random.default_rng(11)
    lengths = rng.integers(1, 40, size=4100, endpoint=True)
    nb = W.pool_blocks_for(lengths, 16)
    b = W.build_static("many_seqs", 4343, "bf16", 4, 2, 64, lengths, num_blocks=nb)
    check(b)


def test_long_context_full_size():
    b = W.long_context()
    check(b, what="8 x 128k, partition 512")


def test_rejected_shapes():
    b = W.llama3_8b_decode(num_seqs=2)
    db = DeviceBatch(b)
    # more than 16 query heads per KV head
    q = torch.zeros((2, 8 * 17, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError, match="query heads per KV head"):
        ops.paged_attention_decode_append(q, db.k_new, db.v_new, db.k_cache, db.v_cache, db.bt, db.lens, b.scale,
                                          torch.empty_like(q), max_context_len=b.max_context_len)
    # k_new of the wrong shape
    with pytest.raises(ValueError):
        ops.paged_attention_decode_append(db.q, db.k_new[:1], db.v_new, db.k_cache, db.v_cache, db.bt, db.lens,
                                          b.scale, db.out, max_context_len=b.max_context_len)
    # fp32 pools
    t = W.tiny_fp32()
    dt = DeviceBatch(t)
    with pytest.raises(ValueError):
        ops.paged_attention_decode_append(dt.q, dt.k_new, dt.v_new, dt.k_cache, dt.v_cache, dt.bt, dt.lens, t.scale,
                                          dt.out, max_context_len=t.max_context_len)


def test_fp32_output_and_two_phase_calls():
    b = W.llama3_8b_decode(num_seqs=9, seed=77)
    say("[append] fp32 output; two-phase calls equal one call")
    # fp32 output from bf16 pools
    a = DeviceBatch(b, out_dtype=torch.float32)
    fused(a, b, 0)
    torch.cuda.synchronize()
    kp, vp = oracle.ref_reshape_and_cache(b.k_new, b.v_new, b.slot_mapping, b.k_pool, b.v_pool)
    assert np.array_equal(to_host_bits(a.k_cache), kp) and np.array_equal(to_host_bits(a.v_cache), vp)
    ref = oracle.ref_paged_attention_decode(b.q, kp, vp, b.block_tables, b.context_lens, b.scale, b.dtype)
    compare(out_f64(a.out), ref, b.dtype, "fused, fp32 out")
    # the decode launch and the reduce called one at a time
    one = DeviceBatch(b)
    fused(one, b, 48)
    two = DeviceBatch(b)
    plan = ops.prepare_decode(two.q, two.k_cache, two.v_cache, two.bt, two.lens, b.scale, two.out, partition_size=48,
                              max_context_len=b.max_context_len, k_new=two.k_new, v_new=two.v_new)
    ops.run_partitions(plan)
    ops.run_reduce(plan)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(one.out), to_host_bits(two.out))
    assert np.array_equal(to_host_bits(one.k_cache), to_host_bits(two.k_cache))
    assert np.array_equal(to_host_bits(one.v_cache), to_host_bits(two.v_cache))
