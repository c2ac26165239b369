"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars (from the contract of the library):
* reshape_and_cache: bit-exact pools;
* decode: max-abs error <= 1e-5 with fp32 KV and <= 2e-2 with bf16 KV
  (fp32 accumulation), with a relative-RMS check beside it because long
  contexts give small outputs that a loose max-abs bound would not catch;
* bit-identical results under physical block permutation, shared-vs-private
  prefix blocks, and repeated runs.
Every workload is poisoned with NaN outside the cached tokens, so any read
past a context end or into an unused block shows up as a non-finite output.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import (DeviceBatch, prompt_run_slots, compare, int_dev, oracle_decode_all, oracle_pools, out_f64, say, to_dev,
                      to_host_bits)
from paged_kv_cache_372_amd import ops
from paged_kv_cache_372_amd.blocks import tables_share_blocks

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ops.load_library()
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def run_and_check(b, partition_size=None, seqs=None, what=""):
    """Cache write + decode on the GPU; compare pools (bit-exact) and outputs
    (every sequence and query head unless ``seqs`` names a subset)."""
    say(f"[{b.name} seed={b.seed} B={b.num_seqs} ps={partition_size if partition_size is not None else b.partition_size}] {what}")
    db = DeviceBatch(b)
    db.write()
    db.decode(partition_size)
    torch.cuda.synchronize()
    kp, vp = oracle_pools(b)
    bits = np.uint32 if b.dtype == "f32" else np.uint16
    assert np.array_equal(to_host_bits(db.k_cache).view(bits), kp.view(bits)), "K pool differs"
    assert np.array_equal(to_host_bits(db.v_cache).view(bits), vp.view(bits)), "V pool differs"
    got = out_f64(db.out)
    if seqs is None:
        ref = oracle_decode_all(b.q, kp, vp, b.block_tables, b.context_lens, b.scale, b.dtype)
        compare(got, ref, b.dtype, f"{b.name} attention, all {b.num_seqs} sequences")
    else:
        ref = oracle.ref_paged_attention_decode(b.q, kp, vp, b.block_tables, b.context_lens, b.scale, b.dtype,
                                                seqs=seqs)
        compare(got[seqs], ref, b.dtype, f"{b.name} attention")
    return db, got


# --------------------------------------------------------------------------
# cache write
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,D", [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128)])
def test_cache_write_bit_exact(dtype, D):
    rng = np.random.default_rng(100 + D)
    NB, Hkv, T = 37, 3, 50
    ks, vs = W.pool_shapes(NB, Hkv, D, 16, dtype)
    bits = np.uint32 if dtype == "f32" else np.uint16
    k_pool = rng.integers(0, np.iinfo(bits).max, size=ks, dtype=bits, endpoint=True)
    v_pool = rng.integers(0, np.iinfo(bits).max, size=vs, dtype=bits, endpoint=True)
    k_new = rng.integers(0, np.iinfo(bits).max, size=(T, Hkv, D), dtype=bits, endpoint=True)
    v_new = rng.integers(0, np.iinfo(bits).max, size=(T, Hkv, D), dtype=bits, endpoint=True)
    slots = rng.choice(NB * 16, size=T, replace=False).astype(np.int64)
    slots[[3, 17]] = -1
    slots[29] = NB * 16 + 5   # outside the pool: skipped by contract
    say(f"[cache_write {dtype} D={D}]")
    host = (lambda a: a.view(np.float32)) if dtype == "f32" else (lambda a: a)
    dk, dv = to_dev(host(k_pool), dtype), to_dev(host(v_pool), dtype)
    ops.reshape_and_cache(to_dev(host(k_new), dtype), to_dev(host(v_new), dtype), int_dev(slots, np.int64), dk, dv)
    torch.cuda.synchronize()
    ref_slots = np.where(slots >= NB * 16, -1, slots)
    kp, vp = oracle.ref_reshape_and_cache(k_new, v_new, ref_slots, k_pool, v_pool)
    assert np.array_equal(to_host_bits(dk).view(bits), kp)
    assert np.array_equal(to_host_bits(dv).view(bits), vp)


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 64), ("bf16", 128)])
def test_cache_write_prompt_runs(dtype, D):
    """Prompt-like writes: runs of consecutive slots (the 16-byte V store
    path) mixed with every case that must fall back to element stores."""
    rng = np.random.default_rng(300 + D)
    NB, Hkv = 64, 2
    slots = prompt_run_slots(rng, NB)
    T = len(slots)
    ks, vs = W.pool_shapes(NB, Hkv, D, 16, dtype)
    bits = np.uint32 if dtype == "f32" else np.uint16
    k_pool = rng.integers(0, np.iinfo(bits).max, size=ks, dtype=bits, endpoint=True)
    v_pool = rng.integers(0, np.iinfo(bits).max, size=vs, dtype=bits, endpoint=True)
    k_new = rng.integers(0, np.iinfo(bits).max, size=(T, Hkv, D), dtype=bits, endpoint=True)
    v_new = rng.integers(0, np.iinfo(bits).max, size=(T, Hkv, D), dtype=bits, endpoint=True)
    say(f"[cache_write prompt runs {dtype} D={D} T={T}]")
    host = (lambda a: a.view(np.float32)) if dtype == "f32" else (lambda a: a)
    dk, dv = to_dev(host(k_pool), dtype), to_dev(host(v_pool), dtype)
    ops.reshape_and_cache(to_dev(host(k_new), dtype), to_dev(host(v_new), dtype), int_dev(slots, np.int64), dk, dv)
    torch.cuda.synchronize()
    ref_slots = np.where(slots >= NB * 16, -1, slots)
    kp, vp = oracle.ref_reshape_and_cache(k_new, v_new, ref_slots, k_pool, v_pool)
    assert np.array_equal(to_host_bits(dk).view(bits), kp)
    assert np.array_equal(to_host_bits(dv).view(bits), vp)


def test_cache_write_empty_is_noop():
    b = W.tiny_fp32()
    db = DeviceBatch(b)
    before = to_host_bits(db.k_cache).copy()
    ops.reshape_and_cache(db.k_new[:0], db.v_new[:0], db.slots[:0], db.k_cache, db.v_cache)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(db.k_cache).view(np.uint32), before.view(np.uint32))


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [W.DEFAULT_SEEDS["tiny_fp32"], 11, 12, 13])
def test_tiny_fp32(seed):
    b = W.tiny_fp32(seed)
    db, got = run_and_check(b)
    # a one-token context returns that token's value row exactly
    s1 = int(np.flatnonzero(b.context_lens == 1)[0])
    assert np.array_equal(got[s1].astype(np.float32), b.v_new[s1].astype(np.float32))


@pytest.mark.parametrize("ps", [0, 16, 48, 256, 1024])
def test_llama3_small(ps):
    run_and_check(W.llama3_8b_decode(num_seqs=6), partition_size=ps)


@pytest.mark.parametrize("seed", [W.DEFAULT_SEEDS["llama3_8b_decode"], 21, 22, 23])
def test_llama3_full_size(seed):
    b = W.llama3_8b_decode(seed)
    run_and_check(b, what="full size, every sequence")


def test_shared_prefix_full_size_and_private_copies():
    b = W.shared_prefix()
    db, got = run_and_check(b, what="full size, every sequence")
    # same content with every sequence holding a private copy of the prefix
    prefix = b.info["prefix_blocks"]
    extra = (b.num_seqs - 1) * len(prefix)
    kp, vp = b.k_pool, b.v_pool
    k2 = np.concatenate([kp, np.repeat(kp[prefix][None], b.num_seqs - 1, 0).reshape((extra,) + kp.shape[1:])])
    v2 = np.concatenate([vp, np.repeat(vp[prefix][None], b.num_seqs - 1, 0).reshape((extra,) + vp.shape[1:])])
    bt2 = b.block_tables.copy()
    for s in range(1, b.num_seqs):
        bt2[s, :len(prefix)] = b.num_blocks + (s - 1) * len(prefix) + np.arange(len(prefix))
    b2 = W.DecodeBatch(**{**b.__dict__, "k_pool": k2, "v_pool": v2, "block_tables": bt2,
                          "num_blocks": b.num_blocks + extra})
    db2 = DeviceBatch(b2)
    db2.write()
    db2.decode()
    torch.cuda.synchronize()
    assert torch.equal(db.out.view(torch.int16), db2.out.view(torch.int16)), "shared vs private prefix differ"


@pytest.mark.parametrize("make", [lambda: W.shared_prefix(num_seqs=16), lambda: W.llama3_8b_decode(num_seqs=6)],
                         ids=["shared_prefix", "llama3"])
def test_shared_blocks_flag_changes_nothing(make):
    """Cached and streaming reads of K/V give bit-identical outputs, equal to the oracle."""
    b = make()
    outs = []
    for shared in (True, False):
        say(f"[{b.name} B={b.num_seqs} shared_blocks={shared}]")
        db = DeviceBatch(b)
        db.write()
        db.decode(shared=shared)
        torch.cuda.synchronize()
        outs.append(db.out.clone())
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    kp, vp = oracle_pools(b)
    ref = oracle.ref_paged_attention_decode(b.q, kp, vp, b.block_tables, b.context_lens, b.scale, b.dtype)
    compare(out_f64(outs[0]), ref, b.dtype, f"{b.name} with cached reads")


def test_long_context_small():
    run_and_check(W.long_context(num_seqs=2, context_len=8192), what="8192 tokens, partition 512")


def test_long_context_full_size():
    b = W.long_context()
    say("generated", b.kv_bytes() / 1e9, "GB of KV")
    run_and_check(b, what="full size, every sequence and head")


def _batching(sim, steps):
    k_pool, v_pool = sim.initial_pools()
    dk, dv = to_dev(k_pool, sim.dtype), to_dev(v_pool, sim.dtype)
    for i in range(steps):
        st = sim.step(i)
        say(f"[continuous_batching B={sim.B}] step {i}: {st.num_prompt_tokens} prompt tokens, "
            f"max context {int(st.context_lens.max())}")
        q = to_dev(st.q, sim.dtype)
        out = torch.full(q.shape, float("nan"), dtype=q.dtype, device="cuda")
        bt, lens = int_dev(st.block_tables, np.int32), int_dev(st.context_lens, np.int32)
        ops.reshape_and_cache(to_dev(st.k_write, sim.dtype), to_dev(st.v_write, sim.dtype),
                              int_dev(st.slot_mapping, np.int64), dk, dv)
        ops.paged_attention_decode(q, dk, dv, bt, lens, sim.scale, out, partition_size=sim.partition_size,
                                   max_context_len=int(st.context_lens.max()),
                                   shared_blocks=tables_share_blocks(st.block_tables, st.context_lens, 16))
        torch.cuda.synchronize()
        k_pool, v_pool = oracle.ref_reshape_and_cache(st.k_write, st.v_write, st.slot_mapping, k_pool, v_pool)
        ref = oracle_decode_all(st.q, k_pool, v_pool, st.block_tables, st.context_lens, sim.scale, sim.dtype)
        compare(out_f64(out), ref, sim.dtype, f"step {i}, all {sim.B} sequences")
        written = np.unique(st.slot_mapping // 16)
        assert np.array_equal(to_host_bits(dk[written]), k_pool[written]), f"step {i}: K pool differs"
        assert np.array_equal(to_host_bits(dv[written]), v_pool[written]), f"step {i}: V pool differs"
    assert np.array_equal(to_host_bits(dk), k_pool) and np.array_equal(to_host_bits(dv), v_pool), "final pools differ"


def test_continuous_batching_small():
    # a quarter of a small batch turns over each step: more slack than 1.5x
    _batching(W.ContinuousBatching(num_seqs=24, steps=4, lmax=1024, replace_frac=0.25, pool_factor=3.0), 4)


def test_continuous_batching_full_size():
    _batching(W.ContinuousBatching(), 10)


# --------------------------------------------------------------------------
# invariances and edge cases
# --------------------------------------------------------------------------

def permuted(b, seed):
    """Same logical content with the physical blocks renumbered."""
    perm = np.random.default_rng(seed).permutation(b.num_blocks)
    k2 = np.empty_like(b.k_pool)
    v2 = np.empty_like(b.v_pool)
    k2[perm] = b.k_pool
    v2[perm] = b.v_pool
    slots = perm[b.slot_mapping // 16] * 16 + b.slot_mapping % 16
    return W.DecodeBatch(**{**b.__dict__, "k_pool": k2, "v_pool": v2, "block_tables": perm[b.block_tables].astype(np.int32),
                            "slot_mapping": slots.astype(np.int64)})


@pytest.mark.parametrize("make", [lambda: W.tiny_fp32(), lambda: W.llama3_8b_decode(num_seqs=5)])
def test_block_permutation_bit_identical(make):
    b = make()
    outs = []
    for bb in (b, permuted(b, 5), permuted(b, 6)):
        db = DeviceBatch(bb)
        db.write()
        db.decode(partition_size=256 if b.dtype == "bf16" else 0)
        torch.cuda.synchronize()
        outs.append(db.out.clone())
    for o in outs[1:]:
        assert torch.equal(outs[0].view(torch.int16), o.view(torch.int16))


def test_run_to_run_deterministic():
    b = W.llama3_8b_decode(num_seqs=8)
    db = DeviceBatch(b)
    db.write()
    db.decode()
    first = db.out.clone()
    for _ in range(3):
        db.out.fill_(float("nan"))
        db.decode()
        torch.cuda.synchronize()
        assert torch.equal(first.view(torch.int16), db.out.view(torch.int16))


@pytest.mark.parametrize("dtype,hq,hkv,D", [("bf16", 4, 4, 64), ("bf16", 8, 1, 128), ("bf16", 16, 1, 64),
                                            ("bf16", 32, 1, 128), ("bf16", 24, 2, 128), ("f32", 8, 2, 128),
                                            ("f32", 16, 2, 64), ("f32", 3, 3, 64), ("f32", 40, 4, 128)])
def test_head_groupings(dtype, hq, hkv, D):
    rng = np.random.default_rng(hq * 100 + hkv * 10 + D)
    lengths = rng.integers(1, 700, size=5)
    nb = W.pool_blocks_for(lengths, 16)
    b = W.build_static("heads", 7, dtype, hq, hkv, D, lengths, nb)
    for ps in (0, 64):
        run_and_check(b, partition_size=ps, what=f"{dtype} {hq}/{hkv} D={D}")


@pytest.mark.parametrize("dtype,hq,hkv,D,ps,kind", [
    ("bf16", 8, 2, 128, 0, "skew"), ("bf16", 8, 2, 64, 0, "skew"), ("bf16", 6, 2, 128, 0, "short"),
    ("bf16", 6, 2, 64, 0, "short"),
    ("f32", 3, 3, 64, 16, "short"), ("f32", 3, 3, 64, 64, "short")])
def test_reduce_shapes(dtype, hq, hkv, D, ps, kind):
    """The split-K merge in each of its forms (for a part with 128 to 1024
    balanced-decode workgroup columns):
    * skew: one 20000-token sequence among 63 short ones.  At most 1024
      ranges for 64 sequences, so one wave merges each row; the long
      sequence's rows (89 pieces or more) are merged by whole workgroups.
    * bf16 short: 33 sequences x 6 heads = 198 rows, so the last workgroup of
      four rows is half empty.
    * fp32, 16-token partitions: up to 44 pieces, one workgroup per row;
      64-token partitions: at most 11, one wave per row, 15 rows."""
    rng = np.random.default_rng([hq, hkv, D, ps, len(kind)])
    if kind == "skew":
        lengths = np.concatenate([[20000], rng.integers(16, 200, size=63)])
    else:
        lengths = rng.integers(1, 700, size=33 if dtype == "bf16" else 5)
    b = W.build_static("reduce", 8, dtype, hq, hkv, D, lengths, W.pool_blocks_for(lengths, 16))
    run_and_check(b, partition_size=ps, what=f"{dtype} {hq}/{hkv} D={D} {kind}")


def test_zero_length_and_single_token():
    b = W.build_static("edge", 9, "bf16", 8, 2, 128, [1, 1, 40, 300], 30)
    db, got = run_and_check(b, partition_size=32)
    # now zero the first two lengths: outputs must be exact zeros, and the rest unchanged
    lens = b.context_lens.copy()
    lens[:2] = 0
    db.lens.copy_(torch.from_numpy(lens))
    db.out.fill_(float("nan"))
    db.decode(partition_size=32)
    torch.cuda.synchronize()
    o = out_f64(db.out)
    assert np.array_equal(o[:2], np.zeros_like(o[:2]))
    assert np.array_equal(o[2:], got[2:])


def test_max_context_len_clamps_lengths():
    b = W.llama3_8b_decode(num_seqs=4)
    cap = 600
    db = DeviceBatch(b)
    db.write()
    db.decode(partition_size=128, max_context_len=cap)
    torch.cuda.synchronize()
    kp, vp = oracle_pools(b)
    ref = oracle.ref_paged_attention_decode(b.q, kp, vp, b.block_tables, np.minimum(b.context_lens, cap), b.scale,
                                            b.dtype)
    compare(out_f64(db.out), ref, b.dtype, "clamped to 600")


def test_two_phase_calls_equal_one_call():
    b = W.llama3_8b_decode(num_seqs=8)
    db = DeviceBatch(b)
    db.write()
    db.decode(partition_size=256)
    one = db.out.clone()
    db.out.fill_(float("nan"))
    a = ops.prepare_decode(db.q, db.k_cache, db.v_cache, db.bt, db.lens, b.scale, db.out, partition_size=256,
                           max_context_len=b.max_context_len)
    ops.run_partitions(a)
    ops.run_reduce(a)
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int16), db.out.view(torch.int16))


@pytest.mark.parametrize("make,ps", [(lambda: W.llama3_8b_decode(num_seqs=8), 0),
                                     (lambda: W.long_context(num_seqs=2, context_len=8192), 512),
                                     (lambda: W.build_static("valu_edge", 29, "bf16", 12, 3, 64, [1, 16, 17, 900], 80), 64)],
                         ids=["gqa4", "gqa8_partition512", "gqa4_d64_edges"])
def test_vector_alu_decode_bf16(make, ps):
    """The measurement aid that runs bf16 decode on the vector ALU meets the bf16 bar too."""
    b = make()
    say(f"[{b.name} B={b.num_seqs} vector ALU, ps={ps}]")
    db = DeviceBatch(b)
    db.write()
    ops.paged_attention_decode_vector_alu(db.q, db.k_cache, db.v_cache, db.bt, db.lens, b.scale, db.out,
                                          partition_size=ps, max_context_len=b.max_context_len)
    torch.cuda.synchronize()
    kp, vp = oracle_pools(b)
    ref = oracle_decode_all(b.q, kp, vp, b.block_tables, b.context_lens, b.scale, b.dtype)
    compare(out_f64(db.out), ref, b.dtype, f"{b.name} vector-ALU decode")


def test_fp32_output_from_bf16_kv():
    b = W.llama3_8b_decode(num_seqs=4)
    db = DeviceBatch(b, out_dtype=torch.float32)
    db.write()
    db.decode()
    torch.cuda.synchronize()
    kp, vp = oracle_pools(b)
    ref = oracle.ref_paged_attention_decode(b.q, kp, vp, b.block_tables, b.context_lens, b.scale, b.dtype)
    err, rel = compare(out_f64(db.out), ref, "bf16", "fp32 out")
    # without the final bf16 rounding the error is far below the bf16 bound
    assert err < 2e-3


def test_workspace_too_small_raises():
    b = W.llama3_8b_decode(num_seqs=4)
    db = DeviceBatch(b)
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(RuntimeError, match="workspace"):
        ops.paged_attention_decode(db.q, db.k_cache, db.v_cache, db.bt, db.lens, b.scale, db.out, partition_size=256,
                                   max_context_len=b.max_context_len, workspace=ws)


def test_workspace_reused_across_call_sizes():
    """One workspace, never cleared, serves calls of different sizes in a row."""
    a = W.llama3_8b_decode(num_seqs=6)                       # many ranges per sequence with the cap below
    b = W.long_context(num_seqs=2, context_len=3000, partition_size=0)
    need = max(ops.decode_workspace_bytes(x.num_seqs, x.num_q_heads, x.num_kv_heads, x.head_dim, x.max_context_len, ps)
               for x, ps in ((a, 48), (b, 0)))
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")   # garbage: NaN patterns
    first = None
    for x, ps in ((a, 48), (b, 0), (a, 48)):
        say(f"[{x.name} B={x.num_seqs} ps={ps}] shared workspace")
        db = DeviceBatch(x)
        db.write()
        ops.paged_attention_decode(db.q, db.k_cache, db.v_cache, db.bt, db.lens, x.scale, db.out, partition_size=ps,
                                   max_context_len=x.max_context_len, workspace=ws)
        torch.cuda.synchronize()
        kp, vp = oracle_pools(x)
        ref = oracle.ref_paged_attention_decode(x.q, kp, vp, x.block_tables, x.context_lens, x.scale, x.dtype)
        compare(out_f64(db.out), ref, x.dtype, f"{x.name} shared workspace")
        if x is a:
            if first is None:
                first = db.out.clone()
            else:
                assert torch.equal(first.view(torch.int16), db.out.view(torch.int16))


def test_more_than_4096_sequences():
    """A batch above one launch's 4096 sequences runs as consecutive launches."""
    rng = np.random.default_rng(4501)
    lengths = rng.integers(1, 41, size=4500)
    b = W.build_static("many", 45, "bf16", 8, 2, 64, lengths, W.pool_blocks_for(lengths, 16))
    run_and_check(b, what="4500 sequences")
    run_and_check(b, partition_size=16, what="4500 sequences, one-block ranges")
