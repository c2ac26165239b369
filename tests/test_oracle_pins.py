"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each pin names what fixes it:

* P1  cache write: after the write the pool differs from before exactly at
      the written slots, which hold the inputs bit for bit -- checked through
      flat offsets computed from the documented pool layout, not through the
      oracle's own indexing.
* PL  table walk: an element-coded pool (every element stores its own
      (block, head, offset, dim) code) gathered through a permuted table.
* P2  identity table == contiguous attention, against torch's
      scaled_dot_product_attention in float64 (a library routine).
* P3  permuting physical blocks leaves the result bit-identical.
* P4  shared prefix blocks give the same result, bit for bit, as private copies.
* P5  brute force with scalar Python loops (math.exp / math.fsum) on tiny inputs.
* P6  closed forms: one token -> its value row; zero query or zero scale ->
      mean of the value rows; identical keys -> mean; one dominant key -> its row.
* P7  split-K: merging per-partition (m, l, o) reproduces the unsplit softmax.
* G   hand-worked examples stored under tests/golden/.

``test_planted_mistakes_are_caught`` plants plausible mistakes in the oracle
(on the CPU) and checks that at least one pin fails for each.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.paged_attention as opa
from workloads import bf16_bits_rne, pool_shapes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# helpers that build pools WITHOUT the oracle (flat offsets from the layout)
# --------------------------------------------------------------------------

def k_flat_offset(b, h, o, d, Hkv, D, bs, x):
    """Documented K layout [NB, Hkv, D/x, bs, x]."""
    c, e = divmod(d, x)
    return ((((b * Hkv + h) * (D // x) + c) * bs + o) * x) + e


def v_flat_offset(b, h, o, d, Hkv, D, bs):
    """Documented V layout [NB, Hkv, D, bs]."""
    return ((b * Hkv + h) * D + d) * bs + o


def place_tokens(kc, vc, table, bs, nb, dtype, fill_nan=True):
    """Put contiguous K/V ``[L, Hkv, D]`` (float values) into pools via flat offsets."""
    L, Hkv, D = kc.shape
    x = 16 // (4 if dtype == "f32" else 2)
    ks, vs = pool_shapes(nb, Hkv, D, bs, dtype)
    store = np.float32 if dtype == "f32" else np.uint16
    kflat = np.full(int(np.prod(ks)), np.nan if dtype == "f32" else 0x7FC0, dtype=store)
    vflat = np.full(int(np.prod(vs)), np.nan if dtype == "f32" else 0x7FC0, dtype=store)
    kbits = kc.astype(np.float32) if dtype == "f32" else bf16_bits_rne(kc)
    vbits = vc.astype(np.float32) if dtype == "f32" else bf16_bits_rne(vc)
    for pos in range(L):
        b, o = int(table[pos // bs]), pos % bs
        for h in range(Hkv):
            for d in range(D):
                kflat[k_flat_offset(b, h, o, d, Hkv, D, bs, x)] = kbits[pos, h, d]
                vflat[v_flat_offset(b, h, o, d, Hkv, D, bs)] = vbits[pos, h, d]
    return kflat.reshape(ks), vflat.reshape(vs)


def exact_values(shape, rng, dtype):
    """Random values exactly representable in the storage dtype, as float64."""
    v = rng.standard_normal(shape).astype(np.float32)
    if dtype == "bf16":
        v = opa.widen(bf16_bits_rne(v), "bf16")
    return v.astype(np.float64)


def storage(v, dtype):
    return v.astype(np.float32) if dtype == "f32" else bf16_bits_rne(v.astype(np.float32))


def torch_sdpa(q, kc, vc, scale):
    """q [Hq, D], kc/vc [L, Hkv, D] float64 -> [Hq, D] via torch SDPA (math path, CPU, fp64)."""
    Hq, D = q.shape
    Hkv = kc.shape[1]
    G = Hq // Hkv
    K = torch.from_numpy(kc).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
    V = torch.from_numpy(vc).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
    Q = torch.from_numpy(q)[None, :, None, :]
    out = torch.nn.functional.scaled_dot_product_attention(Q, K.contiguous(), V.contiguous(), scale=scale)
    return out[0, :, 0, :].numpy()


# --------------------------------------------------------------------------
# pin implementations (reused by the planted-mistake test)
# --------------------------------------------------------------------------

def pin_p1(seed=0, dtype="bf16"):
    rng = np.random.default_rng(seed)
    nb, Hkv, D, bs = 6, 2, 16, 4
    x = 16 // (4 if dtype == "f32" else 2)
    ks, vs = pool_shapes(nb, Hkv, D, bs, dtype)
    bits = np.uint32 if dtype == "f32" else np.uint16
    k_pool = rng.integers(0, np.iinfo(bits).max, size=ks, dtype=bits, endpoint=True)
    v_pool = rng.integers(0, np.iinfo(bits).max, size=vs, dtype=bits, endpoint=True)
    T = 7
    slots = rng.choice(nb * bs, size=T, replace=False).astype(np.int64)
    slots[2] = -1
    k_new = rng.integers(0, np.iinfo(bits).max, size=(T, Hkv, D), dtype=bits, endpoint=True)
    v_new = rng.integers(0, np.iinfo(bits).max, size=(T, Hkv, D), dtype=bits, endpoint=True)
    k_out, v_out = opa.ref_reshape_and_cache(k_new, v_new, slots, k_pool, v_pool)
    kexp, vexp = k_pool.reshape(-1).copy(), v_pool.reshape(-1).copy()
    for t, s in enumerate(slots):
        if s < 0:
            continue
        b, o = divmod(int(s), bs)
        for h in range(Hkv):
            for d in range(D):
                kexp[k_flat_offset(b, h, o, d, Hkv, D, bs, x)] = k_new[t, h, d]
                vexp[v_flat_offset(b, h, o, d, Hkv, D, bs)] = v_new[t, h, d]
    assert np.array_equal(k_out.reshape(-1), kexp)
    assert np.array_equal(v_out.reshape(-1), vexp)
    # inputs untouched
    assert not np.shares_memory(k_out, k_pool)


def pin_layout(seed=1):
    rng = np.random.default_rng(seed)
    nb, Hkv, D, bs, x = 5, 3, 16, 4, 8
    ks, vs = pool_shapes(nb, Hkv, D, bs, "bf16")
    code = lambda b, h, o, d: ((b * 10 + h) * 100 + o) * 1000 + d
    kflat = np.zeros(int(np.prod(ks)), dtype=np.int64)
    vflat = np.zeros(int(np.prod(vs)), dtype=np.int64)
    for b in range(nb):
        for h in range(Hkv):
            for o in range(bs):
                for d in range(D):
                    kflat[k_flat_offset(b, h, o, d, Hkv, D, bs, x)] = code(b, h, o, d)
                    vflat[v_flat_offset(b, h, o, d, Hkv, D, bs)] = -code(b, h, o, d)
    table = rng.permutation(nb)
    L = 17
    kc, vc = opa.gather_contiguous(kflat.reshape(ks), vflat.reshape(vs), table, L)
    for pos in range(L):
        for h in range(Hkv):
            for d in range(D):
                c = code(int(table[pos // bs]), h, pos % bs, d)
                assert kc[pos, h, d] == c and vc[pos, h, d] == -c


def pin_p2(seed=2, dtype="bf16", Hq=8, Hkv=2, D=32, L=45, bs=16, tol=1e-12):
    rng = np.random.default_rng(seed)
    kc = exact_values((L, Hkv, D), rng, dtype)
    vc = exact_values((L, Hkv, D), rng, dtype)
    q = exact_values((1, Hq, D), rng, dtype)
    nblk = -(-L // bs)
    table = np.arange(nblk + 1, dtype=np.int32)  # identity; last entry unused
    k_pool, v_pool = place_tokens(kc, vc, table, bs, nblk + 1, dtype)
    scale = 1.0 / math.sqrt(D)
    got = opa.ref_paged_attention_decode(storage(q, dtype), k_pool, v_pool, table[None], np.array([L]), scale, dtype)[0]
    ref = torch_sdpa(q[0], kc, vc, scale)
    assert np.max(np.abs(got - ref)) <= tol


def _two_placements(seed, dtype, L, Hq, Hkv, D, bs, nb):
    rng = np.random.default_rng(seed)
    kc = exact_values((L, Hkv, D), rng, dtype)
    vc = exact_values((L, Hkv, D), rng, dtype)
    q = storage(exact_values((1, Hq, D), rng, dtype), dtype)
    nblk = -(-L // bs)
    t1 = rng.permutation(nb)[:nblk].astype(np.int32)
    t2 = rng.permutation(nb)[:nblk].astype(np.int32)
    p1 = place_tokens(kc, vc, t1, bs, nb, dtype)
    p2 = place_tokens(kc, vc, t2, bs, nb, dtype)
    return q, (p1, t1), (p2, t2)


def pin_p3(seed=3, dtype="bf16"):
    L, Hq, Hkv, D, bs, nb = 70, 4, 2, 16, 16, 9
    q, (p1, t1), (p2, t2) = _two_placements(seed, dtype, L, Hq, Hkv, D, bs, nb)
    o1 = opa.ref_paged_attention_decode(q, p1[0], p1[1], t1[None], np.array([L]), 0.3, dtype)
    o2 = opa.ref_paged_attention_decode(q, p2[0], p2[1], t2[None], np.array([L]), 0.3, dtype)
    assert np.array_equal(o1, o2)


def pin_p4(seed=4, dtype="bf16"):
    """Two sequences sharing 2 prefix blocks vs. the same content in private blocks."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, bs = 4, 2, 16, 8
    prefix = exact_values((2 * bs, Hkv, D), rng, dtype), exact_values((2 * bs, Hkv, D), rng, dtype)
    suf = [(exact_values((n, Hkv, D), rng, dtype), exact_values((n, Hkv, D), rng, dtype)) for n in (3, 11)]
    q = storage(exact_values((2, Hq, D), rng, dtype), dtype)
    lens = np.array([2 * bs + 3, 2 * bs + 11])
    nb = 12
    # shared: prefix in blocks 5, 1; suffixes in 7 and 3, 9
    shared_tables = np.array([[5, 1, 7, 0], [5, 1, 3, 9]], dtype=np.int32)
    private_tables = np.array([[2, 8, 10, 0], [4, 6, 11, 0]], dtype=np.int32)

    def build(tables):
        ks, vs = pool_shapes(nb, Hkv, D, bs, dtype)
        kp = np.zeros(ks, dtype=np.float32 if dtype == "f32" else np.uint16)
        vp = np.zeros(vs, dtype=kp.dtype)
        for s in range(2):
            kc = np.concatenate([prefix[0], suf[s][0]])
            vc = np.concatenate([prefix[1], suf[s][1]])
            a, b = place_tokens(kc, vc, tables[s], bs, nb, dtype)
            nblk = -(-lens[s] // bs)
            for j in range(nblk):
                kp[tables[s][j]] = a[tables[s][j]]
                vp[tables[s][j]] = b[tables[s][j]]
        return kp, vp

    ks_, vs_ = build(shared_tables)
    kp_, vp_ = build(private_tables)
    o1 = opa.ref_paged_attention_decode(q, ks_, vs_, shared_tables, lens, 0.25, dtype)
    o2 = opa.ref_paged_attention_decode(q, kp_, vp_, private_tables, lens, 0.25, dtype)
    assert np.array_equal(o1, o2)


def brute_force(q, kflat, vflat, table, L, scale, Hq, Hkv, D, bs, x):
    """Scalar loops over the flat pools; float64 via Python floats."""
    G = Hq // Hkv
    out = []
    for h in range(Hq):
        kvh = h // G
        scores = []
        for pos in range(L):
            b, o = int(table[pos // bs]), pos % bs
            scores.append(scale * math.fsum(float(q[h][d]) * float(kflat[k_flat_offset(b, kvh, o, d, Hkv, D, bs, x)])
                                            for d in range(D)))
        m = max(scores)
        w = [math.exp(s - m) for s in scores]
        den = math.fsum(w)
        row = []
        for d in range(D):
            row.append(math.fsum(w[pos] * float(vflat[v_flat_offset(int(table[pos // bs]), kvh, pos % bs, d, Hkv, D, bs)])
                                 for pos in range(L)) / den)
        out.append(row)
    return np.array(out)


def pin_p5(seed=5, dtype="f32", shapes=((4, 2, 8, 1), (2, 2, 16, 23), (8, 2, 8, 40), (4, 4, 64, 37))):
    rng = np.random.default_rng(seed)
    for Hq, Hkv, D, L in shapes:
        bs = 16
        nblk = -(-L // bs)
        nb = nblk + 3
        table = rng.permutation(nb)[:nblk].astype(np.int32)
        kc = exact_values((L, Hkv, D), rng, dtype)
        vc = exact_values((L, Hkv, D), rng, dtype)
        q = exact_values((Hq, D), rng, dtype)
        kp, vp = place_tokens(kc, vc, table, bs, nb, dtype)
        scale = 0.7 / math.sqrt(D)
        got = opa.ref_paged_attention_decode(storage(q[None], dtype), kp, vp, table[None], np.array([L]), scale, dtype)[0]
        kflat = opa.widen(kp.reshape(-1), dtype)
        vflat = opa.widen(vp.reshape(-1), dtype)
        x = 16 // (4 if dtype == "f32" else 2)
        ref = brute_force(q, kflat, vflat, table, L, scale, Hq, Hkv, D, bs, x)
        assert np.max(np.abs(got - ref)) <= 1e-12


def pin_p6(seed=6, dtype="bf16"):
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, bs = 4, 2, 16, 16
    # (a) one token: output is that token's value row, exactly
    kc = exact_values((1, Hkv, D), rng, dtype)
    vc = exact_values((1, Hkv, D), rng, dtype)
    q = storage(exact_values((1, Hq, D), rng, dtype), dtype)
    kp, vp = place_tokens(kc, vc, np.array([2]), bs, 3, dtype)
    out = opa.ref_paged_attention_decode(q, kp, vp, np.array([[2]]), np.array([1]), 0.5, dtype)[0]
    for h in range(Hq):
        assert np.array_equal(out[h], vc[0, h // (Hq // Hkv)])
    # (b) zero scale and (c) zero query: uniform weights -> mean of V
    L = 37
    kc = exact_values((L, Hkv, D), rng, dtype)
    vc = exact_values((L, Hkv, D), rng, dtype)
    table = np.array([4, 0, 2], dtype=np.int32)
    kp, vp = place_tokens(kc, vc, table, bs, 5, dtype)
    for qv, sc in ((q, 0.0), (storage(np.zeros((1, Hq, D)), dtype), 0.3)):
        out = opa.ref_paged_attention_decode(qv, kp, vp, table[None], np.array([L]), sc, dtype)[0]
        for h in range(Hq):
            assert np.max(np.abs(out[h] - vc[:, h // 2].mean(axis=0))) <= 1e-14
    # (d) identical keys -> mean of V
    kc_same = np.repeat(kc[:1], L, axis=0)
    kp2, vp2 = place_tokens(kc_same, vc, table, bs, 5, dtype)
    out = opa.ref_paged_attention_decode(q, kp2, vp2, table[None], np.array([L]), 0.4, dtype)[0]
    for h in range(Hq):
        assert np.max(np.abs(out[h] - vc[:, h // 2].mean(axis=0))) <= 1e-14
    # (e) one key scores 60 above every other: output is its value row (to ~L e^-60)
    kc_dom = np.zeros((L, Hkv, D))
    kc_dom[23, :, 0] = 1.0
    qd = np.zeros((1, Hq, D))
    qd[..., 0] = 1.0
    kp3, vp3 = place_tokens(kc_dom, vc, table, bs, 5, dtype)
    out = opa.ref_paged_attention_decode(storage(qd, dtype), kp3, vp3, table[None], np.array([L]), 60.0, dtype)[0]
    for h in range(Hq):
        assert np.max(np.abs(out[h] - vc[23, h // 2])) <= L * math.exp(-60) * 10


def pin_p7(seed=7):
    rng = np.random.default_rng(seed)
    L, D = 1300, 32
    k = rng.standard_normal((L, D))
    v = rng.standard_normal((L, D))
    q = rng.standard_normal(D) * 2
    ref = opa.softmax_attention(q, k, v, 0.2)
    for ps in (16, 512, 4096):
        got = opa.merge_partitions(opa.partition_stats(q, k, v, 0.2, ps), D)
        assert np.max(np.abs(got - ref)) <= 1e-12
    # empty partitions are ignored
    st = opa.partition_stats(q, k, v, 0.2, 512) + [(-math.inf, 0.0, np.zeros(D))]
    assert np.max(np.abs(opa.merge_partitions(st, D) - ref)) <= 1e-12
    assert np.array_equal(opa.merge_partitions([(-math.inf, 0.0, np.zeros(D))], D), np.zeros(D))


def pin_golden():
    for fn in sorted(os.listdir(GOLDEN)):
        if not fn.startswith("hand_") or not fn.endswith(".json"):
            continue
        g = json.load(open(os.path.join(GOLDEN, fn)))
        dtype = g["dtype"]
        bs, nb, Hkv, D = g["block_size"], g["num_blocks"], g["num_kv_heads"], g["head_dim"]
        kc = np.array(g["keys"], dtype=np.float64)       # [L, Hkv, D]
        vc = np.array(g["values"], dtype=np.float64)
        table = np.array(g["block_table"], dtype=np.int32)
        kp, vp = place_tokens(kc, vc, table, bs, nb, dtype)
        q = storage(np.array(g["query"], dtype=np.float64)[None], dtype)
        out = opa.ref_paged_attention_decode(q, kp, vp, table[None], np.array([len(kc)]), g["scale"], dtype)[0]
        exp = np.array(g["expected"], dtype=np.float64)
        assert np.max(np.abs(out - exp)) <= g["tolerance"], fn


PINS = {"P1": pin_p1, "PL": pin_layout, "P2": pin_p2, "P3": pin_p3, "P4": pin_p4, "P5": pin_p5,
        "P6": pin_p6, "P7": pin_p7, "G": pin_golden}


# --------------------------------------------------------------------------
# the pins as tests
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_p1_cache_write_is_exact_copy(dtype):
    pin_p1(dtype=dtype)


def test_layout_walk_element_codes():
    pin_layout()


@pytest.mark.parametrize("dtype,Hq,Hkv,D,L", [("bf16", 8, 2, 32, 45), ("f32", 4, 4, 64, 37), ("bf16", 32, 8, 128, 300),
                                              ("f32", 3, 1, 16, 16), ("bf16", 16, 1, 64, 1)])
def test_p2_identity_table_equals_sdpa(dtype, Hq, Hkv, D, L):
    pin_p2(dtype=dtype, Hq=Hq, Hkv=Hkv, D=D, L=L)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_p3_permutation_bit_identical(dtype):
    pin_p3(dtype=dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_p4_shared_prefix_bit_identical(dtype):
    pin_p4(dtype=dtype)


def test_p5_brute_force_tiny():
    pin_p5()
    pin_p5(seed=55, dtype="bf16", shapes=((4, 2, 16, 33), (2, 1, 8, 16)))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_p6_closed_forms(dtype):
    pin_p6(dtype=dtype)


def test_p7_split_merge_identity():
    pin_p7()


def test_golden_hand_examples():
    pin_golden()


def test_zero_length_gives_zeros():
    kp, vp = place_tokens(np.zeros((0, 1, 8)), np.zeros((0, 1, 8)), np.array([0]), 16, 1, "bf16")
    out = opa.ref_paged_attention_decode(np.zeros((1, 2, 8), np.uint16), kp, vp, np.array([[0]]), np.array([0]), 1.0, "bf16")
    assert np.array_equal(out, np.zeros((1, 2, 8)))


def test_slot_of_position():
    table = np.array([7, 3, 9])
    assert opa.slot_of_position(table, 0, 16) == 112
    assert opa.slot_of_position(table, 17, 16) == 49
    assert opa.slot_of_position(table, 47, 16) == 159


# --------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# --------------------------------------------------------------------------

def _mut_gqa(monkeypatch):
    monkeypatch.setattr(opa, "kv_head_of", lambda h, Hq, Hkv: h % Hkv)


def _mut_no_scale(monkeypatch):
    orig = opa.softmax_attention
    monkeypatch.setattr(opa, "softmax_attention", lambda q, k, v, scale: orig(q, k, v, 1.0))


def _mut_no_normalise(monkeypatch):
    def f(q, k, v, scale):
        s = scale * (k @ q)
        w = np.exp(s - s.max())
        return w @ v
    monkeypatch.setattr(opa, "softmax_attention", f)


def _mut_drop_last_token(monkeypatch):
    orig = opa.gather_contiguous
    monkeypatch.setattr(opa, "gather_contiguous",
                        lambda kp, vp, row, L, heads=None: tuple(a[:max(L - 1, 0)] for a in orig(kp, vp, row, L, heads)))


def _mut_k_chunks_untransposed(monkeypatch):
    def g(k_pool, v_pool, table_row, context_len, heads=None):
        bs = k_pool.shape[3]
        heads = list(range(k_pool.shape[1])) if heads is None else list(heads)
        D = k_pool.shape[2] * k_pool.shape[4]
        kc = np.empty((context_len, len(heads), D), dtype=k_pool.dtype)
        vc = np.empty((context_len, len(heads), D), dtype=v_pool.dtype)
        for j in range(-(-context_len // bs)):
            p, lo, hi = int(table_row[j]), j * bs, min(context_len, (j + 1) * bs)
            for i, h in enumerate(heads):
                kc[lo:hi, i] = k_pool[p, h][:, :hi - lo, :].reshape(hi - lo, D)  # wrong: no transpose
                vc[lo:hi, i] = v_pool[p, h][:, :hi - lo].T
        return kc, vc
    monkeypatch.setattr(opa, "gather_contiguous", g)


def _mut_ignore_table(monkeypatch):
    orig = opa.gather_contiguous
    monkeypatch.setattr(opa, "gather_contiguous",
                        lambda kp, vp, row, L, heads=None: orig(kp, vp, np.arange(len(row)), L, heads))


def _mut_merge_sign(monkeypatch):
    def m(stats, D):
        live = [(a, b, c) for (a, b, c) in stats if b > 0]
        M = max(a for a, _, _ in live)
        num = sum(math.exp(M - a) * c for a, _, c in live)
        den = sum(math.exp(M - a) * b for a, b, _ in live)
        return num / den
    monkeypatch.setattr(opa, "merge_partitions", m)


def _mut_write_offset(monkeypatch):
    orig = opa.write_v_row
    monkeypatch.setattr(opa, "write_v_row", lambda vp, b, h, o, row: orig(vp, b, h, (o + 1) % vp.shape[3], row))


def _mut_swap_kv_write(monkeypatch):
    ok, ov = opa.write_k_row, opa.write_v_row

    def wk(kp, b, h, o, row):
        ok(kp, b, h, o, row[::-1].copy())
    monkeypatch.setattr(opa, "write_k_row", wk)


MUTANTS = {"gqa_mapping": _mut_gqa, "scale_dropped": _mut_no_scale, "no_normalisation": _mut_no_normalise,
           "last_token_dropped": _mut_drop_last_token, "k_chunks_untransposed": _mut_k_chunks_untransposed,
           "table_ignored": _mut_ignore_table, "merge_weight_sign": _mut_merge_sign,
           "write_offset": _mut_write_offset, "k_row_reversed": _mut_swap_kv_write}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name, monkeypatch):
    MUTANTS[name](monkeypatch)
    failed = []
    for pin, fn in PINS.items():
        try:
            fn()
        except (AssertionError, ValueError, IndexError):
            failed.append(pin)
    assert failed, f"no pin caught the planted mistake {name}"


def test_stored_oracle_values_unchanged():
    """The oracle and the input recipe still reproduce the stored tiny fp32 output."""
    import sys
    sys.path.insert(0, GOLDEN)
    from make_golden import tiny_fp32_expected
    stored = json.load(open(os.path.join(GOLDEN, "oracle_tiny_fp32.json")))
    now = tiny_fp32_expected()
    assert stored["context_lens"] == now["context_lens"]
    assert np.max(np.abs(np.array(stored["expected"]) - np.array(now["expected"]))) <= 1e-15
