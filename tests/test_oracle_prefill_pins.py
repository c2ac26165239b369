"""Pins of the multi-token-query (chunked prefill) oracle to facts outside it.

* Q1  a whole prompt (n = L) through an identity table equals torch's
      scaled_dot_product_attention with is_causal=True, in float64 (a
      library routine); a chunk (n < L) equals SDPA with the causal mask
      aligned at the end of the context.
* Q2  chunking changes nothing: the rows of a chunk equal the last n rows of
      the whole prompt's output over the same cache (causality alone fixes
      this; a mis-aligned mask breaks it).
* Q3  one query per request is decode: equal to the decode oracle, which has
      its own pins.
* Q4  brute force: scalar Python loops with math.exp / math.fsum over the
      flat pools on tiny inputs.
* Q5  closed forms: the first token of a prompt sees only itself (out = its
      value row); a zero query gives the running mean of the value rows.
* Q6  packing: a batch of requests with different chunk lengths, packed row
      after row, equals each request run on its own.

``test_planted_prefill_mistakes_are_caught`` plants plausible mistakes in
the oracle on the CPU and checks that some pin fails for each.
"""
import math

import numpy as np
import pytest
import torch

import oracle.paged_attention as opa
import oracle.prefill as opp
from test_oracle_pins import exact_values, k_flat_offset, place_tokens, storage, v_flat_offset


def sdpa_prefill(q, kc, vc, scale, n):
    """q [n, Hq, D], kc/vc [L, Hkv, D] float64 -> [n, Hq, D]; queries are the last n positions."""
    L, Hkv, D = kc.shape
    Hq = q.shape[1]
    G = Hq // Hkv
    K = torch.from_numpy(kc).permute(1, 0, 2).repeat_interleave(G, dim=0)[None].contiguous()
    V = torch.from_numpy(vc).permute(1, 0, 2).repeat_interleave(G, dim=0)[None].contiguous()
    Q = torch.from_numpy(q).permute(1, 0, 2)[None].contiguous()
    if n == L:
        out = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=scale)
    else:
        allowed = torch.ones(n, L, dtype=torch.bool).tril(diagonal=L - n)
        out = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=allowed, scale=scale)
    return out[0].permute(1, 0, 2).numpy()


def one_request(seed, dtype, L, n, Hq, Hkv, D, bs=16, extra_blocks=3):
    rng = np.random.default_rng(seed)
    kc = exact_values((L, Hkv, D), rng, dtype)
    vc = exact_values((L, Hkv, D), rng, dtype)
    q = exact_values((n, Hq, D), rng, dtype)
    nblk = -(-L // bs)
    nb = nblk + extra_blocks
    table = rng.permutation(nb)[:nblk].astype(np.int32)
    kp, vp = place_tokens(kc, vc, table, bs, nb, dtype)
    return q, kc, vc, table, kp, vp


def run_oracle(q, kp, vp, table, L, scale, dtype):
    n = q.shape[0]
    return opp.ref_paged_attention_prefill(storage(q, dtype), kp, vp, table[None], np.array([L]),
                                           np.array([0, n]), scale, dtype)


def pin_q1(dtype="bf16"):
    for seed, (L, n, Hq, Hkv, D) in enumerate([(45, 45, 8, 2, 32), (70, 70, 4, 4, 16), (70, 19, 8, 2, 32),
                                               (33, 1, 4, 1, 16)]):
        q, kc, vc, table, kp, vp = one_request(100 + seed, dtype, L, n, Hq, Hkv, D)
        scale = 1.0 / math.sqrt(D)
        got = run_oracle(q, kp, vp, table, L, scale, dtype)
        ref = sdpa_prefill(q, kc, vc, scale, n)
        assert np.max(np.abs(got - ref)) <= 1e-12, (L, n)


def pin_q2(dtype="bf16"):
    L, Hq, Hkv, D = 53, 4, 2, 16
    q, kc, vc, table, kp, vp = one_request(200, dtype, L, L, Hq, Hkv, D)
    full = run_oracle(q, kp, vp, table, L, 0.3, dtype)
    for n in (1, 7, 16, 52):
        part = run_oracle(q[L - n:], kp, vp, table, L, 0.3, dtype)
        assert np.array_equal(part, full[L - n:]), n


def pin_q3(dtype="bf16"):
    rng = np.random.default_rng(300)
    B, Hq, Hkv, D, bs, nb = 3, 8, 2, 32, 16, 12
    lens = np.array([1, 17, 40])
    tables = rng.permutation(nb)[:3 * B].reshape(B, 3).astype(np.int32)   # disjoint blocks
    kp = vp = None
    kcs = [exact_values((int(L), Hkv, D), rng, dtype) for L in lens]
    vcs = [exact_values((int(L), Hkv, D), rng, dtype) for L in lens]
    for s in range(B):
        a, b = place_tokens(kcs[s], vcs[s], tables[s], bs, nb, dtype)
        if kp is None:
            kp, vp = a.copy(), b.copy()
        for j in range(-(-int(lens[s]) // bs)):
            kp[tables[s][j]] = a[tables[s][j]]
            vp[tables[s][j]] = b[tables[s][j]]
    q = storage(exact_values((B, Hq, D), rng, dtype), dtype)
    dec = opa.ref_paged_attention_decode(q, kp, vp, tables, lens, 0.2, dtype)
    pre = opp.ref_paged_attention_prefill(q, kp, vp, tables, lens, np.arange(B + 1), 0.2, dtype)
    assert np.max(np.abs(dec - pre)) <= 1e-12


def brute_prefill(q, kflat, vflat, table, L, scale, Hq, Hkv, D, bs, x):
    n = q.shape[0]
    G = Hq // Hkv
    out = np.zeros((n, Hq, D))
    for i in range(n):
        p = L - n + i
        for h in range(Hq):
            kvh = h // G
            sc = []
            for pos in range(p + 1):
                b, o = int(table[pos // bs]), pos % bs
                sc.append(scale * math.fsum(float(q[i, h, d]) * float(kflat[k_flat_offset(b, kvh, o, d, Hkv, D, bs, x)])
                                            for d in range(D)))
            m = max(sc)
            w = [math.exp(s - m) for s in sc]
            den = math.fsum(w)
            for d in range(D):
                out[i, h, d] = math.fsum(w[pos] * float(vflat[v_flat_offset(int(table[pos // bs]), kvh, pos % bs, d,
                                                                             Hkv, D, bs)])
                                         for pos in range(p + 1)) / den
    return out


def pin_q4(dtype="f32"):
    for seed, (L, n, Hq, Hkv, D) in enumerate([(5, 5, 2, 1, 8), (23, 6, 4, 2, 8), (37, 17, 2, 2, 16)]):
        q, kc, vc, table, kp, vp = one_request(400 + seed, dtype, L, n, Hq, Hkv, D)
        scale = 0.6 / math.sqrt(D)
        got = run_oracle(q, kp, vp, table, L, scale, dtype)
        x = 16 // (4 if dtype == "f32" else 2)
        ref = brute_prefill(q, opa.widen(kp.reshape(-1), dtype), opa.widen(vp.reshape(-1), dtype), table, L, scale,
                            Hq, Hkv, D, 16, x)
        assert np.max(np.abs(got - ref)) <= 1e-12, (L, n)


def pin_q5(dtype="bf16"):
    L, Hq, Hkv, D = 29, 4, 2, 16
    q, kc, vc, table, kp, vp = one_request(500, dtype, L, L, Hq, Hkv, D)
    out = run_oracle(q, kp, vp, table, L, 0.5, dtype)
    for h in range(Hq):
        assert np.array_equal(out[0, h], vc[0, h // 2])
    zero = run_oracle(np.zeros_like(q), kp, vp, table, L, 0.5, dtype)
    for i in range(L):
        for h in range(Hq):
            assert np.max(np.abs(zero[i, h] - vc[:i + 1, h // 2].mean(axis=0))) <= 1e-14


def pin_q6(dtype="bf16"):
    rng = np.random.default_rng(600)
    Hq, Hkv, D, bs = 8, 2, 16, 16
    reqs = [(40, 40), (33, 1), (70, 12), (16, 16)]   # (L, n)
    nb = sum(-(-L // bs) for L, _ in reqs) + 2
    perm = rng.permutation(nb).astype(np.int32)
    width = max(-(-L // bs) for L, _ in reqs)
    tables = np.full((len(reqs), width), perm[-1], dtype=np.int32)
    kp = vp = None
    qs, used = [], 0
    for s, (L, n) in enumerate(reqs):
        nblk = -(-L // bs)
        tables[s, :nblk] = perm[used:used + nblk]
        used += nblk
        kc = exact_values((L, Hkv, D), rng, dtype)
        vc = exact_values((L, Hkv, D), rng, dtype)
        a, b = place_tokens(kc, vc, tables[s, :nblk], bs, nb, dtype)
        if kp is None:
            kp, vp = a.copy(), b.copy()
        for j in range(nblk):
            kp[tables[s, j]] = a[tables[s, j]]
            vp[tables[s, j]] = b[tables[s, j]]
        qs.append(storage(exact_values((n, Hq, D), rng, dtype), dtype))
    q = np.concatenate(qs)
    qsl = np.concatenate([[0], np.cumsum([n for _, n in reqs])])
    lens = np.array([L for L, _ in reqs])
    packed = opp.ref_paged_attention_prefill(q, kp, vp, tables, lens, qsl, 0.25, dtype)
    for s, (L, n) in enumerate(reqs):
        alone = opp.ref_paged_attention_prefill(qs[s], kp, vp, tables[s:s + 1], lens[s:s + 1], np.array([0, n]), 0.25,
                                                dtype)
        assert np.array_equal(packed[qsl[s]:qsl[s + 1]], alone)
    # a subset of requests fills only their rows
    part = opp.ref_paged_attention_prefill(q, kp, vp, tables, lens, qsl, 0.25, dtype, seqs=[2])
    assert np.array_equal(part[qsl[2]:qsl[3]], packed[qsl[2]:qsl[3]]) and np.isnan(part[:qsl[2]]).all()


PINS = {"Q1": pin_q1, "Q2": pin_q2, "Q3": pin_q3, "Q4": pin_q4, "Q5": pin_q5, "Q6": pin_q6}


@pytest.mark.parametrize("name", sorted(PINS))
def test_prefill_pin(name):
    PINS[name]()


def test_q1_fp32():
    pin_q1("f32")


def test_more_queries_than_context_gives_zeros():
    q, kc, vc, table, kp, vp = one_request(700, "f32", 3, 3, 2, 1, 8)
    out = opp.ref_paged_attention_prefill(storage(np.concatenate([q, q]), "f32"), kp, vp, table[None], np.array([3]),
                                          np.array([0, 6]), 0.5, "f32")
    assert np.array_equal(out[:3], np.zeros_like(out[:3]))


# --------------------------------------------------------------------------
# planted mistakes
# --------------------------------------------------------------------------

def _mut_top_left(monkeypatch):
    monkeypatch.setattr(opp, "query_positions", lambda L, n: np.arange(0, n, dtype=np.int64))


def _mut_exclude_self(monkeypatch):
    orig = opp.softmax_attention
    monkeypatch.setattr(opp, "softmax_attention", lambda q, k, v, scale: orig(q, k[:-1], v[:-1], scale))


def _mut_see_future(monkeypatch):
    monkeypatch.setattr(opp, "query_positions", lambda L, n: np.full(n, L - 1, dtype=np.int64))


def _mut_gqa_modulo(monkeypatch):
    monkeypatch.setattr(opp, "kv_head_of", lambda h, Hq, Hkv: h % Hkv)


def _mut_rows_reversed(monkeypatch):
    orig = opp.ref_prefill_sequence
    monkeypatch.setattr(opp, "ref_prefill_sequence", lambda q, *a: orig(q[::-1].copy(), *a))


PREFILL_MUTANTS = {"top_left_mask": _mut_top_left, "self_excluded": _mut_exclude_self,
                   "future_visible": _mut_see_future, "gqa_modulo": _mut_gqa_modulo,
                   "query_rows_reversed": _mut_rows_reversed}


@pytest.mark.parametrize("name", sorted(PREFILL_MUTANTS))
def test_planted_prefill_mistakes_are_caught(name, monkeypatch):
    PREFILL_MUTANTS[name](monkeypatch)
    failed = []
    for pin, fn in PINS.items():
        try:
            fn()
        except (AssertionError, ValueError, IndexError):
            failed.append(pin)
    assert failed, f"no pin caught the planted mistake {name}"
