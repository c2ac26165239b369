"""Pins of the fp8 (OCP E4M3) cache oracle to facts outside it.

* F1  closed-form values of the format (smallest subnormal 2^-9, smallest
      normal 2^-6, 1, 1.875, 448, signed zero, the two NaN codes).
* F2  every code decodes as torch's float8_e4m3fn does (a library routine).
* F3  encoding matches torch's round-to-nearest-even cast for every value
      below the rounding threshold 464 (random values, exact midpoints
      between neighbouring codes, subnormals); above it ours saturates to
      +-448 where torch gives NaN.
* F4  encode(decode(c)) == c for every finite code.
* F5  the cache write quantises with a correctly rounded fp32 division by
      the head's scale and stores codes at the documented flat offsets
      (checked against torch's cast, not the oracle's encoder).
* F6  attention over an fp8 cache equals the bf16 oracle over the
      dequantised values when the scales are powers of two (then every
      dequantised value is exact in bf16): bit-identical.
* F7  the same for multi-token (chunked prefill) attention: causal queries
      over an fp8 cache equal the bf16 prefill oracle over the dequantised
      pools, bit for bit, and a single-query request equals fp8 decode.

``test_planted_fp8_mistakes_are_caught`` plants mistakes in the oracle.
"""
import math

import numpy as np
import pytest
import torch

import oracle.fp8 as of8
import oracle.paged_attention as opa
import oracle.prefill as opp
from test_oracle_pins import k_flat_offset, v_flat_offset
from workloads import bf16_bits_rne, pool_shapes


def torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8).copy()).view(torch.float8_e4m3fn).double().numpy()


def torch_encode(y32):
    return torch.from_numpy(np.asarray(y32, dtype=np.float32).copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def pin_f1():
    v = of8.e4m3_value
    assert v(0x00) == 0.0 and math.copysign(1.0, v(0x80)) == -1.0
    assert v(0x01) == 2.0 ** -9 and v(0x07) == 7 * 2.0 ** -9 and v(0x08) == 2.0 ** -6
    assert v(0x38) == 1.0 and v(0x3F) == 1.875 and v(0x40) == 2.0
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0 and v(0xB8) == -1.0
    assert math.isnan(v(0x7F)) and math.isnan(v(0xFF))
    finite = [v(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(finite, finite[1:]))      # increasing magnitudes


def pin_f2():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = of8.e4m3_decode(codes), torch_decode(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def pin_f3():
    rng = np.random.default_rng(8)
    mags = of8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (mags[:-1] + mags[1:]) / 2                          # exact ties (all fit in fp32)
    y = np.concatenate([rng.standard_normal(4000) * 4, rng.standard_normal(1000) * 100,
                        rng.uniform(-2 ** -6, 2 ** -6, 1000), mids, -mids, [0.0, -0.0, 447.9, 455.0, 463.9]])
    y32 = y.astype(np.float32)
    y32 = y32[np.abs(y32) < 464]
    assert np.array_equal(of8.e4m3_encode(y32), torch_encode(y32))
    # saturation above the threshold
    assert of8.e4m3_encode_scalar(464.0) == 0x7E and of8.e4m3_encode_scalar(1e9) == 0x7E
    assert of8.e4m3_encode_scalar(-5000.0) == 0xFE


def pin_f4():
    for c in range(256):
        if c in of8.E4M3_NAN_CODES:
            continue
        assert of8.e4m3_encode_scalar(of8.e4m3_value(c)) == c, hex(c)


def pin_f5():
    rng = np.random.default_rng(9)
    NB, Hkv, D, bs, T = 6, 2, 32, 16, 12
    ks, vs = pool_shapes(NB, Hkv, D, bs, "bf16")
    ks = (NB, Hkv, D // 16, bs, 16)                            # 16 one-byte elements per chunk
    k_pool = rng.integers(0, 255, size=ks, dtype=np.uint8)
    v_pool = rng.integers(0, 255, size=vs, dtype=np.uint8)
    x = rng.standard_normal((2, T, Hkv, D)).astype(np.float32) * 3
    src = bf16_bits_rne(x)                                     # bf16 inputs
    xv = opa.widen(src, "bf16").astype(np.float32)
    scales = [np.array([0.75, 1.3]), np.array([0.02, 2.5])]
    slots = rng.choice(NB * bs, size=T, replace=False)
    slots[3] = -1
    kp, vp = of8.ref_reshape_and_cache_fp8(src[0], src[1], slots, k_pool, v_pool, scales[0], scales[1], "bf16")
    kf, vf = k_pool.reshape(-1).copy(), v_pool.reshape(-1).copy()
    for t in range(T):
        if slots[t] < 0:
            continue
        b, o = divmod(int(slots[t]), bs)
        for h in range(Hkv):
            kc = torch_encode(np.clip(xv[0, t, h] / np.float32(scales[0][h]), -448, 448))
            vc = torch_encode(np.clip(xv[1, t, h] / np.float32(scales[1][h]), -448, 448))
            for d in range(D):
                kf[k_flat_offset(b, h, o, d, Hkv, D, bs, 16)] = kc[d]
                vf[v_flat_offset(b, h, o, d, Hkv, D, bs)] = vc[d]
    assert np.array_equal(kp.reshape(-1), kf) and np.array_equal(vp.reshape(-1), vf)


def pin_f6():
    rng = np.random.default_rng(10)
    NB, Hq, Hkv, D, bs = 8, 8, 2, 32, 16
    kp = rng.integers(0, 0x7F, size=(NB, Hkv, D // 16, bs, 16), dtype=np.uint8) | \
        (rng.integers(0, 2, size=(NB, Hkv, D // 16, bs, 16), dtype=np.uint8) << 7)
    vp = rng.integers(0, 0x7F, size=(NB, Hkv, D, bs), dtype=np.uint8)
    ks, vs = np.array([0.25, 2.0 ** -5]), np.array([4.0, 0.5])
    q = bf16_bits_rne(rng.standard_normal((3, Hq, D)).astype(np.float32) * 0.05)
    tables = rng.permutation(NB)[:6].reshape(3, 2).astype(np.int32)
    lens = np.array([5, 17, 32])
    got = opa.ref_paged_attention_decode(q, kp, vp, tables, lens, 0.3, "fp8", k_scale=ks, v_scale=vs)
    # the same values as a bf16 cache (K chunks of 8 instead of 16 elements)
    kval = of8.dequantize_pool(kp, ks)                          # [NB, Hkv, D/16, bs, 16]
    kval = np.transpose(kval, (0, 1, 3, 2, 4)).reshape(NB, Hkv, bs, D)
    kb = bf16_bits_rne(kval.astype(np.float32)).reshape(NB, Hkv, bs, D // 8, 8).transpose(0, 1, 3, 2, 4).copy()
    vb = bf16_bits_rne(of8.dequantize_pool(vp, vs).astype(np.float32))
    assert np.array_equal(opa.widen(vb, "bf16"), of8.dequantize_pool(vp, vs))   # exact in bf16
    ref = opa.ref_paged_attention_decode(q, kb, vb, tables, lens, 0.3, "bf16")
    assert np.array_equal(got, ref)


def as_bf16_pools(kp, vp, ks, vs):
    """The dequantised values of fp8 pools in the bf16 pool layout (K chunks of 8)."""
    NB, Hkv, _, bs, _ = kp.shape
    D = vp.shape[2]
    kval = np.transpose(of8.dequantize_pool(kp, ks), (0, 1, 3, 2, 4)).reshape(NB, Hkv, bs, D)
    kb = bf16_bits_rne(kval.astype(np.float32)).reshape(NB, Hkv, bs, D // 8, 8).transpose(0, 1, 3, 2, 4).copy()
    vb = bf16_bits_rne(of8.dequantize_pool(vp, vs).astype(np.float32))
    return kb, vb


def pin_f7():
    rng = np.random.default_rng(11)
    NB, Hq, Hkv, D, bs = 10, 4, 2, 32, 16
    kp = rng.integers(0, 0x7F, size=(NB, Hkv, D // 16, bs, 16), dtype=np.uint8) | \
        (rng.integers(0, 2, size=(NB, Hkv, D // 16, bs, 16), dtype=np.uint8) << 7)
    vp = rng.integers(0, 0x7F, size=(NB, Hkv, D, bs), dtype=np.uint8) | \
        (rng.integers(0, 2, size=(NB, Hkv, D, bs), dtype=np.uint8) << 7)
    ks, vs = np.array([0.5, 2.0 ** -4]), np.array([2.0, 0.25])
    lens = np.array([20, 33, 7])
    new = np.array([6, 1, 7])                       # request 1 is a decode row
    qsl = np.concatenate([[0], np.cumsum(new)])
    q = bf16_bits_rne(rng.standard_normal((int(qsl[-1]), Hq, D)).astype(np.float32) * 0.1)
    tables = rng.permutation(NB)[:9].reshape(3, 3).astype(np.int32)
    got = opp.ref_paged_attention_prefill(q, kp, vp, tables, lens, qsl, 0.3, "fp8", k_scale=ks, v_scale=vs)
    kb, vb = as_bf16_pools(kp, vp, ks, vs)
    assert np.array_equal(opa.widen(vb, "bf16"), of8.dequantize_pool(vp, vs))   # exact in bf16
    ref = opp.ref_paged_attention_prefill(q, kb, vb, tables, lens, qsl, 0.3, "bf16")
    assert np.array_equal(got, ref)
    dec = opa.ref_paged_attention_decode(q[qsl[1]:qsl[2]], kp, vp, tables[1:2], lens[1:2], 0.3, "fp8",
                                         k_scale=ks, v_scale=vs)
    assert np.array_equal(got[qsl[1]:qsl[2]], dec)


PINS = {"F1": pin_f1, "F2": pin_f2, "F3": pin_f3, "F4": pin_f4, "F5": pin_f5, "F6": pin_f6, "F7": pin_f7}


@pytest.mark.parametrize("name", sorted(PINS))
def test_fp8_pin(name):
    PINS[name]()


# --------------------------------------------------------------------------
# planted mistakes
# --------------------------------------------------------------------------

def _mut_multiply_scale(monkeypatch):
    orig = of8.quantize_row
    monkeypatch.setattr(of8, "quantize_row", lambda x, d, s: orig(x, d, 1.0 / s))


def _mut_flush_subnormals(monkeypatch):
    table = of8._DECODE_TABLE.copy()
    table[[c for c in range(256) if (c >> 3) & 0xF == 0]] = 0.0
    monkeypatch.setattr(of8, "_DECODE_TABLE", table)


def _mut_ties_away(monkeypatch):
    def enc(y):
        a = abs(y)
        sign = 0x80 if math.copysign(1.0, y) < 0 else 0
        if a >= 448:
            return sign | 0x7E
        mags = of8._DECODE_TABLE[:0x7F]
        i = int(np.searchsorted(mags, a, side="right")) - 1
        lo, hi = mags[i], mags[min(i + 1, 0x7E)]
        return sign | (i if a - lo < hi - a else min(i + 1, 0x7E))
    monkeypatch.setattr(of8, "e4m3_encode_scalar", enc)


def _mut_bias_8(monkeypatch):
    def val(code):
        code = int(code) & 0xFF
        s = -1.0 if code & 0x80 else 1.0
        e, m = (code >> 3) & 0xF, code & 7
        if e == 0xF and m == 7:
            return math.nan
        return s * m * 2.0 ** -10 if e == 0 else s * (1 + m / 8) * 2.0 ** (e - 8)
    monkeypatch.setattr(of8, "_DECODE_TABLE", np.array([val(c) for c in range(256)]))


def _mut_v_scale_from_k(monkeypatch):
    orig = opa.widen_kv
    monkeypatch.setattr(opa, "widen_kv", lambda kc, vc, d, heads, ks=None, vs=None: orig(kc, vc, d, heads, ks, ks))


FP8_MUTANTS = {"scale_multiplied": _mut_multiply_scale, "subnormals_flushed": _mut_flush_subnormals,
               "ties_away_from_zero": _mut_ties_away, "exponent_bias_8": _mut_bias_8,
               "v_scale_from_k": _mut_v_scale_from_k}


@pytest.mark.parametrize("name", sorted(FP8_MUTANTS))
def test_planted_fp8_mistakes_are_caught(name, monkeypatch):
    FP8_MUTANTS[name](monkeypatch)
    failed = []
    for pin, fn in PINS.items():
        try:
            fn()
        except (AssertionError, ValueError, IndexError):
            failed.append(pin)
    assert failed, f"no pin caught the planted mistake {name}"
