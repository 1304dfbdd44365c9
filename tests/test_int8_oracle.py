"""Pins of the INT8 KV-cache oracle (``oracle/int8_kv.py``), on the CPU."""
import numpy as np
import pytest

import oracle
from oracle import int8_kv
from workloads import make_batch, to_u16


def rows(shape, seed, dt="bf16", spread=1.0):
    return to_u16(np.random.default_rng(seed).standard_normal(shape).astype(np.float32) * spread, dt)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_row_maximum_maps_to_127_and_error_is_half_a_step(dt):
    x = rows((50, 4, 128), 1, dt)
    codes, scales = int8_kv.quantize_rows(x, dt)
    xf = oracle.decode_u16(x, dt)
    assert codes.dtype == np.int8 and scales.dtype == np.float32
    assert np.all(np.max(np.abs(codes), axis=-1) == 127)
    arg = np.argmax(np.abs(xf), axis=-1)
    picked = np.take_along_axis(codes.astype(int), arg[..., None], -1)[..., 0]
    assert np.all(picked == np.sign(np.take_along_axis(xf, arg[..., None], -1)[..., 0]) * 127)
    # half a step, plus the float32 rounding of the quotient x / scale (|x / scale| <= 127)
    err = np.abs(int8_kv.dequantize(codes, scales) - xf)
    assert np.all(err <= scales[..., None] * (0.5 + 127 * 2.0 ** -23))
    assert np.all(np.sign(codes) * np.sign(xf) >= 0)       # no sign flips


def test_zero_and_constant_rows():
    z = np.zeros((3, 64), dtype=np.uint16)
    codes, scales = int8_kv.quantize_rows(z, "bf16")
    assert np.all(codes == 0) and np.all(scales == 0)
    c = np.full((2, 64), to_u16(np.array([-0.375], np.float32), "bf16")[0], dtype=np.uint16)
    codes, scales = int8_kv.quantize_rows(c, "bf16")
    assert np.all(codes == -127) and np.allclose(scales, 0.375 / 127, rtol=1e-7)


def test_half_way_ties_round_to_even():
    # amax 127 gives scale exactly 1, so x / scale = x and the ties are exact
    vals = np.array([127.0, 2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5, 126.5], np.float32)
    x = to_u16(vals, "f16")[None, :]
    codes, scales = int8_kv.quantize_rows(x, "f16")
    assert scales[0] == np.float32(1.0)
    assert codes[0].tolist() == [127, 2, 4, -2, -4, 0, 0, 2, 126]


def test_codes_rederived_in_float64():
    """fp32 division re-derived on a different path: a float64 quotient of two float32
    values rounded once to float32 is the correctly rounded float32 quotient."""
    x = rows((200, 128), 3, "bf16", spread=7.0)
    codes, scales = int8_kv.quantize_rows(x, "bf16")
    xf = oracle.decode_u16(x, "bf16")                      # float64, exact
    amax = np.max(np.abs(xf), axis=-1)
    s64 = (amax / 127.0).astype(np.float32)                # one rounding
    assert np.array_equal(s64, scales)
    qt = (xf / s64.astype(np.float64)[:, None]).astype(np.float32)
    assert np.array_equal(np.rint(qt).astype(np.int8), codes)


def _exact_int8_cache(seed, NB, BS, Hkv, D):
    """Codes and power-of-two scales whose products are exact in bf16 (|code| <= 127)."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(-127, 128, (NB, Hkv, BS, D)).astype(np.int8)
    scales = np.ldexp(1.0, rng.integers(-9, -3, (NB, Hkv, BS))).astype(np.float32)
    return codes, scales


def test_decode_equals_16bit_oracle_on_exact_values():
    B, Hq, Hkv, D, BS, NB = 3, 8, 2, 64, 16, 24
    kc, ks = _exact_int8_cache(11, NB, BS, Hkv, D)
    vc, vs = _exact_int8_cache(12, NB, BS, Hkv, D)
    # the same values in the 16-bit token-major layout [NB][BS][Hkv][D]
    kf = int8_kv.dequantize(kc, ks).transpose(0, 2, 1, 3)
    vf = int8_kv.dequantize(vc, vs).transpose(0, 2, 1, 3)
    kbits = to_u16(kf.astype(np.float32), "bf16")
    vbits = to_u16(vf.astype(np.float32), "bf16")
    assert np.array_equal(oracle.decode_u16(kbits, "bf16"), kf)     # exactly representable
    rng = np.random.default_rng(13)
    tables = np.stack([rng.permutation(NB)[:8] for _ in range(B)]).astype(np.int32)
    lens = np.array([1, 77, 128], np.int32)
    q = rows((B, Hq, D), 14)
    ref16 = oracle.paged_decode(q, kbits, vbits, tables, lens, 0.125, "bf16")
    got = int8_kv.paged_decode_int8(q, kc, vc, ks, vs, tables, lens, 0.125, "bf16")
    np.testing.assert_allclose(got, ref16, rtol=0, atol=1e-12)


def test_reshape_and_cache_int8_writes_slots_and_skips_padding():
    b = make_batch(B=3, Hq=4, Hkv=2, D=64, BS=16, dtype="f16", scale=0.125, seed=20,
                   lens_range=(5, 60))
    NB = b.NB
    kc = np.zeros((NB, 2, 16, 64), np.int8); vc = kc.copy()
    ks = np.full((NB, 2, 16), -1.0, np.float32); vs = ks.copy()
    slots = b.slot_mapping_compact.copy()
    slots[1] = -1
    int8_kv.reshape_and_cache_int8(b.key_new, b.value_new, kc, vc, ks, vs, slots, "f16")
    kq, kscale = int8_kv.quantize_rows(b.key_new, "f16")
    for t, s in enumerate(slots):
        if s < 0:
            continue
        assert np.array_equal(kc[s // 16, :, s % 16], kq[t])
        assert np.array_equal(ks[s // 16, :, s % 16], kscale[t])
    untouched = b.slot_mapping_compact[1]
    assert np.all(ks[untouched // 16, :, untouched % 16] == -1.0)


@pytest.mark.parametrize("mutation", ["scale_128", "truncate", "scale_layout"])
def test_pins_catch_planted_mistakes(mutation, monkeypatch):
    real_q = int8_kv.quantize_rows
    real_g = int8_kv.gather_int8
    if mutation == "scale_128":
        def q(bits, dtype):
            c, s = real_q(bits, dtype)
            return c, (s * np.float32(127.0) / np.float32(128.0)).astype(np.float32)
        monkeypatch.setattr(int8_kv, "quantize_rows", q)
    elif mutation == "truncate":
        def q(bits, dtype):
            x = oracle.decode_u16(bits, dtype, out_dtype=np.float32)
            s = (np.max(np.abs(x), -1) / np.float32(127)).astype(np.float32)
            return np.trunc(x / s[..., None]).astype(np.int8), s
        monkeypatch.setattr(int8_kv, "quantize_rows", q)
    else:
        def g(codes, scales, row, L):           # reshape where a transpose is needed
            Hkv, BS, D = codes.shape[1:]
            parts = [int8_kv.dequantize(codes[int(row[j])], scales[int(row[j])]).reshape(BS, Hkv, D)
                     for j in range(oracle.blocks_needed(L, BS))]
            return np.concatenate(parts)[:L]
        monkeypatch.setattr(int8_kv, "gather_int8", g)
    checks = [test_row_maximum_maps_to_127_and_error_is_half_a_step,
              test_half_way_ties_round_to_even, test_codes_rederived_in_float64,
              test_decode_equals_16bit_oracle_on_exact_values]
    failed = False
    for c in checks:
        try:
            c("bf16") if c is test_row_maximum_maps_to_127_and_error_is_half_a_step else c()
        except AssertionError:
            failed = True
    assert failed, mutation
