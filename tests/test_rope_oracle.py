"""Pins of the rotary-embedding oracle (``oracle/rope.py``), on the CPU."""
import numpy as np
import pytest

import oracle
from oracle import rope
from workloads import rope_tables, to_u16


def rows(shape, seed, dt="bf16", spread=1.0):
    return to_u16(np.random.default_rng(seed).standard_normal(shape).astype(np.float32) * spread, dt)


def exact_table(angles_code, half):
    """Rows of exactly representable (cos, sin): code 0 -> 0, 1 -> pi/2, 2 -> pi, 3 -> 3pi/2."""
    c = np.array([1, 0, -1, 0], np.float32)[angles_code]
    s = np.array([0, 1, 0, -1], np.float32)[angles_code]
    return np.repeat(c[:, None], half, 1), np.repeat(s[:, None], half, 1)


# ------------------------------------------------------------------ 16-bit rounding
def test_encode_round_trips_every_finite_pattern():
    for dt in ("bf16", "f16"):
        bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
        with np.errstate(invalid="ignore"):
            v = oracle.decode_u16(bits, dt, out_dtype=np.float32)
        fin = np.isfinite(v)
        assert np.array_equal(rope.encode_u16(v[fin], dt), bits[fin]), dt
        nan = np.isnan(v)
        with np.errstate(invalid="ignore"):
            assert np.all(np.isnan(oracle.decode_u16(rope.encode_u16(v[nan], dt), dt))), dt


def test_bf16_rounding_is_nearest_even_by_brute_force():
    rng = np.random.default_rng(5)
    u = rng.integers(0, 0x7F7F0000, 20000, dtype=np.uint32)
    u[:1000] = (u[:1000] & 0xFFFF0000) | 0x8000                 # exact ties
    x = (u | (rng.integers(0, 2, u.size, dtype=np.uint32) << 31)).view(np.float32)
    got = rope.encode_u16(x, "bf16")
    lo = (x.view(np.uint32) >> 16).astype(np.uint16)
    hi = lo + np.uint16(1)
    dl = np.abs(oracle.decode_u16(lo, "bf16") - x.astype(np.float64))
    dh = np.abs(oracle.decode_u16(hi, "bf16") - x.astype(np.float64))
    want = np.where(dl < dh, lo, np.where(dh < dl, hi, np.where(lo % 2 == 0, lo, hi)))
    assert np.array_equal(got, want)


# ------------------------------------------------------------------ rotation
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_quarter_turns_are_exact(dt):
    """theta = 0, pi/2, pi, 3pi/2 map (x1, x2) to (x1, x2), (-x2, x1), (-x1, -x2), (x2, -x1)."""
    T, H, D = 8, 3, 64
    x = rows((T, H, D), 1, dt)
    cos, sin = exact_table(np.array([0, 1, 2, 3]), D // 2)
    pos = np.arange(T) % 4
    y = oracle.decode_u16(rope.rotate(x, pos, cos, sin, dt), dt)
    xf = oracle.decode_u16(x, dt)
    x1, x2 = xf[..., :D // 2], xf[..., D // 2:]
    want = {0: (x1, x2), 1: (-x2, x1), 2: (-x1, -x2), 3: (x2, -x1)}
    for t in range(T):
        a, b = want[t % 4]
        assert np.array_equal(y[t], np.concatenate([a[t], b[t]], -1)), t


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_equals_complex_multiplication(dt):
    """Pair i as the complex number x1_i + j x2_i, multiplied by cos_i + j sin_i (complex128):
    the float32 result is within two float32 roundings of it."""
    T, H, D = 40, 4, 128
    x = rows((T, H, D), 2, dt, spread=3.0)
    cos, sin = rope_tables(4096, D)
    pos = np.random.default_rng(3).integers(0, 4096, T)
    y = rope.rotate_f32(x, pos, cos, sin, dt).astype(np.float64)
    xf = oracle.decode_u16(x, dt)
    z = (xf[..., :D // 2] + 1j * xf[..., D // 2:]) * (cos[pos] + 1j * sin[pos].astype(np.float64))[:, None]
    mag = np.abs(xf[..., :D // 2]) + np.abs(xf[..., D // 2:])
    bound = 2.0 ** -22 * mag
    assert np.all(np.abs(y[..., :D // 2] - z.real) <= bound)
    assert np.all(np.abs(y[..., D // 2:] - z.imag) <= bound)
    # and the 16-bit result is that float32 value rounded once
    assert np.array_equal(rope.rotate(x, pos, cos, sin, dt), rope.encode_u16(y.astype(np.float32), dt))


def test_norm_and_inverse_with_negated_sin():
    """A rotation keeps each pair's length, and the pages' backward (the same map with -sin)
    undoes it up to the 16-bit roundings."""
    T, H, D, dt = 30, 2, 128, "f16"
    x = rows((T, H, D), 4, dt)
    cos, sin = rope_tables(2048, D, base=5.0e5)
    pos = np.random.default_rng(6).integers(0, 2048, T)
    y = rope.rotate(x, pos, cos, sin, dt)
    xf, yf = oracle.decode_u16(x, dt), oracle.decode_u16(y, dt)
    n_x = xf[..., :D // 2] ** 2 + xf[..., D // 2:] ** 2
    n_y = yf[..., :D // 2] ** 2 + yf[..., D // 2:] ** 2
    np.testing.assert_allclose(n_y, n_x, rtol=3 * 2.0 ** -10, atol=1e-6)
    back = oracle.decode_u16(rope.rotate(y, pos, cos, -sin, dt), dt)
    np.testing.assert_allclose(back, xf, rtol=0, atol=4 * 2.0 ** -10 * np.abs(xf).max())


def test_scores_depend_on_relative_position_only():
    """<R_a q, R_b k> = <R_{a+d} q, R_{b+d} k>: what makes the embedding positional."""
    D = 128
    cos, sin = rope_tables(8192, D)
    rng = np.random.default_rng(7)
    q = to_u16(rng.standard_normal((1, 1, D)).astype(np.float32), "f16")
    k = to_u16(rng.standard_normal((1, 1, D)).astype(np.float32), "f16")
    for a, b in [(5, 2), (100, 37), (4000, 3000)]:
        s0 = float(rope.rotate_f32(q, [a], cos, sin, "f16").ravel() @
                   rope.rotate_f32(k, [b], cos, sin, "f16").ravel())
        for dlt in (1, 17, 1000):
            s1 = float(rope.rotate_f32(q, [a + dlt], cos, sin, "f16").ravel() @
                       rope.rotate_f32(k, [b + dlt], cos, sin, "f16").ravel())
            assert abs(s1 - s0) < 2e-3 * (1 + abs(s0)), (a, b, dlt)


# ------------------------------------------------------------------ fused step
def test_fused_step_writes_rotated_keys_and_plain_values():
    T, Hq, Hkv, D, BS, NB, dt = 7, 8, 2, 64, 16, 6, "bf16"
    q, k, v = rows((T, Hq, D), 10, dt), rows((T, Hkv, D), 11, dt), rows((T, Hkv, D), 12, dt)
    cos, sin = rope_tables(500, D)
    pos = np.array([0, 3, 499, 500, -1, 17, 250])      # 500 and -1 are outside the table
    slots = np.array([0, 17, 95, 5, 6, -1, NB * BS])   # -1 and NB*BS write nothing
    kc = np.full((NB, BS, Hkv, D), 0x1234, np.uint16); vc = kc.copy()
    q_out = rope.rope_reshape_and_cache(q, k, v, kc, vc, pos, cos, sin, slots, dt)
    ok = [0, 1, 2, 5, 6]
    assert np.array_equal(q_out[ok], rope.rotate(q[ok], pos[ok], cos, sin, dt))
    assert np.array_equal(q_out[[3, 4]], q[[3, 4]])
    written = {0: 0, 1: 17, 2: 95}
    for t, s in written.items():
        assert np.array_equal(kc[s // BS, s % BS], rope.rotate(k[t:t + 1], pos[t:t + 1], cos, sin, dt)[0])
        assert np.array_equal(vc[s // BS, s % BS], v[t])
    untouched = np.ones(NB * BS, bool)
    untouched[list(written.values())] = False
    assert np.all(kc.reshape(NB * BS, Hkv, D)[untouched] == 0x1234)
    assert np.all(vc.reshape(NB * BS, Hkv, D)[untouched] == 0x1234)
    assert rope.rope_reshape_and_cache(None, k, v, kc, vc, pos, cos, sin, slots, dt) is None


@pytest.mark.parametrize("mutation", ["interleaved", "sign", "swap_cos_sin", "position_is_index",
                                      "fma"])
def test_pins_catch_planted_mistakes(mutation, monkeypatch):
    def planted(x_bits, positions, cos, sin, dtype):
        x = oracle.decode_u16(x_bits, dtype, out_dtype=np.float32)
        D = x.shape[-1]
        pos = np.asarray(positions, np.int64)
        if mutation == "position_is_index":
            pos = np.arange(len(pos))
        c = np.asarray(cos, np.float32)[pos][:, None, :]
        s = np.asarray(sin, np.float32)[pos][:, None, :]
        if mutation == "interleaved":
            x1, x2 = x[..., 0::2], x[..., 1::2]
            y = np.empty_like(x)
            y[..., 0::2] = x1 * c - x2 * s
            y[..., 1::2] = x2 * c + x1 * s
            return y
        if mutation == "swap_cos_sin":
            c, s = s, c
        x1, x2 = x[..., :D // 2], x[..., D // 2:]
        if mutation == "sign":
            return np.concatenate([x1 * c + x2 * s, x2 * c - x1 * s], -1)
        if mutation == "fma":   # products not rounded before the sum
            y1 = (x1.astype(np.float64) * c - x2.astype(np.float64) * s).astype(np.float32)
            y2 = (x2.astype(np.float64) * c + x1.astype(np.float64) * s).astype(np.float32)
            return np.concatenate([y1, y2], -1)
        return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], -1)   # mutated c, s or pos

    monkeypatch.setattr(rope, "rotate_f32", planted)
    checks = [lambda: test_quarter_turns_are_exact("bf16"), lambda: test_equals_complex_multiplication("bf16"),
              test_fma_rounding_is_pinned]
    failed = False
    for c in checks:
        try:
            c()
        except (AssertionError, IndexError):
            failed = True
    assert failed, mutation


def test_fma_rounding_is_pinned():
    """Separately rounded products differ from a fused form on inputs built for it: x1 c and
    x2 s each round in float32, and their difference cancels so the rounding shows."""
    # x1 = x2 = 1 + 2^-7 (exact in bf16), c = 1 + 2^-20 + 2^-23, s = 1 + 2^-20:
    # x1 c = 1 + 2^-7 + 2^-20 + 2^-23 + 2^-27 + 2^-30 -> float32 drops the last two terms,
    # x2 s = 1 + 2^-7 + 2^-20 + 2^-27 -> float32 drops 2^-27; the rounded difference is 2^-23,
    # the exact one 2^-23 + 2^-30.
    x = to_u16(np.full((1, 1, 2), 1 + 2.0 ** -7, np.float32), "bf16")
    c = np.array([[1 + 2.0 ** -20 + 2.0 ** -23]], np.float32)
    s = np.array([[1 + 2.0 ** -20]], np.float32)
    y = rope.rotate_f32(x, [0], c, s, "bf16")
    assert y[0, 0, 0] == np.float32(2.0 ** -23)
