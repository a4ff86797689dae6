"""Pins of the RoPE oracle against facts that are not its own formula: the
complex-number form of the rotation, a hand-derived worked example, the
relative-position property that motivates RoPE, orthogonality, the angle
addition theorem on the tables, and the Qwen3 implementation that ships with
transformers (a library routine, run on CPU in float64). Planted mistakes at
the bottom must fail at least one pin each.
"""
import numpy as np
import pytest
import torch

import oracle.rope as R


def _x(T, H, d, seed):
    return np.random.default_rng(seed).standard_normal((T, H, d))


def pin_complex_form(orc):
    """Pair j is the complex number x_j + i x_{j+d/2}; RoPE multiplies it by
    exp(i pos f_j)."""
    T, H, d, base = 9, 3, 16, 500.0
    x = _x(T, H, d, 1)
    pos = np.array([0, 1, 2, 5, 17, 33, 100, 7, 63])
    cos, sin = orc.rope_tables_ref(128, d, base)
    y = orc.rope_ref(x, pos, cos, sin)
    f = base ** (-np.arange(d // 2) * 2.0 / d)
    z = (x[..., :d // 2] + 1j * x[..., d // 2:]) * np.exp(1j * pos[:, None, None] * f)
    np.testing.assert_allclose(y, np.concatenate([z.real, z.imag], -1), rtol=0, atol=1e-12)


def pin_worked_example(orc):
    """d = 4, base 100: f = (1, 0.1). e_0 at position 1 turns into
    (cos 1, 0, sin 1, 0); e_1 at position 2 into (0, cos 0.2, 0, sin 0.2);
    e_2 at position 3 into (-sin 3, 0, cos 3, 0)."""
    cos, sin = orc.rope_tables_ref(4, 4, 100.0)
    x = np.zeros((3, 1, 4))
    x[0, 0, 0] = x[1, 0, 1] = x[2, 0, 2] = 1.0
    y = orc.rope_ref(x, [1, 2, 3], cos, sin)[:, 0]
    want = np.array([[np.cos(1), 0, np.sin(1), 0],
                     [0, np.cos(0.2), 0, np.sin(0.2)],
                     [-np.sin(3), 0, np.cos(3), 0]])
    np.testing.assert_allclose(y, want, rtol=0, atol=1e-15)


def pin_relative_position(orc):
    """<R(m) q, R(n) k> depends on m - n only."""
    d = 32
    cos, sin = orc.rope_tables_ref(400, d, 10000.0)
    q, k = _x(1, 1, d, 2), _x(1, 1, d, 3)
    ref = float((orc.rope_ref(q, [37], cos, sin) * k).sum())
    for m, n in [(37, 0), (40, 3), (137, 100), (399, 362)]:
        got = float((orc.rope_ref(q, [m], cos, sin) * orc.rope_ref(k, [n], cos, sin)).sum())
        assert abs(got - ref) < 1e-11, (m, n, got, ref)


def pin_orthogonal(orc):
    """Position 0 is the identity, every pair keeps its length, and the
    inverse undoes the rotation."""
    d = 64
    x = _x(11, 2, d, 4)
    pos = np.arange(0, 1100, 100)
    cos, sin = orc.rope_tables_ref(1100, d, 1e6)
    y = orc.rope_ref(x, pos, cos, sin)
    np.testing.assert_array_equal(y[0], x[0])
    h = d // 2
    np.testing.assert_allclose(y[..., :h] ** 2 + y[..., h:] ** 2,
                               x[..., :h] ** 2 + x[..., h:] ** 2, rtol=1e-12)
    np.testing.assert_allclose(orc.rope_ref(y, pos, cos, sin, inverse=True), x, atol=1e-12)


def pin_angle_addition(orc):
    """Table rows satisfy cos(a + b) = cos a cos b - sin a sin b for the
    positions 1 and p: row p + 1 follows from rows 1 and p; and column d/4
    has frequency base ** -1/2."""
    d, base = 128, 1e6
    cos, sin = orc.rope_tables_ref(300, d, base)
    p = np.arange(1, 299)
    np.testing.assert_allclose(cos[p + 1], cos[p] * cos[1] - sin[p] * sin[1], atol=1e-12)
    np.testing.assert_allclose(sin[p + 1], sin[p] * cos[1] + cos[p] * sin[1], atol=1e-12)
    np.testing.assert_allclose(cos[7, d // 4], np.cos(7 / np.sqrt(base)), rtol=1e-15)


def pin_transformers_qwen3(orc):
    """transformers' Qwen3 RoPE on CPU in float64. apply_rotary_pos_emb fixes
    the pairing and the sign: fed this oracle's tables, it must give the same
    rotated q and k. Qwen3RotaryEmbedding fixes the frequencies: it computes
    its angles in float32, so its tables are compared at positions below 64,
    where float32 angles are good to 1e-5."""
    from transformers import Qwen3Config
    from transformers.models.qwen3.modeling_qwen3 import (Qwen3RotaryEmbedding,
                                                          apply_rotary_pos_emb)
    H, Hk, d, T = 4, 2, 128, 50
    pos = np.random.default_rng(5).integers(0, 4000, size=T)
    q, k = _x(T, H, d, 6), _x(T, Hk, d, 7)
    cos, sin = orc.rope_tables_ref(4096, d, 1e6)
    c = torch.from_numpy(np.concatenate([cos[pos], cos[pos]], -1))[None]  # [1, T, d]
    s = torch.from_numpy(np.concatenate([sin[pos], sin[pos]], -1))[None]
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]  # [1, H, T, d]
    kt = torch.from_numpy(k).permute(1, 0, 2)[None]
    qr, kr = apply_rotary_pos_emb(qt, kt, c, s)
    np.testing.assert_allclose(orc.rope_ref(q, pos, cos, sin), qr[0].permute(1, 0, 2).numpy(),
                               rtol=0, atol=1e-12)
    np.testing.assert_allclose(orc.rope_ref(k, pos, cos, sin), kr[0].permute(1, 0, 2).numpy(),
                               rtol=0, atol=1e-12)
    cfg = Qwen3Config(hidden_size=H * d, num_attention_heads=H, num_key_value_heads=Hk,
                      head_dim=d, rope_theta=1e6, max_position_embeddings=4096)
    small = torch.arange(64)[None]
    ce, se = Qwen3RotaryEmbedding(cfg)(qt.float(), small)
    np.testing.assert_allclose(cos[:64], ce[0, :, :d // 2].double().numpy(), rtol=0, atol=1e-5)
    np.testing.assert_allclose(sin[:64], se[0, :, :d // 2].double().numpy(), rtol=0, atol=1e-5)


def pin_positions(orc):
    """Token positions of a packed batch and of a chunked prefill."""
    np.testing.assert_array_equal(orc.varlen_positions([0, 3, 3, 5]), [0, 1, 2, 0, 1])
    np.testing.assert_array_equal(orc.chunk_positions([0, 2, 2, 5], [10, 4, 3]),
                                  [8, 9, 0, 1, 2])


PINS = [pin_complex_form, pin_worked_example, pin_relative_position, pin_orthogonal,
        pin_angle_addition, pin_transformers_qwen3, pin_positions]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_rope_oracle_pin(pin):
    pin(R)


def pin_fp16_single_rounding(orc):
    """rope_fp16_ref rounds the exact rotation to fp16 once, to nearest even.
    Hand-derived values (fp16 has 10 fraction bits, spacing 2^-10 on [1, 2),
    smallest subnormal 2^-24):
      * position 0 is the identity, so the fp64 input itself is rounded:
        1 + 2^-11 + 2^-40 lies just above the midpoint of 1 and 1 + 2^-10 and
        gives 1 + 2^-10; 1 + 2^-11 - 2^-40 lies just below it and gives 1;
        1 + 2^-11 exactly is a tie and goes to the even neighbour 1;
        1 + 3 * 2^-11 is a tie between 1 + 2^-10 and 1 + 2^-9 and goes to
        1 + 2^-9; 2^-25 + 2^-60 passes half the smallest subnormal and gives
        2^-24, 2^-25 - 2^-60 gives 0;
      * with cos = 0, sin = 1 (a quarter turn, given as explicit tables) the
        pair (a, b) becomes (-b, a), and the rounding acts on the rotated
        value: b = 1 + 2^-11 + 2^-40 gives -(1 + 2^-10) in slot 0.
    Rounding through fp32 first (a plausible mistake) drops the 2^-40 and
    2^-60 terms and turns the first and fifth cases into ties."""
    e = 2.0 ** -40
    vals = [1 + 2 ** -11 + e, 1 + 2 ** -11 - e, 1 + 2 ** -11, 1 + 3 * 2 ** -11,
            2 ** -25 + 2 ** -60, 2 ** -25 - 2 ** -60]
    want = [1 + 2 ** -10, 1.0, 1.0, 1 + 2 ** -9, 2 ** -24, 0.0]
    cos, sin = orc.rope_tables_ref(1, 2 * len(vals), 10000.0)
    x = np.array(vals + [0.0] * len(vals), dtype=np.float64)[None, None, :]
    y = orc.rope_fp16_ref(x, [0], cos, sin)
    assert y.dtype == np.float16
    np.testing.assert_array_equal(y[0, 0, :len(vals)].astype(np.float64), want)
    np.testing.assert_array_equal(y[0, 0, len(vals):].astype(np.float64), 0.0)
    quarter_c = np.array([[1.0], [0.0]])
    quarter_s = np.array([[0.0], [1.0]])
    xq = np.array([[[1 + 2 ** -11 - e, 1 + 2 ** -11 + e]]])
    yq = orc.rope_fp16_ref(xq, [1], quarter_c, quarter_s)
    np.testing.assert_array_equal(yq[0, 0].astype(np.float64), [-(1 + 2 ** -10), 1.0])
    # The inverse quarter turn maps (a, b) to (b, -a).
    yi = orc.rope_fp16_ref(xq, [1], quarter_c, quarter_s, inverse=True)
    np.testing.assert_array_equal(yi[0, 0].astype(np.float64), [1 + 2 ** -10, -1.0])


def test_rope_fp16_is_round_to_nearest():
    pin_fp16_single_rounding(R)


# Planted mistakes.
_orig_tables = R.rope_tables_ref
_orig_rope = R.rope_ref


def _tables_freq_j_over_d(max_pos, d, base):
    j = np.arange(d // 2, dtype=np.float64)
    ang = np.arange(max_pos)[:, None] * np.power(float(base), -j / d)[None, :]
    return np.cos(ang), np.sin(ang)


def _tables_swapped(max_pos, d, base):
    c, s = _orig_tables(max_pos, d, base)
    return s, c


def _rope_interleaved(x, pos, cos, sin, inverse=False):
    x = np.asarray(x, np.float64)
    c, s = cos[pos][:, None, :], sin[pos][:, None, :]
    s = -s if inverse else s
    y = x.copy()
    y[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
    y[..., 1::2] = x[..., 1::2] * c + x[..., 0::2] * s
    return y


def _rope_wrong_sign(x, pos, cos, sin, inverse=False):
    return _orig_rope(x, pos, cos, sin, not inverse)


def _rope_fp16_via_fp32(x, pos, cos, sin, inverse=False):
    return R.rope_ref(x, pos, cos, sin, inverse).astype(np.float32).astype(np.float16)


def _rope_fp16_truncating(x, pos, cos, sin, inverse=False):
    y = R.rope_ref(x, pos, cos, sin, inverse)
    r = y.astype(np.float16)
    over = np.abs(r.astype(np.float64)) > np.abs(y)
    return np.where(over, np.nextafter(r, np.float16(0)), r).astype(np.float16)


def _rope_off_by_one(x, pos, cos, sin, inverse=False):
    return _orig_rope(x, np.asarray(pos) + 1, np.vstack([cos, cos[-1:]]),
                      np.vstack([sin, sin[-1:]]), inverse)


MUTANTS = [
    ("rope_tables_ref", _tables_freq_j_over_d, [pin_complex_form, pin_worked_example,
                                                pin_angle_addition, pin_transformers_qwen3]),
    ("rope_tables_ref", _tables_swapped, [pin_complex_form, pin_worked_example,
                                          pin_orthogonal]),
    ("rope_ref", _rope_interleaved, [pin_complex_form, pin_worked_example,
                                     pin_transformers_qwen3]),
    ("rope_ref", _rope_wrong_sign, [pin_complex_form, pin_worked_example,
                                    pin_transformers_qwen3]),
    ("rope_ref", _rope_off_by_one, [pin_complex_form, pin_worked_example, pin_orthogonal]),
    ("rope_fp16_ref", _rope_fp16_via_fp32, [pin_fp16_single_rounding]),
    ("rope_fp16_ref", _rope_fp16_truncating, [pin_fp16_single_rounding]),
]


@pytest.mark.parametrize("name,fn,pins", MUTANTS, ids=[f"{m[0]}:{m[1].__name__}" for m in MUTANTS])
def test_rope_pins_catch_planted_mistake(monkeypatch, name, fn, pins):
    monkeypatch.setattr(R, name, fn)
    for pin in pins:
        with pytest.raises(Exception):
            pin(R)
