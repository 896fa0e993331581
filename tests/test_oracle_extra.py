"""Pins of the oracle functions beyond sparse_attn itself (CPU only): the YaRN form of the
rotary table. Each pin checks a property the pages or the mathematics fix, computed
independently of the oracle's own formula."""
import math

import numpy as np
import pytest


# ------------------------------------------------------------------ YaRN rotary table
YARN = dict(original_seq_len=65536, factor=16.0, beta_fast=32.0, beta_slow=1.0)   # model config


@pytest.mark.parametrize("rd,base", [(64, 160000.0), (64, 10000.0), (128, 160000.0)])
def test_yarn_keeps_fast_pairs_and_scales_slow_pairs(orc, rd, base):
    """precompute_freqs_cis with YaRN (attention output page): pairs whose wavelength fits
    more than beta_fast times into the training context keep their frequency, pairs that fit
    fewer than beta_slow times have it divided by factor, and the band between is blended
    linearly and monotonically. Rotations are counted here in f64 from the definition of
    the wavelength, not from the oracle's corrected_dim."""
    L, fac = YARN["original_seq_len"], YARN["factor"]
    plain = orc.freqs_cis(rd, 2, base)
    yarn = orc.freqs_cis(rd, 2, base, **YARN)
    f_plain = np.arctan2(plain[1, :, 1].astype(np.float64), plain[1, :, 0])
    f_yarn = np.arctan2(yarn[1, :, 1].astype(np.float64), yarn[1, :, 0])
    i = np.arange(rd // 2)
    rotations = L * base ** (-2.0 * i / rd) / (2 * math.pi)   # turns over the context
    fast, slow = rotations > YARN["beta_fast"], rotations < YARN["beta_slow"]
    assert fast.any()
    assert slow.any() or base < 100000          # base 10000: even the slowest pair turns > once
    assert np.array_equal(yarn[:, fast], plain[:, fast])          # bit for bit: unchanged
    assert np.allclose(f_yarn[slow], f_plain[slow] / fac, rtol=1e-6, atol=0)
    w = (f_plain - f_yarn) / (f_plain - f_plain / fac)              # 0 kept .. 1 scaled
    assert np.all(w >= -1e-6) and np.all(w <= 1 + 1e-6)
    assert np.all(np.diff(w) >= -1e-6), "the blend must not go back"
    band = (w > 1e-6) & (w < 1 - 1e-6)
    if band.sum() >= 3:                                               # linear in the pair index
        assert np.allclose(np.diff(w[band], 2), 0.0, atol=2e-5)


def test_yarn_off_is_the_plain_table(orc):
    t0 = orc.freqs_cis(64, 300, 10000.0)
    t1 = orc.freqs_cis(64, 300, 10000.0, original_seq_len=0, factor=16.0)
    assert np.array_equal(t0, t1)


def test_yarn_table_entries_are_rotations(orc):
    """Every entry is a unit complex number, and the angle at position p is p times the
    angle at position 1 (a rotation by a fixed frequency per pair)."""
    t = orc.freqs_cis(64, 5000, 160000.0, **YARN).astype(np.float64)
    assert np.allclose(t[..., 0] ** 2 + t[..., 1] ** 2, 1.0, atol=1e-6)
    f = np.arctan2(t[1, :, 1], t[1, :, 0])
    for p in (2, 3, 17, 500, 4999):
        ang = np.float32(p) * f.astype(np.float32)
        assert np.allclose(t[p, :, 0], np.cos(ang.astype(np.float64)), atol=4e-6 * max(1, p / 100))
        assert np.allclose(t[p, :, 1], np.sin(ang.astype(np.float64)), atol=4e-6 * max(1, p / 100))
