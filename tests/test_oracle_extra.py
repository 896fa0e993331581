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


# ------------------------------------------------------------------ KV write path
import torch  # noqa: E402


def _rows(seed, b, s, d, tail_pairs_unit=False):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(b, s, d, generator=g)
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _f32(u):
    return torch.from_numpy(np.ascontiguousarray(u).view(np.int16)).view(torch.bfloat16).float().numpy()


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_kv_write_ring_worked_example(orc):
    """The ring-cache paragraph's sequence (12 tokens into 8 slots, then decode steps 12 and
    13) through the write path: token t's row carries t + 1 in its first element, which the
    fp8 round trip keeps exactly, so the ring reads back as tokens."""
    import os
    g = {}
    with open(os.path.join(os.path.dirname(__file__), "golden", "ring_cache_12_into_8.txt")) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                k, *v = line.split()
                g[k] = [int(t) for t in v]
    Wn, S, d, rd = 8, 12, 64, 16
    x = np.zeros((1, 14, d), np.float32)
    x[0, :, 0] = np.arange(1, 15)                     # token id + 1, exact in e4m3 (<= 4 bits)
    x[0, :, 1:] = np.random.default_rng(0).standard_normal((14, d - 1))
    xu = _bf16(x)
    cs = orc.freqs_cis(rd, 16, 10000.0)
    ring = np.zeros((1, Wn, d), np.uint16)
    rows = orc.kv_write(xu[:, :S], np.arange(S)[None], rd, cs, Wn, Wn, cache_bf16=ring)
    assert (_f32(ring[0, :, 0]) - 1).astype(int).tolist() == g["ring_after_prefill"]
    assert np.array_equal(ring[0], rows[0, S - Wn:][np.argsort(np.arange(S - Wn, S) % Wn)])
    for P in (12, 13):
        before = ring.copy()
        orc.kv_write(xu[:, P:P + 1], np.array([[P]]), rd, cs, Wn, Wn, cache_bf16=ring)
        changed = np.nonzero((ring != before).any(axis=-1)[0])[0].tolist()
        assert changed == g[f"decode_{P}_writes_slot"]
        assert (_f32(ring[0, :, 0]) - 1).astype(int).tolist() == g[f"ring_after_decode_{P}"]


def test_kv_write_quantises_after_rotating(orc):
    """The stored rows are fp8 round-trip fixed points (quantised last); the blocks before the
    rope tail equal the round trip of the unrotated row; the fp8 storage form decodes to the
    bf16 form."""
    b, s, d, rd, W = 2, 40, 512, 64, 16
    x = _rows(3, b, s, d)
    cs = orc.freqs_cis(rd, 100, 10000.0)
    pos = np.tile(np.arange(s), (b, 1)) + np.array([[0], [50]])
    ring = np.zeros((b, W, d), np.uint16)
    codes = np.zeros((b, W, d), np.uint8)
    scales = np.zeros((b, W, d // 32), np.uint8)
    rows = orc.kv_write(x, pos, rd, cs, W, W, cache_bf16=ring, cache_codes=codes, cache_scales=scales)
    flat = rows.reshape(-1, d)
    assert np.array_equal(orc.act_quant(flat)[0], flat)
    head = orc.act_quant(x.reshape(-1, d))[0][:, : d - rd]
    assert np.array_equal(flat[:, : d - rd], head)
    assert np.array_equal(orc.fp8_storage_decode(codes.reshape(-1, d), scales.reshape(-1, d // 32)),
                          ring.reshape(-1, d))


def test_kv_write_rotates_forward_at_the_row_position(orc):
    """Tail pairs (1, 0) become (cos, sin) of position x frequency, the forward direction of
    apply_rotary_emb, computed here in f64 from the definition (frequency base^(-2i/rd)),
    within the fp8 step (3 mantissa bits)."""
    d, rd, s = 64, 16, 9
    x = np.zeros((1, s, d), np.float32)
    x[0, :, d - rd::2] = 1.0
    pos = np.array([[0, 1, 2, 3, 10, 33, 100, 250, 499]])
    cs = orc.freqs_cis(rd, 500, 10000.0)
    rows = _f32(orc.kv_write(_bf16(x), pos, rd, cs, 0, s, row0=np.zeros(1, np.int32)))
    i = np.arange(rd // 2)
    ang = pos[0][:, None] * 10000.0 ** (-2.0 * i / rd)[None, :]
    got_c, got_s = rows[0, :, d - rd::2], rows[0, :, d - rd + 1::2]
    assert np.allclose(got_c, np.cos(ang), atol=1 / 16 + 1e-3)
    assert np.allclose(got_s, np.sin(ang), atol=1 / 16 + 1e-3)
    assert np.all(rows[0, :, : d - rd] == 0)


def test_kv_write_linear_store_and_invalid_rows(orc):
    """window 0: row t lands at row0[n] + t; rows whose destination falls outside the cache
    or whose position is outside the table are not stored; other rows are untouched."""
    b, s, d, rd, R = 2, 6, 128, 32, 10
    x = _rows(5, b, s, d)
    cs = orc.freqs_cis(rd, 64, 10000.0)
    pos = np.array([[0, 4, 8, 12, 16, 20], [1, 99, 3, 4, 5, 6]])         # 99: outside the table
    row0 = np.array([2, 7], np.int32)                                    # sequence 1 runs past R
    cache = np.full((b, R, d), 0x7777, np.uint16)
    rows = orc.kv_write(x, pos, rd, cs, 0, R, row0=row0, cache_bf16=cache)
    assert np.array_equal(cache[0, 2:8], rows[0])
    assert np.all(cache[0, :2] == 0x7777) and np.all(cache[0, 8:] == 0x7777)
    assert np.array_equal(cache[1, 7], rows[1, 0]) and np.array_equal(cache[1, 9], rows[1, 2])
    assert np.all(cache[1, 8] == 0x7777)                                 # position 99: nothing
    assert np.all(cache[1, :7] == 0x7777)
