"""Pins of the oracle's numeric helpers (bf16, pow2_ceil, e4m3, block-32 ue8m0 round trip)
against things other than the oracle itself: exhaustive comparison with torch's casts,
frexp, closed forms and invariants. CPU only."""
import math

import numpy as np
import pytest
import torch


# ------------------------------------------------------------------ bf16 <-> f32
def test_bf16_roundtrip_exhaustive(orc):
    allb = np.arange(1 << 16, dtype=np.uint16)
    f = orc.bf16_to_f32(allb)
    back = orc.f32_to_bf16(f)
    finite = ~np.isnan(f)
    assert np.array_equal(back[finite], allb[finite])
    # bf16 -> f32 is the upper half of the f32 pattern, as torch does it
    t = torch.from_numpy(allb.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(f[finite], t[finite])


def test_f32_to_bf16_matches_torch_rne(orc):
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 32, 200_000, dtype=np.uint64).astype(np.uint32)
    # force exact ties (lower half 0x8000) on a quarter of them
    bits[::4] = (bits[::4] & 0xFFFF0000) | 0x8000
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    ours = orc.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


# ------------------------------------------------------------------ pow2_ceil
def _pow2_ceil_frexp(v):
    m, e = math.frexp(v)            # v = m * 2^e, m in [0.5, 1)
    return math.ldexp(1.0, e - 1 if m == 0.5 else e)


def test_pow2_ceil_against_frexp(orc):
    rng = np.random.default_rng(1)
    vals = []
    for E in range(1, 254):         # every normal exponent
        for M in (0, 1, (1 << 23) - 1, int(rng.integers(1, 1 << 23))):
            vals.append(np.array([(E << 23) | M], np.uint32).view(np.float32)[0])
    for v in vals:
        v = float(v)
        expect = _pow2_ceil_frexp(v)
        if expect > 3.4028234663852886e38:
            continue
        assert orc.pow2_ceil(v) == expect, v
    for k in range(-126, 128):
        assert orc.pow2_ceil(math.ldexp(1.0, k)) == math.ldexp(1.0, k)


# ------------------------------------------------------------------ e4m3
def _all_bf16_finite():
    allb = np.arange(1 << 16, dtype=np.uint16)
    f = torch.from_numpy(allb.view(np.int16)).view(torch.bfloat16).float().numpy()
    return f[np.isfinite(f)]


def test_e4m3_encode_exhaustive_vs_torch(orc):
    f = _all_bf16_finite()
    inside = f[np.abs(f) <= 448.0]
    ref = torch.from_numpy(inside).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([orc.e4m3_encode(float(v)) for v in inside], np.uint8)
    assert np.array_equal(ours, ref)


def test_e4m3_clamps_before_rounding(orc):
    # beyond 448 the reading is "clamped": 460, 500, 1e30 all land on the largest code
    for v in (448.0, 449.0, 460.0, 500.0, 1e30):
        assert orc.e4m3_encode(v) == 0x7E
        assert orc.e4m3_encode(-v) == 0xFE
    assert orc.e4m3_decode(0x7E) == 448.0


def test_e4m3_ties_to_even(orc):
    cases = {1.5 * 2**-9: 2**-8, 2.5 * 2**-9: 2**-8, 17.0: 16.0, 19.0: 20.0, 248.0: 256.0,
             0.5 * 2**-9: 0.0}
    for x, y in cases.items():
        assert orc.e4m3_decode(orc.e4m3_encode(x)) == y, x


def test_e4m3_decode_all_codes_vs_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    ours = np.array([orc.e4m3_decode(int(c)) for c in codes], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))  # -0 too


# ------------------------------------------------------------------ block-32 ue8m0
def _lognormal_rows(seed, rows, d):
    g = torch.Generator().manual_seed(seed)
    mag = torch.exp(torch.randn(rows, d // 32, 1, generator=g) * 4.0)
    x = torch.randn(rows, d // 32, 32, generator=g) * mag
    return x.reshape(rows, d).to(torch.bfloat16)


def _u16(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _f32(u16):
    return torch.from_numpy(u16.view(np.int16)).view(torch.bfloat16).float().numpy()


def test_act_quant_scale_rule(orc):
    """The scale is the unique power of two s with amax/448 <= s < amax/224, i.e.
    max(amax, 1e-4)/s lies in (224, 448] -- which fixes pow2_ceil(max(amax,1e-4)/448)."""
    x = _lognormal_rows(0, 512, 512)
    y, codes, scales = orc.act_quant(_u16(x))
    xf = x.float().numpy().reshape(512, 16, 32)
    amax = np.maximum(np.abs(xf).max(-1), np.float32(1e-4))
    s = np.ldexp(1.0, scales.astype(np.int64) - 127)
    r = amax / s
    assert np.all(r > 224.0) and np.all(r <= 448.0)


def test_act_quant_zero_block(orc):
    x = np.zeros((2, 64), np.uint16)
    y, codes, scales = orc.act_quant(x)
    # pow2_ceil(1e-4 / 448 = 2.23e-7) = 2^-22 -> biased exponent 105
    assert np.all(scales == 105) and np.all(codes == 0) and np.all(y == 0)


def test_act_quant_matches_torch_fp8_cast(orc):
    """y = e4m3(x / s) * s with torch's own e4m3fn cast as the encoder (scale from the
    oracle's scale bytes, which the previous test pins)."""
    x = _lognormal_rows(1, 256, 512)
    y, codes, scales = orc.act_quant(_u16(x))
    s = torch.from_numpy(np.ldexp(1.0, scales.astype(np.int64) - 127).astype(np.float32))
    xs = x.float().view(256, 16, 32) / s.unsqueeze(-1)
    q = xs.clamp(-448, 448).to(torch.float8_e4m3fn)
    assert np.array_equal(codes.reshape(256, 16, 32), q.view(torch.uint8).numpy())
    yt = (q.float() * s.unsqueeze(-1)).reshape(256, 512)
    assert torch.equal(yt.to(torch.bfloat16).float(), yt)           # bf16-exact
    assert np.array_equal(_f32(y), yt.numpy())


def test_act_quant_idempotent_and_lossless_storage(orc):
    x = _lognormal_rows(2, 1024, 512)
    y, codes, scales = orc.act_quant(_u16(x))
    y2, _, _ = orc.act_quant(y)
    assert np.array_equal(y, y2)                    # rt(rt(x)) == rt(x), value-wise
    dec = orc.fp8_storage_decode(codes, scales)
    assert np.array_equal(dec, y)                   # fp8 storage reproduces the bf16 rt
    # error bound of RNE into e4m3: half a step of the grid at the value's binade
    xf, yf = x.float().numpy(), _f32(y)
    s = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=-1)
    a = np.abs(xf) / s
    step = np.where(a < 2**-6, 2.0**-9, np.ldexp(1.0, np.floor(np.log2(np.maximum(a, 2**-6))).astype(np.int64) - 3))
    assert np.all(np.abs(xf - yf) <= 0.5 * step * s * (1 + 1e-6))


def test_act_quant_d64_two_blocks(orc):
    x = _lognormal_rows(3, 7, 64)
    y, codes, scales = orc.act_quant(_u16(x))
    assert scales.shape == (7, 2)
    with pytest.raises(ValueError):
        orc.act_quant(np.zeros((2, 48), np.uint16))
