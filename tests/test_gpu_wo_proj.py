"""The grouped output projection (sa_grouped_proj) against the oracle: bf16 outputs within
the bf16 tolerance on random inputs, bit for bit on exact integer inputs, and the fp8-weight
form bit for bit equal to the bf16 form on the decoded weights."""
import sys

import numpy as np
import pytest
import torch

import oracle
from sa_harness import assert_close, u16

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def sa():
    import sparse_latent_attention_attn_amd as sa
    sa.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return sa


def _inputs(seed, m, g, r, kg, integer=False):
    gen = torch.Generator().manual_seed(seed)
    if integer:
        o = torch.randint(-4, 5, (m, g * kg), generator=gen).float()
        w = torch.randint(-4, 5, (g, r, kg), generator=gen).float()
    else:
        o = torch.randn(m, g * kg, generator=gen)
        w = torch.randn(g, r, kg, generator=gen) * kg ** -0.5
    return o.to(torch.bfloat16), w.to(torch.bfloat16)


CASES = [
    (1, 64, 8, 1024, 4096, False),     # decode: 64 tokens, 64 heads of 512 in 8 groups
    (2, 5, 2, 256, 512, False),        # the LDS-staged decode kernel with one 16-token block
    (3, 300, 3, 256, 640, False),      # the tiled kernel with a ragged token tail
    (4, 40, 2, 128, 1024, True),       # exact arithmetic, LDS-staged, 40 of 64 token rows
    (5, 270, 2, 256, 192, True),       # exact arithmetic, tiled, k not a multiple of 512
    (6, 20, 3, 48, 512, False),        # rows not a multiple of 32: the operand-load decode kernel
    (7, 33, 1, 32, 256, True),         # one 32-row block, one k chunk, 33 tokens
    (8, 17, 2, 64, 768, False),        # two 16-token blocks, three k chunks (one stage reused)
]


@pytest.mark.parametrize("seed,m,g,r,kg,integer", CASES)
def test_grouped_proj_vs_oracle(sa, seed, m, g, r, kg, integer):
    _say("grouped proj", m, g, r, kg, integer)
    o, w = _inputs(seed, m, g, r, kg, integer)
    out = sa.grouped_proj(o.cuda(), w.cuda())
    ref = oracle.grouped_proj(u16(o).reshape(m, g, kg), u16(w))
    if integer:
        assert np.array_equal(u16(out), ref)
    else:
        assert_close(u16(out), ref, "grouped proj")


@pytest.mark.parametrize("m,g,r,kg", [(64, 8, 1024, 8192), (300, 2, 256, 512), (7, 3, 64, 1024),
                                      (20, 2, 48, 512), (33, 2, 32, 1280)])
def test_fp8_weights_equal_bf16_on_decoded_weights(sa, m, g, r, kg):
    """Weights stored as e4m3 + block-32 scales (sa_quant_kv_fp8 on rows of kg): the result
    is bit for bit the bf16 product with the decoded weights (the decode is exact), and
    matches the oracle on them."""
    _say("grouped proj fp8", m, g, r, kg)
    o, w = _inputs(7 + m, m, g, r, kg)
    codes, scales = sa.quant_kv_fp8(w.cuda(), want=("codes", "scales"))
    w_dec = oracle.fp8_storage_decode(codes.cpu().numpy().reshape(-1, kg), scales.cpu().numpy().reshape(-1, kg // 32))
    w_dec_t = torch.from_numpy(w_dec.view(np.int16)).view(torch.bfloat16).reshape(g, r, kg)
    out8 = sa.grouped_proj(o.cuda(), codes, w_scale=scales)
    out16 = sa.grouped_proj(o.cuda(), w_dec_t.cuda())
    assert torch.equal(out8.view(torch.int16), out16.view(torch.int16))
    sel = np.unique(np.linspace(0, m - 1, min(m, 16)).round().astype(np.int64))
    ref = oracle.grouped_proj(u16(o[sel]).reshape(sel.size, g, kg), w_dec.reshape(g, r, kg))
    assert_close(u16(out8)[sel], ref, "grouped proj fp8")


def test_grouped_proj_full_size_prefill(sa):
    """The long prefill's output (8192 tokens, 128 heads of 512 = 8 groups of 8192) into 8
    groups of 1024: sampled tokens against the oracle, every output finite; tokens read from
    sparse_attn's [b][s][h][d] output layout."""
    m, g, r, kg = 8192, 8, 1024, 8192
    o, w = _inputs(9, m, g, r, kg)
    od = o.cuda().view(1, m, 128, 512)
    out = sa.grouped_proj(od, w.cuda())
    assert bool(torch.isfinite(out.float()).all())
    sel = np.array([0, 1, 255, 256, 4095, 4096, 8000, 8191])
    ref = oracle.grouped_proj(u16(o[sel]).reshape(sel.size, g, kg), u16(w))
    assert_close(u16(out)[sel], ref, "grouped proj full size")
