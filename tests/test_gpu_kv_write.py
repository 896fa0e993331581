"""The KV write path (sa_kv_write) against the oracle's composition of forward RoPE, the
block-32 fp8 round trip and the ring / linear store: stored rows, codes, scale bytes and the
returned rows bit for bit; then the written ring feeds sparse_attn like the pages' decode."""
import sys

import numpy as np
import pytest
import torch

import oracle
import sa_workloads as W
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


def _rows(seed, b, s, d):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(b, s, d, generator=g).to(torch.bfloat16)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_ring_sequence_write_then_attend(sa, fmt):
    """Prefill 12 tokens into an 8-slot ring, then decode steps 12 and 13 (the ring-cache
    paragraph): after each write the ring (bf16 rows, or codes and scale bytes) equals the
    oracle's bit for bit, and sparse_attn over it matches the oracle's attention."""
    cfg = W.tiny_ring()
    Wn, h, d, rd = cfg["window"], cfg["h"], cfg["d"], cfg["rd"]
    sink, scale = cfg["sink"], cfg["scale"]
    table = sa.rope_table(rd, 16, 10000.0, "cuda")
    cs = oracle.freqs_cis(rd, 16, 10000.0)
    if fmt == "bf16":
        ring = torch.zeros(1, Wn, d, dtype=torch.bfloat16, device="cuda")
        scales = None
    else:
        ring = torch.zeros(1, Wn, d, dtype=torch.uint8, device="cuda")
        scales = torch.zeros(1, Wn, d // 32, dtype=torch.uint8, device="cuda")
    o_ring = np.zeros((1, Wn, d), np.uint16)
    o_codes = np.zeros((1, Wn, d), np.uint8)
    o_scales = np.zeros((1, Wn, d // 32), np.uint8)
    for step in cfg["steps"]:
        P, q, x = step["start_pos"], step["q"], step["kv_rows"]
        S = q.shape[1]
        _say("kv write ring", fmt, step["kind"], P)
        pos = (torch.arange(S, dtype=torch.int32) + P).view(1, S)
        rows = torch.empty(1, S, d, dtype=torch.bfloat16, device="cuda")
        sa.kv_write(x.view(1, S, d).cuda(), pos.cuda(), ring, rope=table, window=Wn,
                    cache_scale=scales, rows_out=rows)
        o_rows = oracle.kv_write(u16(x).reshape(1, S, d), pos.numpy(), rd, cs, Wn, Wn,
                                 cache_bf16=o_ring, cache_codes=o_codes, cache_scales=o_scales)
        assert np.array_equal(u16(rows), o_rows)
        if fmt == "bf16":
            assert np.array_equal(u16(ring), o_ring)
        else:
            assert np.array_equal(ring.cpu().numpy(), o_codes)
            assert np.array_equal(scales.cpu().numpy(), o_scales)
        # attend: prefill reads the chunk's rows, decode the ring
        if step["kind"] == "prefill":
            kv, kv_scale = rows, None
            idx = sa.window_topk_idxs(Wn, S, 1, device="cuda")
            kv_o, idx_o = o_rows, oracle.window_topk_idxs(Wn, S)
        else:
            kv, kv_scale = ring, scales
            idx = sa.window_topk_idxs(Wn, 1, 1, start_pos=torch.tensor([P], dtype=torch.int32, device="cuda"))
            kv_o, idx_o = o_ring, oracle.window_topk_idxs(Wn, 1, [P])
        out = sa.sparse_attn(q.cuda(), kv, sink.cuda(), idx, scale, kv_scale=kv_scale,
                             rope=(table, pos.cuda()))
        ref = oracle.sparse_attn(u16(q), kv_o, sink.numpy(), idx_o, scale)
        ref = oracle.apply_rotary(ref, rd, cs, pos.numpy().reshape(-1), inverse=True)
        assert_close(u16(out).reshape(-1, h, d), ref, f"ring {fmt} {step['kind']} {P}")


@pytest.mark.parametrize("seed,name,b,s,d,rd,window,fmt", [
    (21, "prefill chunk of 4096 tokens", 1, 4096, 512, 64, 128, "bf16"),
    (22, "prefill chunk of 4096 tokens, fp8", 1, 4096, 512, 64, 128, "fp8"),
    (27, "the long prefill's 8192 tokens", 1, 8192, 512, 64, 128, "bf16"),
    (23, "decode, 64 sequences", 64, 1, 512, 64, 128, "bf16"),
    (24, "decode, 64 sequences, fp8", 64, 1, 512, 64, 128, "fp8"),
    (25, "short chunks, d 128", 3, 37, 128, 32, 16, "bf16"),
    (26, "d 256, fp8", 2, 50, 256, 64, 64, "fp8"),
])
def test_ring_write_bit_exact(sa, seed, name, b, s, d, rd, window, fmt):
    _say("kv write", name)
    x = _rows(seed, b, s, d)
    g = torch.Generator().manual_seed(7)
    start = torch.randint(0, 60000, (b, 1), generator=g, dtype=torch.int32) if s == 1 else torch.zeros(b, 1, dtype=torch.int32)
    pos = start + torch.arange(s, dtype=torch.int32)[None]
    max_pos = int(pos.max()) + 1
    table = sa.rope_table(rd, max_pos, 10000.0, "cuda")
    cs = oracle.freqs_cis(rd, max_pos, 10000.0)
    fill = torch.Generator().manual_seed(9)
    if fmt == "bf16":
        init = torch.randn(b, window, d, generator=fill).to(torch.bfloat16)
        ring = init.cuda()
        scales = None
    else:
        init = torch.randint(0, 255, (b, window, d), generator=fill, dtype=torch.uint8)
        ring = init.cuda()
        scales = torch.randint(0, 255, (b, window, d // 32), generator=fill, dtype=torch.uint8).cuda()
    sc_before = None if scales is None else scales.cpu().numpy().copy()
    rows = torch.empty(b, s, d, dtype=torch.bfloat16, device="cuda")
    sa.kv_write(x.cuda(), pos.cuda(), ring, rope=table, window=window, cache_scale=scales, rows_out=rows)
    if fmt == "bf16":
        o_ring = u16(init).copy()
        o_rows = oracle.kv_write(u16(x), pos.numpy(), rd, cs, window, window, cache_bf16=o_ring)
        assert np.array_equal(u16(ring), o_ring)
    else:
        o_codes, o_scales = init.numpy().copy(), sc_before.copy()
        o_rows = oracle.kv_write(u16(x), pos.numpy(), rd, cs, window, window,
                                 cache_codes=o_codes, cache_scales=o_scales)
        assert np.array_equal(ring.cpu().numpy(), o_codes)
        assert np.array_equal(scales.cpu().numpy(), o_scales)
    assert np.array_equal(u16(rows), o_rows)


def test_linear_store_and_reported_rows(sa):
    """window 0 (a linear cache such as the compressed one, rows at row0[n] + t, positions
    j * ratio): bit for bit with the oracle; rows whose position lies outside the table or
    whose destination lies outside the cache are not stored, and bit value 4 is reported."""
    b, s, d, rd, R = 4, 300, 512, 64, 16384
    x = _rows(11, b, s, d)
    row0 = torch.tensor([0, 100, 5000, 16200], dtype=torch.int32)     # sequence 3 runs past R
    pos = (row0[:, None] + torch.arange(s, dtype=torch.int32)[None]) * 4
    pos[1, 7] = -1
    max_pos = 65536
    pos[2, 9] = max_pos                                                 # outside the table
    table = sa.rope_table(rd, max_pos, 160000.0, "cuda", original_seq_len=65536, factor=16.0)
    cs = oracle.freqs_cis(rd, max_pos, 160000.0, original_seq_len=65536, factor=16.0)
    init = torch.zeros(b, R, d, dtype=torch.bfloat16)
    cache = init.cuda()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    sa.kv_write(x.cuda(), pos.cuda(), cache, rope=table, window=0, row0=row0.cuda(),
                err_word=err, check_idx=True)
    o_cache = u16(init).copy()
    oracle.kv_write(u16(x), pos.numpy(), rd, cs, 0, R, row0=row0.numpy(), cache_bf16=o_cache,
                    want_rows=False)
    assert np.array_equal(u16(cache), o_cache)
    assert int(err.item()) == 4
    err.zero_()
    ok = pos.clone()
    ok[1, 7], ok[2, 9] = 0, 0
    sa.kv_write(x[:3].cuda(), ok[:3].cuda(), cache[:3], rope=table, window=0, row0=row0[:3].cuda(),
                err_word=err, check_idx=True)
    assert int(err.item()) == 0


def test_decode_write_at_the_last_table_row(sa):
    """64 decode rows at position 65535, the last row of a 65536-row (cos, sin) table, into
    slot 65535 mod 128 = 127 of each ring: rows and ring bit for bit against the oracle."""
    b, s, d, rd, window, p = 64, 1, 512, 64, 128, 65535
    _say("kv write at the last table row", b, p)
    x = _rows(28, b, s, d)
    pos = torch.full((b, s), p, dtype=torch.int32)
    table = sa.rope_table(rd, p + 1, 10000.0, "cuda")
    cs = oracle.freqs_cis(rd, p + 1, 10000.0)
    init = torch.randn(b, window, d, generator=torch.Generator().manual_seed(10)).to(torch.bfloat16)
    ring = init.cuda()
    rows = torch.empty(b, s, d, dtype=torch.bfloat16, device="cuda")
    sa.kv_write(x.cuda(), pos.cuda(), ring, rope=table, window=window, rows_out=rows)
    o_ring = u16(init).copy()
    o_rows = oracle.kv_write(u16(x), pos.numpy(), rd, cs, window, window, cache_bf16=o_ring)
    assert np.array_equal(u16(ring), o_ring)
    assert np.array_equal(u16(rows), o_rows)
    # only slot 127 of each ring changed
    changed = (u16(ring) != u16(init)).any(axis=2)
    assert not changed[:, :127].any()
