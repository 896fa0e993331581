"""Parity of the HIP path (called through the C ABI) with the CPU oracle, on the same
seeded inputs. Indices and fp8 codes must match bit for bit; bf16 outputs must satisfy
|gpu - oracle| <= 8e-3 + 1.6e-2 |oracle| elementwise."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import sa_workloads as W
from sa_harness import (ATOL, RTOL, assert_close, f32_of_u16, gpu_indices, gpu_inputs, gpu_run,
                        oracle_core, oracle_indices, oracle_rotate, oracle_run, u16)

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def sa():
    import sparse_latent_attention_attn_amd as sa
    sa.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return sa


# ------------------------------------------------------------------ window index lists
@pytest.mark.parametrize("window,seqlen", [(1, 5), (8, 12), (8, 3), (128, 1), (128, 130), (128, 4096), (16, 300)])
def test_prefill_lists_bit_exact(sa, window, seqlen):
    _say("prefill lists", window, seqlen)
    got = sa.window_topk_idxs(window, seqlen, 2, device="cuda").cpu().numpy()
    ref = oracle.window_topk_idxs(window, seqlen, nseq=2)
    assert np.array_equal(got, ref)


def test_decode_lists_bit_exact(sa):
    g = torch.Generator().manual_seed(0)
    P = torch.cat([torch.tensor([1, 2, 6, 7, 8, 12, 13, 127, 128, 65535], dtype=torch.int32),
                   torch.randint(1, 70000, (200,), generator=g, dtype=torch.int32)])
    for window in (8, 128, 5):
        _say("decode lists", window)
        got = sa.window_topk_idxs(window, 1, P.numel(), start_pos=P.cuda()).cpu().numpy()
        ref = oracle.window_topk_idxs(window, 1, P.numpy())
        assert np.array_equal(got, ref)


@pytest.mark.parametrize("positions", [[0], [0, 0, 0], [0, 5, 1]])
def test_decode_lists_at_position_zero(sa, positions):
    """A decode step at position 0 (the ring holds token 0 only), alone and beside other
    sequences: the whole ring's list, against the oracle."""
    P = torch.tensor(positions, dtype=torch.int32)
    for window in (8, 128):
        got = sa.window_topk_idxs(window, 1, P.numel(), start_pos=P.cuda()).cpu().numpy()
        ref = oracle.window_topk_idxs(window, 1, P.numpy())
        assert got.shape == ref.shape == (P.numel(), 1, window)
        assert np.array_equal(got, ref)


def test_decode_lists_negative_position(sa):
    """A negative position is a caller error (the oracle rejects it); the library writes a
    row of -1 for it, as include/sa.h documents, and the other rows as usual."""
    P = torch.tensor([-3, 5], dtype=torch.int32)
    got = sa.window_topk_idxs(8, 1, 2, start_pos=P.cuda()).cpu().numpy()
    assert got[0, 0].tolist() == [-1] * 8
    assert np.array_equal(got[1:], oracle.window_topk_idxs(8, 1, [5]))


def test_lists_written_in_place_leave_other_columns(sa):
    _say("in-place lists")
    buf = torch.full((4, 1, 640), 777, dtype=torch.int32, device="cuda")
    P = torch.tensor([65535, 200, 3, 128], dtype=torch.int32)
    sa.window_topk_idxs(128, 1, 4, start_pos=P.cuda(), out=buf)
    b = buf.cpu().numpy()
    assert np.array_equal(b[:, :, :128], oracle.window_topk_idxs(128, 1, P.numpy()))
    assert np.all(b[:, :, 128:] == 777)


# ------------------------------------------------------------------ fp8 quantisation
def _lognormal(seed, rows, d):
    g = torch.Generator().manual_seed(seed)
    mag = torch.exp(torch.randn(rows, d // 32, 1, generator=g) * 6.0)
    x = (torch.randn(rows, d // 32, 32, generator=g) * mag).reshape(rows, d)
    x[0, :32] = 0.0                                   # an all-zero block
    x[1, :32] = 1e-30                                  # below the 1e-4 floor
    x[2, 5] = 3.0e38                                   # near the bf16 maximum
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("rows,d", [(64, 512), (33, 64), (7, 256), (1000, 128)])
def test_quant_bit_exact(sa, rows, d):
    _say("quant", rows, d)
    x = _lognormal(rows + d, rows, d)
    codes, scales, rt = sa.quant_kv_fp8(x.cuda(), want=("codes", "scales", "roundtrip"))
    y, c_ref, s_ref = oracle.act_quant(u16(x))
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    assert np.array_equal(u16(rt), y)


@pytest.mark.parametrize("k", [0, -20, 30])
def test_quant_every_bf16_value(sa, k):
    """Every finite bf16 value of magnitude up to 448, times 2^k, in blocks whose first
    element 448 * 2^k fixes the scale at 2^k: all of e4m3fn's normal, subnormal, tie and
    saturating cases go through the kernel's encode and round trip, against the oracle."""
    _say("quant every bf16 value, scale 2^", k)
    u = np.arange(65536, dtype=np.uint32)
    v = (u << 16).view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 448.0)]
    per = 31
    nblk = -(-v.size // per)
    vals = np.zeros(nblk * per, np.float32)
    vals[:v.size] = v
    blocks = np.concatenate([np.full((nblk, 1), 448.0, np.float32), vals.reshape(nblk, per)], axis=1)
    rows = -(-nblk // 16)
    x = np.zeros((rows * 16, 32), np.float32)
    x[:nblk] = blocks
    xt = (torch.from_numpy(x.reshape(rows, 512)) * 2.0 ** k).to(torch.bfloat16)   # exact unless it underflows
    codes, scales, rt = sa.quant_kv_fp8(xt.cuda(), want=("codes", "scales", "roundtrip"))
    y, c_ref, s_ref = oracle.act_quant(u16(xt))
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    assert np.array_equal(u16(rt), y)


def test_quant_in_place(sa):
    x = _lognormal(5, 16, 512)
    xd = x.cuda()
    sa.quant_kv_fp8(xd, roundtrip=xd, want=("roundtrip",))
    assert np.array_equal(u16(xd), oracle.act_quant(u16(x))[0])


# ------------------------------------------------------------------ sparse_attn
def test_ring_cache_sequence(sa):
    """Prefill 12 tokens into an 8-slot ring, then decode 12 and 13 with the same ring
    (the three regimes of the attention API docs' ring-cache example); the output of
    every step against the oracle, bf16 and fp8 storage."""
    cfg = W.tiny_ring()
    Wn, h, d, rd = cfg["window"], cfg["h"], cfg["d"], cfg["rd"]
    sink = cfg["sink"]
    for fmt in ("bf16", "fp8"):
        ring_dev = torch.zeros(1, Wn, d, dtype=torch.bfloat16, device="cuda")
        ring_orc = np.zeros((Wn, d), np.uint16)
        table = sa.rope_table(rd, 16, device="cuda")
        cs = oracle.freqs_cis(rd, 16, 10000.0)
        for step in cfg["steps"]:
            _say("ring", fmt, step["kind"], step["start_pos"])
            q, rows = step["q"], step["kv_rows"]
            S = q.shape[1]
            P = step["start_pos"]
            rows_dev = rows.cuda()
            rows_orc = u16(rows)
            if fmt == "fp8":
                (rows_dev,) = sa.quant_kv_fp8(rows_dev.contiguous(), want=("roundtrip",))
                rows_orc = oracle.act_quant(rows_orc)[0]
            if step["kind"] == "prefill":
                kv_dev = rows_dev.view(1, S, d)
                idx = sa.window_topk_idxs(Wn, S, 1, device="cuda")
                kv_orc = rows_orc.reshape(1, S, d)
                idx_orc = oracle.window_topk_idxs(Wn, S)
                pos = torch.arange(S, dtype=torch.int32).view(1, S)
                for p_ in range(max(0, S - Wn), S):             # ring writes of the prefill
                    ring_dev[0, p_ % Wn] = rows_dev[p_]
                oracle.ring_prefill(ring_orc, rows_orc)
            else:
                ring_dev[0, P % Wn] = rows_dev[0]
                oracle.ring_decode(ring_orc, rows_orc[0], P)
                kv_dev = ring_dev
                idx = sa.window_topk_idxs(Wn, 1, 1, start_pos=torch.tensor([P], dtype=torch.int32, device="cuda"))
                kv_orc = ring_orc.reshape(1, Wn, d)
                idx_orc = oracle.window_topk_idxs(Wn, 1, [P])
                pos = torch.tensor([[P]], dtype=torch.int32)
            assert np.array_equal(idx.cpu().numpy(), idx_orc)
            assert np.array_equal(u16(ring_dev[0]), ring_orc)
            if fmt == "fp8":
                codes, scales = sa.quant_kv_fp8(kv_dev.contiguous(), want=("codes", "scales"))
                out = sa.sparse_attn(q.cuda(), codes, sink.cuda(), idx, cfg["scale"], kv_scale=scales,
                                     rope=(table, pos.cuda()))
            else:
                out = sa.sparse_attn(q.cuda(), kv_dev, sink.cuda(), idx, cfg["scale"], rope=(table, pos.cuda()))
            ref = oracle.sparse_attn(u16(q), kv_orc, sink.numpy(), idx_orc, cfg["scale"])
            ref = oracle.apply_rotary(ref, rd, cs, pos.numpy().reshape(-1), inverse=True)
            assert_close(u16(out).reshape(-1, h, d), ref, f"ring {fmt} {step['kind']} {P}")


@pytest.mark.parametrize("name", ["decode_window", "prefill_window", "decode_compress", "prefill_compress"])
@pytest.mark.parametrize("fmt,rope", [("bf16", True), ("bf16", False), ("fp8", True)])
def test_small_workloads(sa, name, fmt, rope):
    w = W.small_variant(name)
    _say("small", name, fmt, rope, tuple(w.q.shape), w.topk)
    out, idx = gpu_run(w, fmt, rope)
    assert np.array_equal(idx.cpu().numpy(), oracle_indices(w))
    ref = oracle_run(w, rope=rope, round_trip=w.kv_roundtrip or fmt == "fp8")
    assert_close(u16(out).reshape(-1, w.h, w.d), ref, f"{name} {fmt} rope={rope}")


@pytest.mark.parametrize("seed,b,s,h,d,rows,topk,hole,dup", [
    (1, 1, 3, 1, 64, 40, 7, 0.0, False),
    (2, 2, 5, 20, 128, 100, 33, 0.3, True),
    (3, 3, 2, 100, 512, 300, 100, 0.1, False),
    (4, 1, 4, 160, 256, 64, 64, 0.5, True),
    (5, 2, 1, 128, 512, 2000, 1000, 0.02, False),
    (6, 1, 2, 64, 64, 9, 1, 0.0, False),
    (7, 4, 3, 16, 512, 50, 31, 0.9, True),
])
def test_random_problems(sa, seed, b, s, h, d, rows, topk, hole, dup):
    _say("random", seed, b, s, h, d, rows, topk)
    q, kv, sink, idx = W.rand_problem(seed, b, s, h, d, rows, topk, hole, dup, sink_std=2.0)
    scale = float(np.float32(d ** -0.5))
    out = sa.sparse_attn(q.cuda(), kv.cuda(), sink.cuda(), idx.cuda(), scale)
    ref = oracle.sparse_attn(u16(q), u16(kv), sink.numpy(), idx.numpy(), scale)
    assert_close(u16(out).reshape(-1, h, d), ref, f"random {seed}")


@pytest.mark.parametrize("seed,b,s,h,rows,topk,hole", [
    (61, 1, 300, 128, 200, 70, 0.1),     # 300 workgroups of 128 heads: two head blocks per wave
    (62, 2, 140, 160, 100, 40, 0.3),     # 160 heads: the second workgroup's last 96 heads are padding
])
def test_wide_waves(sa, seed, b, s, h, rows, topk, hole):
    """Enough queries at d = 512 and >= 128 heads for the plan with two blocks of 16 heads
    per wave (one gathered K or V operand feeds two MFMAs)."""
    _say("wide", seed, b, s, h, rows, topk)
    q, kv, sink, idx = W.rand_problem(seed, b, s, h, 512, rows, topk, hole, False)
    scale = float(np.float32(512 ** -0.5))
    # a late key far above the rest for a few queries: the second key pass on this plan too
    for t in range(0, s, 37):
        kv[0, int(idx[0, t, topk - 1]) if idx[0, t, topk - 1] >= 0 else 0] = (q[0, t, 3].float() * 2).to(torch.bfloat16)
    out = sa.sparse_attn(q.cuda(), kv.cuda(), sink.cuda(), idx.cuda(), scale)
    ref = oracle.sparse_attn(u16(q), u16(kv), sink.numpy(), idx.numpy(), scale)
    assert_close(u16(out).reshape(-1, h, 512), ref, f"wide {seed}")


@pytest.mark.parametrize("seed,b,s,h,rows,topk,hole,dup", [
    (71, 1, 300, 64, 500, 200, 0.1, False),   # 600 two-wave workgroups, a ragged last tile
    (72, 2, 150, 40, 90, 256, 0.3, True),     # 40 heads: the second workgroup half padding
    (73, 1, 520, 48, 300, 33, 0.0, False),    # two tiles, the second with one column
])
def test_compact_plan(sa, seed, b, s, h, rows, topk, hole, dup):
    """Short lists (at most 256 columns) at d = 512 with enough queries for two workgroups
    per compute unit: the compact plan (two-wave workgroups, a two-tile ring), including a
    late key far above the rest for some queries (the second key pass)."""
    _say("compact", seed, b, s, h, rows, topk)
    q, kv, sink, idx = W.rand_problem(seed, b, s, h, 512, rows, topk, hole, dup)
    scale = float(np.float32(512 ** -0.5))
    for t in range(0, s, 41):
        r = int(idx[0, t, topk - 1])
        kv[0, r if r >= 0 else 0] = (q[0, t, 1].float() * 2).to(torch.bfloat16)
    out = sa.sparse_attn(q.cuda(), kv.cuda(), sink.cuda(), idx.cuda(), scale)
    ref = oracle.sparse_attn(u16(q), u16(kv), sink.numpy(), idx.numpy(), scale)
    assert_close(u16(out).reshape(-1, h, 512), ref, f"compact {seed}")
    assert bool(torch.isfinite(out.float()).all())


# seed, b, s, h, d, rows, topk, hole, dup, fmt, rope_dim: one case per plan family
SWEEP = [
    (81, 3, 5, 16, 64, 40, 40, 0.2, False, "bf16", 16),       # one-wave workgroups
    (82, 2, 33, 24, 128, 300, 260, 0.1, True, "fp8", 0),       # ragged heads and tiles, fp8 (d 128)
    (83, 1, 3, 64, 256, 5000, 4500, 0.1, False, "bf16", 64),   # two splits and the combine kernel
    (84, 2, 1, 64, 512, 1000, 700, 0.05, False, "fp8", 64),    # key groups, fp8 in-kernel conversion
    (85, 4, 1, 128, 512, 2000, 640, 0.02, False, "bf16", 64),  # two key groups (window + compressed decode)
    (86, 1, 7, 16, 512, 64, 64, 0.0, False, "bf16", 0),        # one head block, short lists
    (87, 1, 700, 40, 512, 300, 100, 0.1, False, "bf16", 64),   # compact plan, ragged heads
    (88, 1, 260, 128, 512, 600, 300, 0.1, False, "fp8", 64),   # dequantised rows, two head blocks per wave
    (89, 2, 1, 64, 128, 9000, 5000, 0.3, True, "fp8", 0),      # fp8 at d 128 with splits
    (90, 3, 20, 16, 256, 500, 1, 0.0, False, "bf16", 32),      # one column per list
    (91, 8, 1, 64, 512, 128, 128, 0.0, False, "fp8", 64),      # window-decode shape, fp8
    (92, 1, 64, 128, 64, 2048, 2048, 0.5, True, "fp8", 0),     # long lists at d 64, half holes
]


@pytest.mark.parametrize("seed,b,s,h,d,rows,topk,hole,dup,fmt,rd", SWEEP)
def test_plan_sweep(sa, seed, b, s, h, d, rows, topk, hole, dup, fmt, rd):
    """Random problems across the planner's branches (workgroup widths, head blocks per wave,
    key groups, splits, the compact layout, dequantised rows), bf16 and fp8 storage, with and
    without the inverse-RoPE epilogue, against the oracle on the same (round-tripped) rows."""
    _say("sweep", seed, b, s, h, d, rows, topk, fmt, rd)
    q, kv, sink, idx = W.rand_problem(seed, b, s, h, d, rows, topk, hole, dup)
    scale = float(np.float32(d ** -0.5))
    kv_scale = None
    if fmt == "fp8":
        codes, kv_scale = sa.quant_kv_fp8(kv.cuda(), want=("codes", "scales"))
        kv_dev = codes
        kv_ref = oracle.act_quant(u16(kv))[0]
    else:
        kv_dev = kv.cuda()
        kv_ref = u16(kv)
    rope = None
    pos = torch.randint(0, 5000, (b, s), generator=torch.Generator().manual_seed(seed), dtype=torch.int32)
    if rd:
        rope = (sa.rope_table(rd, 5000, 10000.0, "cuda"), pos.cuda())
    out = sa.sparse_attn(q.cuda(), kv_dev, sink.cuda(), idx.cuda(), scale, kv_scale=kv_scale, rope=rope)
    got = u16(out).reshape(-1, h, d)
    assert np.all(np.isfinite(f32_of_u16(got)))
    ref = oracle.sparse_attn(u16(q), kv_ref.reshape(b, rows, d), sink.numpy(), idx.numpy(), scale)
    if rd:
        ref = oracle.apply_rotary(ref, rd, oracle.freqs_cis(rd, 5000, 10000.0), pos.view(-1).numpy(), inverse=True)
    assert_close(got, ref, f"sweep {seed}")


def test_strided_sequences(sa):
    """Per-sequence blocks inside larger buffers (non-packed sequence strides)."""
    q, kv, sink, idx = W.rand_problem(21, 3, 2, 32, 128, 50, 40, 0.1, False)
    qb = torch.zeros(3, 4, 32, 128, dtype=torch.bfloat16)
    qb[:, :2] = q
    kvb = torch.zeros(3, 70, 128, dtype=torch.bfloat16)
    kvb[:, :50] = kv
    ib = torch.full((3, 5, 40), -1, dtype=torch.int32)
    ib[:, :2] = idx
    qd, kvd, idd = qb.cuda(), kvb.cuda(), ib.cuda()
    outb = torch.zeros(3, 6, 32, 128, dtype=torch.bfloat16, device="cuda")
    sa.sparse_attn(qd[:, :2], kvd[:, :50], sink.cuda(), idd[:, :2], 0.088, out=outb[:, :2])
    ref = oracle.sparse_attn(u16(q), u16(kv), sink.numpy(), idx.numpy(), 0.088)
    assert_close(u16(outb[:, :2]).reshape(-1, 32, 128), ref, "strided")
    assert torch.all(outb[:, 2:] == 0)


@pytest.mark.parametrize("boost,where,fmt", [
    (0.0, 70, "bf16"),      # nothing special: scores within a few units of each other
    (4.0, 70, "bf16"),      # a late key ~45 log2 units above the first tile: second pass
    (13.0, 70, "bf16"),     # ~150 log2 units above: 2^150 would overflow without it
    (13.0, 3, "bf16"),      # the large key in the first tile: no second pass
    (-13.0, 70, "bf16"),    # a very negative late score
    (4.0, 70, "fp8"),
])
def test_late_large_scores(sa, boost, where, fmt):
    """Scores far above the first tile's maximum (kv row = boost * q of head 0): the
    softmax stays exact, including the second pass over the keys."""
    _say("late large", boost, where, fmt)
    q, kv, sink, idx = W.rand_problem(51, 1, 2, 16, 64, 120, 96, 0.0, False)
    for t in range(2):
        row = int(idx[0, t, where])
        kv[0, row] = (q[0, t, 0].float() * boost).to(torch.bfloat16)
    scale = 0.125
    kvd = kv.cuda()
    kv_scale = None
    if fmt == "fp8":
        kvd, kv_scale = sa.quant_kv_fp8(kvd, want=("codes", "scales"))
        kv_ref = oracle.act_quant(u16(kv).reshape(-1, 64))[0].reshape(kv.shape)
    else:
        kv_ref = u16(kv)
    out = sa.sparse_attn(q.cuda(), kvd, sink.cuda(), idx.cuda(), scale, kv_scale=kv_scale)
    assert torch.isfinite(out.float()).all()
    ref = oracle.sparse_attn(u16(q), kv_ref, sink.numpy(), idx.numpy(), scale)
    assert_close(u16(out).reshape(-1, 16, 64), ref, f"late large {boost} {where} {fmt}")


@pytest.mark.parametrize("seed,b,s,h,rows,topk,hole,boost", [
    (81, 1, 3, 16, 40, 20, 0.0, 0.0),       # one wave per workgroup, a single tile
    (82, 2, 2, 32, 100, 64, 0.3, 0.0),      # two waves, two tiles (the shortest pipeline)
    (83, 1, 4, 64, 200, 96, 0.1, 0.0),      # four waves, three tiles
    (84, 2, 3, 128, 500, 300, 0.5, 0.0),    # ten tiles, half the columns skipped
    (85, 1, 2, 64, 4000, 3200, 0.02, 0.0),  # more columns than one workgroup stages: splits
    (86, 1, 2, 48, 60, 50, 1.0, 0.0),       # every column skipped
    (87, 1, 3, 64, 300, 200, 0.0, 4.0),     # a late large score: the second key pass
    (88, 2, 1, 64, 1200, 1024, 0.05, 4.0),  # decode-shaped: two key groups, merge and second pass
    # enough workgroups to fill the GPU and rows named only a few times each: the pipelined
    # loop with in-kernel conversion (one and four waves), also with the second pass
    (89, 4, 64, 16, 2000, 200, 0.1, 0.0),
    (90, 2, 128, 64, 3000, 300, 0.2, 0.0),
    (91, 2, 130, 64, 3000, 300, 0.1, 4.0),
])
def test_fp8_pipeline(sa, seed, b, s, h, rows, topk, hole, boost):
    """fp8 storage at d = 512 converted inside the kernel (codes and scales gathered into raw
    slots ahead of the tile they fill and converted to bf16 tiles between the products, in the
    pipelined loop or, for short lists that leave compute units idle, by the key groups)
    against the oracle on the round-tripped rows."""
    _say("fp8 pipeline", seed, b, s, h, rows, topk, hole, boost)
    q, kv, sink, idx = W.rand_problem(seed, b, s, h, 512, rows, topk, hole, False)
    if boost:
        # a late row aligned with head 2's query: its score (about boost/2 * 0.8 * 512 raw,
        # 50 and more in log2 units) runs far past the first tile's reference, while its
        # values stay at +-boost/2 (P is rounded to bf16 for the PV product, an error of up to
        # 2^-9 of the largest |value| per output element)
        for t in range(s):
            col = topk - 5
            if idx[0, t, col] >= 0:
                kv[0, int(idx[0, t, col])] = (torch.sign(q[0, t, 2].float()) * (boost / 2)).to(torch.bfloat16)
    scale = float(np.float32(512 ** -0.5))
    codes, kv_scale = sa.quant_kv_fp8(kv.cuda(), want=("codes", "scales"))
    kv_ref = oracle.act_quant(u16(kv).reshape(-1, 512))[0].reshape(kv.shape)
    out = sa.sparse_attn(q.cuda(), codes, sink.cuda(), idx.cuda(), scale, kv_scale=kv_scale)
    ref = oracle.sparse_attn(u16(q), kv_ref, sink.numpy(), idx.numpy(), scale)
    assert_close(u16(out).reshape(-1, h, 512), ref, f"fp8 pipeline {seed}")


@pytest.mark.parametrize("d,plan", [(512, "key groups"), (256, "splits")])
def test_late_large_scores_across_splits(sa, d, plan):
    """A decode-shaped problem with few queries: at d = 512 the waves of a workgroup split the
    tiles between key groups (merged in LDS), at other widths the planner splits them across
    workgroups (f32 partials and a combine kernel). Large late scores sit in tiles of
    different groups or splits, so the second key pass and the merge meet."""
    _say("late large across", d, plan)
    q, kv, sink, idx = W.rand_problem(52, 2, 1, 64, d, 1200, 1024, 0.0, False)
    for b, col in ((0, 900), (1, 950)):
        row = int(idx[b, 0, col])
        kv[b, row] = (q[b, 0, 5].float() * 2.0).to(torch.bfloat16)
    scale = float(np.float32(d ** -0.5))
    args = sa.make_args(q.cuda(), kv.cuda(), sink.cuda(), idx.cuda(), scale, torch.empty_like(q.cuda()))
    ws = sa.sparse_attn_workspace_bytes(args)
    assert (ws > 0) == (plan == "splits"), f"expected a plan with {plan}"
    out = sa.sparse_attn(q.cuda(), kv.cuda(), sink.cuda(), idx.cuda(), scale)
    ref = oracle.sparse_attn(u16(q), u16(kv), sink.numpy(), idx.numpy(), scale)
    assert_close(u16(out).reshape(-1, 64, d), ref, f"late large {plan}")


@pytest.mark.parametrize("seed,b,h,topk,hole", [
    (71, 40, 128, 600, 0.1),     # 40 queries x 128 heads: two key groups of 32 heads
    (72, 30, 96, 700, 0.05),     # four key groups of 16 heads; 22 tiles, the last super tile half full
    (73, 6, 64, 520, 0.3),       # four key groups; 17 tiles, three groups idle in the last super tile
])
def test_key_groups(sa, seed, b, h, topk, hole):
    """Decode-shaped problems (one query per sequence, d = 512) with long key lists and few
    queries, which the planner gives to key groups (the waves of a workgroup share out each
    query's tiles) instead of splits; ragged tile counts leave groups idle at the end, and a
    query whose list names nothing leaves every group empty, and a query with a single tile
    leaves every group but the first without rows."""
    _say("key groups", seed, b, h, topk)
    q, kv, sink, idx = W.rand_problem(seed, b, 1, h, 512, 400, topk, hole, False)
    idx[b // 2, 0] = -1
    idx[b // 3, 0, 20:] = -1          # one tile only: the other key groups have no rows
    scale = float(np.float32(512 ** -0.5))
    args = sa.make_args(q.cuda(), kv.cuda(), sink.cuda(), idx.cuda(), scale, torch.empty_like(q.cuda()))
    assert sa.sparse_attn_workspace_bytes(args) == 0
    for sk in (sink, torch.full_like(sink, -math.inf)):
        out = sa.sparse_attn(q.cuda(), kv.cuda(), sk.cuda(), idx.cuda(), scale)
        o = out.float().cpu()
        assert torch.isfinite(o).all()
        assert torch.all(o[b // 2] == 0) or sk[0] != -math.inf
        ref = oracle.sparse_attn(u16(q), u16(kv), sk.numpy(), idx.numpy(), scale)
        assert_close(u16(out).reshape(-1, h, 512), ref, f"key groups {seed}")


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_key_groups_with_splits(sa, fmt):
    """A list longer than one workgroup stages (4500 columns: 4096 with bf16 storage, 3072
    with fp8) on a decode-shaped problem: key groups inside each workgroup and two splits
    merged by the combine kernel, with a late large score in the second split."""
    _say("key groups + splits", fmt)
    q, kv, sink, idx = W.rand_problem(74, 2, 1, 64, 512, 6000, 4500, 0.05, False)
    row = int(idx[1, 0, 4400]) if idx[1, 0, 4400] >= 0 else 0
    kv[1, row] = (q[1, 0, 7].float() * 2.0).to(torch.bfloat16)
    scale = float(np.float32(512 ** -0.5))
    kvd, kv_scale, kv_ref = kv.cuda(), None, u16(kv)
    if fmt == "fp8":
        kvd, kv_scale = sa.quant_kv_fp8(kvd, want=("codes", "scales"))
        kv_ref = oracle.act_quant(u16(kv).reshape(-1, 512))[0].reshape(kv.shape)
    args = sa.make_args(q.cuda(), kvd, sink.cuda(), idx.cuda(), scale, torch.empty_like(q.cuda()), kv_scale=kv_scale)
    assert sa.sparse_attn_workspace_bytes(args) > 0, "expected a plan with splits"
    out = sa.sparse_attn(q.cuda(), kvd, sink.cuda(), idx.cuda(), scale, kv_scale=kv_scale)
    ref = oracle.sparse_attn(u16(q), kv_ref, sink.numpy(), idx.numpy(), scale)
    assert_close(u16(out).reshape(-1, 64, 512), ref, f"key groups + splits {fmt}")


@pytest.mark.parametrize("seed,b,s,h,rows,topk,hole", [
    (91, 40, 1, 128, 900, 600, 0.1),   # key groups: decode-shaped, 40 queries x 128 heads
    (92, 2, 24, 64, 700, 300, 0.2),    # the pipelined loop, one head block per wave
    (93, 1, 256, 128, 300, 96, 0.3),   # the pipelined loop, two head blocks per wave
])
def test_skipped_columns_read_nothing(sa, seed, b, s, h, rows, topk, hole):
    """Every kv row that no index names holds NaN, row 0 among them: a skipped column (-1)
    must bring no row's values into the tile, so the output stays finite and matches the
    oracle (which reads named rows only)."""
    _say("skipped columns read nothing", seed, b, s, h)
    q, kv, sink, idx = W.rand_problem(seed, b, s, h, 512, rows, topk, hole, False)
    idx[idx == 0] = -1
    for bi in range(b):
        named = torch.zeros(rows, dtype=torch.bool)
        v = idx[bi].reshape(-1)
        named[v[v >= 0].long()] = True
        assert not named.all()
        kv[bi, ~named] = float("nan")
    scale = float(np.float32(512 ** -0.5))
    out = sa.sparse_attn(q.cuda(), kv.cuda(), sink.cuda(), idx.cuda(), scale)
    assert torch.isfinite(out.float()).all()
    ref = oracle.sparse_attn(u16(q), u16(kv), sink.numpy(), idx.numpy(), scale)
    assert_close(u16(out).reshape(-1, h, 512), ref, f"skipped columns {seed}")


def test_empty_lists_and_no_sink(sa):
    q, kv, sink, idx = W.rand_problem(31, 1, 3, 16, 64, 20, 40, 0.0, False)
    idx[0, 1] = -1
    idx[0, 2, 5:] = -9
    for sk in (sink, torch.full_like(sink, -math.inf)):
        out = sa.sparse_attn(q.cuda(), kv.cuda(), sk.cuda(), idx.cuda(), 0.125)
        o = out.float().cpu()
        assert torch.isfinite(o).all()
        assert torch.all(o[0, 1] == 0)
        ref = oracle.sparse_attn(u16(q), u16(kv), sk.numpy(), idx.numpy(), 0.125)
        assert_close(u16(out).reshape(-1, 16, 64), ref, "empty/no-sink")


def test_check_idx_flag(sa):
    q, kv, sink, idx = W.rand_problem(41, 1, 2, 16, 64, 20, 10, 0.0, False)
    bad = idx.clone()
    bad[0, 1, 3] = 20                      # == kv_rows: out of range
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = sa.sparse_attn(q.cuda(), kv.cuda(), sink.cuda(), bad.cuda(), 0.125, err_word=err, check_idx=True)
    assert int(err.item()) & 1
    skip = idx.clone()
    skip[0, 1, 3] = -1                     # the bad column is treated as a skip
    ref = oracle.sparse_attn(u16(q), u16(kv), sink.numpy(), skip.numpy(), 0.125)
    assert_close(u16(out).reshape(-1, 16, 64), ref, "check_idx")
    err.zero_()
    sa.sparse_attn(q.cuda(), kv.cuda(), sink.cuda(), idx.cuda(), 0.125, err_word=err, check_idx=True)
    assert int(err.item()) == 0


def test_deterministic_and_order_free(sa):
    w = W.small_variant("decode_compress")
    q, kv, _, sink, idx = gpu_inputs(w)
    a = sa.sparse_attn(q, kv, sink, idx, w.scale)
    b = sa.sparse_attn(q, kv, sink, idx, w.scale)
    assert torch.equal(a, b)
    perm = torch.randperm(idx.shape[-1], generator=torch.Generator().manual_seed(1)).cuda()
    c = sa.sparse_attn(q, kv, sink, idx[..., perm].contiguous(), w.scale)
    assert_close(u16(c), u16(a), "column order")


@pytest.mark.parametrize("name", ["decode_compress", "prefill_window"])
def test_graph_replays_match_eager(sa, name):
    """The step (window lists, then sparse_attn with the RoPE epilogue and, for the decode
    shape, a split plan and its combine) captured in a HIP graph and replayed several times,
    with new inputs copied in eagerly between replays: every replay equals an eager run on
    the same inputs, bit for bit."""
    w = W.small_variant(name)
    q, kv, _, sink, idx = gpu_inputs(w)
    table = sa.rope_table(w.rd, w.max_pos, w.rope_base, "cuda")
    pos = w.pos.cuda()
    sp = None if w.win_start_pos is None else w.win_start_pos.cuda()
    view = idx.view(w.win_nseq, w.win_seqlen, w.topk)
    args = sa.make_args(q, kv, sink, idx, w.scale, torch.empty_like(q), rope=(table, pos))
    nws = sa.sparse_attn_workspace_bytes(args)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device="cuda") if nws else None
    out = torch.empty_like(q)

    def step():
        sa.window_topk_idxs(w.window, w.win_seqlen, w.win_nseq, start_pos=sp, out=view)
        sa.sparse_attn(q, kv, sink, idx, w.scale, out=out, rope=(table, pos), workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(7)
    for r in range(4):
        q.copy_(torch.randn(q.shape, generator=gen).to(torch.bfloat16))
        if sp is not None:
            sp.copy_(torch.randint(w.window - 1, 4 * w.window, sp.shape, generator=gen, dtype=torch.int32))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref_idx = torch.empty_like(idx)
        if w.comp_idx is not None:
            ref_idx.copy_(idx)
        sa.window_topk_idxs(w.window, w.win_seqlen, w.win_nseq, start_pos=sp,
                            out=ref_idx.view(w.win_nseq, w.win_seqlen, w.topk))
        assert torch.equal(ref_idx, idx), f"replay {r}: index lists"
        ref = sa.sparse_attn(q, kv, sink, ref_idx, w.scale, rope=(table, pos))
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"replay {r}: output differs from the eager call"


# ------------------------------------------------------------------ rotary table
@pytest.mark.parametrize("rd,max_pos,base,yarn", [
    (16, 300, 10000.0, False), (64, 70000, 10000.0, False), (64, 70000, 160000.0, True),
    (128, 1000, 160000.0, True),
])
def test_rope_table_vs_oracle(sa, rd, max_pos, base, yarn):
    """sa_rope_table against the oracle's precompute_freqs_cis (f32 roundings of the page):
    the frequencies and angles agree bit for bit, so cos and sin differ by at most one f32
    rounding of the same angle."""
    kw = dict(original_seq_len=65536, factor=16.0, beta_fast=32.0, beta_slow=1.0) if yarn else {}
    got = sa.rope_table(rd, max_pos, base, "cuda", **kw).cpu().numpy()
    ref = oracle.freqs_cis(rd, max_pos, base, **kw)
    assert got.shape == ref.shape
    diff = np.abs(got.astype(np.float64) - ref)
    assert diff.max() <= 6e-8, diff.max()
    # the oracle's libm cosf/sinf are within one ulp of the correctly rounded value
    assert (diff == 0).mean() > 0.95


# ------------------------------------------------------------------ full sizes
def _full_selection(w):
    """Every query of the decode workloads; for the prefills 72 (64) queries: 9 (8) per XCD
    slot of the kernel's work order (a query's slot is its index mod 8), from the first
    queries (short, partly -1 lists) to the last (the longest lists)."""
    nq = w.b * w.s
    if nq <= 64:
        return np.arange(nq, dtype=np.int64)
    ks = [0, 2, 7, 15, 40, 200, 511, 700, 1023] if nq >= 8192 else [0, 2, 7, 15, 40, 200, 400, 511]
    sel = np.array(sorted(8 * k + r for k in ks for r in range(8) if 8 * k + r < nq), np.int64)
    assert set(sel % 8) == set(range(8))
    return sel


_FULL = {}


def _full(name):
    """(workload, selection, oracle core of the selection); one workload cached at a time."""
    if name not in _FULL:
        _FULL.clear()
        w = W.make(name)
        sel = _full_selection(w)
        core = oracle_core(w, qsel=sel)
        _FULL[name] = (w, sel, core)
    return _FULL[name]


FULL_CASES = [(n, f, r) for n in ("decode_window", "decode_compress", "prefill_window", "prefill_compress")
              for f, r in (("bf16", True), ("bf16", False), ("fp8", True))]


@pytest.mark.parametrize("name,fmt,rope", FULL_CASES)
def test_full_size(sa, name, fmt, rope):
    """The workload at full size in the launch configuration the bench times (bf16 storage
    with the epilogue), and also without the epilogue and with fp8 storage: index lists bit
    for bit, the whole output finite, and the selected queries against the oracle."""
    w, sel, core = _full(name)
    _say("full", name, fmt, "rope" if rope else "no epilogue", f"{sel.size} queries")
    out, idx = gpu_run(w, fmt, rope)
    assert np.array_equal(idx.cpu().numpy(), oracle_indices(w))
    assert bool(torch.isfinite(out.float()).all()), "non-finite output"
    got = u16(out.view(-1, w.h, w.d)[torch.from_numpy(sel).cuda()])
    ref = oracle_rotate(w, core, sel) if rope else core
    assert_close(got, ref, f"full {name} {fmt} rope={rope}")
    del out, idx
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ edge cases of the softmax
@pytest.mark.parametrize("d,b,s,h,topk,empty,want_ws", [
    (64, 1, 3, 16, 64, [(0, 32)], False),              # pipelined loop, a leading empty tile
    (512, 2, 3, 64, 160, [(0, 64)], False),            # d = 512, two leading empty tiles
    (512, 1, 160, 256, 96, [(0, 32)], False),          # two head blocks per wave
    (256, 2, 1, 64, 1024, [(0, 256)], True),           # four splits, split 0 (the sink's) empty
    (256, 2, 1, 64, 1024, [(512, 768)], True),         # a middle split empty
])
def test_no_sink_with_empty_tiles(sa, d, b, s, h, topk, empty, want_ws):
    """sink = -inf (no sink) with tiles or whole splits whose columns are all -1 ahead of the
    rows: the empty tiles and splits contribute exactly nothing (no NaN from -inf - -inf)."""
    _say("no sink, empty tiles", d, b, s, h, topk, empty)
    q, kv, sink, idx = W.rand_problem(110 + d + topk, b, s, h, d, 4 * topk, topk, 0.05, False)
    for lo, hi in empty:
        idx[..., lo:hi] = -1
    sk = torch.full_like(sink, -math.inf)
    scale = float(np.float32(d ** -0.5))
    args = sa.make_args(q.cuda(), kv.cuda(), sk.cuda(), idx.cuda(), scale, torch.empty_like(q.cuda()))
    assert (sa.sparse_attn_workspace_bytes(args) > 0) == want_ws
    out = sa.sparse_attn(q.cuda(), kv.cuda(), sk.cuda(), idx.cuda(), scale)
    assert bool(torch.isfinite(out.float()).all())
    ref = oracle.sparse_attn(u16(q), u16(kv), sk.numpy(), idx.numpy(), scale)
    assert_close(u16(out).reshape(-1, h, d), ref, f"no sink {d} {empty}")


def test_no_sink_key_group_without_rows_in_second_pass(sa):
    """Key groups (decode-shaped, d = 512): every tile of key group 0 is empty while a late
    large score in group 1 triggers the second pass over the keys; with no sink, group 0 must
    still contribute exactly nothing to the merge."""
    q, kv, sink, idx = W.rand_problem(121, 2, 1, 64, 512, 1200, 1024, 0.0, False)
    for t0 in range(0, 1024, 128):                      # tiles 0, 4, 8, ... (four key groups)
        idx[..., t0:t0 + 32] = -1
    for bb in range(2):
        row = int(idx[bb, 0, 5 * 32 + 3])               # tile 5: group 1's second tile
        kv[bb, row] = (q[bb, 0, 5].float() * 2.0).to(torch.bfloat16)
    sk = torch.full_like(sink, -math.inf)
    scale = float(np.float32(512 ** -0.5))
    args = sa.make_args(q.cuda(), kv.cuda(), sk.cuda(), idx.cuda(), scale, torch.empty_like(q.cuda()))
    assert sa.sparse_attn_workspace_bytes(args) == 0, "expected the key-group plan"
    for s_ in (sk, sink):
        out = sa.sparse_attn(q.cuda(), kv.cuda(), s_.cuda(), idx.cuda(), scale)
        assert bool(torch.isfinite(out.float()).all())
        ref = oracle.sparse_attn(u16(q), u16(kv), s_.numpy(), idx.numpy(), scale)
        assert_close(u16(out).reshape(-1, 64, 512), ref, "key group 0 empty")


@pytest.mark.parametrize("d,b,s,h,topk", [
    (64, 1, 4, 16, 40),         # one workgroup per query, epilogue in the key-loop kernel
    (512, 2, 2, 64, 1024),      # key groups, the merged epilogue
    (256, 2, 2, 64, 1024),      # splits: the combine kernel runs the epilogue
])
def test_check_idx_reports_positions_outside_the_table(sa, d, b, s, h, topk):
    """With the epilogue on, a query whose position has no row in the (cos, sin) table is
    left unrotated and, with SA_FLAG_CHECK_IDX, sets bit value 2 of the error word; the other
    queries are rotated as usual."""
    _say("check_idx positions", d, b, s, h, topk)
    q, kv, sink, idx = W.rand_problem(130 + d, b, s, h, d, 2000, topk, 0.1, False)
    rd, max_pos = min(64, d // 4), 50
    pos = torch.arange(b * s, dtype=torch.int32).view(b, s) * 7 % max_pos
    bad = [(b - 1, s - 1, max_pos), (0, 0, -3)] if b * s > 1 else [(0, 0, max_pos)]
    for bb, tt, v in bad:
        pos[bb, tt] = v
    scale = float(np.float32(d ** -0.5))
    table = sa.rope_table(rd, max_pos, 10000.0, "cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = sa.sparse_attn(q.cuda(), kv.cuda(), sink.cuda(), idx.cuda(), scale, rope=(table, pos.cuda()),
                         err_word=err, check_idx=True)
    assert int(err.item()) == 2
    core = oracle.sparse_attn(u16(q), u16(kv), sink.numpy(), idx.numpy(), scale)
    cs = oracle.freqs_cis(rd, max_pos, 10000.0)
    flat = pos.view(-1).numpy()
    ok = (flat >= 0) & (flat < max_pos)
    ref = core.copy()
    ref[ok] = oracle.apply_rotary(core[ok], rd, cs, flat[ok], inverse=True)
    assert_close(u16(out).reshape(-1, h, d), ref, "positions outside the table")
    # without the flag the rows are the same and nothing is reported
    err.zero_()
    out2 = sa.sparse_attn(q.cuda(), kv.cuda(), sink.cuda(), idx.cuda(), scale, rope=(table, pos.cuda()))
    assert torch.equal(out, out2) and int(err.item()) == 0


@pytest.mark.parametrize("seed,b,s,h,d,rows,topk,hole,dup", [
    (101, 2, 3, 16, 64, 50, 40, 0.2, True),
    (102, 1, 4, 48, 128, 300, 200, 0.1, False),
    (103, 2, 2, 64, 256, 100, 64, 0.3, True),
    (104, 1, 2, 32, 256, 3000, 2500, 0.05, False),     # splits and the combine kernel
    (105, 3, 2, 100, 128, 900, 700, 0.5, False),
])
def test_fp8_storage_other_head_dims(sa, seed, b, s, h, d, rows, topk, hole, dup):
    """fp8 storage (e4m3 codes + block-32 scale bytes) at head dims 64, 128 and 256, where the
    tiles are converted by a plain loop, against the oracle on the round-tripped rows, with
    the epilogue on."""
    _say("fp8 other d", seed, d, topk)
    q, kv, sink, idx = W.rand_problem(seed, b, s, h, d, rows, topk, hole, dup)
    scale = float(np.float32(d ** -0.5))
    codes, kv_scale = sa.quant_kv_fp8(kv.cuda(), want=("codes", "scales"))
    kv_ref = oracle.act_quant(u16(kv).reshape(-1, d))[0].reshape(kv.shape)
    rd = d // 4
    pos = torch.randint(0, 3000, (b, s), generator=torch.Generator().manual_seed(seed), dtype=torch.int32)
    table = sa.rope_table(rd, 3000, 10000.0, "cuda")
    out = sa.sparse_attn(q.cuda(), codes, sink.cuda(), idx.cuda(), scale, kv_scale=kv_scale,
                         rope=(table, pos.cuda()))
    core = oracle.sparse_attn(u16(q), kv_ref, sink.numpy(), idx.numpy(), scale)
    ref = oracle.apply_rotary(core, rd, oracle.freqs_cis(rd, 3000, 10000.0), pos.view(-1).numpy(), inverse=True)
    assert_close(u16(out).reshape(-1, h, d), ref, f"fp8 d={d}")


@pytest.mark.parametrize("seed,b,s,h,d,rows,topk,hole,dup", [
    (111, 2, 64, 32, 512, 96, 80, 0.1, False),       # bf16 kernels on the dequantised rows
    (112, 1, 40, 64, 128, 50, 45, 0.2, True),
    (113, 2, 2, 16, 256, 300, 5000, 0.05, True),     # dequantised rows and split partials
])
def test_fp8_dequantised_rows_plan(sa, seed, b, s, h, d, rows, topk, hole, dup):
    """fp8 storage whose rows are each named by many (query, column) pairs: the plan turns the
    cache into bf16 rows in the workspace first (reported by the workspace query) and runs the
    bf16 kernels on them; against the oracle on the round-tripped rows, epilogue on."""
    _say("fp8 dequantised rows", seed, d, rows, topk)
    q, kv, sink, idx = W.rand_problem(seed, b, s, h, d, rows, topk, hole, dup)
    scale = float(np.float32(d ** -0.5))
    codes, kv_scale = sa.quant_kv_fp8(kv.cuda(), want=("codes", "scales"))
    rd = 64 if d == 512 else d // 4
    pos = torch.randint(0, 3000, (b, s), generator=torch.Generator().manual_seed(seed), dtype=torch.int32)
    table = sa.rope_table(rd, 3000, 10000.0, "cuda")
    out = torch.empty_like(q, device="cuda")
    args = sa.make_args(q.cuda(), codes, sink.cuda(), idx.cuda(), scale, out, kv_scale=kv_scale,
                        rope=(table, pos.cuda()))
    assert sa.sparse_attn_workspace_bytes(args) >= b * rows * d * 2
    out = sa.sparse_attn(q.cuda(), codes, sink.cuda(), idx.cuda(), scale, kv_scale=kv_scale,
                         rope=(table, pos.cuda()))
    kv_ref = oracle.act_quant(u16(kv).reshape(-1, d))[0].reshape(kv.shape)
    core = oracle.sparse_attn(u16(q), kv_ref, sink.numpy(), idx.numpy(), scale)
    ref = oracle.apply_rotary(core, rd, oracle.freqs_cis(rd, 3000, 10000.0), pos.view(-1).numpy(), inverse=True)
    assert_close(u16(out).reshape(-1, h, d), ref, f"fp8 dequantised rows {seed}")


# ------------------------------------------------------------------ fused window lists
def _fused_case(w, fmt):
    """(explicit output, fused output, idx with the window columns poisoned)."""
    import sparse_latent_attention_attn_amd as sa
    q, kv, kv_scale, sink, idx = gpu_inputs(w, fmt)
    pos = w.pos.cuda()
    table = sa.rope_table(w.rd, w.max_pos, w.rope_base, "cuda")
    ref = sa.sparse_attn(q, kv, sink, idx, w.scale, kv_scale=kv_scale, rope=(table, pos))
    poisoned = idx.clone()
    poisoned[..., :w.win_cols] = 10 ** 9                   # never read in the fused mode
    mode = "chunk" if w.win_start_pos is None else "ring"
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = sa.sparse_attn(q, kv, sink, poisoned, w.scale, kv_scale=kv_scale, rope=(table, pos),
                         window=(w.window, mode, pos), err_word=err, check_idx=True)
    torch.cuda.synchronize()
    assert int(err.item()) == 0, "a window column was read from idx"
    return ref, got


@pytest.mark.parametrize("name", ["decode_window", "prefill_window", "decode_compress", "prefill_compress"])
@pytest.mark.parametrize("size", ["small", "full"])
def test_fused_window_lists_equal_explicit_lists(sa, name, size):
    """The window lists generated inside sparse_attn from the positions (ring lists for the
    decode workloads and the long prefill's per-query lists, chunk lists for the window-only
    prefill) give the same output, bit for bit, as the lists of sa_window_topk_idxs."""
    _say("fused window", name, size)
    w = W.small_variant(name) if size == "small" else W.make(name)
    for fmt in (("bf16", "fp8") if size == "small" else ("bf16",)):
        ref, got = _fused_case(w, fmt)
        assert torch.equal(ref.view(torch.int16), got.view(torch.int16)), f"{name} {fmt}"


def test_fused_ring_with_unreached_slots(sa):
    """Fused ring lists (128 slots, two key groups at d 512) at positions before, at and past
    the ring's first tiles, with every slot the position has not reached holding NaN: the
    output matches the oracle on the lists of sa_window_topk_idxs and is finite."""
    b, h, d, window = 8, 64, 512, 128
    q, kv, sink, _ = W.rand_problem(161, b, 1, h, d, window, window, 0.0, False)
    pos = torch.tensor([0, 5, 31, 40, 62, 63, 64, 500], dtype=torch.int32).view(b, 1)
    for bi in range(b):
        p = int(pos[bi, 0])
        if p + 1 < window:
            kv[bi, p + 1:] = float("nan")
    win = oracle.window_topk_idxs(window, 1, pos.view(-1).numpy())
    full = torch.from_numpy(win.reshape(b, 1, window))
    poisoned = torch.full((b, 1, window), 10 ** 9, dtype=torch.int32)
    rd = 64
    table = sa.rope_table(rd, 1024, 10000.0, "cuda")
    posd = pos.cuda()
    scale = float(np.float32(d ** -0.5))
    out = sa.sparse_attn(q.cuda(), kv.cuda(), sink.cuda(), poisoned.cuda(), scale, rope=(table, posd),
                         window=(window, "ring", posd))
    got = u16(out).reshape(-1, h, d)
    assert np.all(np.isfinite(f32_of_u16(got)))
    core = oracle.sparse_attn(u16(q), u16(kv), sink.numpy(), full.numpy(), scale)
    ref = oracle.apply_rotary(core, rd, oracle.freqs_cis(rd, 1024, 10000.0), pos.view(-1).numpy(), inverse=True)
    assert_close(got, ref, "ring with unreached slots")


def test_fused_window_across_splits_and_against_oracle(sa):
    """A 300-slot ring list inside 4500-column lists (split plans: the generated columns run
    into the second split), d = 256, and a chunk list at d = 64, against the oracle."""
    for d, window, mode, topk, rows in ((256, 300, "ring", 4500, 6000), (64, 40, "chunk", 40, 90)):
        _say("fused window splits", d, window, mode)
        b, s, h = (2, 1, 32) if mode == "ring" else (1, 90, 16)
        q, kv, sink, idx = W.rand_problem(140 + d, b, s, h, d, rows, topk, 0.05, False)
        if mode == "ring":
            pos = torch.tensor([[70000], [123]], dtype=torch.int32)
            win = oracle.window_topk_idxs(window, 1, pos.view(-1).numpy())
        else:
            pos = torch.arange(s, dtype=torch.int32).view(1, s)
            win = oracle.window_topk_idxs(window, s)
        ncol = win.shape[-1]
        full = idx.clone()
        full[..., :ncol] = torch.from_numpy(win.reshape(b, s, ncol))
        rd = d // 4
        table = sa.rope_table(rd, 70001, 10000.0, "cuda")
        posd = pos.cuda()
        out = sa.sparse_attn(q.cuda(), kv.cuda(), sink.cuda(), idx.cuda(), float(np.float32(d ** -0.5)),
                             rope=(table, posd), window=(window, mode, posd))
        core = oracle.sparse_attn(u16(q), u16(kv), sink.numpy(), full.numpy(), float(np.float32(d ** -0.5)))
        ref = oracle.apply_rotary(core, rd, oracle.freqs_cis(rd, 70001, 10000.0), pos.view(-1).numpy(), inverse=True)
        assert_close(u16(out).reshape(-1, h, d), ref, f"fused {mode}")
