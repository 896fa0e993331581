"""Pins of the oracle's window index lists, ring writes, sparse_attn and rotary epilogue:
the ring-cache worked example of the attention API docs (tests/golden), brute force by an
independent formulation, closed forms, and reductions to torch routines. CPU only."""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import sa_workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, *v = line.split()
        out[k] = [int(x) for x in v]
    return out


def _u16(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _f32(u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).float()


# ------------------------------------------------------------------ window indices / ring
def test_ring_cache_worked_example(orc):
    """The 12-tokens-into-8-slots example, followed with one ring through all three regimes."""
    g = _golden("ring_cache_12_into_8.txt")
    Wn, S = g["window"][0], g["prefill_tokens"][0]
    # token t's kv row is the constant row t, so the ring contents read back as tokens
    rows = np.repeat(np.arange(16, dtype=np.uint16)[:, None], 4, axis=1)
    ring = np.full((Wn, 4), 0xFFFF, np.uint16)
    orc.ring_prefill(ring, rows[:S])
    assert ring[:, 0].tolist() == g["ring_after_prefill"]
    # prefill lists: one causal window per query into the chunk
    idx = orc.window_topk_idxs(Wn, S)[0]
    assert idx.shape == (S, Wn)
    assert idx[0].tolist() == [0] + [-1] * 7
    assert idx[3].tolist() == [0, 1, 2, 3] + [-1] * 4
    assert idx[7].tolist() == list(range(8))
    assert idx[11].tolist() == list(range(4, 12))
    for P, key in ((12, "decode_12"), (13, "decode_13")):
        orc.ring_decode(ring, rows[P], P)
        assert P % Wn == g[key + "_writes_slot"][0]
        assert ring[:, 0].tolist() == g["ring_after_" + key]
        lst = orc.window_topk_idxs(Wn, 1, [P])[0, 0]
        assert lst.tolist() == g[key + "_reads_slots"]
        # oldest first: the tokens read are strictly increasing and end with P
        toks = ring[lst, 0].astype(int).tolist()
        assert toks == sorted(toks) and toks[-1] == P and len(set(toks)) == Wn


def _simulate_ring(window, P):
    """Independent formulation: write tokens 0..P one by one into slot t mod window; the
    decode list is the occupied slots ordered by the token they hold, -1 padded."""
    holder = [-1] * window
    for t in range(P + 1):
        holder[t % window] = t
    occ = sorted((tok, slot) for slot, tok in enumerate(holder) if tok >= 0)
    return [slot for _, slot in occ] + [-1] * (window - len(occ))


def test_decode_lists_brute_force(orc):
    for window in range(1, 17):
        for P in range(0, 64):
            got = orc.window_topk_idxs(window, 1, [P])[0, 0].tolist()
            assert got == _simulate_ring(window, P), (window, P)
    # several sequences at their own positions in one call
    Ps = [1, 5, 7, 8, 100, 0]
    got = orc.window_topk_idxs(8, 1, Ps)
    for n, P in enumerate(Ps):
        assert got[n, 0].tolist() == _simulate_ring(8, P)


def test_prefill_lists_brute_force(orc):
    for window in (1, 3, 8, 16):
        for S in (2, 5, 8, 17, 40):
            got = orc.window_topk_idxs(window, S, nseq=2)
            cols = min(S, window)
            assert got.shape == (2, S, cols)
            for t in range(S):
                visible = [j for j in range(S) if t - window < j <= t]
                assert got[0, t].tolist() == visible + [-1] * (cols - len(visible))
            assert np.array_equal(got[0], got[1])


def test_window_rejects_chunked_prefill(orc):
    with pytest.raises(ValueError):
        orc.window_topk_idxs(8, 4, [3])
    with pytest.raises(ValueError):
        orc.window_topk_idxs(0, 4)
    with pytest.raises(ValueError):
        orc.window_topk_idxs(8, 1, [-1])


# ------------------------------------------------------------------ sparse_attn
def _sdpa_reference(q, kv, sink, idx, scale, dtype=torch.float64):
    """sparse_attn written as torch's scaled_dot_product_attention over the gathered rows
    plus one appended all-zero key/value whose additive bias is the sink: its score is
    exactly the sink, and it adds nothing to the weighted sum."""
    b, s, h, d = q.shape
    out = torch.zeros(b, s, h, d, dtype=dtype)
    for bi in range(b):
        for t in range(s):
            sel = [int(j) for j in idx[bi, t] if j >= 0]
            rows = kv[bi, sel].to(dtype)
            keys = torch.cat([rows, torch.zeros(1, d, dtype=dtype)], 0)
            bias = torch.zeros(h, 1, keys.shape[0], dtype=dtype)
            bias[:, 0, -1] = sink.to(dtype)
            o = F.scaled_dot_product_attention(q[bi, t].to(dtype).unsqueeze(1), keys.unsqueeze(0),
                                               keys.unsqueeze(0), attn_mask=bias, scale=scale)
            out[bi, t] = o[:, 0]
    return out


@pytest.mark.parametrize("seed,b,s,h,d,rows,topk,hole,dup", [
    (0, 1, 3, 4, 64, 16, 16, 0.2, False),
    (1, 2, 2, 3, 32, 9, 12, 0.3, True),
    (2, 1, 1, 8, 64, 40, 7, 0.0, False),
    (3, 3, 1, 2, 16, 5, 5, 0.5, True),
])
def test_sparse_attn_vs_sdpa(orc, seed, b, s, h, d, rows, topk, hole, dup):
    q, kv, sink, idx = W.rand_problem(seed, b, s, h, d, rows, topk, hole, dup)
    scale = float(np.float32(d ** -0.5))          # the oracle takes the scale as an f32
    ref = _sdpa_reference(q, kv, sink, idx, scale)
    o64 = orc.sparse_attn_f64(_u16(q), _u16(kv), sink.numpy(), idx.numpy(), scale)
    assert np.allclose(o64.reshape(ref.shape), ref.numpy(), rtol=1e-12, atol=1e-13)
    o = _f32(orc.sparse_attn(_u16(q), _u16(kv), sink.numpy(), idx.numpy(), scale))
    # the f32 path, rounded once to bf16: within a bf16 half-ulp plus f32 summation error
    assert torch.allclose(o.reshape(ref.shape).double(), ref, rtol=2 ** -8, atol=1e-6)


def test_sink_only_in_denominator(orc):
    """sum_j p_j < 1 and 1 - sum_j p_j = e^sink / (sum_j e^s_j + e^sink)."""
    q, kv, sink, idx = W.rand_problem(7, 1, 2, 4, 64, 32, 24, 0.25, False)
    scale = 0.125
    for qi in range(2):
        for hh in range(4):
            w, share = orc.sparse_attn_weights_f64(_u16(q), _u16(kv), sink.numpy(), idx.numpy(),
                                                   scale, qi, hh)
            sel = [int(j) for j in idx[0, qi] if j >= 0]
            sc = (q[0, qi, hh].double() @ kv[0, sel].double().T) * scale
            closed = math.exp(sink[hh]) / (torch.exp(sc).sum().item() + math.exp(sink[hh]))
            assert w.sum() < 1.0
            assert abs((1.0 - w.sum()) - closed) < 1e-12 and abs(share - closed) < 1e-12


def test_constant_rows_and_zero_query(orc):
    h, d, rows, topk = 4, 64, 10, 8
    g = torch.Generator().manual_seed(3)
    u = torch.randn(d, generator=g).to(torch.bfloat16)
    q = torch.randn(1, 1, h, d, generator=g).to(torch.bfloat16)
    sink = torch.randn(h, generator=g)
    kv = u.view(1, 1, d).expand(1, rows, d).contiguous()
    idx = torch.tensor([[[0, 3, -1, 5, 5, 9, -1, 2]]], dtype=torch.int32)
    n = 6
    o = orc.sparse_attn_f64(_u16(q), _u16(kv), sink.numpy(), idx.numpy(), 0.125)[0]
    s_ = (q[0, 0].double() @ u.double()) * 0.125               # same score for every row
    factor = n * torch.exp(s_) / (n * torch.exp(s_) + torch.exp(sink.double()))
    assert np.allclose(o, (factor[:, None] * u.double()[None]).numpy(), rtol=1e-12, atol=1e-14)
    # q = 0: every score is 0, so o = sum_j kv_j / (|J| + e^sink)
    q0 = torch.zeros(1, 1, h, d, dtype=torch.bfloat16)
    kv2 = torch.randn(1, rows, d, generator=g).to(torch.bfloat16)
    o = orc.sparse_attn_f64(_u16(q0), _u16(kv2), sink.numpy(), idx.numpy(), 0.125)[0]
    sel = [0, 3, 5, 5, 9, 2]
    expect = kv2[0, sel].double().sum(0)[None] / (n + torch.exp(sink.double()))[:, None]
    assert np.allclose(o, expect.numpy(), rtol=1e-12, atol=1e-14)


def test_no_sink_is_plain_attention(orc):
    q, kv, sink, idx = W.rand_problem(9, 1, 2, 4, 64, 30, 20, 0.2, False)
    sink = torch.full((4,), -math.inf)
    o = orc.sparse_attn_f64(_u16(q), _u16(kv), sink.numpy(), idx.numpy(), 0.125)
    for t in range(2):
        sel = [int(j) for j in idx[0, t] if j >= 0]
        K = kv[0, sel].double()
        ref = F.scaled_dot_product_attention(q[0, t].double().unsqueeze(1), K[None], K[None],
                                             scale=0.125)[:, 0]
        assert np.allclose(o[t], ref.numpy(), rtol=1e-12, atol=1e-14)


def test_empty_selection_gives_zero(orc):
    q, kv, sink, idx = W.rand_problem(5, 1, 3, 2, 32, 8, 6, 0.0, False)
    idx[0, 1] = -1
    idx[0, 2, :] = -7                       # any negative index is a skip
    o = orc.sparse_attn(_u16(q), _u16(kv), sink.numpy(), idx.numpy(), 0.2)
    assert np.all(o[1] == 0) and np.all(o[2] == 0) and np.any(o[0] != 0)
    o = orc.sparse_attn(_u16(q), _u16(kv), np.full(2, -np.inf, np.float32), idx.numpy(), 0.2)
    assert np.all(o[1] == 0)


def test_f32_oracle_close_to_f64_and_order_free(orc):
    q, kv, sink, idx = W.rand_problem(11, 2, 4, 4, 64, 64, 48, 0.15, True)
    o32 = _f32(orc.sparse_attn(_u16(q), _u16(kv), sink.numpy(), idx.numpy(), 0.125)).double()
    o64 = torch.from_numpy(orc.sparse_attn_f64(_u16(q), _u16(kv), sink.numpy(), idx.numpy(), 0.125))
    assert torch.allclose(o32, o64, rtol=2 ** -8, atol=1e-6)
    perm = torch.randperm(48, generator=torch.Generator().manual_seed(0))
    o64p = orc.sparse_attn_f64(_u16(q), _u16(kv), sink.numpy(), idx[..., perm].contiguous().numpy(), 0.125)
    assert np.allclose(o64p, o64.numpy(), rtol=1e-12, atol=1e-14)


def test_query_subset_matches_full(orc):
    q, kv, sink, idx = W.rand_problem(12, 2, 5, 3, 32, 20, 10, 0.1, False)
    full = orc.sparse_attn(_u16(q), _u16(kv), sink.numpy(), idx.numpy(), 0.3)
    sel = np.array([9, 0, 4, 5], np.int64)
    part = orc.sparse_attn(_u16(q), _u16(kv), sink.numpy(), idx.numpy(), 0.3, qsel=sel)
    assert np.array_equal(part, full[sel])


def test_out_of_range_index_rejected(orc):
    q, kv, sink, idx = W.rand_problem(13, 1, 1, 2, 32, 8, 4, 0.0, False)
    idx[0, 0, 1] = 8
    with pytest.raises(ValueError):
        orc.sparse_attn(_u16(q), _u16(kv), sink.numpy(), idx.numpy(), 0.3)


# ------------------------------------------------------------------ rotary epilogue
def test_freqs_table(orc):
    rd, n = 16, 300
    cs = orc.freqs_cis(rd, n, 10000.0).astype(np.float64)
    assert np.all(cs[0, :, 0] == 1.0) and np.all(cs[0, :, 1] == 0.0)
    # pair 0 has frequency 1: its angle is the position itself
    ang = np.arange(n, dtype=np.float64)
    assert np.allclose(cs[:, 0, 0], np.cos(ang), atol=2e-6)
    assert np.allclose(cs[:, 0, 1], np.sin(ang), atol=2e-6)
    # pair i at position 1 has angle base^(-2i/rd)
    theta = 10000.0 ** (-np.arange(0, rd, 2) / rd)
    assert np.allclose(np.arctan2(cs[1, :, 1], cs[1, :, 0]), theta, atol=1e-6)
    assert np.allclose(cs[..., 0] ** 2 + cs[..., 1] ** 2, 1.0, atol=1e-6)


def test_rotary_vs_complex_multiply(orc):
    """The printed formula, evaluated by torch: view pairs as complex, multiply by
    freqs_cis (conjugated for the inverse), back to bf16."""
    g = torch.Generator().manual_seed(4)
    n, h, d, rd = 6, 3, 64, 16
    x = torch.randn(n, h, d, generator=g).to(torch.bfloat16)
    pos = torch.tensor([0, 1, 5, 77, 1000, 4095], dtype=torch.int32)
    cs = orc.freqs_cis(rd, 4096, 10000.0)
    fc = torch.complex(torch.from_numpy(cs[..., 0]), torch.from_numpy(cs[..., 1]))
    for inverse in (False, True):
        got = _f32(orc.apply_rotary(_u16(x), rd, cs, pos.numpy(), inverse))
        f = fc[pos.long()].conj() if inverse else fc[pos.long()]
        xc = torch.view_as_complex(x[..., -rd:].float().unflatten(-1, (-1, 2)).contiguous())
        rot = torch.view_as_real(xc * f[:, None, :]).flatten(-2).to(torch.bfloat16).float()
        assert torch.equal(got[..., :-rd], x[..., :-rd].float())
        diff = (got[..., -rd:] - rot).abs()
        ulp = rot.abs().clamp_min(1e-30) * 2 ** -7
        assert torch.all(diff <= ulp)                 # at most one bf16 ulp (FMA in torch)
        assert (diff == 0).float().mean() > 0.99


def test_rotary_identity_and_inverse(orc):
    g = torch.Generator().manual_seed(5)
    x = torch.randn(4, 2, 64, generator=g).to(torch.bfloat16)
    cs = orc.freqs_cis(16, 100, 10000.0)
    assert np.array_equal(orc.apply_rotary(_u16(x), 16, cs, np.zeros(4, np.int32), True), _u16(x))
    assert np.array_equal(orc.apply_rotary(_u16(x), 0, cs, np.zeros(4, np.int32), True), _u16(x))
    pos = np.array([3, 17, 50, 99], np.int32)
    fw = orc.apply_rotary(_u16(x), 16, cs, pos, False)
    back = _f32(orc.apply_rotary(fw, 16, cs, pos, True))
    assert torch.allclose(back, x.float(), rtol=2 ** -6, atol=2 ** -6)
    # a rotation keeps each pair's length (up to two bf16 roundings)
    a = _f32(fw)[..., -16:].unflatten(-1, (-1, 2)).norm(dim=-1)
    b = x.float()[..., -16:].unflatten(-1, (-1, 2)).norm(dim=-1)
    assert torch.allclose(a, b, rtol=2 ** -6, atol=1e-6)
