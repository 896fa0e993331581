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


# ------------------------------------------------------------------ indexer (compressed top-k)
def _index_inputs(seed, b, s, h, d, n_pos, integer=False):
    g = torch.Generator().manual_seed(seed)
    if integer:
        q = torch.randint(-3, 4, (b, s, h, d), generator=g).float()
        k = torch.randint(-3, 4, (b, n_pos, d), generator=g).float()
        w = 2.0 ** torch.randint(-2, 2, (b, s, h), generator=g).float()
    else:
        q = torch.randn(b, s, h, d, generator=g)
        k = torch.randn(b, n_pos, d, generator=g)
        w = torch.randn(b, s, h, generator=g) * (d ** -0.5 * h ** -0.5)
    qb, kb = q.to(torch.bfloat16), k.to(torch.bfloat16)
    return (qb.view(torch.int16).numpy().view(np.uint16), kb.view(torch.int16).numpy().view(np.uint16),
            w.numpy().astype(np.float32), qb.double(), kb.double(), w.double())


def test_index_scores_vs_einsum(orc):
    """The indexer's score as torch evaluates the page's einsum, in f64: relu(q . k) times
    the head weights, summed over heads; -inf beyond each query's (pos+1)//ratio visible
    positions and outside the candidate mask."""
    b, s, h, d, n_pos, ratio = 2, 7, 8, 64, 40, 4
    q, k, w, qd, kd, wd = _index_inputs(1, b, s, h, d, n_pos)
    pos = np.array([[0, 3, 4, 50, 100, 159, 200], [7, 8, 9, 10, 11, 12, 300]], np.int32)
    cand = (np.random.default_rng(2).random((b, s, n_pos)) < 0.7).astype(np.uint8)
    got = orc.index_scores(q, k, w, pos, ratio, cand)
    ref = (torch.einsum("bshd,btd->bsht", qd, kd).relu() * wd[..., None]).sum(2).numpy()
    vis = np.minimum((pos + 1) // ratio, n_pos)
    t = np.arange(n_pos)
    live = (t[None, None, :] < vis[..., None]) & (cand == 1)
    assert np.all(np.isneginf(got[~live]))
    assert np.allclose(got[live], ref[live], rtol=1e-5, atol=1e-6)


def _rank_select(scores, topk):
    """Brute force by ranks: a finite position is chosen when fewer than topk positions beat
    it (a higher score, or the same score at a lower position)."""
    n = scores.size
    chosen = []
    for t in range(n):
        if not np.isfinite(scores[t]):
            continue
        beat = sum(1 for u in range(n) if np.isfinite(scores[u]) and
                   (scores[u] > scores[t] or (scores[u] == scores[t] and u < t)))
        if beat < topk:
            chosen.append(t)
    return chosen


@pytest.mark.parametrize("integer", [False, True])
def test_index_topk_brute_force(orc, integer):
    """Top-k, re-sorted by position, shifted by the offset, -1 padded (Indexer.forward's last
    lines), against rank counting; integer scores make ties common, which go to the lower
    position."""
    b, s, h, d, n_pos, ratio, topk, off = 2, 9, 4, 32, 24, 2, 7, 128
    q, k, w, *_ = _index_inputs(3, b, s, h, d, n_pos, integer=integer)
    pos = np.array([[0, 1, 2, 5, 9, 13, 20, 40, 60]] * b, np.int32)
    sc = orc.index_scores(q, k, w, pos, ratio)
    if integer:
        assert len(np.unique(sc[np.isfinite(sc)])) < np.isfinite(sc).sum()   # ties present
    idx = orc.index_topk(sc, topk, off)
    for bi in range(b):
        for si in range(s):
            want = _rank_select(sc[bi, si], topk)
            row = idx[bi, si]
            assert row[: len(want)].tolist() == [t + off for t in want]
            assert np.all(row[len(want):] == -1)


def test_index_topk_lists_every_visible_position_when_few(orc):
    """With at most topk visible positions the list is all of them in order: offset ..
    offset + (p+1)//ratio - 1, then -1 (closed form of the causal prefill)."""
    b, s, h, d, n_pos, ratio, topk = 1, 64, 4, 32, 16, 4, 16
    q, k, w, *_ = _index_inputs(4, b, s, h, d, n_pos)
    pos = np.arange(s, dtype=np.int32)[None]
    idx = orc.index_topk(orc.index_scores(q, k, w, pos, ratio), topk, 128)
    for t in range(s):
        v = min((t + 1) // ratio, n_pos)
        assert idx[0, t].tolist() == list(range(128, 128 + v)) + [-1] * (topk - v)


def _blocks_brute(row, length, topk_blocks, bs):
    n = row.size
    nblk = -(-n // bs)
    last = (length - 1) // bs                                     # Python floor division
    sc = []
    for j in range(nblk):
        vals = [row[t] if t < n else -np.inf for t in range(j * bs, (j + 1) * bs)]
        sc.append(np.inf if j == last else max(vals))
    keep = []
    for j in range(nblk):
        beat = sum(1 for u in range(nblk) if sc[u] > sc[j] or (sc[u] == sc[j] and u < j))
        keep.append(beat < min(topk_blocks, nblk) and sc[j] > -np.inf)
    return np.repeat(np.array(keep, np.uint8), bs)[:n]


@pytest.mark.parametrize("topk_blocks", [1, 3, 6, 50])
def test_candidate_blocks_brute_force(orc, topk_blocks):
    """select_candidate_blocks against rank counting over block maxima, with the newest
    partly filled block pinned; blocks with no finite logit are never kept."""
    b, s, h, d, n_pos, ratio, bs = 1, 12, 4, 32, 45, 2, 8
    q, k, w, *_ = _index_inputs(5, b, s, h, d, n_pos, integer=True)
    pos = np.array([[0, 1, 2, 9, 16, 17, 30, 47, 60, 70, 89, 200]], np.int32)
    logits = orc.index_scores(q, k, w, pos, ratio)
    mask = orc.candidate_blocks(logits, pos, ratio, topk_blocks, bs)
    for si in range(s):
        length = (int(pos[0, si]) + 1) // ratio
        assert np.array_equal(mask[0, si], _blocks_brute(logits[0, si], length, topk_blocks, bs)), si
        if length == 0:
            assert not mask[0, si].any()
        elif length <= n_pos:
            assert mask[0, si, length - 1] == 1                  # the pinned block


def test_candidate_blocks_keep_every_reachable_block_when_few(orc):
    """With at least as many picks as blocks (the config's 2048 blocks of 8 at 16384
    positions), every block holding a visible position is kept and nothing else."""
    b, s, h, d, n_pos, ratio, bs = 1, 5, 4, 32, 64, 4, 8
    q, k, w, *_ = _index_inputs(6, b, s, h, d, n_pos)
    pos = np.array([[3, 40, 100, 255, 1000]], np.int32)
    mask = orc.candidate_blocks(orc.index_scores(q, k, w, pos, ratio), pos, ratio, 8, bs)
    for si in range(s):
        v = min((int(pos[0, si]) + 1) // ratio, n_pos)
        want = np.zeros(n_pos, np.uint8)
        want[: -(-v // bs) * bs] = 1
        assert np.array_equal(mask[0, si], want[:n_pos])


def test_two_level_selection_stays_inside_the_candidates(orc):
    """Level two masks its own scores to the level-one candidates: every listed position is
    a candidate and visible."""
    b, s, h, d, n_pos, ratio, bs = 2, 6, 8, 64, 96, 2, 8
    q, k, w, *_ = _index_inputs(7, b, s, h, d, n_pos)
    q2, _, w2, *_ = _index_inputs(8, b, s, h, d, n_pos)
    pos = np.array([[10, 50, 90, 120, 150, 191]] * b, np.int32)
    cand = orc.candidate_blocks(orc.index_scores(q, k, w, pos, ratio), pos, ratio, 3, bs)
    idx = orc.index_topk(orc.index_scores(q2, k, w2, pos, ratio, cand), 10, 0)
    for bi in range(b):
        for si in range(s):
            sel = idx[bi, si][idx[bi, si] >= 0]
            vis = (pos[bi, si] + 1) // ratio
            assert sel.size == min(10, int(cand[bi, si, :vis].sum()))
            assert np.all(cand[bi, si, sel] == 1) and np.all(sel < (pos[bi, si] + 1) // ratio)


# ------------------------------------------------------------------ grouped output projection
def _proj_inputs(seed, m, g, r, kg, integer=False):
    gen = torch.Generator().manual_seed(seed)
    if integer:
        o = torch.randint(-4, 5, (m, g, kg), generator=gen).float()
        w = torch.randint(-4, 5, (g, r, kg), generator=gen).float()
    else:
        o = torch.randn(m, g, kg, generator=gen)
        w = torch.randn(g, r, kg, generator=gen) * kg ** -0.5
    return o.to(torch.bfloat16), w.to(torch.bfloat16)


def test_grouped_proj_vs_einsum(orc):
    """The page's einsum "bsgd,grd->bsgr" evaluated by torch in f64, then rounded to bf16:
    the f32 oracle differs by at most one bf16 rounding step."""
    o, w = _proj_inputs(1, 7, 4, 24, 96)
    got = _f32(orc.grouped_proj(o.view(torch.int16).numpy().view(np.uint16), w.view(torch.int16).numpy().view(np.uint16)))
    ref = torch.einsum("mgd,grd->mgr", o.double(), w.double())
    refb = ref.to(torch.bfloat16).double()
    assert np.all(np.abs(got - refb.numpy()) <= np.abs(ref.numpy()) * 2 ** -8 + 1e-6)
    assert (got == refb.numpy()).mean() > 0.97


def test_grouped_proj_exact_and_block_diagonal(orc):
    """Small integers: every partial sum is exact, so the oracle equals the exact einsum;
    changing one group's input changes only that group's output (block-diagonal wo_a)."""
    o, w = _proj_inputs(2, 5, 3, 16, 64, integer=True)
    ou = lambda t: t.view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    got = orc.grouped_proj(ou(o), ou(w))
    ref = torch.einsum("mgd,grd->mgr", o.double(), w.double()).to(torch.bfloat16)
    assert np.array_equal(got, ou(ref))
    o2 = o.clone()
    o2[:, 1] = -o2[:, 1]
    got2 = orc.grouped_proj(ou(o2), ou(w))
    assert np.array_equal(got2[:, [0, 2]], got[:, [0, 2]])
    assert np.array_equal(_f32(got2[:, 1]), -_f32(got[:, 1]))
