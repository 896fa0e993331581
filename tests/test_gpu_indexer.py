"""The indexer (sa_indexer_topk) and the candidate blocks (sa_candidate_blocks) against the
oracle. Scores come from bf16 MFMA with f32 accumulation, so on random inputs they agree
with the oracle's to rounding (a bound derived from the magnitudes); the selections the
scores decide are compared bit for bit with the oracle's selection run on the GPU's own
scores, and on inputs whose arithmetic is exact (small integers, power-of-two weights) the
whole chain is compared bit for bit."""
import sys

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def sa():
    import sparse_latent_attention_attn_amd as sa
    sa.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return sa


def _u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _inputs(seed, b, s, h, d, n_pos, integer=False):
    g = torch.Generator().manual_seed(seed)
    if integer:
        q = torch.randint(-3, 4, (b, s, h, d), generator=g).float()
        k = torch.randint(-3, 4, (b, n_pos, d), generator=g).float()
        w = 2.0 ** torch.randint(-2, 2, (b, s, h), generator=g).float()
        w = w * torch.where(torch.rand(b, s, h, generator=g) < 0.2, -1.0, 1.0)
    else:
        q = torch.randn(b, s, h, d, generator=g)
        k = torch.randn(b, n_pos, d, generator=g)
        w = torch.randn(b, s, h, generator=g) * (d ** -0.5 * h ** -0.5)
    return q.to(torch.bfloat16), k.to(torch.bfloat16), w.float()


def _score_bound(q, k, w, rel=2e-6):
    """|gpu - oracle| bound of a score: both sum the same products in f32 in different orders;
    rel times the sum of magnitudes sum_h |w_h| sum_d |q_hd k_ud| (f64) covers it."""
    mag = torch.einsum("bshd,bud->bshu", q.double().abs(), k.double().abs())
    return (mag * w.double().abs()[..., None]).sum(2).numpy() * rel + 1e-30


def _check_structure(idx, scores, topk, offset):
    """Listed positions ascending, shifted by offset, finite-scored; then -1; as many as
    min(topk, finite scores)."""
    b, s, _ = idx.shape
    for bi in range(b):
        for si in range(s):
            row = idx[bi, si, :topk]
            v = row[row >= 0]
            nfin = int(np.isfinite(scores[bi, si]).sum())
            assert v.size == min(topk, nfin)
            assert np.all(row[v.size:] == -1) and np.all(np.diff(v) > 0)
            assert np.all(np.isfinite(scores[bi, si, v - offset]))


@pytest.mark.parametrize("seed,b,s,h,d,n_pos,ratio,topk,integer", [
    (1, 2, 5, 32, 128, 300, 4, 16, False),
    (2, 3, 7, 16, 64, 77, 2, 10, True),
    (3, 1, 33, 64, 128, 129, 1, 40, False),
    (4, 2, 4, 32, 256, 1000, 4, 100, True),
    (5, 4, 1, 64, 64, 5000, 4, 512, False),
    (6, 2, 3, 32, 64, 3000, 1, 700, True),
    (7, 1, 2, 16, 64, 20000, 1, 2000, True),
])
def test_indexer_against_oracle(sa, seed, b, s, h, d, n_pos, ratio, topk, integer):
    _say("indexer", seed, b, s, h, d, n_pos, ratio, topk, "integer" if integer else "random")
    q, k, w = _inputs(seed, b, s, h, d, n_pos, integer)
    g = torch.Generator().manual_seed(seed + 100)
    pos = torch.randint(0, ratio * n_pos + 20, (b, s), generator=g, dtype=torch.int32)
    pos[0, 0] = 0                                    # nothing visible yet for ratio > 1
    off = 128
    sc, idx = sa.indexer_topk(q.cuda(), k.cuda(), w.cuda(), pos.cuda(), ratio, topk=topk, offset=off)
    sc, idx = sc.cpu().numpy(), idx.cpu().numpy()
    ref = oracle.index_scores(_u16(q), _u16(k), w.numpy(), pos.numpy(), ratio)
    assert np.array_equal(np.isneginf(sc), np.isneginf(ref))
    fin = np.isfinite(ref)
    if integer:
        assert np.array_equal(sc[fin], ref[fin])
        assert np.array_equal(idx, oracle.index_topk(ref, topk, off))
    else:
        assert np.all(np.abs(sc[fin] - ref[fin]) <= _score_bound(q, k, w)[fin])
    assert np.array_equal(idx, oracle.index_topk(sc, topk, off))
    _check_structure(idx, sc, topk, off)


@pytest.mark.parametrize("seed,b,s,d,n_pos,ratio,integer,cand", [
    (51, 1, 37, 128, 700, 4, False, False),   # 37 queries = 4 workgroups of 8 + 5; 700 = 10 x 64 + 60 positions
    (52, 2, 20, 64, 333, 2, True, False),     # d 64, exact integer sums; 333 = 5 x 64 + 13
    (53, 2, 17, 128, 129, 1, True, True),     # a candidate mask; 17 = 2 x 8 + 1: one live query in the last pair
    (54, 1, 72, 128, 2048, 4, False, False),  # causal positions from -8: the first workgroup sees nothing
])
def test_indexer_32_heads_prefill(sa, seed, b, s, d, n_pos, ratio, integer, cand):
    """32 index heads with 8 or more queries per sequence (the model's indexer shape in
    prefill): ragged query groups and position tiles, d 64 and 128, a candidate mask,
    workgroups with no visible position. Scores against the oracle (exact for integer
    inputs), lists against the oracle's selection."""
    _say("indexer 32 heads", seed, b, s, d, n_pos, ratio, "integer" if integer else "random", "cand" if cand else "")
    h, topk, off = 32, 50, 128
    q, k, w = _inputs(seed, b, s, h, d, n_pos, integer)
    g = torch.Generator().manual_seed(seed + 100)
    if seed == 54:
        pos = (torch.arange(s, dtype=torch.int32) - 8)[None].repeat(b, 1)
    else:
        pos = torch.randint(0, ratio * n_pos + 20, (b, s), generator=g, dtype=torch.int32)
    cm = (torch.rand(b, s, n_pos, generator=g) < 0.5).to(torch.uint8) if cand else None
    sc, idx = sa.indexer_topk(q.cuda(), k.cuda(), w.cuda(), pos.cuda(), ratio, topk=topk, offset=off,
                              cand=None if cm is None else cm.cuda())
    sc, idx = sc.cpu().numpy(), idx.cpu().numpy()
    ref = oracle.index_scores(_u16(q), _u16(k), w.numpy(), pos.numpy(), ratio, None if cm is None else cm.numpy())
    assert np.array_equal(np.isneginf(sc), np.isneginf(ref))
    fin = np.isfinite(ref)
    if integer:
        assert np.array_equal(sc[fin], ref[fin])
    else:
        assert np.all(np.abs(sc[fin] - ref[fin]) <= _score_bound(q, k, w)[fin])
    assert np.array_equal(idx, oracle.index_topk(sc, topk, off))
    _check_structure(idx, sc, topk, off)


@pytest.mark.parametrize("n_pos", [5000, 16384])
@pytest.mark.parametrize("shape", ["all_equal", "tie_at_threshold", "outliers", "few_selectable"])
def test_indexer_topk_adversarial_scores(sa, n_pos, shape):
    """Score distributions that defeat a sampled bracket, for the several-waves-per-query
    search (4 and 16 waves): every query's q_h is the first unit vector and the weights sum
    to 1, so score_t = relu(k_t[0]) exactly. Lists bit for bit against the oracle's selection
    on the oracle's scores."""
    _say("indexer top-k", shape, n_pos)
    b, s, h, d, topk = 2, 1, 32, 64, 512
    g = torch.Generator().manual_seed(n_pos)
    q = torch.zeros(b, s, h, d)
    q[..., 0] = 1.0
    w = torch.full((b, s, h), 1.0 / h)
    k0 = torch.ones(b, n_pos)
    if shape == "tie_at_threshold":        # 300 higher keys, then a tie across the rest
        k0[:, torch.randperm(n_pos, generator=g)[:300]] = 2.0
    elif shape == "outliers":              # 5 far above (a sample of 64 misses them), a band, the rest equal
        k0[:, torch.randperm(n_pos, generator=g)[:5]] = 4096.0
        k0[:, torch.arange(n_pos) % 7 == 0] = 3.0
    elif shape == "few_selectable":        # most scores 0 (relu of a negative key), a band of small ones
        k0 = -torch.ones(b, n_pos)
        k0[:, torch.randperm(n_pos, generator=g)[:700]] = torch.randint(1, 9, (700,), generator=g).float()
    k = torch.zeros(b, n_pos, d)
    k[..., 0] = k0
    k[..., 1:] = torch.randint(-3, 4, (b, n_pos, d - 1), generator=g).float()   # no effect on the score
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    pos = torch.full((b, s), 4 * n_pos + 3, dtype=torch.int32)
    if shape == "few_selectable":
        pos[1, 0] = 4 * 300 - 1             # sequence 1 sees 300 positions: fewer than topk
    sc, idx = sa.indexer_topk(q.cuda(), k.cuda(), w.cuda(), pos.cuda(), 4, topk=topk, offset=0)
    sc, idx = sc.cpu().numpy(), idx.cpu().numpy()
    ref = oracle.index_scores(_u16(q), _u16(k), w.numpy(), pos.numpy(), 4)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isneginf(sc), np.isneginf(ref))
    assert np.array_equal(sc[fin], ref[fin])
    assert np.array_equal(idx, oracle.index_topk(ref, topk, 0))
    _check_structure(idx, sc, topk, 0)


def test_indexer_candidates_and_two_levels(sa):
    """The candidate source's scores give the level-one blocks; level two scores its own
    queries inside them. Each GPU result equals the oracle's on the same GPU inputs."""
    b, s, h, d, n_pos, ratio, bs = 2, 9, 32, 128, 600, 4, 8
    q, k, w = _inputs(11, b, s, h, d, n_pos, integer=True)
    q2, _, w2 = _inputs(12, b, s, h, d, n_pos, integer=True)
    pos = torch.tensor([[0, 3, 7, 100, 511, 1024, 1500, 2000, 2399]] * b, dtype=torch.int32)
    sc, _ = sa.indexer_topk(q.cuda(), k.cuda(), w.cuda(), pos.cuda(), ratio)
    for topk_blocks in (1, 5, 20, 2048):
        mask = sa.candidate_blocks(sc, pos.cuda(), ratio, topk_blocks, bs).cpu().numpy()
        ref = oracle.candidate_blocks(sc.cpu().numpy(), pos.numpy(), ratio, topk_blocks, bs)
        assert np.array_equal(mask, ref), topk_blocks
    cand = sa.candidate_blocks(sc, pos.cuda(), ratio, 6, bs)
    sc2, idx2 = sa.indexer_topk(q2.cuda(), k.cuda(), w2.cuda(), pos.cuda(), ratio, topk=30, offset=0, cand=cand)
    ref2 = oracle.index_scores(_u16(q2), _u16(k), w2.numpy(), pos.numpy(), ratio, cand.cpu().numpy())
    fin = np.isfinite(ref2)
    assert np.array_equal(np.isneginf(sc2.cpu().numpy()), np.isneginf(ref2))
    assert np.array_equal(sc2.cpu().numpy()[fin], ref2[fin])
    assert np.array_equal(idx2.cpu().numpy(), oracle.index_topk(ref2, 30, 0))


def test_candidate_blocks_random_logits(sa):
    """Random logits with -inf beyond each query's visible positions, several block sizes
    (rows of whole 16-byte pieces with blocks of 4, 8 or 16 take one, four or sixteen waves
    per query with blocks inside lanes; other powers of two up to 64 take block maxima by lane
    exchanges, the rest by LDS atomics), ragged last blocks, selections that keep every
    visible block and ones that choose, and small-integer logits whose block maxima tie."""
    g = torch.Generator().manual_seed(21)
    for b, s, n_pos, ratio, tb, bs, ints in (
            (2, 6, 1000, 4, 17, 8, False), (1, 3, 16384, 4, 2048, 8, False), (3, 4, 999, 1, 3, 7, False),
            (2, 5, 1001, 2, 40, 16, False), (2, 3, 4096, 4, 64, 64, False), (1, 4, 777, 1, 500, 4, False),
            (2, 3, 2048, 4, 9, 1, False),
            (2, 5, 2048, 4, 17, 8, False), (2, 5, 2048, 1, 17, 8, True), (1, 4, 4096, 1, 100, 16, True),
            (2, 3, 8192, 2, 300, 4, False), (1, 3, 16384, 4, 100, 8, True), (1, 2, 20000, 1, 1000, 8, False),
            (3, 2, 512, 1, 5, 16, True)):
        pos = torch.randint(0, ratio * n_pos, (b, s), generator=g, dtype=torch.int32)
        lg = torch.randint(-3, 4, (b, s, n_pos), generator=g).float() if ints else torch.randn(b, s, n_pos, generator=g)
        vis = torch.clamp((pos.long() + 1) // ratio, max=n_pos)
        lg[torch.arange(n_pos)[None, None, :] >= vis[..., None]] = -float("inf")
        mask = sa.candidate_blocks(lg.cuda(), pos.cuda(), ratio, tb, bs).cpu().numpy()
        assert np.array_equal(mask, oracle.candidate_blocks(lg.numpy(), pos.numpy(), ratio, tb, bs))


def _full_case(name):
    if name == "decode":      # 64 sequences at position 65535: 16384 compressed positions
        return dict(b=64, s=1, n_pos=16384, pos=lambda b, s: torch.full((b, s), 65535, dtype=torch.int32))
    return dict(b=1, s=8192, n_pos=2048, pos=lambda b, s: torch.arange(s, dtype=torch.int32)[None].repeat(b, 1))


@pytest.mark.parametrize("name", ["decode", "prefill"])
def test_indexer_full_size(sa, name):
    """The indexer at the sizes of the window + compressed decode (64 x 1 query, 16384
    positions) and the long prefill (8192 queries, 2048 positions): 32 index heads of 128,
    ratio 4, 512 picks offset by the 128 window rows, written after the window part of each
    list. Scores of sampled queries against the oracle; every list bit for bit against the
    oracle's selection on the GPU's scores; the window part untouched."""
    c = _full_case(name)
    b, s, n_pos, h, d, topk = c["b"], c["s"], c["n_pos"], 32, 128, 512
    _say("indexer full", name)
    q, k, w = _inputs(31, b, s, h, d, n_pos)
    pos = c["pos"](b, s)
    lists = torch.full((b, s, 128 + topk), 777, dtype=torch.int32, device="cuda")
    sc, _ = sa.indexer_topk(q.cuda(), k.cuda(), w.cuda(), pos.cuda(), 4, topk=topk, offset=128,
                            idx=lists[:, :, 128:])
    sc_h = sc.cpu().numpy()
    got = lists.cpu().numpy()
    assert np.all(got[:, :, :128] == 777)
    assert np.array_equal(got[:, :, 128:], oracle.index_topk(sc_h, topk, 128))
    _check_structure(got[:, :, 128:], sc_h, topk, 128)
    sel = np.unique(np.linspace(0, b * s - 1, 24).round().astype(np.int64))
    bs_, ss_ = sel // s, sel % s
    qs = q[bs_, ss_][:, None] if s > 1 else q[bs_]
    ws = w[bs_, ss_][:, None] if s > 1 else w[bs_]
    ps = pos[bs_, ss_].view(-1, 1)
    ks = k[bs_] if b > 1 else k.expand(sel.size, -1, -1)
    ref = oracle.index_scores(_u16(qs.reshape(-1, 1, h, d)), _u16(ks.contiguous()), ws.reshape(-1, 1, h).numpy(),
                              ps.numpy(), 4)
    got_sc = sc_h[bs_, ss_][:, None]
    fin = np.isfinite(ref)
    assert np.array_equal(np.isneginf(got_sc), np.isneginf(ref))
    bound = _score_bound(qs.reshape(-1, 1, h, d), ks.contiguous(), ws.reshape(-1, 1, h))
    assert np.all(np.abs(got_sc[fin] - ref[fin]) <= bound[fin])
