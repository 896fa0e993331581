"""Host-side checks that need no GPU: the seeded generators keep the index-list contract of
the indexer page (Indexer.forward: compressed positions ascending, shifted by the offset of
the window rows, -1 where unreachable, causal visibility (t+1)//ratio in prefill and
end_pos//ratio in decode), and the parity comparison rejects what it must."""
import numpy as np
import pytest
import torch

import sa_workloads as W
from sa_harness import assert_close


def _check_compressed(comp, window, n_comp, visible):
    """comp: int32 [s][Tc] of one sequence; visible[t]: causal compressed positions of
    query t. Valid entries: strictly ascending (hence distinct), in [window, window+visible),
    i.e. shifted by the window rows and causal."""
    for t in range(comp.shape[0]):
        row = comp[t]
        v = row[row >= 0]
        assert np.all(row[row < 0] == -1), "the only skip marker is -1"
        assert np.all(np.diff(v) > 0), f"query {t}: not strictly ascending"
        assert v.size == 0 or (v.min() >= window and v.max() < window + min(visible[t], n_comp)), \
            f"query {t}: outside the causal compressed rows"


def test_prefill_compress_contract_full_size():
    """The long-prefill workload (8192 queries, ratio 4, 2048 compressed rows after 128 window
    rows): query t names exactly its (t+1)//4 causal compressed positions, all of them, as a
    prefix, ascending, offset by 128, then -1."""
    w = W.make("prefill_compress")
    comp = w.comp_idx[0].numpy()
    S, Tc = comp.shape
    assert (S, Tc) == (8192, 2048) and w.window == 128 and w.kv_rows == 128 + 2048
    t = np.arange(S)
    nvis = (t + 1) // 4
    counts = (comp >= 0).sum(axis=1)
    assert np.array_equal(counts, nvis)
    c = np.arange(Tc)[None, :]
    expect = np.where(c < nvis[:, None], c + 128, -1)
    assert np.array_equal(comp, expect)
    # the window half is the decode list at position t: positions start at 0 and step by 1
    assert np.array_equal(w.win_start_pos.numpy(), t) and np.array_equal(w.pos.numpy()[0], t)


def test_decode_compress_contract_full_size():
    """The window + compressed decode workload (64 sequences at position 65535, 16384
    compressed rows after 128 window rows): 512 distinct positions per query, sorted, offset
    by 128, every one causal (65536 // 4 = 16384 visible), about 2% of them -1 in place."""
    w = W.make("decode_compress")
    comp = w.comp_idx.numpy()
    assert comp.shape == (64, 1, 512) and w.kv_rows == 128 + 16384
    assert np.all(w.win_start_pos.numpy() == 65535)
    for b in range(64):
        _check_compressed(comp[b], 128, 16384, [65536 // 4])
    holes = int((comp < 0).sum())
    # binomial(32768, 0.02): mean 655, sd 25
    assert 500 < holes < 820, holes
    # holes sit anywhere, not only at the end
    first_hole = [int(np.argmax(comp[b, 0] < 0)) for b in range(64) if (comp[b, 0] < 0).any()]
    assert min(first_hole) < 400


@pytest.mark.parametrize("name", ["decode_compress", "prefill_compress"])
def test_small_variants_keep_the_contract(name):
    w = W.small_variant(name)
    comp = w.comp_idx.numpy()
    n_comp = w.kv_rows - w.window
    for b in range(w.b):
        if name == "prefill_compress":
            vis = [(t + 1) // 4 for t in range(w.s)]
            assert np.array_equal((comp[b] >= 0).sum(axis=1), vis)
        else:
            vis = [(int(w.win_start_pos[b]) + 1) // 4]
        _check_compressed(comp[b], w.window, n_comp, vis)


def test_generators_are_deterministic():
    a, b = W.small_variant("decode_compress"), W.small_variant("decode_compress")
    assert torch.equal(a.q, b.q) and torch.equal(a.kv, b.kv) and torch.equal(a.comp_idx, b.comp_idx)
    c = W.small_variant("decode_compress", seed=99)
    assert not torch.equal(a.q, c.q)


def _bf16(vals):
    return torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_assert_close_accepts_within_bound():
    ref = _bf16([1.0, -2.0, 0.0, 100.0])
    got = _bf16([1.0078125, -2.0, 0.0078125, 101.0])
    assert_close(got, ref, "within")


@pytest.mark.parametrize("bad", [[1.5, -2.0, 0.0, 100.0], [float("nan")] * 4,
                                 [1.0, float("nan"), 0.0, 100.0], [1.0, -2.0, float("inf"), 100.0]])
def test_assert_close_rejects_outside_and_non_finite(bad):
    ref = _bf16([1.0, -2.0, 0.0, 100.0])
    with pytest.raises(AssertionError):
        assert_close(_bf16(bad), ref, "bad")


def test_assert_close_rejects_nan_in_the_oracle():
    with pytest.raises(AssertionError):
        assert_close(_bf16([1.0, 2.0]), _bf16([1.0, float("nan")]), "nan oracle")
