"""The C-ABI library without a GPU: it loads, exports every function include/sa.h declares,
and rejects bad arguments on the host before making any HIP call."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sa.h")


@pytest.fixture(scope="module")
def sa():
    import sparse_latent_attention_attn_amd as sa
    if not os.path.exists(sa.LIB_PATH):
        from sparse_latent_attention_attn_amd import build_lib
        build_lib.build()
    sa.lib()
    return sa


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("sa_sparse_attn", "sa_sparse_attn_workspace", "sa_window_topk_idxs",
              "sa_quant_kv_fp8", "sa_status_string", "sa_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol(sa):
    L = sa.lib()
    for n in _declared_functions():
        assert hasattr(L, n), n
    assert L.sa_abi_version() == 2
    assert L.sa_status_string(0) == b"ok"
    assert b"invalid" in L.sa_status_string(-1)


def test_no_symbol_leaks_beyond_the_header(sa):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", sa.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert {n for n in exported if n.startswith("sa_")} == set(_declared_functions())


def _args(sa, **kw):
    a = sa.AttnArgs()
    a.b, a.s, a.h, a.d, a.topk, a.kv_rows = 1, 1, 16, 64, 8, 8
    a.q_seq_stride, a.kv_seq_stride, a.idx_seq_stride, a.out_seq_stride = 1024, 512, 8, 1024
    a.scale = 0.125
    # non-null, 16-byte aligned fake device pointers: validation never dereferences them
    for f in ("q", "kv", "sink", "idx", "out"):
        setattr(a, f, 0x10000)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("b", 0, -1), ("h", 0, -1), ("topk", 0, -1), ("kv_rows", 0, -1),
    ("d", 96, -2), ("d", 1024, -2), ("kv_format", 7, -1), ("flags", 2, -1),
    ("rope_dim", 3, -1), ("rope_dim", 128, -1), ("q", 0, -1), ("idx", 0, -1),
    ("q", 0x10008, -1), ("scale", float("inf"), -1), ("q_seq_stride", 12, -1),
])
def test_sparse_attn_rejects_before_any_hip_call(sa, field, value, status):
    a = _args(sa, **{field: value})
    assert sa.lib().sa_sparse_attn(C.byref(a), None) == status


def test_sparse_attn_requires_scales_for_fp8_and_pointers_for_rope(sa):
    assert sa.lib().sa_sparse_attn(C.byref(_args(sa, kv_format=1)), None) == -1
    assert sa.lib().sa_sparse_attn(C.byref(_args(sa, rope_dim=16)), None) == -1
    assert sa.lib().sa_sparse_attn(C.byref(_args(sa, flags=1)), None) == -1
    assert sa.lib().sa_sparse_attn(None, None) == -1


def test_batched_strides_are_checked(sa):
    a = _args(sa, b=2, q_seq_stride=8)      # smaller than s*h*d
    assert sa.lib().sa_sparse_attn(C.byref(a), None) == -1


def test_window_idxs_validation(sa):
    L = sa.lib()
    cols = C.c_int32(0)
    fake = C.c_void_p(0x10000)
    assert L.sa_window_topk_idxs(0, 4, 1, None, fake, 16, 4, C.byref(cols), None) == -1
    assert L.sa_window_topk_idxs(8, 4, 1, fake, fake, 16, 4, C.byref(cols), None) == -2   # chunked prefill
    assert L.sa_window_topk_idxs(8, 12, 1, None, fake, 96, 4, C.byref(cols), None) == -1  # row stride < cols
    assert L.sa_window_topk_idxs(8, 1, 2, fake, fake, 4, 8, C.byref(cols), None) == -1    # seq stride
    assert L.sa_window_topk_idxs(8, 1, 1, None, None, 8, 8, C.byref(cols), None) == -1


def test_quant_validation(sa):
    L = sa.lib()
    fake = C.c_void_p(0x10000)
    assert L.sa_quant_kv_fp8(fake, 4, 48, fake, None, None, None) == -1       # d % 32
    assert L.sa_quant_kv_fp8(fake, 4, 64, None, None, None, None) == -1       # no output
    assert L.sa_quant_kv_fp8(None, 4, 64, fake, None, None, None) == -1
    assert L.sa_quant_kv_fp8(fake, 0, 64, fake, None, None, None) == 0        # nothing to do


def test_split_plans_keep_the_combine_grid_in_int32(sa):
    """A list longer than one workgroup stages (5000 columns) forces a split plan; with
    b * s * h above the int32 range the combine kernel's wave index would overflow, so the
    call is refused on the host."""
    a = _args(sa, s=32768, h=65536, d=256, topk=5000, kv_rows=8, q_seq_stride=0,
              out_seq_stride=0, kv_seq_stride=0, idx_seq_stride=0)
    n = C.c_size_t(0)
    assert sa.lib().sa_sparse_attn_workspace(C.byref(a), C.byref(n)) == 0 and n.value > 0
    assert sa.lib().sa_sparse_attn(C.byref(a), None) == -2


def test_fp8_prefill_plans_take_dequantised_rows(sa):
    """fp8 storage: a prefill shape (each row named by thousands of (query, column) pairs)
    asks for a workspace holding the cache as bf16 rows; a decode shape (each row named about
    once) converts inside the kernel and needs none."""
    n = C.c_size_t(0)
    a = _args(sa, b=1, s=8192, h=128, d=512, topk=2176, kv_rows=2176, kv_format=1,
              q_seq_stride=0, out_seq_stride=0, kv_seq_stride=0, idx_seq_stride=0)
    assert sa.lib().sa_sparse_attn_workspace(C.byref(a), C.byref(n)) == 0
    assert n.value == 2176 * 512 * 2
    a = _args(sa, b=64, s=1, h=128, d=512, topk=640, kv_rows=16512, kv_format=1,
              q_seq_stride=128 * 512, out_seq_stride=128 * 512, kv_seq_stride=16512 * 512,
              idx_seq_stride=640, kv_scale_seq_stride=16512 * 16)
    assert sa.lib().sa_sparse_attn_workspace(C.byref(a), C.byref(n)) == 0 and n.value == 0


def test_rope_table_validation(sa):
    L = sa.lib()
    fake = C.c_void_p(0x10000)
    ok = (64, 16, 0, 10000.0, 1.0, 32.0, 1.0, fake, None)
    for i, bad in ((0, 3), (0, 0), (1, 0), (2, -1), (3, 1.0), (3, float("nan")), (7, None)):
        args = list(ok)
        args[i] = bad
        assert L.sa_rope_table(*args) == -1, (i, bad)
    yarn = list(ok)
    yarn[2] = 65536
    for i, bad in ((4, 0.0), (5, 1.0), (6, 0.0), (5, float("inf"))):
        args = list(yarn)
        args[i] = bad
        assert L.sa_rope_table(*args) == -1, (i, bad)


def _kv_args(sa, **kw):
    a = sa.KvWriteArgs()
    a.b, a.s, a.d, a.rope_dim = 1, 4, 64, 16
    a.x = a.pos = a.cache = a.rope_cos_sin = 0x10000
    a.max_pos, a.window, a.cache_rows, a.kv_format = 16, 8, 8, 0
    a.x_seq_stride, a.pos_seq_stride, a.cache_seq_stride = 256, 4, 512
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("b", 0, -1), ("s", 0, -1), ("d", 96, -2), ("rope_dim", 3, -1), ("rope_dim", 80, -1),
    ("kv_format", 3, -1), ("flags", 2, -1), ("x", 0, -1), ("pos", 0, -1), ("cache", 0, -1),
    ("cache_rows", 4, -1), ("window", -1, -1), ("x", 0x10008, -1), ("x_seq_stride", 12, -1),
    ("kv_format", 1, -1),          # fp8 without cache_scale
    ("flags", 1, -1),              # checking without err_word
])
def test_kv_write_rejects_before_any_hip_call(sa, field, value, status):
    a = _kv_args(sa, **{field: value})
    assert sa.lib().sa_kv_write(C.byref(a), None) == status


def test_kv_write_rejects_2_to_31_rows(sa):
    """b * s >= 2^31 rows is outside what the kernel indexes (32-bit row split)."""
    assert sa.lib().sa_kv_write(C.byref(_kv_args(sa, b=2, s=2 ** 30)), None) == -2


def test_kv_write_linear_needs_row0(sa):
    assert sa.lib().sa_kv_write(C.byref(_kv_args(sa, window=0)), None) == -1
    assert sa.lib().sa_kv_write(None, None) == -1


def test_grouped_proj_validation(sa):
    L = sa.lib()

    def args(**kw):
        a = sa.GroupedProjArgs()
        a.m, a.g, a.r, a.kg = 300, 2, 256, 512
        a.o = a.w = a.out = 0x10000
        a.o_stride, a.out_stride = 1024, 512
        for k, v in kw.items():
            setattr(a, k, v)
        return a
    for kw, st in (({"m": 0}, -1), ({"w_format": 5}, -1), ({"o": 0}, -1), ({"w_format": 1}, -1),
                   ({"o_stride": 1000}, -1), ({"out_stride": 100}, -1), ({"r": 200}, -2),
                   ({"kg": 96, "o_stride": 192}, -2), ({"o": 0x10008}, -1),
                   # fp8 scale bytes are read as words; a decode shape no kernel takes
                   ({"w_format": 1, "w_scale": 0x10002}, -1), ({"m": 40, "r": 48, "kg": 256}, -2)):
        assert L.sa_grouped_proj(C.byref(args(**kw)), None) == st, kw
    assert L.sa_grouped_proj(None, None) == -1


def test_fused_window_validation(sa):
    for kw in ({"window": -1}, {"window": 8, "window_mode": 3}, {"window": 8, "window_mode": 1},
               {"window": 9, "window_mode": 1, "pos": 0x10000}, {"window": 4, "window_mode": 1, "pos": 0x10002}):
        # topk is 8: a ring of 9 slots does not fit, and a window needs 4-byte aligned positions
        a = _args(sa, **kw)
        assert sa.lib().sa_sparse_attn(C.byref(a), None) == -1, kw


def _indexer_args(sa, **kw):
    a = sa.IndexerArgs()
    a.b, a.s, a.h, a.d, a.n_pos, a.ratio = 2, 4, 32, 128, 1000, 4
    a.q = a.k = a.w = a.pos = a.scores = 0x10000
    a.q_seq_stride, a.k_seq_stride = 4 * 32 * 128, 1000 * 128
    a.w_seq_stride, a.pos_seq_stride, a.scores_seq_stride = 4 * 32, 4, 4 * 1000
    a.topk, a.offset = 64, 0
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    ({"b": 0}, -1), ({"ratio": 0}, -1), ({"d": 96}, -2), ({"h": 48}, -2), ({"h": 64, "d": 256}, -2),
    ({"q": 0}, -1), ({"q": 0x10008}, -1), ({"scores": 0x10002}, -1), ({"q_seq_stride": 12}, -1),
    ({"k_seq_stride": 999 * 128}, -1), ({"scores_seq_stride": 3999}, -1),
    ({"n_pos": (1 << 28) + 1, "k_seq_stride": ((1 << 28) + 1) * 128, "scores_seq_stride": 4 * ((1 << 28) + 1)}, -2),
    ({"idx": 0x10000, "topk": 0, "idx_row_stride": 64, "idx_seq_stride": 256}, -1),
    ({"idx": 0x10000, "idx_row_stride": 32, "idx_seq_stride": 256}, -1),
    ({"idx": 0x10000, "idx_row_stride": 64, "idx_seq_stride": 100}, -1),
    ({"idx": 0x10000, "idx_row_stride": 64, "idx_seq_stride": 256, "n_pos": 40000,
      "k_seq_stride": 40000 * 128, "scores_seq_stride": 4 * 40000}, -2),
])
def test_indexer_rejects_before_any_hip_call(sa, kw, status):
    """sa_indexer_topk: bad sizes, pointers, alignments and strides are refused on the host,
    shapes no kernel takes are unsupported (no launch is ever attempted here)."""
    assert sa.lib().sa_indexer_topk(C.byref(_indexer_args(sa, **kw)), None) == status
    assert sa.lib().sa_indexer_topk(None, None) == -1


@pytest.mark.parametrize("kw,status", [
    ({"b": 0}, -1), ({"topk_blocks": 0}, -1), ({"block_size": 0}, -1), ({"logits": 0}, -1),
    ({"logits": 0x10002}, -1), ({"mask": 0}, -1), ({"logits_seq_stride": 100}, -1),
    ({"mask_seq_stride": 100}, -1), ({"n_pos": 40000, "block_size": 1, "logits_seq_stride": 120000,
                                      "mask_seq_stride": 120000}, -2),
])
def test_candidate_blocks_rejects_before_any_hip_call(sa, kw, status):
    a = sa.CandidateArgs()
    a.b, a.s, a.n_pos, a.ratio, a.topk_blocks, a.block_size = 2, 3, 1000, 4, 16, 8
    a.logits = a.pos = a.mask = 0x10000
    a.logits_seq_stride, a.pos_seq_stride, a.mask_seq_stride = 3000, 3, 3000
    for k, v in kw.items():
        setattr(a, k, v)
    assert sa.lib().sa_candidate_blocks(C.byref(a), None) == status
    assert sa.lib().sa_candidate_blocks(None, None) == -1
