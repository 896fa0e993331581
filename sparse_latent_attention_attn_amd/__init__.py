"""MI355X (gfx950) sparse latent attention of DeepSeek-V4.1: Python binding of libsa.so.

This module only marshals arguments: it checks tensor dtypes, shapes and devices, then
passes raw device pointers and the current HIP stream to the C ABI declared in
``include/sa.h``. Every step of the computation runs in the library's HIP kernels. The
library must be built (``python -m sparse_latent_attention_attn_amd.build_lib``); importing
a function from here without it raises, there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

__all__ = [
    "SaError", "lib", "sparse_attn", "sparse_attn_noalloc", "sparse_attn_workspace_bytes", "window_topk_idxs",
    "quant_kv_fp8", "rope_table", "kv_write", "KvWriteArgs", "indexer_topk", "candidate_blocks",
    "IndexerArgs", "CandidateArgs", "grouped_proj", "GroupedProjArgs", "KV_BF16", "KV_FP8", "FLAG_CHECK_IDX", "AttnArgs",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsa.so")

SA_OK, SA_ERR_INVALID, SA_ERR_UNSUPPORTED, SA_ERR_HIP, SA_ERR_WORKSPACE, SA_ERR_SCRATCH = 0, -1, -2, -3, -4, -5
NOALLOC_SCRATCH_BYTES = 64 << 20
KV_BF16, KV_FP8 = 0, 1
FLAG_CHECK_IDX = 1
WINDOW_RING, WINDOW_CHUNK = 1, 2


class SaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib().sa_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


class AttnArgs(C.Structure):
    """Mirror of sa_attn_args in include/sa.h (field order and types must match)."""
    _fields_ = [
        ("b", C.c_int32), ("s", C.c_int32), ("h", C.c_int32), ("d", C.c_int32),
        ("topk", C.c_int32), ("kv_rows", C.c_int32),
        ("q", C.c_void_p), ("q_seq_stride", C.c_int64),
        ("kv", C.c_void_p), ("kv_seq_stride", C.c_int64),
        ("kv_scale", C.c_void_p), ("kv_scale_seq_stride", C.c_int64),
        ("kv_format", C.c_int32),
        ("sink", C.c_void_p),
        ("idx", C.c_void_p), ("idx_seq_stride", C.c_int64),
        ("scale", C.c_float),
        ("out", C.c_void_p), ("out_seq_stride", C.c_int64),
        ("rope_dim", C.c_int32),
        ("rope_cos_sin", C.c_void_p), ("max_pos", C.c_int32),
        ("pos", C.c_void_p), ("pos_seq_stride", C.c_int64),
        ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t),
        ("flags", C.c_uint32), ("err_word", C.c_void_p),
        ("window", C.c_int32), ("window_mode", C.c_int32),
    ]


class KvWriteArgs(C.Structure):
    """Mirror of sa_kv_write_args in include/sa.h (field order and types must match)."""
    _fields_ = [
        ("b", C.c_int32), ("s", C.c_int32), ("d", C.c_int32), ("rope_dim", C.c_int32),
        ("x", C.c_void_p), ("x_seq_stride", C.c_int64),
        ("rope_cos_sin", C.c_void_p), ("max_pos", C.c_int32),
        ("pos", C.c_void_p), ("pos_seq_stride", C.c_int64),
        ("window", C.c_int32), ("row0", C.c_void_p), ("cache_rows", C.c_int32),
        ("kv_format", C.c_int32),
        ("cache", C.c_void_p), ("cache_seq_stride", C.c_int64),
        ("cache_scale", C.c_void_p), ("cache_scale_seq_stride", C.c_int64),
        ("rows_out", C.c_void_p), ("rows_out_seq_stride", C.c_int64),
        ("flags", C.c_uint32), ("err_word", C.c_void_p),
    ]


class IndexerArgs(C.Structure):
    """Mirror of sa_indexer_args in include/sa.h (field order and types must match)."""
    _fields_ = [
        ("b", C.c_int32), ("s", C.c_int32), ("h", C.c_int32), ("d", C.c_int32),
        ("n_pos", C.c_int32), ("ratio", C.c_int32),
        ("q", C.c_void_p), ("q_seq_stride", C.c_int64),
        ("k", C.c_void_p), ("k_seq_stride", C.c_int64),
        ("w", C.c_void_p), ("w_seq_stride", C.c_int64),
        ("pos", C.c_void_p), ("pos_seq_stride", C.c_int64),
        ("cand", C.c_void_p), ("cand_seq_stride", C.c_int64),
        ("scores", C.c_void_p), ("scores_seq_stride", C.c_int64),
        ("topk", C.c_int32), ("offset", C.c_int32),
        ("idx", C.c_void_p), ("idx_seq_stride", C.c_int64), ("idx_row_stride", C.c_int64),
    ]


class CandidateArgs(C.Structure):
    """Mirror of sa_candidate_args in include/sa.h."""
    _fields_ = [
        ("b", C.c_int32), ("s", C.c_int32), ("n_pos", C.c_int32), ("ratio", C.c_int32),
        ("topk_blocks", C.c_int32), ("block_size", C.c_int32),
        ("logits", C.c_void_p), ("logits_seq_stride", C.c_int64),
        ("pos", C.c_void_p), ("pos_seq_stride", C.c_int64),
        ("mask", C.c_void_p), ("mask_seq_stride", C.c_int64),
    ]


class GroupedProjArgs(C.Structure):
    """Mirror of sa_grouped_proj_args in include/sa.h."""
    _fields_ = [
        ("m", C.c_int32), ("g", C.c_int32), ("r", C.c_int32), ("kg", C.c_int32),
        ("o", C.c_void_p), ("o_stride", C.c_int64),
        ("w_format", C.c_int32), ("w", C.c_void_p), ("w_scale", C.c_void_p),
        ("out", C.c_void_p), ("out_stride", C.c_int64),
    ]


_lib = None


def lib():
    """Load libsa.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_latent_attention_attn_amd.build_lib`")
        L = C.CDLL(LIB_PATH)
        P, I32, I64 = C.c_void_p, C.c_int32, C.c_int64
        L.sa_abi_version.restype = C.c_int
        L.sa_abi_version.argtypes = []
        L.sa_status_string.restype = C.c_char_p
        L.sa_status_string.argtypes = [C.c_int]
        L.sa_sparse_attn.restype = C.c_int
        L.sa_sparse_attn.argtypes = [C.POINTER(AttnArgs), P]
        L.sa_sparse_attn_noalloc.restype = C.c_int
        L.sa_sparse_attn_noalloc.argtypes = [C.POINTER(AttnArgs), P]
        L.sa_sparse_attn_workspace.restype = C.c_int
        L.sa_sparse_attn_workspace.argtypes = [C.POINTER(AttnArgs), C.POINTER(C.c_size_t)]
        L.sa_window_topk_idxs.restype = C.c_int
        L.sa_window_topk_idxs.argtypes = [I32, I32, I32, P, P, I64, I64, C.POINTER(I32), P]
        L.sa_rope_table.restype = C.c_int
        L.sa_rope_table.argtypes = [I32, I32, I32, C.c_float, C.c_float, C.c_float, C.c_float, P, P]
        L.sa_indexer_topk.restype = C.c_int
        L.sa_indexer_topk.argtypes = [C.POINTER(IndexerArgs), P]
        L.sa_candidate_blocks.restype = C.c_int
        L.sa_candidate_blocks.argtypes = [C.POINTER(CandidateArgs), P]
        L.sa_grouped_proj.restype = C.c_int
        L.sa_grouped_proj.argtypes = [C.POINTER(GroupedProjArgs), P]
        L.sa_kv_write.restype = C.c_int
        L.sa_kv_write.argtypes = [C.POINTER(KvWriteArgs), P]
        L.sa_quant_kv_fp8.restype = C.c_int
        L.sa_quant_kv_fp8.argtypes = [P, I64, I32, P, P, P, P]
        if L.sa_abi_version() != 2:
            raise RuntimeError("libsa.so ABI version mismatch")
        _lib = L
    return _lib


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check(fn, status):
    if status != SA_OK:
        raise SaError(fn, status)


def _need(t, dtype, name, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _seq_major(t, name, inner_ndim):
    """Per-sequence blocks must be contiguous; the sequence stride may be anything."""
    inner = t[0] if t.shape[0] > 0 else t
    if not inner.is_contiguous():
        raise ValueError(f"{name}: each sequence's block must be contiguous")
    return t.stride(0)


def make_args(q, kv, sink, idx, scale, out, *, kv_scale=None, rope=None, workspace=None,
              err_word=None, check_idx=False, window=None) -> AttnArgs:
    """Build sa_attn_args from tensors. q [b][s][h][d] bf16, kv [b][R][d] bf16 or uint8
    (fp8 codes, with kv_scale uint8 [b][R][d/32]), sink f32 [h], idx int32 [b][s][topk],
    out like q. rope = (cos_sin f32 [max_pos][rd/2][2], pos int32 [b][s]) or None.
    window = (W, "ring" | "chunk", pos int32 [b][s]) fuses the window lists: the first
    W (ring) or min(s, W) (chunk) columns are generated from the positions."""
    dev = q.device
    _need(q, torch.bfloat16, "q", dev)
    _need(out, torch.bfloat16, "out", dev)
    _need(sink, torch.float32, "sink", dev)
    _need(idx, torch.int32, "idx", dev)
    if q.dim() != 4 or kv.dim() != 3 or idx.dim() != 3 or out.shape != q.shape:
        raise ValueError("shapes: q/out [b][s][h][d], kv [b][R][d], idx [b][s][topk]")
    b, s, h, d = q.shape
    fmt = KV_BF16
    if kv.dtype == torch.bfloat16:
        _need(kv, torch.bfloat16, "kv", dev)
    else:
        _need(kv, torch.uint8, "kv", dev)
        if kv_scale is None:
            raise ValueError("fp8 kv needs kv_scale")
        _need(kv_scale, torch.uint8, "kv_scale", dev)
        fmt = KV_FP8
    if kv.shape[0] != b or kv.shape[2] != d or idx.shape[:2] != (b, s) or sink.shape != (h,):
        raise ValueError("inconsistent shapes")
    a = AttnArgs()
    a.b, a.s, a.h, a.d, a.topk, a.kv_rows = b, s, h, d, idx.shape[2], kv.shape[1]
    a.q, a.q_seq_stride = _ptr(q), _seq_major(q, "q", 3)
    a.kv, a.kv_seq_stride = _ptr(kv), _seq_major(kv, "kv", 2)
    if fmt == KV_FP8:
        a.kv_scale, a.kv_scale_seq_stride = _ptr(kv_scale), _seq_major(kv_scale, "kv_scale", 2)
    a.kv_format = fmt
    if not sink.is_contiguous():
        raise ValueError("sink must be contiguous")
    a.sink = _ptr(sink)
    a.idx, a.idx_seq_stride = _ptr(idx), _seq_major(idx, "idx", 2)
    a.scale = float(scale)
    a.out, a.out_seq_stride = _ptr(out), _seq_major(out, "out", 3)
    if rope is not None:
        cs, pos = rope
        _need(cs, torch.float32, "rope cos_sin", dev)
        _need(pos, torch.int32, "pos", dev)
        if not cs.is_contiguous() or cs.dim() != 3 or pos.shape != (b, s):
            raise ValueError("rope table [max_pos][rd/2][2] contiguous, pos [b][s]")
        a.rope_dim = cs.shape[1] * 2
        a.rope_cos_sin, a.max_pos = _ptr(cs), cs.shape[0]
        a.pos, a.pos_seq_stride = _ptr(pos), _seq_major(pos, "pos", 1)
    if workspace is not None:
        a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    if check_idx:
        if err_word is None:
            raise ValueError("check_idx needs err_word")
        _need(err_word, torch.int32, "err_word", dev)
        a.flags, a.err_word = FLAG_CHECK_IDX, _ptr(err_word)
    if window is not None:
        wn, mode, wpos = window
        _need(wpos, torch.int32, "window pos", dev)
        if wpos.shape != (b, s):
            raise ValueError("window positions must be [b][s]")
        if rope is not None and wpos.data_ptr() != rope[1].data_ptr():
            raise ValueError("the fused window lists and the epilogue read the same positions")
        a.window, a.window_mode = wn, {"ring": WINDOW_RING, "chunk": WINDOW_CHUNK}[mode]
        a.pos, a.pos_seq_stride = _ptr(wpos), _seq_major(wpos, "pos", 1)
    return a


def sparse_attn_workspace_bytes(args: AttnArgs) -> int:
    n = C.c_size_t(0)
    _check("sa_sparse_attn_workspace", lib().sa_sparse_attn_workspace(C.byref(args), C.byref(n)))
    return n.value


def sparse_attn(q, kv, sink, idx, scale, *, out=None, kv_scale=None, rope=None,
                workspace=None, err_word=None, check_idx=False, window=None):
    """sparse_attn on the GPU (see include/sa.h). Returns out (bf16, like q). A workspace
    is allocated with torch when none is given and the plan needs one. window: see
    make_args."""
    if out is None:
        out = torch.empty_like(q)
    a = make_args(q, kv, sink, idx, scale, out, kv_scale=kv_scale, rope=rope,
                  err_word=err_word, check_idx=check_idx, window=window)
    need = sparse_attn_workspace_bytes(a)
    if need > 0:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    _check("sa_sparse_attn", lib().sa_sparse_attn(C.byref(a), C.c_void_p(_stream(q.device))))
    return out


def sparse_attn_noalloc(q, kv, sink, idx, scale, *, out, kv_scale=None, rope=None,
                       err_word=None, check_idx=False):
    """sparse_attn through sa_sparse_attn_noalloc (include/sa.h): no workspace and no
    allocation by the library; `out` must be given. Returns out."""
    a = make_args(q, kv, sink, idx, scale, out, kv_scale=kv_scale, rope=rope,
                  err_word=err_word, check_idx=check_idx)
    _check("sa_sparse_attn_noalloc", lib().sa_sparse_attn_noalloc(C.byref(a), C.c_void_p(_stream(q.device))))
    return out


def window_topk_idxs(window: int, seqlen: int, nseq: int, start_pos=None, *, out=None,
                     device=None):
    """Window index lists (include/sa.h). start_pos None: prefill from position 0, returns
    int32 [nseq][seqlen][min(seqlen, window)]. start_pos (device int32 [nseq]): decode
    (seqlen 1), returns [nseq][1][window]. With `out` (int32 [nseq][seqlen][>= cols]) the
    lists are written into its first cols columns and out is returned."""
    if start_pos is not None:
        _need(start_pos, torch.int32, "start_pos")
        device = start_pos.device
        cols = window
    else:
        cols = min(seqlen, window)
    if out is None:
        out = torch.empty(nseq, seqlen, cols, dtype=torch.int32, device=device or "cuda")
    _need(out, torch.int32, "out")
    if out.dim() != 3 or out.stride(2) != 1 or out.shape[0] != nseq or out.shape[1] != seqlen:
        raise ValueError("out must be [nseq][seqlen][>=cols] with unit column stride")
    c = C.c_int32(0)
    _check("sa_window_topk_idxs", lib().sa_window_topk_idxs(
        window, seqlen, nseq, _ptr(start_pos), _ptr(out), out.stride(0), out.stride(1),
        C.byref(c), C.c_void_p(_stream(out.device))))
    assert c.value == cols
    return out


def quant_kv_fp8(kv, *, codes=None, scales=None, roundtrip=None, want=("codes", "scales")):
    """Block-32 ue8m0 fp8 quantisation of bf16 rows kv [..., d]. Returns the tuple of the
    requested outputs among codes (uint8 like kv), scales (uint8 [..., d/32]) and
    roundtrip (bf16 like kv; may be kv itself for in-place)."""
    _need(kv, torch.bfloat16, "kv")
    if not kv.is_contiguous():
        raise ValueError("kv must be contiguous")
    d = kv.shape[-1]
    rows = kv.numel() // d
    if "codes" in want and codes is None:
        codes = torch.empty(kv.shape, dtype=torch.uint8, device=kv.device)
    if "scales" in want and scales is None:
        scales = torch.empty(kv.shape[:-1] + (d // 32,), dtype=torch.uint8, device=kv.device)
    if "roundtrip" in want and roundtrip is None:
        roundtrip = torch.empty_like(kv)
    _check("sa_quant_kv_fp8", lib().sa_quant_kv_fp8(
        _ptr(kv), rows, d, _ptr(codes), _ptr(scales), _ptr(roundtrip),
        C.c_void_p(_stream(kv.device))))
    res = {"codes": codes, "scales": scales, "roundtrip": roundtrip}
    return tuple(res[w] for w in want)


def kv_write(x, pos, cache, *, rope=None, window=0, row0=None, cache_scale=None,
             rows_out=None, err_word=None, check_idx=False):
    """The KV write path (sa_kv_write in include/sa.h). x: bf16 [b][s][d] normalised rows;
    pos: int32 [b][s]; cache: bf16 [b][R][d] (bf16 storage) or uint8 [b][R][d] with
    cache_scale uint8 [b][R][d/32] (fp8 storage); rope = cos_sin table f32
    [max_pos][rd/2][2] or None; window > 0: ring of `window` slots, else row0 int32 [b].
    rows_out: optional bf16 [b][s][d]. Returns rows_out."""
    dev = x.device
    _need(x, torch.bfloat16, "x", dev)
    _need(pos, torch.int32, "pos", dev)
    if x.dim() != 3 or pos.shape != x.shape[:2] or cache.dim() != 3 or cache.shape[0] != x.shape[0] \
            or cache.shape[2] != x.shape[2]:
        raise ValueError("shapes: x [b][s][d], pos [b][s], cache [b][R][d]")
    a = KvWriteArgs()
    a.b, a.s, a.d = x.shape
    a.x, a.x_seq_stride = _ptr(x), _seq_major(x, "x", 2)
    a.pos, a.pos_seq_stride = _ptr(pos), _seq_major(pos, "pos", 1)
    if rope is not None:
        _need(rope, torch.float32, "rope", dev)
        if not rope.is_contiguous() or rope.dim() != 3:
            raise ValueError("rope table [max_pos][rd/2][2] contiguous")
        a.rope_dim, a.rope_cos_sin, a.max_pos = rope.shape[1] * 2, _ptr(rope), rope.shape[0]
    a.window = window
    if row0 is not None:
        _need(row0, torch.int32, "row0", dev)
        a.row0 = _ptr(row0)
    a.cache_rows = cache.shape[1]
    if cache.dtype == torch.bfloat16:
        _need(cache, torch.bfloat16, "cache", dev)
        a.kv_format = KV_BF16
    else:
        _need(cache, torch.uint8, "cache", dev)
        if cache_scale is None:
            raise ValueError("fp8 cache needs cache_scale")
        _need(cache_scale, torch.uint8, "cache_scale", dev)
        a.kv_format = KV_FP8
        a.cache_scale, a.cache_scale_seq_stride = _ptr(cache_scale), _seq_major(cache_scale, "cache_scale", 2)
    a.cache, a.cache_seq_stride = _ptr(cache), _seq_major(cache, "cache", 2)
    if rows_out is not None:
        _need(rows_out, torch.bfloat16, "rows_out", dev)
        if rows_out.shape != x.shape:
            raise ValueError("rows_out must be shaped like x")
        a.rows_out, a.rows_out_seq_stride = _ptr(rows_out), _seq_major(rows_out, "rows_out", 2)
    if check_idx:
        if err_word is None:
            raise ValueError("check_idx needs err_word")
        _need(err_word, torch.int32, "err_word", dev)
        a.flags, a.err_word = FLAG_CHECK_IDX, _ptr(err_word)
    _check("sa_kv_write", lib().sa_kv_write(C.byref(a), C.c_void_p(_stream(dev))))
    return rows_out


def indexer_topk(q, k, w, pos, ratio: int, *, topk: int | None = None, offset: int = 0,
                 cand=None, scores=None, idx=None):
    """The indexer (sa_indexer_topk in include/sa.h). q bf16 [b][s][h][d], k bf16
    [b][n_pos][d], w f32 [b][s][h], pos int32 [b][s], cand uint8 [b][s][n_pos] or None.
    Returns (scores f32 [b][s][n_pos], idx int32 [b][s][>= topk] or None); with topk None
    only the scores are computed. idx may be a view into a larger list buffer (its first
    topk columns are written)."""
    dev = q.device
    _need(q, torch.bfloat16, "q", dev)
    _need(k, torch.bfloat16, "k", dev)
    _need(w, torch.float32, "w", dev)
    _need(pos, torch.int32, "pos", dev)
    if q.dim() != 4 or k.dim() != 3 or k.shape[0] != q.shape[0] or k.shape[2] != q.shape[3] \
            or w.shape != q.shape[:3] or pos.shape != q.shape[:2]:
        raise ValueError("shapes: q [b][s][h][d], k [b][n_pos][d], w [b][s][h], pos [b][s]")
    b, s, h, d = q.shape
    n_pos = k.shape[1]
    if scores is None:
        scores = torch.empty(b, s, n_pos, dtype=torch.float32, device=dev)
    _need(scores, torch.float32, "scores", dev)
    a = IndexerArgs()
    a.b, a.s, a.h, a.d, a.n_pos, a.ratio = b, s, h, d, n_pos, ratio
    a.q, a.q_seq_stride = _ptr(q), _seq_major(q, "q", 3)
    a.k, a.k_seq_stride = _ptr(k), _seq_major(k, "k", 2)
    a.w, a.w_seq_stride = _ptr(w), _seq_major(w, "w", 2)
    a.pos, a.pos_seq_stride = _ptr(pos), _seq_major(pos, "pos", 1)
    if cand is not None:
        _need(cand, torch.uint8, "cand", dev)
        if cand.shape != (b, s, n_pos):
            raise ValueError("cand must be [b][s][n_pos]")
        a.cand, a.cand_seq_stride = _ptr(cand), _seq_major(cand, "cand", 2)
    if scores.shape != (b, s, n_pos):
        raise ValueError("scores must be [b][s][n_pos]")
    a.scores, a.scores_seq_stride = _ptr(scores), _seq_major(scores, "scores", 2)
    if topk is not None:
        if idx is None:
            idx = torch.empty(b, s, topk, dtype=torch.int32, device=dev)
        _need(idx, torch.int32, "idx", dev)
        if idx.dim() != 3 or idx.shape[:2] != (b, s) or idx.shape[2] < topk or idx.stride(2) != 1:
            raise ValueError("idx must be [b][s][>= topk] with unit column stride")
        a.topk, a.offset = topk, offset
        a.idx, a.idx_seq_stride, a.idx_row_stride = _ptr(idx), idx.stride(0), idx.stride(1)
    _check("sa_indexer_topk", lib().sa_indexer_topk(C.byref(a), C.c_void_p(_stream(dev))))
    return scores, idx


def candidate_blocks(logits, pos, ratio: int, topk_blocks: int, block_size: int, *, mask=None):
    """select_candidate_blocks (sa_candidate_blocks in include/sa.h): logits f32
    [b][s][n_pos], pos int32 [b][s]; returns the uint8 mask [b][s][n_pos]."""
    dev = logits.device
    _need(logits, torch.float32, "logits", dev)
    _need(pos, torch.int32, "pos", dev)
    if logits.dim() != 3 or pos.shape != logits.shape[:2]:
        raise ValueError("shapes: logits [b][s][n_pos], pos [b][s]")
    b, s, n_pos = logits.shape
    if mask is None:
        mask = torch.empty(b, s, n_pos, dtype=torch.uint8, device=dev)
    _need(mask, torch.uint8, "mask", dev)
    a = CandidateArgs()
    a.b, a.s, a.n_pos, a.ratio, a.topk_blocks, a.block_size = b, s, n_pos, ratio, topk_blocks, block_size
    a.logits, a.logits_seq_stride = _ptr(logits), _seq_major(logits, "logits", 2)
    a.pos, a.pos_seq_stride = _ptr(pos), _seq_major(pos, "pos", 1)
    a.mask, a.mask_seq_stride = _ptr(mask), _seq_major(mask, "mask", 2)
    _check("sa_candidate_blocks", lib().sa_candidate_blocks(C.byref(a), C.c_void_p(_stream(dev))))
    return mask


def grouped_proj(o, w, *, w_scale=None, out=None):
    """The grouped output projection (sa_grouped_proj in include/sa.h). o: bf16 holding m
    tokens of g * kg elements (e.g. sparse_attn's output [b][s][h][d]; viewed as [m][g * kg]
    without a copy); w: bf16 [g][r][kg], or uint8 e4m3 codes [g][r][kg] with w_scale uint8
    [g][r][kg/32]. Returns out, bf16 [m][g][r]."""
    dev = o.device
    _need(o, torch.bfloat16, "o", dev)
    if w.dim() != 3:
        raise ValueError("w must be [g][r][kg]")
    g, r, kg = w.shape
    if o.numel() % (g * kg) != 0:
        raise ValueError("o must hold whole tokens of g * kg elements")
    tok = o.view(-1, g * kg)
    m = tok.shape[0]
    if out is None:
        out = torch.empty(m, g, r, dtype=torch.bfloat16, device=dev)
    _need(out, torch.bfloat16, "out", dev)
    if tuple(out.shape) != (m, g, r) or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 [m][g][r]")
    if not w.is_contiguous():
        raise ValueError("w must be contiguous")
    a = GroupedProjArgs()
    a.m, a.g, a.r, a.kg = m, g, r, kg
    a.o, a.o_stride = _ptr(tok), tok.stride(0)
    if w.dtype == torch.bfloat16:
        _need(w, torch.bfloat16, "w", dev)
        a.w_format = KV_BF16
    else:
        _need(w, torch.uint8, "w", dev)
        if w_scale is None:
            raise ValueError("fp8 weights need w_scale")
        _need(w_scale, torch.uint8, "w_scale", dev)
        a.w_format, a.w_scale = KV_FP8, _ptr(w_scale)
    a.w = _ptr(w)
    a.out, a.out_stride = _ptr(out), g * r
    _check("sa_grouped_proj", lib().sa_grouped_proj(C.byref(a), C.c_void_p(_stream(dev))))
    return out


def rope_table(rope_dim: int, max_pos: int, base: float = 10000.0, device="cuda", *,
               original_seq_len: int = 0, factor: float = 1.0, beta_fast: float = 32.0,
               beta_slow: float = 1.0, out=None):
    """The (cos, sin) table of the inverse-RoPE epilogue, f32 [max_pos][rope_dim/2][2],
    computed by sa_rope_table on the device (include/sa.h)."""
    if out is None:
        out = torch.empty(max_pos, rope_dim // 2, 2, dtype=torch.float32, device=device)
    _need(out, torch.float32, "out")
    if not out.is_contiguous() or tuple(out.shape) != (max_pos, rope_dim // 2, 2):
        raise ValueError("out must be a contiguous f32 [max_pos][rope_dim/2][2]")
    _check("sa_rope_table", lib().sa_rope_table(
        rope_dim, max_pos, original_seq_len, base, factor, beta_fast, beta_slow, _ptr(out),
        C.c_void_p(_stream(out.device))))
    return out
