"""Plain CPU oracle for DeepSeek-V4.1 sparse latent attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package. The GPU library never uses it, and the two share no code.

This module is argument marshalling (numpy <-> ctypes) over ``liboracle.so``, built from
``sa_oracle.c`` by :func:`build`. The arithmetic, and the citation of the passage each
function follows, is in that C file.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sa_oracle.c")
# SA_ORACLE_LIB names another build of the same source (the sanitizer build of the tests)
_LIB_PATH = os.environ.get("SA_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=all"]


def build(force: bool = True, out: str | None = None, sanitize: bool = False) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, no FMA contraction, OpenMP). With
    sanitize, an AddressSanitizer + UndefinedBehaviorSanitizer build at -O1 (load it with
    libasan preloaded)."""
    out = out or _LIB_PATH
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        opt = SANITIZE_FLAGS if sanitize else ["-O2"]
        cmd = ["gcc", *opt, "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


class AttnProblem(C.Structure):
    _fields_ = [
        ("b", C.c_int32), ("s", C.c_int32), ("h", C.c_int32), ("d", C.c_int32),
        ("topk", C.c_int32), ("kv_rows", C.c_int32),
        ("q", C.c_void_p), ("q_seq_stride", C.c_int64),
        ("kv", C.c_void_p), ("kv_seq_stride", C.c_int64),
        ("sink", C.c_void_p),
        ("idx", C.c_void_p), ("idx_seq_stride", C.c_int64),
        ("scale", C.c_float),
    ]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = C.CDLL(_LIB_PATH)
        P, I32, I64, F = C.c_void_p, C.c_int32, C.c_int64, C.c_float
        sig = {
            "orc_bf16_to_f32": (F, [C.c_uint16]),
            "orc_f32_to_bf16": (C.c_uint16, [F]),
            "orc_f32_to_bf16_array": (None, [P, P, I64]),
            "orc_bf16_to_f32_array": (None, [P, P, I64]),
            "orc_pow2_ceil": (F, [F]),
            "orc_e4m3_encode": (C.c_uint8, [F]),
            "orc_e4m3_decode": (F, [C.c_uint8]),
            "orc_act_quant_rows": (C.c_int, [P, I64, I32, P, P, P]),
            "orc_fp8_storage_decode": (C.c_int, [P, P, I64, I32, P]),
            "orc_window_cols": (C.c_int, [I32, I32, P, I32, P]),
            "orc_window_topk_idxs": (C.c_int, [I32, I32, P, I32, P, P]),
            "orc_ring_prefill": (None, [P, I32, I32, P, I32]),
            "orc_ring_decode": (None, [P, I32, I32, P, I32]),
            "orc_sparse_attn": (C.c_int, [C.POINTER(AttnProblem), P, I64, P, I32]),
            "orc_sparse_attn_f64": (C.c_int, [C.POINTER(AttnProblem), P, I64, P, I32]),
            "orc_sparse_attn_weights_f64": (C.c_int, [C.POINTER(AttnProblem), I64, I32, P, P]),
            "orc_freqs_cis": (None, [I32, I32, F, P]),
            "orc_freqs_cis_yarn": (C.c_int, [I32, I32, I32, F, F, F, F, P]),
            "orc_apply_rotary": (C.c_int, [P, I64, I32, I32, I32, P, I32, P, I32]),
            "orc_max_threads": (I32, []),
            "orc_kv_write": (C.c_int, [P, I32, I32, I32, I32, P, I32, P, I32, P, I32, P, P, P, P]),
            "orc_index_scores": (C.c_int, [P, P, P, P, P, I32, I32, I32, I32, I32, I32, P, I32]),
            "orc_index_topk": (C.c_int, [P, I32, I32, I32, I32, I32, P]),
            "orc_candidate_blocks": (C.c_int, [P, P, I32, I32, I32, I32, I32, I32, P]),
            "orc_grouped_proj": (C.c_int, [P, I64, P, I32, I32, I32, I32, P, I32]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _u16(a) -> np.ndarray:
    """bf16 payload as uint16 (accepts uint16 arrays or torch bf16 tensors)."""
    if hasattr(a, "view") and hasattr(a, "dtype") and str(a.dtype) == "torch.bfloat16":
        a = a.contiguous().view(__import__("torch").int16).numpy().view(np.uint16)
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def max_threads() -> int:
    return int(lib().orc_max_threads())


# ---------------------------------------------------------------- scalar/vector numerics
def bf16_to_f32(x) -> np.ndarray:
    x = _u16(x)
    y = np.empty(x.shape, np.float32)
    lib().orc_bf16_to_f32_array(_ptr(x), _ptr(y), x.size)
    return y


def f32_to_bf16(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, np.uint16)
    lib().orc_f32_to_bf16_array(_ptr(x), _ptr(y), x.size)
    return y


def pow2_ceil(v: float) -> float:
    return float(lib().orc_pow2_ceil(float(v)))


def e4m3_encode(v: float) -> int:
    return int(lib().orc_e4m3_encode(float(v)))


def e4m3_decode(c: int) -> float:
    return float(lib().orc_e4m3_decode(int(c)))


# ---------------------------------------------------------------- fp8 block-32 round trip
def act_quant(x, d: int | None = None):
    """Block-32 ue8m0 round trip of bf16 rows. Returns (y_bf16, e4m3 codes, e8m0 bytes)."""
    x = _u16(x)
    d = d or x.shape[-1]
    rows = x.size // d
    y = np.empty_like(x)
    codes = np.empty(x.shape, np.uint8)
    scales = np.empty(x.shape[:-1] + (d // 32,), np.uint8)
    rc = lib().orc_act_quant_rows(_ptr(x), rows, d, _ptr(y), _ptr(codes), _ptr(scales))
    if rc:
        raise ValueError("orc_act_quant_rows rejected its arguments")
    return y, codes, scales


def fp8_storage_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    d = codes.shape[-1]
    y = np.empty(codes.shape, np.uint16)
    rc = lib().orc_fp8_storage_decode(_ptr(codes), _ptr(scales), codes.size // d, d, _ptr(y))
    if rc:
        raise ValueError("orc_fp8_storage_decode rejected its arguments")
    return y


# ---------------------------------------------------------------- window indices / ring
def window_topk_idxs(window: int, seqlen: int, start_pos=None, nseq: int = 1) -> np.ndarray:
    """int32 [nseq][seqlen][cols]. start_pos None: prefill of nseq sequences from position 0;
    otherwise a decode step, one position per sequence. Raises on the cases the oracle
    rejects."""
    if start_pos is None:
        sp, n = None, nseq
    else:
        sp = np.ascontiguousarray(np.atleast_1d(np.asarray(start_pos, np.int32)))
        n = sp.size
    spp = None if sp is None else _ptr(sp)
    cols = np.zeros(1, np.int32)
    rc = lib().orc_window_cols(window, seqlen, spp, n, _ptr(cols))
    if rc:
        raise ValueError(f"window_topk_idxs: status {rc}")
    out = np.empty((n, seqlen, int(cols[0])), np.int32)
    rc = lib().orc_window_topk_idxs(window, seqlen, spp, n, _ptr(out), _ptr(cols))
    if rc:
        raise ValueError(f"window_topk_idxs: status {rc}")
    return out


def ring_prefill(ring: np.ndarray, chunk_rows: np.ndarray) -> None:
    assert ring.dtype == np.uint16 and chunk_rows.dtype == np.uint16 and ring.flags.c_contiguous
    chunk_rows = np.ascontiguousarray(chunk_rows)
    lib().orc_ring_prefill(_ptr(ring), ring.shape[0], ring.shape[1], _ptr(chunk_rows),
                           chunk_rows.shape[0])


def ring_decode(ring: np.ndarray, row: np.ndarray, pos: int) -> None:
    assert ring.dtype == np.uint16 and ring.flags.c_contiguous
    row = np.ascontiguousarray(row, np.uint16)
    lib().orc_ring_decode(_ptr(ring), ring.shape[0], ring.shape[1], _ptr(row), pos)


# ---------------------------------------------------------------- sparse_attn
def _problem(q, kv, sink, idx, scale, keep):
    """q [b][s][h][d] bf16(u16), kv [b][R][d] bf16(u16), sink f32 [h], idx int32 [b][s][T]."""
    q, kv = _u16(q), _u16(kv)
    sink = np.ascontiguousarray(sink, np.float32)
    idx = np.ascontiguousarray(idx, np.int32)
    b, s, h, d = q.shape
    assert kv.ndim == 3 and kv.shape[0] == b and kv.shape[2] == d
    assert idx.shape[:2] == (b, s) and sink.shape == (h,)
    keep.extend([q, kv, sink, idx])
    return AttnProblem(b, s, h, d, idx.shape[2], kv.shape[1],
                       q.ctypes.data, s * h * d, kv.ctypes.data, kv.shape[1] * d,
                       sink.ctypes.data, idx.ctypes.data, s * idx.shape[2], float(scale))


def sparse_attn(q, kv, sink, idx, scale, qsel=None, nthreads: int = 0) -> np.ndarray:
    """bf16 (uint16) output [nsel][h][d] for the flattened queries qsel (all if None)."""
    keep = []
    p = _problem(q, kv, sink, idx, scale, keep)
    sel = None if qsel is None else np.ascontiguousarray(qsel, np.int64)
    n = p.b * p.s if sel is None else sel.size
    out = np.empty((n, p.h, p.d), np.uint16)
    rc = lib().orc_sparse_attn(C.byref(p), None if sel is None else _ptr(sel), n, _ptr(out),
                               nthreads)
    if rc:
        raise ValueError("orc_sparse_attn rejected its arguments")
    return out


def sparse_attn_f64(q, kv, sink, idx, scale, qsel=None, nthreads: int = 0) -> np.ndarray:
    keep = []
    p = _problem(q, kv, sink, idx, scale, keep)
    sel = None if qsel is None else np.ascontiguousarray(qsel, np.int64)
    n = p.b * p.s if sel is None else sel.size
    out = np.empty((n, p.h, p.d), np.float64)
    rc = lib().orc_sparse_attn_f64(C.byref(p), None if sel is None else _ptr(sel), n,
                                   _ptr(out), nthreads)
    if rc:
        raise ValueError("orc_sparse_attn_f64 rejected its arguments")
    return out


def sparse_attn_weights_f64(q, kv, sink, idx, scale, query: int, head: int):
    keep = []
    p = _problem(q, kv, sink, idx, scale, keep)
    w = np.empty(p.topk, np.float64)
    share = np.zeros(1, np.float64)
    rc = lib().orc_sparse_attn_weights_f64(C.byref(p), query, head, _ptr(w), _ptr(share))
    if rc:
        raise ValueError("orc_sparse_attn_weights_f64 rejected its arguments")
    return w, float(share[0])


# ---------------------------------------------------------------- rotary
def freqs_cis(rd: int, max_pos: int, base: float = 10000.0, original_seq_len: int = 0,
              factor: float = 1.0, beta_fast: float = 32.0, beta_slow: float = 1.0) -> np.ndarray:
    """f32 [max_pos][rd/2][2] of (cos, sin); YaRN when original_seq_len > 0."""
    out = np.empty((max_pos, rd // 2, 2), np.float32)
    if original_seq_len == 0:
        lib().orc_freqs_cis(rd, max_pos, float(base), _ptr(out))
        return out
    rc = lib().orc_freqs_cis_yarn(rd, max_pos, original_seq_len, float(base), float(factor),
                                  float(beta_fast), float(beta_slow), _ptr(out))
    if rc:
        raise ValueError("orc_freqs_cis_yarn rejected its arguments")
    return out


def apply_rotary(x: np.ndarray, rd: int, cos_sin: np.ndarray, pos, inverse: bool) -> np.ndarray:
    """x: bf16 (u16) [n][h][d]; returns a rotated copy."""
    y = np.array(_u16(x), copy=True)
    n, h, d = y.shape
    cs = np.ascontiguousarray(cos_sin, np.float32)
    pos = np.ascontiguousarray(pos, np.int32)
    rc = lib().orc_apply_rotary(_ptr(y), n, h, d, rd, _ptr(cs), cs.shape[0], _ptr(pos),
                                1 if inverse else 0)
    if rc:
        raise ValueError("orc_apply_rotary rejected its arguments")
    return y


# ---------------------------------------------------------------- KV write path
def kv_write(x, pos, rd: int, cos_sin, window: int, cache_rows: int, row0=None,
             cache_bf16=None, cache_codes=None, cache_scales=None, want_rows: bool = True):
    """x: bf16 (u16) [b][s][d]; pos int32 [b][s]. Updates the given caches in place
    ([b][cache_rows][d] u16, [b][cache_rows][d] u8, [b][cache_rows][d/32] u8) and returns the
    processed rows (bf16 u16 [b][s][d]) when want_rows."""
    x = _u16(x)
    b, s, d = x.shape
    pos = np.ascontiguousarray(pos, np.int32).reshape(b, s)
    cs = np.ascontiguousarray(cos_sin, np.float32) if rd > 0 else np.zeros((1, 1, 2), np.float32)
    r0 = None if row0 is None else np.ascontiguousarray(row0, np.int32)
    for c in (cache_bf16, cache_codes, cache_scales):
        assert c is None or (c.flags.c_contiguous and c.shape[0] == b and c.shape[1] == cache_rows)
    rows = np.empty_like(x) if want_rows else None
    rc = lib().orc_kv_write(_ptr(x), b, s, d, rd, _ptr(cs), cs.shape[0], _ptr(pos), window,
                            None if r0 is None else _ptr(r0), cache_rows,
                            None if cache_bf16 is None else _ptr(cache_bf16),
                            None if cache_codes is None else _ptr(cache_codes),
                            None if cache_scales is None else _ptr(cache_scales),
                            None if rows is None else _ptr(rows))
    if rc:
        raise ValueError("orc_kv_write rejected its arguments")
    return rows


# ---------------------------------------------------------------- indexer
def index_scores(q, k, w, pos, ratio: int, cand=None, nthreads: int = 0) -> np.ndarray:
    """q bf16 (u16) [b][s][h][d], k bf16 (u16) [b][n_pos][d], w f32 [b][s][h], pos int32
    [b][s], cand uint8 [b][s][n_pos] or None -> f32 [b][s][n_pos]."""
    q, k = _u16(q), _u16(k)
    b, s, h, d = q.shape
    n_pos = k.shape[1]
    w = np.ascontiguousarray(w, np.float32).reshape(b, s, h)
    pos = np.ascontiguousarray(pos, np.int32).reshape(b, s)
    c = None if cand is None else np.ascontiguousarray(cand, np.uint8).reshape(b, s, n_pos)
    out = np.empty((b, s, n_pos), np.float32)
    rc = lib().orc_index_scores(_ptr(q), _ptr(k), _ptr(w), _ptr(pos), None if c is None else _ptr(c),
                                b, s, h, d, n_pos, ratio, _ptr(out), nthreads)
    if rc:
        raise ValueError("orc_index_scores rejected its arguments")
    return out


def index_topk(scores, topk: int, offset: int) -> np.ndarray:
    scores = np.ascontiguousarray(scores, np.float32)
    b, s, n_pos = scores.shape
    out = np.empty((b, s, topk), np.int32)
    if lib().orc_index_topk(_ptr(scores), b, s, n_pos, topk, offset, _ptr(out)):
        raise ValueError("orc_index_topk rejected its arguments")
    return out


def candidate_blocks(logits, pos, ratio: int, topk_blocks: int, block_size: int) -> np.ndarray:
    logits = np.ascontiguousarray(logits, np.float32)
    b, s, n_pos = logits.shape
    pos = np.ascontiguousarray(pos, np.int32).reshape(b, s)
    out = np.empty((b, s, n_pos), np.uint8)
    if lib().orc_candidate_blocks(_ptr(logits), _ptr(pos), b, s, n_pos, ratio, topk_blocks,
                                  block_size, _ptr(out)):
        raise ValueError("orc_candidate_blocks rejected its arguments")
    return out


# ---------------------------------------------------------------- grouped output projection
def grouped_proj(o, w, nthreads: int = 0) -> np.ndarray:
    """o: bf16 (u16) [m][g][kg]; w: bf16 (u16) [g][r][kg] -> bf16 (u16) [m][g][r]."""
    o, w = _u16(o), _u16(w)
    m, g, kg = o.shape
    r = w.shape[1]
    assert w.shape == (g, r, kg)
    out = np.empty((m, g, r), np.uint16)
    if lib().orc_grouped_proj(_ptr(o), g * kg, _ptr(w), m, g, r, kg, _ptr(out), nthreads):
        raise ValueError("orc_grouped_proj rejected its arguments")
    return out
