"""Runs a seeded workload through the GPU library and, independently, through the CPU
oracle. The two sides share only the raw draws from sa_workloads: each does its own fp8
round trip of the KV rows, its own window index lists and its own rotary table."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import sa_workloads as W

# The acceptance bound on bf16 outputs, elementwise: |gpu - oracle| <= ATOL + RTOL*|oracle|.
ATOL, RTOL = 8e-3, 1.6e-2


def u16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32_of_u16(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).float().numpy()


# ------------------------------------------------------------------ GPU side
def gpu_indices(w: W.Workload, device="cuda") -> torch.Tensor:
    import sparse_latent_attention_attn_amd as sa
    idx = torch.empty(w.b, w.s, w.topk, dtype=torch.int32, device=device)
    view = idx.view(w.win_nseq, w.win_seqlen, w.topk)
    sp = None if w.win_start_pos is None else w.win_start_pos.to(device)
    sa.window_topk_idxs(w.window, w.win_seqlen, w.win_nseq, start_pos=sp, out=view)
    if w.comp_idx is not None:
        idx[:, :, w.win_cols:] = w.comp_idx.to(device)
    return idx


def gpu_inputs(w: W.Workload, kv_format: str = "bf16", device="cuda"):
    """Device tensors for sparse_attn: (q, kv, kv_scale, sink, idx)."""
    import sparse_latent_attention_attn_amd as sa
    q = w.q.to(device)
    kv_raw = w.kv.to(device)
    sink = w.sink.to(device)
    idx = gpu_indices(w, device)
    kv_scale = None
    if kv_format == "fp8":
        codes, scales = sa.quant_kv_fp8(kv_raw, want=("codes", "scales"))
        kv, kv_scale = codes, scales
    elif w.kv_roundtrip:
        (kv,) = sa.quant_kv_fp8(kv_raw, want=("roundtrip",))
    else:
        kv = kv_raw
    return q, kv, kv_scale, sink, idx


def gpu_run(w: W.Workload, kv_format: str = "bf16", rope: bool = True, device="cuda"):
    import sparse_latent_attention_attn_amd as sa
    q, kv, kv_scale, sink, idx = gpu_inputs(w, kv_format, device)
    rp = (sa.rope_table(w.rd, w.max_pos, w.rope_base, device), w.pos.to(device)) if rope else None
    out = sa.sparse_attn(q, kv, sink, idx, w.scale, kv_scale=kv_scale, rope=rp)
    torch.cuda.synchronize()
    return out, idx


# ------------------------------------------------------------------ oracle side
def oracle_indices(w: W.Workload) -> np.ndarray:
    sp = None if w.win_start_pos is None else w.win_start_pos.numpy()
    win = oracle.window_topk_idxs(w.window, w.win_seqlen, sp, nseq=w.win_nseq).reshape(w.b, w.s, -1)
    if w.comp_idx is None:
        return np.ascontiguousarray(win)
    return np.ascontiguousarray(np.concatenate([win, w.comp_idx.numpy()], axis=-1))


def oracle_kv(w: W.Workload, round_trip: bool, seqs=None, idx=None, qsel=None) -> np.ndarray:
    """The kv rows the oracle reads: the raw draws, or their block-32 fp8 round trip. With
    idx and qsel given, only the rows the selected queries name are round-tripped (the
    oracle reads no other row)."""
    kv = u16(w.kv)
    if not round_trip:
        return kv
    out = kv.copy()
    for sq in (range(w.b) if seqs is None else seqs):
        if idx is None or qsel is None:
            out[sq] = oracle.act_quant(kv[sq])[0]
            continue
        q_of_seq = [int(i) % w.s for i in qsel if int(i) // w.s == sq]
        named = idx[sq, q_of_seq].reshape(-1)
        rows = np.unique(named[named >= 0])
        if rows.size:
            out[sq, rows] = oracle.act_quant(np.ascontiguousarray(kv[sq, rows]))[0]
    return out


def oracle_core(w: W.Workload, qsel=None, round_trip=None, nthreads: int = 0):
    """sparse_attn of the oracle, before the epilogue: bf16 (u16) [nsel][h][d]."""
    rt = w.kv_roundtrip if round_trip is None else round_trip
    seqs = None if qsel is None else sorted({int(i) // w.s for i in qsel})
    idx = oracle_indices(w)
    kv = oracle_kv(w, rt, seqs, idx, qsel)
    return oracle.sparse_attn(u16(w.q), kv, w.sink.numpy(), idx, w.scale, qsel=qsel,
                              nthreads=nthreads)


def oracle_rotate(w: W.Workload, core: np.ndarray, qsel=None):
    """The inverse-RoPE epilogue of the oracle on core outputs of the queries qsel."""
    cs = oracle.freqs_cis(w.rd, w.max_pos, w.rope_base)
    pos = w.pos.numpy().reshape(-1)
    pos = pos if qsel is None else pos[np.asarray(qsel)]
    return oracle.apply_rotary(core, w.rd, cs, pos, inverse=True)


def oracle_run(w: W.Workload, qsel=None, rope: bool = True, round_trip=None, nthreads: int = 0):
    """bf16 (u16) [nsel][h][d] for the flattened queries qsel (all if None)."""
    out = oracle_core(w, qsel, round_trip, nthreads)
    return oracle_rotate(w, out, qsel) if rope else out


def assert_close(gpu_u16: np.ndarray, ref_u16: np.ndarray, what: str = ""):
    g = f32_of_u16(gpu_u16).astype(np.float64)
    r = f32_of_u16(ref_u16).astype(np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    err = np.abs(g - r)
    bound = ATOL + RTOL * np.abs(r)
    # NaN in either side is a failure: ~(err <= bound) is True where err is NaN
    bad = ~(err <= bound)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(np.isnan(err), np.inf, err - bound)), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements outside "
                             f"|gpu-oracle| <= {ATOL} + {RTOL}|oracle|; worst at {i}: "
                             f"gpu {g[i]} oracle {r[i]}")
    return float(err.max())
