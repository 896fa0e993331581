"""Seeded synthetic inputs for sparse latent attention, shared by the tests, the smoke check
and the bench.

This module draws random numbers and lays them out; it holds none of the method's
arithmetic. The block-32 fp8 round trip of the KV rows, the window index lists, the
rotary table and the attention itself are computed separately by the GPU library and by
the CPU oracle from the raw draws returned here.

Workloads follow the shapes of DeepSeek-V4.1 attention (Attention.__init__ and the model
config on the pages: head_dim 512, rope_head_dim 64, window_size 128, index_topk 512,
compress ratio 4 for the compressed layers, softmax_scale = head_dim^-0.5):

  tiny_ring        1 sequence, window 8, prefill 12 tokens then decode steps 12 and 13
                   (the ring-cache worked example of the attention API docs); h=4, d=64, rd=16
  decode_window    32 sequences x 1 query, h=64, d=512, full 128-slot ring, topk 128
  prefill_window   1 sequence of 4096 queries, h=64, d=512, causal window 128 into the chunk
  decode_compress  64 sequences x 1 query, h=128, d=512, 128 ring rows + 16384 compressed
                   rows (context 65536, ratio 4), topk 128 + 512 (about 2% holes)
  prefill_compress 1 sequence of 8192 queries, h=128, d=512, 128 window rows + 2048
                   compressed rows (ratio 4), topk 128 + 2048 (causal, -1 padded)

Recipe (same for all): a CPU torch.Generator seeded with the workload's seed; draws in the
order q, kv, sink, then index randomness; q and kv are randn in f32 rounded to bf16, the
sink is randn * sink_std in f32 (std 1 for tiny_ring, 0.5 otherwise). ``kv_roundtrip``
says whether the consumer must pass kv through the block-32 fp8 round trip before use.
"""
from __future__ import annotations

import dataclasses

import torch

__all__ = ["Workload", "WORKLOADS", "make", "small_variant"]


@dataclasses.dataclass
class Workload:
    name: str
    b: int                   # sequences
    s: int                   # queries per sequence
    h: int
    d: int
    rd: int                  # rope dims at the end of each head's row (epilogue)
    window: int
    kv_rows: int             # rows of kv per sequence
    # "window sequences": how the window index builder sees the queries; the c5-style
    # workload treats each query t as a decode step at position t
    win_nseq: int
    win_seqlen: int
    win_start_pos: torch.Tensor | None
    comp_idx: torch.Tensor | None   # int32 [b][s][Tc], already offset, -1 = skip
    q: torch.Tensor                 # bf16 [b][s][h][d]
    kv: torch.Tensor                # bf16 [b][kv_rows][d], raw draws
    sink: torch.Tensor              # f32 [h]
    pos: torch.Tensor               # int32 [b][s] absolute positions (epilogue)
    kv_roundtrip: bool
    scale: float
    seed: int
    rope_base: float = 10000.0

    @property
    def win_cols(self) -> int:
        if self.win_start_pos is None:
            return min(self.win_seqlen, self.window)
        return self.window

    @property
    def topk(self) -> int:
        return self.win_cols + (0 if self.comp_idx is None else self.comp_idx.shape[-1])

    @property
    def max_pos(self) -> int:
        return int(self.pos.max().item()) + 1


def _scale(d: int) -> float:
    # softmax_scale = head_dim ** -0.5, held as an f32 (Attention.__init__)
    return float(torch.tensor(d ** -0.5, dtype=torch.float32).item())


def _rd(d: int) -> int:
    # rope_head_dim 64 of the model config; smaller heads keep a quarter of their width
    return 64 if d >= 256 else d // 4


def _draw(g, b, s, h, d, rows, sink_std):
    q = torch.randn(b, s, h, d, generator=g, dtype=torch.float32).to(torch.bfloat16)
    kv = torch.randn(b, rows, d, generator=g, dtype=torch.float32).to(torch.bfloat16)
    sink = torch.randn(h, generator=g, dtype=torch.float32) * sink_std
    return q, kv, sink


def tiny_ring(seed: int = 1):
    """The three regimes of the ring-cache example: returns a list of three step dicts.
    Step 0 is the 12-token prefill (kv = the chunk's own rows), steps 1 and 2 decode
    tokens 12 and 13 (kv = the ring after writing the new token)."""
    g = torch.Generator().manual_seed(seed)
    W, h, d, rd, S = 8, 4, 64, 16, 12
    q_pre = torch.randn(1, S, h, d, generator=g).to(torch.bfloat16)
    kv_pre = torch.randn(S, d, generator=g).to(torch.bfloat16)
    sink = torch.randn(h, generator=g, dtype=torch.float32)
    steps = [dict(kind="prefill", q=q_pre, kv_rows=kv_pre, start_pos=0)]
    for P in (12, 13):
        qd = torch.randn(1, 1, h, d, generator=g).to(torch.bfloat16)
        kvd = torch.randn(1, d, generator=g).to(torch.bfloat16)
        steps.append(dict(kind="decode", q=qd, kv_rows=kvd, start_pos=P))
    return dict(window=W, h=h, d=d, rd=rd, sink=sink, scale=_scale(d), steps=steps, seed=seed)


def decode_window(seed: int = 2, b: int = 32, h: int = 64, d: int = 512, window: int = 128):
    g = torch.Generator().manual_seed(seed)
    q, kv, sink = _draw(g, b, 1, h, d, window, 0.5)
    P = torch.randint(window - 1, 65536, (b,), generator=g, dtype=torch.int64).to(torch.int32)
    return Workload(name="decode_window", b=b, s=1, h=h, d=d, rd=_rd(d), window=window,
                    kv_rows=window, win_nseq=b, win_seqlen=1, win_start_pos=P.clone(),
                    comp_idx=None, q=q, kv=kv, sink=sink, pos=P.view(b, 1).clone(),
                    kv_roundtrip=True, scale=_scale(d), seed=seed)


def prefill_window(seed: int = 3, S: int = 4096, h: int = 64, d: int = 512, window: int = 128):
    g = torch.Generator().manual_seed(seed)
    q, kv, sink = _draw(g, 1, S, h, d, S, 0.5)
    pos = torch.arange(S, dtype=torch.int32).view(1, S)
    return Workload(name="prefill_window", b=1, s=S, h=h, d=d, rd=_rd(d), window=window,
                    kv_rows=S, win_nseq=1, win_seqlen=S, win_start_pos=None, comp_idx=None,
                    q=q, kv=kv, sink=sink, pos=pos, kv_roundtrip=True, scale=_scale(d),
                    seed=seed)


def decode_compress(seed: int = 4, b: int = 64, h: int = 128, d: int = 512, window: int = 128,
                    n_comp: int = 16384, n_sel: int = 512, hole_p: float = 0.02,
                    context: int = 65536):
    g = torch.Generator().manual_seed(seed)
    rows = window + n_comp
    q, kv, sink = _draw(g, b, 1, h, d, rows, 0.5)
    P = torch.full((b,), context - 1, dtype=torch.int32)
    comp = torch.empty(b, 1, n_sel, dtype=torch.int32)
    for i in range(b):
        pick = torch.randperm(n_comp, generator=g)[:n_sel].sort().values
        comp[i, 0] = (pick + window).to(torch.int32)
    holes = torch.rand(b, 1, n_sel, generator=g) < hole_p
    comp[holes] = -1
    return Workload(name="decode_compress", b=b, s=1, h=h, d=d, rd=_rd(d), window=window,
                    kv_rows=rows, win_nseq=b, win_seqlen=1, win_start_pos=P.clone(),
                    comp_idx=comp, q=q, kv=kv, sink=sink, pos=P.view(b, 1).clone(),
                    kv_roundtrip=True, scale=_scale(d), seed=seed)


def prefill_compress(seed: int = 5, S: int = 8192, h: int = 128, d: int = 512,
                     window: int = 128, ratio: int = 4):
    """Window part: query t sees positions t-window+1..t through the 128 ring rows (row
    p mod window), oldest first -- the decode list at position t. Compressed part: all
    (t+1)//ratio causal compressed positions, ascending, offset by the window rows, -1
    padded (never more than the 2048 columns, so no random selection is needed)."""
    g = torch.Generator().manual_seed(seed)
    n_comp = S // ratio
    rows = window + n_comp
    q, kv, sink = _draw(g, 1, S, h, d, rows, 0.5)
    t = torch.arange(S).view(S, 1)
    c = torch.arange(n_comp).view(1, n_comp)
    comp = torch.where(c < (t + 1) // ratio, c + window, torch.full_like(c, -1))
    comp = comp.to(torch.int32).view(1, S, n_comp)
    pos = torch.arange(S, dtype=torch.int32)
    return Workload(name="prefill_compress", b=1, s=S, h=h, d=d, rd=_rd(d), window=window,
                    kv_rows=rows, win_nseq=S, win_seqlen=1, win_start_pos=pos.clone(),
                    comp_idx=comp, q=q, kv=kv, sink=sink, pos=pos.view(1, S).clone(),
                    kv_roundtrip=True, scale=_scale(d), seed=seed)


WORKLOADS = {
    "decode_window": decode_window,
    "prefill_window": prefill_window,
    "decode_compress": decode_compress,
    "prefill_compress": prefill_compress,
}


def make(name: str, **kw) -> Workload:
    return WORKLOADS[name](**kw)


def small_variant(name: str, seed: int | None = None) -> Workload:
    """Shapes the oracle finishes in about a second that still span several key tiles,
    head tiles and a ragged tail."""
    if name == "decode_window":
        return decode_window(seed=seed or 12, b=5, h=64, d=512)
    if name == "prefill_window":
        return prefill_window(seed=seed or 13, S=301, h=64, d=512)
    if name == "decode_compress":
        return decode_compress(seed=seed or 14, b=3, h=128, d=512, n_comp=2048, n_sel=512)
    if name == "prefill_compress":
        return prefill_compress(seed=seed or 15, S=611, h=128, d=512, ratio=4)
    raise KeyError(name)


def rand_problem(seed: int, b: int, s: int, h: int, d: int, rows: int, topk: int,
                 hole_p: float = 0.1, dup: bool = False, sink_std: float = 1.0):
    """A generic random problem: idx drawn uniformly from [0, rows) with holes (-1) and,
    optionally, repeated entries. Returns (q, kv, sink, idx)."""
    g = torch.Generator().manual_seed(seed)
    q, kv, sink = _draw(g, b, s, h, d, rows, sink_std)
    if dup or topk > rows:
        idx = torch.randint(0, rows, (b, s, topk), generator=g, dtype=torch.int64)
    else:
        idx = torch.stack([torch.stack([torch.randperm(rows, generator=g)[:topk]
                                        for _ in range(s)]) for _ in range(b)])
    holes = torch.rand(b, s, topk, generator=g) < hole_p
    idx = idx.to(torch.int32)
    idx[holes] = -1
    return q, kv, sink, idx
