"""sa_sparse_attn_noalloc (the allocation-free variant) against sa_sparse_attn, called
through the C ABI on plans that need a workspace (split partials, dequantised fp8 rows): two
calls in a row, the second on a smaller problem, each bit for bit equal to the workspace
entry point and within the tolerance of the oracle; and a plan larger than the static buffer
is refused."""
import ctypes as C
import sys

import numpy as np
import pytest
import torch

import oracle
import sa_workloads as W
from sa_harness import assert_close, u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sa():
    import sparse_latent_attention_attn_amd as sa
    sa.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return sa


def _call(sa, fn, q, kv, sink, idx, scale, out, kv_scale=None, rope=None, ws=None):
    a = sa.make_args(q, kv, sink, idx, scale, out, kv_scale=kv_scale, rope=rope, workspace=ws)
    st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    return getattr(sa.lib(), fn)(C.byref(a), st), a


# (seed, b, s, h, d, rows, topk, fmt): each pair runs big then small
PAIRS = [
    [(201, 3, 2, 64, 256, 3000, 2000, "bf16"), (202, 1, 1, 32, 256, 800, 700, "bf16")],
    [(203, 2, 1, 64, 512, 9000, 5000, "bf16"), (204, 1, 2, 16, 512, 6000, 4200, "bf16")],
    [(205, 2, 1, 48, 128, 4000, 3500, "fp8"), (206, 1, 1, 16, 64, 900, 640, "fp8")],
    # fp8 rows named by many queries: the workspace holds the dequantised rows (and, the
    # first time, split partials behind them)
    [(208, 1, 40, 16, 256, 4600, 4400, "fp8"), (209, 1, 64, 32, 512, 96, 80, "fp8")],
]


@pytest.mark.parametrize("pair", PAIRS, ids=["d256", "d512-long", "fp8", "fp8-dequantised"])
def test_noalloc_matches_workspace_entry_point(sa, pair):
    for seed, b, s, h, d, rows, topk, fmt in pair:
        print("[case] noalloc", seed, b, s, h, d, topk, fmt, file=sys.stderr, flush=True)
        q, kv, sink, idx = W.rand_problem(seed, b, s, h, d, rows, topk, 0.05, False)
        scale = float(np.float32(d ** -0.5))
        qd, sd, idd = q.cuda(), sink.cuda(), idx.cuda()
        kvd, kv_scale, kv_ref = kv.cuda(), None, u16(kv)
        if fmt == "fp8":
            kvd, kv_scale = sa.quant_kv_fp8(kvd, want=("codes", "scales"))
            kv_ref = oracle.act_quant(u16(kv).reshape(-1, d))[0].reshape(kv.shape)
        rd, max_pos = d // 4, 4096
        pos = torch.randint(0, max_pos, (b, s), generator=torch.Generator().manual_seed(seed),
                            dtype=torch.int32).cuda()
        rope = (sa.rope_table(rd, max_pos, 10000.0, "cuda"), pos)
        out_ws = torch.full_like(qd, float("nan"))
        out_na = torch.full_like(qd, float("nan"))
        probe = sa.make_args(qd, kvd, sd, idd, scale, out_ws, kv_scale=kv_scale, rope=rope)
        need = sa.sparse_attn_workspace_bytes(probe)
        assert 0 < need <= sa.NOALLOC_SCRATCH_BYTES, need
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        rc, _ = _call(sa, "sa_sparse_attn", qd, kvd, sd, idd, scale, out_ws, kv_scale, rope, ws)
        assert rc == 0
        rc, _ = _call(sa, "sa_sparse_attn_noalloc", qd, kvd, sd, idd, scale, out_na, kv_scale, rope)
        assert rc == 0
        torch.cuda.synchronize()
        assert torch.equal(out_na.view(torch.int16), out_ws.view(torch.int16))
        core = oracle.sparse_attn(u16(q), kv_ref, sink.numpy(), idx.numpy(), scale)
        ref = oracle.apply_rotary(core, rd, oracle.freqs_cis(rd, max_pos, 10000.0),
                                  pos.view(-1).cpu().numpy(), inverse=True)
        assert_close(u16(out_na).reshape(-1, h, d), ref, f"noalloc {seed}")


def test_noalloc_without_splits_and_too_large_plans(sa):
    """A plan without splits needs no buffer at all; one needing more than the static buffer
    is refused with SA_ERR_SCRATCH before any launch (out stays untouched)."""
    q, kv, sink, idx = W.rand_problem(207, 2, 3, 32, 64, 100, 60, 0.1, False)
    out = torch.zeros_like(q.cuda())
    rc, _ = _call(sa, "sa_sparse_attn_noalloc", q.cuda(), kv.cuda(), sink.cuda(), idx.cuda(), 0.125, out)
    assert rc == 0
    ref = oracle.sparse_attn(u16(q), u16(kv), sink.numpy(), idx.numpy(), 0.125)
    assert_close(u16(out).reshape(-1, 32, 64), ref, "noalloc no splits")
    # 256 sequences x 128 heads x d 512 with 5000 columns: ~135 MB of partials
    big = sa.AttnArgs()
    big.b, big.s, big.h, big.d, big.topk, big.kv_rows = 256, 1, 128, 512, 5000, 8
    for f in ("q", "kv", "sink", "idx", "out"):
        setattr(big, f, 0x10000)
    big.q_seq_stride = big.out_seq_stride = 128 * 512
    big.kv_seq_stride, big.idx_seq_stride, big.scale = 8 * 512, 5000, 0.04
    n = C.c_size_t(0)
    assert sa.lib().sa_sparse_attn_workspace(C.byref(big), C.byref(n)) == 0
    assert n.value > sa.NOALLOC_SCRATCH_BYTES
    assert sa.lib().sa_sparse_attn_noalloc(C.byref(big), None) == sa.SA_ERR_SCRATCH
    assert b"scratch" in sa.lib().sa_status_string(sa.SA_ERR_SCRATCH)
