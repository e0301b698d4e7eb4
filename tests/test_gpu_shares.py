"""GPU parity of one GPU's share under Ulysses context parallelism and under
tensor parallelism, against the fp64 oracle (oracle/shares.py).

Ulysses: the receive-side layouts of both all-to-alls (attn_ulysses_gather,
attn_ulysses_unpack_o) are pure data movement and must be bit-exact; the
rank's attention (attn_heads_forward on its heads over the full sequence) is
compared with the oracle, and running every rank's share reproduces the
one-shot attention over all heads bit for bit (the per-head arithmetic does
not depend on which heads share a launch).

Tensor parallelism: each rank's partial output (attn_block_create_shard) is
compared with the oracle's, and the partial outputs summed over ranks with
the unsharded block (the all-reduce identity).

Workloads: the Ulysses share of rank 0 at seq 32768, hidden 4096, 32 heads
over 8 ranks (4 heads over the full sequence), and the TP share at seq 8192,
hidden 4096, 8 ranks, on seeded sampled rows; small shapes on every row.
Inputs: long_context_self_amd.synthetic."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from oracle import shares
from long_context_self_amd import binding as B
from long_context_self_amd.synthetic import attention_inputs, block_inputs, sample_rows

from .gpu_util import REL_L2_F32, assert_close, dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    B.lib()


def _vt(v):
    """[H][S][d] -> [H][d][ATTN_VT_LD(S)] (zero padding)."""
    hh, s, d = v.shape
    out = np.zeros((hh, d, B.vt_ld(s)), dtype=v.dtype)
    out[:, :, :s] = v.transpose(0, 2, 1)
    return out


# ------------------------------------------------------------------ Ulysses
@pytest.mark.parametrize("n,hl,s,d,dt", [(8, 4, 2048, 128, np.float16), (4, 2, 512, 128, np.float16),
                                         (2, 3, 48, 64, np.float32)])
def test_ulysses_gather_is_exact(n, hl, s, d, dt):
    say(f"Ulysses gather N={n} Hl={hl} S={s} d={d} {dt.__name__}")
    rng = np.random.default_rng(11)
    hh = n * hl
    t_q = rng.standard_normal((hh, s, d)).astype(dt)
    t_k = rng.standard_normal((hh, s, d)).astype(dt)
    t_vt = rng.standard_normal((hh, d, s)).astype(dt)
    tdt = torch.float16 if dt == np.float16 else torch.float32
    for r in (0, n - 1):
        rq, rk = shares.ulysses_recv_qk(t_q, n, r), shares.ulysses_recv_qk(t_k, n, r)
        rvt = shares.ulysses_recv_vt(t_vt, n, r)
        q = torch.empty((hl, s, d), dtype=tdt, device="cuda")
        k = torch.empty_like(q)
        vt = torch.empty((hl, d, B.vt_ld(s)), dtype=tdt, device="cuda")
        B.attn_ulysses_gather(n, hl, d, s, dev(rq), dev(rk), dev(rvt), q, k, vt, dtype=tdt)
        assert np.array_equal(host(q), shares.ulysses_gather_qk(rq).astype(dt))
        assert np.array_equal(host(k), shares.ulysses_gather_qk(rk).astype(dt))
        assert np.array_equal(host(vt), shares.ulysses_gather_vt(rvt).astype(dt))


@pytest.mark.parametrize("n,hh,rows,d", [(8, 32, 512, 128), (4, 8, 40, 128), (3, 6, 8, 64)])
def test_ulysses_unpack_is_exact(n, hh, rows, d):
    say(f"Ulysses unpack N={n} H={hh} rows={rows}")
    rng = np.random.default_rng(12)
    dt = np.float16 if d == 128 else np.float32
    tdt = torch.float16 if dt == np.float16 else torch.float32
    recv = rng.standard_normal((n, rows, hh // n * d)).astype(dt)
    o = torch.empty((rows, hh * d), dtype=tdt, device="cuda")
    B.attn_ulysses_unpack_o(n, hh, d, rows, dev(recv), o, dtype=tdt)
    assert np.array_equal(host(o), shares.ulysses_unpack_o(recv))


def _ulysses_rank(q, k, vt_full, n, r, s, d, lse=True):
    """One rank's share on the GPU: receive blocks (built from the head-major
    tensors by the all-to-all layout), gather, attention of its heads."""
    hh = q.shape[0]
    hl = hh // n
    rq = dev(shares.ulysses_recv_qk(q, n, r))
    rk = dev(shares.ulysses_recv_qk(k, n, r))
    rvt = dev(shares.ulysses_recv_vt(vt_full[:, :, :s], n, r))
    gq = torch.empty((hl, s, d), dtype=torch.float16, device="cuda")
    gk = torch.empty_like(gq)
    gvt = torch.empty((hl, d, B.vt_ld(s)), dtype=torch.float16, device="cuda")
    B.attn_ulysses_gather(n, hl, d, s, rq, rk, rvt, gq, gk, gvt)
    del rq, rk, rvt
    o = torch.empty((s, hl * d), dtype=torch.float16, device="cuda")
    ls = torch.empty((hl, s), dtype=torch.float32, device="cuda") if lse else None
    B.attn_heads_forward(hl, d, gq, gk, gvt, s, o, hl * d, ls)
    return o, ls


def test_ulysses_share_small_all_rows():
    n, hh, s, d = 4, 8, 2048, 128
    say(f"Ulysses share N={n} H={hh} S={s}")
    q, k, v = attention_inputs(hh, s, s, d, seed=21)
    vt = _vt(v)
    for r in (0, n - 1):
        o, lse = _ulysses_rank(q, k, vt, n, r, s, d)
        o_ref, lse_ref = shares.ulysses_share(q, k, v, n, r)
        assert_close(host(o), o_ref, what=f"rank {r} O")
        assert_close(host(lse), lse_ref, what=f"rank {r} LSE")


def test_ulysses_all_ranks_equal_one_shot_attention():
    # Below 1024 keys no launch plan splits keys, so the share of any head
    # count runs the same per-row arithmetic as the one-shot call.
    n, hh, s, d = 8, 16, 960, 128
    say(f"Ulysses: all {n} ranks' shares vs one attention over all {hh} heads (bit-exact)")
    q, k, v = attention_inputs(hh, s, s, d, seed=22)
    vt = _vt(v)
    full = torch.empty((s, hh * d), dtype=torch.float16, device="cuda")
    full_lse = torch.empty((hh, s), dtype=torch.float32, device="cuda")
    B.attn_heads_forward(hh, d, dev(q), dev(k), dev(vt), s, full, hh * d, full_lse)
    hl = hh // n
    for r in range(n):
        o, lse = _ulysses_rank(q, k, vt, n, r, s, d)
        assert torch.equal(o, full[:, r * hl * d:(r + 1) * hl * d]), f"rank {r} O differs"
        assert torch.equal(lse, full_lse[r * hl:(r + 1) * hl]), f"rank {r} LSE differs"


def test_ulysses_share_config_seq32768_rank0_sampled():
    n, hh, s, d = 8, 32, 32768, 128
    say("Ulysses share: rank 0 of 8, seq 32768, 32 heads (4 local), sampled rows")
    q, k, v = attention_inputs(hh, s, s, d, seed=23)
    vt = _vt(v)
    o, lse = _ulysses_rank(q, k, vt, n, 0, s, d)
    rows = sample_rows(s, 128, seed=23, must=[s // 8 * i for i in range(9)])
    o_r, lse_r = host(o[rows]), host(lse[:, rows])
    del o, lse
    hl = hh // n
    o_ref, lse_ref = oracle.partial_attention(q[:hl, rows], k[:hl], v[:hl])
    assert_close(o_r, oracle.merge_heads(o_ref), what="rank 0 O (sampled)")
    assert_close(lse_r, lse_ref, what="rank 0 LSE (sampled)")


# ------------------------------------------------------- tensor parallelism
def _tp_partials(x, ws, nh, n, ranks, seq):
    outs = {}
    for r in ranks:
        blk = B.AttnBlock(*(dev(w) for w in ws), nh, seq, n_ranks=n, rank=r)
        outs[r] = blk.forward(dev(x))
        blk.close()
    return outs


@pytest.mark.parametrize("seq,h,nh,n", [(1000, 512, 4, 2), (300, 1024, 8, 4)])
def test_tp_share_f16_small_all_rows(seq, h, nh, n):
    say(f"TP share S={seq} h={h} H={nh} N={n}")
    x, [ws] = block_inputs(seq, h, 1, dtype=np.float16, seed=31)
    outs = _tp_partials(x, ws, nh, n, range(n), seq)
    total = np.zeros((seq, h))
    for r, y in outs.items():
        yr = host(y)
        assert_close(yr, shares.tp_share(x, *ws, nh, n, r), what=f"rank {r} partial y")
        total += yr
    assert_close(total, oracle.block_forward(x, *ws, nh), what="sum of partials (all-reduce)")


@pytest.mark.parametrize("seq,h,nh,n", [(2048, 1024, 8, 4), (1500, 512, 4, 2)])
def test_tp_share_key_split_all_rows(seq, h, nh, n):
    # few heads per rank: the attention splits its keys into ranges merged by LSE
    say(f"TP share with key-split attention S={seq} h={h} H={nh} N={n}")
    x, [ws] = block_inputs(seq, h, 1, dtype=np.float16, seed=34)
    hl, d = nh // n, h // nh
    for r in (0, n - 1):
        blk = B.AttnBlock(*(dev(w) for w in ws), nh, seq, n_ranks=n, rank=r)
        attn = torch.empty((seq, hl * d), dtype=torch.float16, device="cuda")
        lse = torch.empty((hl, seq), dtype=torch.float32, device="cuda")
        y = blk.forward(dev(x), taps=B.Taps(None, None, None, attn.data_ptr(), lse.data_ptr(), 0))
        blk.close()
        assert_close(host(y), shares.tp_share(x, *ws, nh, n, r), what=f"rank {r} partial y")
        ref = oracle.block_forward(x, *ws, nh, taps=True)
        assert_close(host(attn), ref["o"][:, r * hl * d:(r + 1) * hl * d], what=f"rank {r} attention output")
        assert_close(host(lse), ref["lse"][r * hl:(r + 1) * hl], what=f"rank {r} LSE")


def test_tp_share_tiny_fp32():
    seq, h, nh, n = 256, 256, 4, 4
    say("TP share tiny fp32, 4 ranks")
    x, [ws] = block_inputs(seq, h, 1, dtype=np.float32, seed=32)
    outs = _tp_partials(x, ws, nh, n, range(n), seq)
    for r, y in outs.items():
        assert_close(host(y), shares.tp_share(x, *ws, nh, n, r), rel=REL_L2_F32, mabs=1e-5, what=f"rank {r}")


def test_tp_share_with_taps_holds_local_heads():
    seq, h, nh, n, r = 512, 1024, 8, 4, 2
    x, [ws] = block_inputs(seq, h, 1, dtype=np.float16, seed=33)
    hl, d = nh // n, h // nh
    blk = B.AttnBlock(*(dev(w) for w in ws), nh, seq, n_ranks=n, rank=r)
    attn = torch.empty((seq, hl * d), dtype=torch.float16, device="cuda")
    lse = torch.empty((hl, seq), dtype=torch.float32, device="cuda")
    blk.forward(dev(x), taps=B.Taps(None, None, None, attn.data_ptr(), lse.data_ptr(), 0))
    blk.close()
    ref = oracle.block_forward(x, *ws, nh, taps=True)
    assert_close(host(attn), ref["o"][:, r * hl * d:(r + 1) * hl * d], what="local heads' attention output")
    assert_close(host(lse), ref["lse"][r * hl:(r + 1) * hl], what="local heads' LSE")


def test_tp_share_config_seq8192_hidden4096_sampled():
    seq, h, nh, n = 8192, 4096, 32, 8
    say("TP share seq 8192 hidden 4096, 8 ranks: ranks 0 and 7 on sampled rows")
    x, [ws] = block_inputs(seq, h, 1, dtype=np.float16, seed=0)
    outs = _tp_partials(x, ws, nh, n, (0, 7), seq)
    rows = sample_rows(seq, 128, seed=0)
    for r, y in outs.items():
        assert_close(host(y[rows]), shares.tp_share(x, *ws, nh, n, r, rows=rows), what=f"rank {r} partial y")
