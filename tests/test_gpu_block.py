"""GPU parity of the whole block (attn_block_forward) and of the
context-parallel rank share against the fp64 oracle.

Small and ragged shapes are compared element by element on every row. The
full-size workloads -- seq 8192 / 16384 / 32768 / 65536 at hidden 4096 with 32
heads, seq 8192 at hidden 8192 with 64 heads, the rank share (a 1/8 query chunk
of seq 32768 against K/V streamed in 8 blocks), and 6 stacked blocks at seq
32768 -- run in the same launch configuration the benchmark times and are
compared on seeded sampled rows that the oracle computes exactly (K and V
always over all rows). Inputs: the seeded recipe of
long_context_self_amd.synthetic."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from long_context_self_amd import binding as B
from long_context_self_amd.synthetic import block_inputs, sample_rows

from .gpu_util import (REL_L2_F32, REL_L2_SPLIT, assert_close, dev, host, rel_l2, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    B.lib()


def _taps(seq, h, nh, d, dtype, lse=True, qkv_only=False, v_rows=False):
    t = {
        "q_scaled": torch.empty((nh, seq, d), dtype=dtype, device="cuda"),
        "k": torch.empty((nh, seq, d), dtype=dtype, device="cuda"),
        "v_t": torch.zeros((nh, d, B.vt_ld(seq)), dtype=dtype, device="cuda"),
        "attn_out": torch.empty((seq, h), dtype=dtype, device="cuda"),
        "lse": torch.empty((nh, seq), dtype=torch.float32, device="cuda") if lse else None,
        "v": torch.empty((nh, seq, d), dtype=dtype, device="cuda") if v_rows else None,
    }
    c = B.Taps(t["q_scaled"].data_ptr(), t["k"].data_ptr(), t["v_t"].data_ptr(), t["attn_out"].data_ptr(),
               t["lse"].data_ptr() if lse else None, 1 if qkv_only else 0, None,
               t["v"].data_ptr() if v_rows else None)
    return t, c


def _block(ws, nh, max_tokens):
    wq, wk, wv, wo = (dev(w) for w in ws)
    return B.AttnBlock(wq, wk, wv, wo, nh, max_tokens)


def _check_all_rows(seq, h, nh, dtype, rel, mabs):
    say(f"block S={seq} h={h} H={nh} {dtype.__name__}")
    x, [ws] = block_inputs(seq, h, 1, dtype=dtype, seed=0)
    d = h // nh
    tdt = torch.float16 if dtype == np.float16 else torch.float32
    blk = _block(ws, nh, seq)
    t, c = _taps(seq, h, nh, d, tdt, v_rows=True)
    y = blk.forward(dev(x), taps=c)
    ref = oracle.block_forward(x, *ws, nh, taps=True)
    # the row-major V tap is the exact transpose of the V^T tap
    assert torch.equal(t["v"], t["v_t"][:, :, :seq].transpose(1, 2))
    assert_close(host(t["v"]), ref["v"], rel=rel, mabs=mabs, what="v")
    assert_close(host(y), ref["y"], rel=rel, mabs=mabs, what="y")
    assert_close(host(t["q_scaled"]), ref["q_scaled"], rel=rel, mabs=mabs, what="q_scaled")
    assert_close(host(t["k"]), ref["k"], rel=rel, mabs=mabs, what="k")
    vt = host(t["v_t"])[:, :, :seq]
    assert_close(vt, ref["v"].transpose(0, 2, 1), rel=rel, mabs=mabs, what="v_t")
    assert_close(host(t["attn_out"]), ref["o"], rel=rel, mabs=mabs, what="attn_out")
    assert_close(host(t["lse"]), ref["lse"], rel=rel, mabs=mabs, what="lse")
    # the same block without taps gives the same y, bit for bit
    y2 = blk.forward(dev(x))
    assert torch.equal(y, y2)
    blk.close()


def test_tiny_config_fp32_block():
    # seq 256, hidden 256, 4 heads of 64, fp32, seed 0
    _check_all_rows(256, 256, 4, np.float32, REL_L2_F32, 1e-5)


def test_tiny_config_fp32_rank_share_four_chunks():
    say("tiny fp32: QKV taps, K/V split into 4 chunks, LSE merge")
    seq, h, nh, d = 256, 256, 4, 64
    x, [ws] = block_inputs(seq, h, 1, dtype=np.float32, seed=0)
    blk = _block(ws, nh, seq)
    t, c = _taps(seq, h, nh, d, torch.float32, lse=False, qkv_only=True)
    blk.forward(dev(x), taps=c)
    ld = B.vt_ld(seq)
    o_parts = torch.empty((4, nh, seq, d), dtype=torch.float32, device="cuda")
    lse_parts = torch.empty((4, nh, seq), dtype=torch.float32, device="cuda")
    for b in range(4):
        B.attn_partial_forward_vt(nh, d, t["q_scaled"], seq, seq * d, t["k"][:, 64 * b:], 64, seq * d,
                               t["v_t"][:, :, 64 * b:], d * ld, ld, o_parts[b], lse_parts[b], dtype=torch.float32)
    o = torch.empty((seq, h), dtype=torch.float32, device="cuda")
    B.attn_merge_lse(4, nh, d, seq, o_parts, lse_parts, o, torch.float32)
    ref = oracle.block_forward(x, *ws, nh, taps=True)
    assert_close(host(o), ref["o"], rel=REL_L2_F32, mabs=1e-5, what="merged attention output")
    blk.close()


# 40 heads of 2000 rows run their attention in 384-row workgroups, which fit
# one round of 256 CUs; 48 heads of 2000 rows run rows [0, 1920) so and the
# last 80 rows of every head in 256-row workgroups over 4 key ranges, merged by
# LSE; the others take 256-row workgroups.
@pytest.mark.parametrize("seq,h,nh", [(1000, 512, 4), (300, 384, 3), (1, 256, 2), (7, 128, 1), (520, 1024, 8),
                                      (2000, 256, 2), (2000, 5120, 40), (2000, 6144, 48)])
def test_block_f16_small_all_rows(seq, h, nh):
    _check_all_rows(seq, h, nh, np.float16, 5e-3, 2e-2)


def test_block_every_row_every_launch():
    """Every row of every output is written on every launch (outputs are
    filled with NaN before each), repeated launches give the same bits, and
    all rows match the oracle, at a size with more attention workgroups (512)
    than CUs."""
    seq, h, nh = 4096, 4096, 32
    say(f"block S={seq} h={h} H={nh}, 3 launches, all rows")
    x, [ws] = block_inputs(seq, h, 1, dtype=np.float16, seed=3)
    blk = _block(ws, nh, seq)
    xd = dev(x)
    attn = torch.empty((seq, h), dtype=torch.float16, device="cuda")
    lse = torch.empty((nh, seq), dtype=torch.float32, device="cuda")
    y = torch.empty((seq, h), dtype=torch.float16, device="cuda")
    outs = []
    for _ in range(3):
        for t in (attn, lse, y):
            t.fill_(float("nan"))
        blk.forward(xd, y, taps=B.Taps(None, None, None, attn.data_ptr(), lse.data_ptr(), 0))
        torch.cuda.synchronize()
        assert torch.isfinite(attn).all() and torch.isfinite(lse).all() and torch.isfinite(y).all()
        outs.append((attn.clone(), lse.clone(), y.clone()))
    for o in outs[1:]:
        assert all(torch.equal(a, b) for a, b in zip(o, outs[0]))
    blk.close()
    ref = oracle.block_forward(x, *ws, nh, taps=True)
    assert_close(host(outs[0][0]), ref["o"], what="attn_out, all rows")
    assert_close(host(outs[0][1]), ref["lse"], what="lse, all rows")
    assert_close(host(outs[0][2]), ref["y"], what="y, all rows")


def test_block_f32_head_dim_128():
    _check_all_rows(200, 512, 4, np.float32, REL_L2_F32, 1e-5)


def test_block_seq_zero_and_capacity():
    x, [ws] = block_inputs(64, 256, 1, dtype=np.float16, seed=0)
    blk = _block(ws, 2, 64)
    y = torch.full((64, 256), 3.0, dtype=torch.float16, device="cuda")
    B.attn_block_forward(blk.handle, dev(x), y, 0)
    assert torch.all(y == 3.0)
    with pytest.raises(B.AttnError):
        B.attn_block_forward(blk.handle, dev(x), y, 65)
    with pytest.raises(B.AttnError) as ei:
        B.attn_block_forward(blk.handle, dev(x), y, 32, batch=2)
    assert ei.value.status == B.ATTN_E_UNSUPPORTED
    blk.close()


# ------------------------------------------------------------ full-size configs
def _sampled_block(seq, h, nh, seed=0):
    say(f"block S={seq} h={h} H={nh} fp16 (sampled rows)")
    x, [ws] = block_inputs(seq, h, 1, dtype=np.float16, seed=seed)
    d = h // nh
    blk = _block(ws, nh, seq)
    attn = torch.empty((seq, h), dtype=torch.float16, device="cuda")
    lse = torch.empty((nh, seq), dtype=torch.float32, device="cuda")
    taps = B.Taps(None, None, None, attn.data_ptr(), lse.data_ptr(), 0)
    y = blk.forward(dev(x), taps=taps)
    rows = sample_rows(seq, 256, seed=seed, must=[seq // 8 * r for r in range(9)])
    yr, ar, lr = host(y[rows]), host(attn[rows]), host(lse[:, rows])
    blk.close()
    del y, attn, lse
    ref = oracle.block_forward(x, *ws, nh, rows=rows, taps=True)
    assert_close(yr, ref["y"], what=f"y S={seq}")
    assert_close(ar, ref["o"], what=f"attn_out S={seq}")
    assert_close(lr, ref["lse"], what=f"lse S={seq}")


def test_config_seq8192_hidden4096():
    _sampled_block(8192, 4096, 32)


@pytest.mark.parametrize("seq", [16384, 32768, 65536])
def test_config_seq_sweep_hidden4096(seq):
    _sampled_block(seq, 4096, 32)


def test_config_seq8192_hidden8192():
    _sampled_block(8192, 8192, 64)


def _rank_share(x, ws, seq, h, nh, ranks=8, check_ranks=(0, 7)):
    """Rank r's share: per K/V block, attn_partial_forward on row-major K/V
    (the k and v taps) and attn_partial_forward_vt on the v_t tap -- equal bit
    for bit -- then the LSE merge; and the same chunk against all keys in one
    call."""
    d = h // nh
    blk = _block(ws, nh, seq)
    t, c = _taps(seq, h, nh, d, torch.float16, lse=False, qkv_only=True, v_rows=True)
    blk.forward(dev(x), taps=c)
    ld = B.vt_ld(seq)
    chunk = seq // ranks
    results = {}
    for r in check_ranks:
        q = t["q_scaled"][:, r * chunk:]
        o_parts = torch.empty((ranks, nh, chunk, d), dtype=torch.float32, device="cuda")
        lse_parts = torch.empty((ranks, nh, chunk), dtype=torch.float32, device="cuda")
        o_rows = torch.empty_like(o_parts)
        lse_rows = torch.empty_like(lse_parts)
        for b in range(ranks):
            B.attn_partial_forward_vt(nh, d, q, chunk, seq * d, t["k"][:, b * chunk:], chunk, seq * d,
                                      t["v_t"][:, :, b * chunk:], d * ld, ld, o_parts[b], lse_parts[b])
            B.attn_partial_forward(nh, d, q, chunk, seq * d, t["k"][:, b * chunk:], t["v"][:, b * chunk:], chunk,
                                   seq * d, o_rows[b], lse_rows[b])
        assert torch.equal(o_rows, o_parts) and torch.equal(lse_rows, lse_parts), "row-major V differs from V^T"
        o = torch.empty((chunk, h), dtype=torch.float16, device="cuda")
        lse = torch.empty((nh, chunk), dtype=torch.float32, device="cuda")
        B.attn_merge_lse(ranks, nh, d, chunk, o_parts, lse_parts, o, torch.float16, lse)
        # AllGather-KV share: one call over all keys
        o1 = torch.empty((1, nh, chunk, d), dtype=torch.float32, device="cuda")
        l1 = torch.empty((1, nh, chunk), dtype=torch.float32, device="cuda")
        B.attn_partial_forward_vt(nh, d, q, chunk, seq * d, t["k"], seq, seq * d, t["v_t"], d * ld, ld, o1[0], l1[0])
        o_one = torch.empty((chunk, h), dtype=torch.float16, device="cuda")
        B.attn_merge_lse(1, nh, d, chunk, o1, l1, o_one, torch.float16)
        split_vs_one = rel_l2(host(o), host(o_one))
        say(f"  rank {r}: split-merge vs one-shot rel_l2={split_vs_one:.3e}")
        assert split_vs_one <= REL_L2_SPLIT
        results[r] = (host(o), host(lse))
    blk.close()
    return results


def test_config_rank_share_seq32768():
    seq, h, nh = 32768, 4096, 32
    say("rank share: chunk 1/8 of S=32768 vs K/V in 8 blocks")
    x, [ws] = block_inputs(seq, h, 1, dtype=np.float16, seed=0)
    res = _rank_share(x, ws, seq, h, nh)
    chunk = seq // 8
    for r, (o, lse) in res.items():
        local = sample_rows(chunk, 128, seed=r, must=[0, chunk - 1])
        ref = oracle.block_forward(x, *ws, nh, rows=r * chunk + local, taps=True)
        assert_close(o[local], ref["o"], what=f"rank {r} merged O")
        assert_close(lse[:, local], ref["lse"], what=f"rank {r} merged LSE")


def test_rank_share_small_all_rows():
    seq, h, nh = 2048, 512, 4
    say("rank share small (all rows)")
    x, [ws] = block_inputs(seq, h, 1, dtype=np.float16, seed=1)
    res = _rank_share(x, ws, seq, h, nh, check_ranks=range(8))
    ref = oracle.block_forward(x, *ws, nh, taps=True)
    chunk = seq // 8
    for r, (o, lse) in res.items():
        assert_close(o, ref["o"][r * chunk:(r + 1) * chunk], what=f"rank {r} O")
        assert_close(lse, ref["lse"][:, r * chunk:(r + 1) * chunk], what=f"rank {r} LSE")


def _stack(x, layers, nh, seq):
    blocks = [_block(ws, nh, seq) for ws in layers]
    outs = []
    cur = dev(x)
    for blk in blocks:
        cur = blk.forward(cur)
        outs.append(cur)
    for blk in blocks:
        blk.close()
    return outs


def test_six_stack_small_all_rows():
    seq, h, nh = 2048, 4096, 32
    say("6-stack S=2048 h=4096 vs full fp64 6-layer oracle")
    x, layers = block_inputs(seq, h, 6, dtype=np.float16, seed=0)
    outs = _stack(x, layers, nh, seq)
    ref = oracle.stack_forward(x, layers, nh)
    assert_close(host(outs[-1]), ref, what="6-stack output")


@pytest.mark.timeout(900)
def test_config_six_stack_seq32768():
    """Every layer of the 6-block stack at seq 32768, teacher-forced: layer l's
    oracle input is the GPU's own fp16 output of layer l-1 (x for layer 0),
    K and V over all 32768 rows, and layer l's GPU output is compared on
    sampled rows at the block's gates."""
    seq, h, nh = 32768, 4096, 32
    say("6-stack S=32768: every layer teacher-forced on the previous layer's GPU output, sampled rows")
    x, layers = block_inputs(seq, h, 6, dtype=np.float16, seed=0)
    outs = _stack(x, layers, nh, seq)
    rows = sample_rows(seq, 128, seed=0, must=[seq // 8 * r for r in range(9)])
    prev = x
    for li, (o, ws) in enumerate(zip(outs, layers)):
        got = host(o[rows])
        ref = oracle.block_forward(prev, *ws, nh, rows=rows)
        spread = np.linalg.norm(got - got.mean(0)) / np.linalg.norm(got)
        say(f"  layer {li}: relative row spread of the GPU output {spread:.3e}")
        assert_close(got, ref, what=f"layer {li} (input: {'x' if li == 0 else f'GPU layer {li - 1}'})")
        prev = o.cpu().numpy()  # the exact fp16 values the next GPU layer read
    del outs
