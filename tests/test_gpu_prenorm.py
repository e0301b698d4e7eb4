"""GPU parity of the block with RMSNorm pre-norm (attn_block_set_prenorm)
against the fp64 oracle's block_forward(..., norm=(gain, eps)).

Reading (the pages list RMSNorm in the model without placement or
parameters): pre-norm on the block input, eps 1e-6, unit gain unless given.
Tiny fp32 and small fp16 shapes are compared on every row and every tap; the
headline size (seq 8192, hidden 4096) on seeded sampled rows; a 6-block stack
with pre-norm against the full fp64 stack. Inputs: the seeded recipe of
long_context_self_amd.synthetic (norm_gain for non-unit gains)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from long_context_self_amd import binding as B
from long_context_self_amd.synthetic import block_inputs, norm_gain, sample_rows

from .gpu_util import REL_L2_F32, assert_close, dev, host, say

pytestmark = pytest.mark.gpu

EPS = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    B.lib()


def _block(ws, nh, max_tokens, gain, eps=EPS):
    blk = B.AttnBlock(*(dev(w) for w in ws), nh, max_tokens)
    blk.set_prenorm(None if gain is None else dev(gain), eps)
    return blk


def _all_rows(seq, h, nh, dtype, rel, mabs, unit_gain, eps=EPS, seed=0):
    say(f"pre-norm block S={seq} h={h} H={nh} {dtype.__name__} unit_gain={unit_gain} eps={eps}")
    x, [ws] = block_inputs(seq, h, 1, dtype=dtype, seed=seed)
    # rows of very different magnitudes, so the per-row factor matters
    x = (x.astype(np.float32) * np.linspace(0.05, 4.0, seq, dtype=np.float32)[:, None]).astype(dtype)
    g = None if unit_gain else norm_gain(h, dtype=dtype, seed=seed)
    d = h // nh
    tdt = torch.float16 if dtype == np.float16 else torch.float32
    blk = _block(ws, nh, seq, g, eps)
    q = torch.empty((nh, seq, d), dtype=tdt, device="cuda")
    k = torch.empty((nh, seq, d), dtype=tdt, device="cuda")
    lse = torch.empty((nh, seq), dtype=torch.float32, device="cuda")
    taps = B.Taps(q.data_ptr(), k.data_ptr(), None, None, lse.data_ptr(), 0)
    y = blk.forward(dev(x), taps=taps)
    ref = oracle.block_forward(x, *ws, nh, taps=True, norm=(g, eps))
    assert_close(host(q), ref["q_scaled"], rel=rel, mabs=mabs, what="q_scaled")
    assert_close(host(k), ref["k"], rel=rel, mabs=mabs, what="k")
    assert_close(host(lse), ref["lse"], rel=rel, mabs=mabs, what="lse")
    assert_close(host(y), ref["y"], rel=rel, mabs=mabs, what="y")
    blk.close()


def test_prenorm_tiny_fp32_with_gain():
    _all_rows(256, 256, 4, np.float32, REL_L2_F32, 1e-5, unit_gain=False)


def test_prenorm_tiny_fp32_large_eps():
    # eps comparable to the mean square of the small rows: eps inside the root matters
    _all_rows(256, 256, 4, np.float32, REL_L2_F32, 1e-5, unit_gain=True, eps=0.5)


@pytest.mark.parametrize("seq,h,nh,unit", [(1000, 512, 4, False), (300, 384, 3, True), (7, 128, 1, False)])
def test_prenorm_f16_small_all_rows(seq, h, nh, unit):
    _all_rows(seq, h, nh, np.float16, 5e-3, 2e-2, unit_gain=unit)


def test_prenorm_config_seq8192_hidden4096_sampled():
    seq, h, nh = 8192, 4096, 32
    say("pre-norm block S=8192 h=4096 (sampled rows, unit gain)")
    x, [ws] = block_inputs(seq, h, 1, dtype=np.float16, seed=0)
    blk = _block(ws, nh, seq, None)
    y = blk.forward(dev(x))
    rows = sample_rows(seq, 256, seed=0)
    yr = host(y[rows])
    blk.close()
    ref = oracle.block_forward(x, *ws, nh, rows=rows, norm=(None, EPS))
    assert_close(yr, ref, what="y S=8192 pre-norm")


def test_prenorm_six_stack_small_all_rows():
    seq, h, nh = 1024, 4096, 32
    say("6-stack with pre-norm S=1024 h=4096 vs full fp64 6-layer oracle")
    x, layers = block_inputs(seq, h, 6, dtype=np.float16, seed=0)
    blocks = [_block(ws, nh, seq, None) for ws in layers]
    cur = dev(x)
    for blk in blocks:
        cur = blk.forward(cur)
    out = host(cur)
    for blk in blocks:
        blk.close()
    ref = oracle.stack_forward(x, layers, nh, norms=[(None, EPS)] * 6)
    assert_close(out, ref, what="6-stack output with pre-norm")


def test_prenorm_cannot_be_set_twice():
    x, [ws] = block_inputs(64, 256, 1, dtype=np.float16, seed=0)
    blk = _block(ws, 2, 64, None)
    with pytest.raises(B.AttnError) as ei:
        blk.set_prenorm(None, EPS)
    assert ei.value.status == B.ATTN_E_INVALID_ARG
    blk.close()
