"""GPU tests of Ring-style K/V streaming (attn_ring_*): parity with the fp64
oracle (attention over the keys of all blocks, which the per-block partials
merged by log-sum-exp must equal), and bit-for-bit equality with the same
blocks run one by one through attn_partial_forward + attn_merge_lse -- any
copy that overwrote a staging slot still being read would break it. Blocks
come from device memory and from pinned host memory (the stand-in for a
peer's link). Full size: rank 0 of 8 at seq 32768 (its 4096-row query chunk
against 8 blocks of 4096 keys from the block's own projection). Inputs:
long_context_self_amd.synthetic."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from long_context_self_amd import binding as B
from long_context_self_amd.synthetic import attention_inputs, block_inputs, sample_rows

from .gpu_util import REL_L2_F32, REL_L2_SPLIT, assert_close, dev, host, rel_l2, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    B.lib()


def _blocks(k, v, lens, pinned=False):
    """Split head-major K [H][S][d], V [H][S][d] into owner layouts: K_b
    [H][len][d], V_b^T [H][d][ATTN_VT_LD(len)]."""
    kb, vb, a = [], [], 0
    for n in lens:
        kk = np.ascontiguousarray(k[:, a:a + n])
        vt = np.zeros((k.shape[0], k.shape[2], B.vt_ld(n)), dtype=v.dtype)
        vt[:, :, :n] = v[:, a:a + n].transpose(0, 2, 1)
        if pinned:
            kb.append(torch.from_numpy(kk).pin_memory())
            vb.append(torch.from_numpy(vt).pin_memory())
        else:
            kb.append(dev(kk))
            vb.append(dev(vt))
        a += n
    return kb, vb


def _sequential(q, sq, kb, vb, lens, hh, d, dtype=torch.float16):
    o_parts = torch.empty((len(lens), hh, sq, d), dtype=torch.float32, device="cuda")
    lse_parts = torch.empty((len(lens), hh, sq), dtype=torch.float32, device="cuda")
    for b, n in enumerate(lens):
        kd = kb[b].cuda() if n else None
        vd = vb[b].cuda() if n else None
        ld = B.vt_ld(n)
        B.attn_partial_forward_vt(hh, d, q, sq, sq * d, kd, n, n * d, vd, d * ld, ld, o_parts[b], lse_parts[b],
                               dtype=dtype)
    o = torch.empty((sq, hh * d), dtype=dtype, device="cuda")
    lse = torch.empty((hh, sq), dtype=torch.float32, device="cuda")
    B.attn_merge_lse(len(lens), hh, d, sq, o_parts, lse_parts, o, dtype, lse)
    return o, lse


def _ring(q, sq, kb, vb, lens, hh, d, dtype=torch.float16, ring=None):
    own = ring is None
    if own:
        ring = B.AttnRing(hh, d, len(lens), sq, max(max(lens), 1), dtype)
    o = torch.empty((sq, hh * d), dtype=dtype, device="cuda")
    lse = torch.empty((hh, sq), dtype=torch.float32, device="cuda")
    ring.forward(q, sq, kb, vb, lens, o, lse)
    torch.cuda.synchronize()
    if own:
        ring.close()
    return o, lse


@pytest.mark.parametrize("pinned", [False, True])
def test_ring_small_ragged_blocks(pinned):
    hh, sq, d = 4, 300, 128
    lens = [256, 100, 0, 513, 64]
    say(f"ring: H={hh} sq={sq} blocks={lens} pinned={pinned}")
    q, k, v = attention_inputs(hh, sq, sum(lens), d, seed=41)
    kb, vb = _blocks(k, v, lens, pinned)
    qd = dev(q)
    o, lse = _ring(qd, sq, kb, vb, lens, hh, d)
    o_ref, lse_ref = oracle.partial_attention(q, k, v)
    assert_close(host(o).reshape(sq, hh, d).transpose(1, 0, 2), o_ref, what="ring O")
    assert_close(host(lse), lse_ref, what="ring LSE")
    o2, lse2 = _sequential(qd, sq, kb, vb, lens, hh, d)
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "ring differs from partials + merge"


def test_ring_reused_across_calls():
    hh, sq, d = 2, 256, 128
    lens = [128, 128, 128, 128]
    say("ring reused for two inputs")
    ring = B.AttnRing(hh, d, len(lens), sq, 128)
    for seed in (42, 43):
        q, k, v = attention_inputs(hh, sq, sum(lens), d, seed=seed)
        kb, vb = _blocks(k, v, lens)
        o, lse = _ring(dev(q), sq, kb, vb, lens, hh, d, ring=ring)
        o_ref, _ = oracle.partial_attention(q, k, v)
        assert_close(host(o).reshape(sq, hh, d).transpose(1, 0, 2), o_ref, what=f"ring O seed {seed}")
    ring.close()


def test_ring_tiny_fp32():
    hh, sq, d = 4, 256, 64
    lens = [64, 64, 64, 64]
    say("ring tiny fp32, 4 blocks of 64 keys")
    q, k, v = attention_inputs(hh, sq, sum(lens), d, dtype=np.float32, seed=44)
    kb, vb = _blocks(k, v, lens)
    o, lse = _ring(dev(q), sq, kb, vb, lens, hh, d, dtype=torch.float32)
    o_ref, lse_ref = oracle.partial_attention(q, k, v)
    assert_close(host(o).reshape(sq, hh, d).transpose(1, 0, 2), o_ref, rel=REL_L2_F32, mabs=1e-5, what="O")
    assert_close(host(lse), lse_ref, rel=REL_L2_F32, mabs=1e-5, what="LSE")


def test_ring_device_resident_blocks_one_launch():
    # Every block in device memory: one launch over (block, head, query rows) for
    # all blocks. Blocks of 1024 keys or more may be split by the per-block calls'
    # plan, so the two agree within the split-merge gate; both meet the oracle's.
    hh, sq, d = 8, 1000, 128
    lens = [2048, 1500, 0, 3000, 64]
    say(f"ring, device-resident blocks {lens}, H={hh} sq={sq}")
    q, k, v = attention_inputs(hh, sq, sum(lens), d, seed=45)
    kb, vb = _blocks(k, v, lens)
    qd = dev(q)
    o, lse = _ring(qd, sq, kb, vb, lens, hh, d)
    o_ref, lse_ref = oracle.partial_attention(q[:2], k[:2], v[:2])
    got = host(o).reshape(sq, hh, d).transpose(1, 0, 2)
    assert_close(got[:2], o_ref, what="ring O (one launch)")
    assert_close(host(lse)[:2], lse_ref, what="ring LSE (one launch)")
    o2, lse2 = _sequential(qd, sq, kb, vb, lens, hh, d)
    r = rel_l2(host(o).astype(np.float64), host(o2).astype(np.float64))
    say(f"  one launch vs per-block partials + merge: rel_l2={r:.2e}")
    assert r <= REL_L2_SPLIT
    assert rel_l2(host(lse), host(lse2)) <= REL_L2_SPLIT
    o3, lse3 = _ring(qd, sq, kb, vb, lens, hh, d)
    assert torch.equal(o, o3) and torch.equal(lse, lse3), "one-launch ring not deterministic"


def test_ring_equal_device_blocks_read_as_one_sequence():
    # Equal power-of-two blocks in device memory: the ring reads them as one key
    # sequence in a single planned launch (no per-block partials), which equals
    # attn_partial_forward_vt over the concatenated K/V bit for bit (after the
    # same fp16 rounding), and meets the oracle's gates.
    hh, sq, d = 8, 700, 128
    lens = [1024] * 4
    say(f"ring, equal device-resident blocks {lens}, H={hh} sq={sq}")
    q, k, v = attention_inputs(hh, sq, sum(lens), d, seed=46)
    kb, vb = _blocks(k, v, lens)
    qd = dev(q)
    o, lse = _ring(qd, sq, kb, vb, lens, hh, d)
    o_ref, lse_ref = oracle.partial_attention(q[:2], k[:2], v[:2])
    got = host(o).reshape(sq, hh, d).transpose(1, 0, 2)
    assert_close(got[:2], o_ref, what="ring O (one sequence)")
    assert_close(host(lse)[:2], lse_ref, what="ring LSE (one sequence)")
    skv = sum(lens)
    ld = B.vt_ld(skv)
    vt = np.zeros((hh, d, ld), dtype=np.float16)
    vt[:, :, :skv] = v.transpose(0, 2, 1)
    o32 = torch.empty((hh, sq, d), dtype=torch.float32, device="cuda")
    l32 = torch.empty((hh, sq), dtype=torch.float32, device="cuda")
    B.attn_partial_forward_vt(hh, d, qd, sq, sq * d, dev(k), skv, skv * d, dev(vt), d * ld, ld, o32, l32)
    torch.cuda.synchronize()
    o_cat = o32.transpose(0, 1).reshape(sq, hh * d).to(torch.float16)
    assert torch.equal(o, o_cat) and torch.equal(lse, l32), "ring differs from one partial over the concatenated keys"
    o2, lse2 = _sequential(qd, sq, kb, vb, lens, hh, d)
    assert rel_l2(host(o).astype(np.float64), host(o2).astype(np.float64)) <= REL_L2_SPLIT
    assert rel_l2(host(lse), host(lse2)) <= REL_L2_SPLIT


@pytest.mark.parametrize("hh,sq,blen,nb,heads", [(40, 3100, 256, 4, [0, 17, 39]), (40, 2400, 512, 4, [0, 23, 39])])
def test_ring_equal_device_blocks_main_launch_and_tail(hh, sq, blen, nb, heads):
    # The one-sequence launch under the two tail plans: 40 heads of 3100 rows over
    # 1024 keys run rows [0, 2304) in 384-row workgroups and the rest over all keys
    # in 256-row ones; 40 heads of 2400 rows over 2048 keys run the last 96 rows in
    # 256-row workgroups over 4 key ranges, merged by LSE. Against the oracle on
    # three heads, and bit for bit against one partial over the concatenated keys.
    d = 128
    lens = [blen] * nb
    say(f"ring, equal device blocks with a planned tail: H={hh} sq={sq} {nb} x {blen}")
    q, k, v = attention_inputs(hh, sq, sum(lens), d, seed=60 + nb)
    kb, vb = _blocks(k, v, lens)
    qd = dev(q)
    o, lse = _ring(qd, sq, kb, vb, lens, hh, d)
    o_ref, lse_ref = oracle.partial_attention(q[heads], k[heads], v[heads])
    got = host(o).reshape(sq, hh, d).transpose(1, 0, 2)
    assert_close(got[heads], o_ref, what="ring O")
    assert_close(host(lse)[heads], lse_ref, what="ring LSE")
    skv = sum(lens)
    ld = B.vt_ld(skv)
    vt = np.zeros((hh, d, ld), dtype=np.float16)
    vt[:, :, :skv] = v.transpose(0, 2, 1)
    o32 = torch.empty((hh, sq, d), dtype=torch.float32, device="cuda")
    l32 = torch.empty((hh, sq), dtype=torch.float32, device="cuda")
    B.attn_partial_forward_vt(hh, d, qd, sq, sq * d, dev(k), skv, skv * d, dev(vt), d * ld, ld, o32, l32)
    torch.cuda.synchronize()
    o_cat = o32.transpose(0, 1).reshape(sq, hh * d).to(torch.float16)
    assert torch.equal(o, o_cat) and torch.equal(lse, l32), "ring differs from one partial over the concatenated keys"


@pytest.mark.parametrize("hh,sq,blen,nb", [(3, 77, 64, 5), (1, 400, 512, 16), (2, 1, 128, 3), (40, 2000, 256, 4)])
def test_ring_equal_device_blocks_edge_shapes(hh, sq, blen, nb):
    # the one-sequence path at its edges: the shortest block (64 keys), the most
    # blocks one launch takes (16), a single query row, and 40 heads of 2000 rows
    # (384-row workgroups; the others take 256-row ones); all rows against the
    # oracle and bit for bit against one partial over the concatenated keys
    d = 128
    lens = [blen] * nb
    say(f"ring, equal device blocks: H={hh} sq={sq} {nb} x {blen}")
    q, k, v = attention_inputs(hh, sq, sum(lens), d, seed=47 + nb)
    kb, vb = _blocks(k, v, lens)
    qd = dev(q)
    o, lse = _ring(qd, sq, kb, vb, lens, hh, d)
    o_ref, lse_ref = oracle.partial_attention(q, k, v)
    assert_close(host(o).reshape(sq, hh, d).transpose(1, 0, 2), o_ref, what="ring O")
    assert_close(host(lse), lse_ref, what="ring LSE")
    skv = sum(lens)
    ld = B.vt_ld(skv)
    vt = np.zeros((hh, d, ld), dtype=np.float16)
    vt[:, :, :skv] = v.transpose(0, 2, 1)
    o32 = torch.empty((hh, sq, d), dtype=torch.float32, device="cuda")
    l32 = torch.empty((hh, sq), dtype=torch.float32, device="cuda")
    B.attn_partial_forward_vt(hh, d, qd, sq, sq * d, dev(k), skv, skv * d, dev(vt), d * ld, ld, o32, l32)
    torch.cuda.synchronize()
    o_cat = o32.transpose(0, 1).reshape(sq, hh * d).to(torch.float16)
    assert torch.equal(o, o_cat) and torch.equal(lse, l32), "ring differs from one partial over the concatenated keys"


def test_ring_config_seq32768_rank0_pinned():
    seq, h, nh, ranks = 32768, 4096, 32, 8
    d, ch = h // nh, seq // ranks
    say("ring: rank 0 of 8 at seq 32768, K/V blocks in pinned host memory, sampled rows")
    x, [ws] = block_inputs(seq, h, 1, dtype=np.float16, seed=0)
    blk = B.AttnBlock(*(dev(w) for w in ws), nh, seq)
    q = torch.empty((nh, seq, d), dtype=torch.float16, device="cuda")
    k = torch.empty_like(q)
    vt = torch.zeros((nh, d, B.vt_ld(seq)), dtype=torch.float16, device="cuda")
    blk.forward(dev(x), taps=B.Taps(q.data_ptr(), k.data_ptr(), vt.data_ptr(), None, None, 1))
    blk.close()
    q0 = q[:, :ch].contiguous()
    kb = [k[:, b * ch:(b + 1) * ch].contiguous().cpu().pin_memory() for b in range(ranks)]
    vb = [vt[:, :, b * ch:(b + 1) * ch].contiguous().cpu().pin_memory() for b in range(ranks)]
    lens = [ch] * ranks
    o, lse = _ring(q0, ch, kb, vb, lens, nh, d)
    o2, lse2 = _sequential(q0, ch, kb, vb, lens, nh, d)
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "ring differs from partials + merge"
    rows = sample_rows(ch, 128, seed=0)
    o_r, l_r = host(o[rows]), host(lse[:, rows])
    kh, vh = host(k), host(vt)[:, :, :seq].transpose(0, 2, 1)
    o_ref, lse_ref = oracle.partial_attention(host(q0)[:, rows], kh, vh)
    assert_close(o_r, oracle.merge_heads(o_ref), what="ring O (sampled rows)")
    assert_close(l_r, lse_ref, what="ring LSE (sampled rows)")
