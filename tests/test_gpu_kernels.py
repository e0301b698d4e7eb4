"""GPU parity of the attention kernel (attn_partial_forward_vt, and
attn_partial_forward with V row-major) and the LSE merge (attn_merge_lse)
against the fp64 oracle, at sizes that span several tiles with ragged tails,
plus the method's degenerate cases and the GPU-only properties (split-merge vs
unsplit, row-chunk bit-exactness, determinism, row-major V = V^T bit for
bit)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from long_context_self_amd import binding as B
from long_context_self_amd.synthetic import attention_inputs

from .gpu_util import (REL_L2_F16, REL_L2_F32, REL_L2_SPLIT, assert_close, dev, host, max_abs, partial,
                       partial_rows, rel_l2, say, to_vt)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    B.lib()


def _run(h, sq, skv, d=128, dtype=np.float16, seed=0, score_std=1.0):
    q, k, v = attention_inputs(h, sq, skv, d, dtype=dtype, seed=seed, score_std=score_std)
    tdt = torch.float16 if dtype == np.float16 else torch.float32
    vt = to_vt(v)
    o, lse = partial(dev(q), dev(k), dev(vt), sq, skv, vt.shape[2], dtype=tdt)
    return (q, k, v), host(o), host(lse)


@pytest.mark.parametrize("h,sq,skv", [(2, 300, 200), (3, 1000, 1000), (1, 257, 4097), (2, 64, 63)])
def test_partial_f16_vs_oracle(h, sq, skv):
    say(f"partial f16 H={h} sq={sq} skv={skv}")
    (q, k, v), o, lse = _run(h, sq, skv)
    o_ref, lse_ref = oracle.partial_attention(q, k, v)
    assert_close(o, o_ref, what="o_part")
    assert_close(lse, lse_ref, what="lse_part")


def test_planned_split_tail_vs_oracle():
    # 32 heads, 3500 query rows: 320 workgroups of 384 rows would leave the
    # second round of 256 CUs mostly idle, so the launch plan runs rows
    # [0, 3072) whole and splits the last 428 rows of every head over key
    # ranges (in 256-row workgroups), merged by LSE. Both parts, and the border between them, against
    # the oracle on two heads (all rows).
    h, sq, skv, d = 32, 3500, 3500, 128
    say(f"planned launch with a split tail: H={h} sq={sq} skv={skv}")
    q, k, v = attention_inputs(h, sq, skv, d, seed=9)
    vt = to_vt(v)
    o, lse = partial(dev(q), dev(k), dev(vt), sq, skv, vt.shape[2])
    heads = [0, h - 1]
    o_ref, lse_ref = oracle.partial_attention(q[heads], k[heads], v[heads])
    assert_close(host(o)[heads], o_ref, what="o_part (whole rows and split tail)")
    assert_close(host(lse)[heads], lse_ref, what="lse_part (whole rows and split tail)")
    o2, lse2 = partial(dev(q), dev(k), dev(vt), sq, skv, vt.shape[2])
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "planned launch not deterministic"


@pytest.mark.parametrize("ramp", [False, True])
def test_partial_f16_384_row_workgroups_vs_oracle(ramp):
    # 40 heads of 2000 query rows: 240 workgroups of 384 rows fit one round of
    # 256 CUs and 320 of 256 rows would not, so the launch plan takes the
    # 384-row form (the small shapes above get 256-row workgroups). Ragged in
    # both query rows (2000 = 5 x 384 + 80) and keys, with peaked scores, or
    # with keys ordered so that every tile moves the running max by far more
    # than the 2^8 lazy-rescale threshold.
    h, sq, d = 40, 2000, 128
    skv = 640 if ramp else 1000
    say(f"partial f16 384-row workgroups H={h} sq={sq} skv={skv} ramp={ramp}")
    if ramp:
        rng = np.random.default_rng(15)
        q = np.full((h, sq, d), 0.05, np.float16)
        base = rng.standard_normal((h, skv, d)).astype(np.float32) * 0.1
        k = (base + np.linspace(0.0, 30.0, skv, dtype=np.float32)[None, :, None]).astype(np.float16)
        v = rng.standard_normal((h, skv, d)).astype(np.float16)
    else:
        q, k, v = attention_inputs(h, sq, skv, d, seed=14, score_std=8.0)
    vt = to_vt(v)
    o, lse = partial(dev(q), dev(k), dev(vt), sq, skv, vt.shape[2])
    heads = [0, 17, h - 1]
    o_ref, lse_ref = oracle.partial_attention(q[heads], k[heads], v[heads])
    assert_close(host(o)[heads], o_ref, what="o_part (384-row workgroups)")
    assert_close(host(lse)[heads], lse_ref, what="lse_part (384-row workgroups)")


def test_partial_f16_peaked_scores_exercise_rescale():
    # score std 8: running maxima keep growing by more than the 2^8 lazy-rescale threshold
    say("partial f16 peaked scores")
    (q, k, v), o, lse = _run(2, 500, 3000, score_std=8.0, seed=3)
    o_ref, lse_ref = oracle.partial_attention(q, k, v)
    assert_close(o, o_ref, what="o_part peaked")
    assert_close(lse, lse_ref, what="lse peaked")


def test_partial_f16_increasing_keys_force_every_rescale():
    # keys ordered so each tile's max exceeds the previous by far more than 2^8
    say("partial f16 increasing scores")
    h, sq, skv, d = 1, 64, 640, 128
    rng = np.random.default_rng(5)
    q = np.full((h, sq, d), 0.05, np.float16)
    base = rng.standard_normal((h, skv, d)).astype(np.float32) * 0.1
    ramp = np.linspace(0.0, 30.0, skv, dtype=np.float32)[None, :, None]
    k = (base + ramp).astype(np.float16)
    v = rng.standard_normal((h, skv, d)).astype(np.float16)
    vt = to_vt(v)
    o, lse = partial(dev(q), dev(k), dev(vt), sq, skv, vt.shape[2])
    o_ref, lse_ref = oracle.partial_attention(q, k, v)
    assert_close(host(o), o_ref, what="o ramp")
    assert_close(host(lse), lse_ref, what="lse ramp")


def test_partial_zero_query_gives_mean_of_v():
    say("zero query -> mean of V")
    h, sq, skv, d = 2, 70, 333, 128
    _, k, v = attention_inputs(h, sq, skv, d, seed=1)
    q = np.zeros((h, sq, d), np.float16)
    vt = to_vt(v)
    o, lse = partial(dev(q), dev(k), dev(vt), sq, skv, vt.shape[2])
    mean_v = v.astype(np.float64).mean(axis=1, keepdims=True)
    assert_close(host(o), np.broadcast_to(mean_v, (h, sq, d)), rel=1e-5, mabs=1e-5, what="mean of V")
    assert np.allclose(host(lse), np.log(skv), atol=1e-5)


def test_partial_single_key_returns_its_value():
    say("single key")
    h, sq, skv, d = 2, 100, 1, 128
    q, k, v = attention_inputs(h, sq, skv, d, seed=2)
    vt = to_vt(v)
    o, lse = partial(dev(q), dev(k), dev(vt), sq, skv, vt.shape[2])
    # exp(s - m) of the only key is 1 up to the rounding of s*log2(e) in the
    # exp2-domain softmax, so O equals that V row to fp32 rounding.
    assert np.allclose(host(o), np.broadcast_to(v.astype(np.float64), (h, sq, d)), rtol=1e-6, atol=0)
    score = np.einsum("hqd,hkd->hq", q.astype(np.float64), k.astype(np.float64))
    assert np.allclose(host(lse), score, atol=1e-4)


def test_partial_empty_kv_block():
    say("skv = 0")
    h, sq, d = 2, 50, 128
    q = dev(attention_inputs(h, sq, 1, d)[0])
    o = torch.full((h, sq, d), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.zeros((h, sq), dtype=torch.float32, device="cuda")
    B.attn_partial_forward_vt(h, d, q, sq, q.stride(0), None, 0, 0, None, 0, 0, o, lse)
    assert np.all(host(o) == 0.0)
    assert np.all(np.isneginf(host(lse)))


def test_partial_single_query_row():
    say("sq = 1")
    (q, k, v), o, lse = _run(4, 1, 777, seed=4)
    o_ref, lse_ref = oracle.partial_attention(q, k, v)
    assert_close(o, o_ref, what="o sq=1")
    assert_close(lse, lse_ref, what="lse sq=1")


def test_split_merge_equals_unsplit():
    say("split-merge vs unsplit")
    h, sq, skv, d = 3, 600, 2000, 128
    q, k, v = attention_inputs(h, sq, skv, d, seed=6)
    qd = dev(q)
    vt_full = to_vt(v)
    o_full, lse_full = partial(qd, dev(k), dev(vt_full), sq, skv, vt_full.shape[2])
    cuts = [0, 512, 1000, 1001, 1600, 2000]  # uneven, with a size-1 block
    n = len(cuts) - 1
    o_parts = torch.empty((n, h, sq, d), dtype=torch.float32, device="cuda")
    lse_parts = torch.empty((n, h, sq), dtype=torch.float32, device="cuda")
    for b, (a0, a1) in enumerate(zip(cuts[:-1], cuts[1:])):
        vt = to_vt(np.ascontiguousarray(v[:, a0:a1]))
        ob, lb = partial(qd, dev(np.ascontiguousarray(k[:, a0:a1])), dev(vt), sq, a1 - a0, vt.shape[2])
        o_parts[b].copy_(ob)
        lse_parts[b].copy_(lb)
    o_m = torch.empty((sq, h * d), dtype=torch.float16, device="cuda")
    lse_m = torch.empty((h, sq), dtype=torch.float32, device="cuda")
    B.attn_merge_lse(n, h, d, sq, o_parts, lse_parts, o_m, torch.float16, lse_m)
    o_m_heads = host(o_m).reshape(sq, h, d).transpose(1, 0, 2)
    r = rel_l2(o_m_heads, host(o_full))
    say(f"  merged vs unsplit rel_l2={r:.3e}")
    assert r <= REL_L2_SPLIT
    # Each partial's row sum adds the fp16-rounded probabilities (relative
    # error below the fp16 unit roundoff 2^-11), so each LSE is within
    # ln(1 + 2^-11) < 2^-11 of its exact value, and two of them within 2^-10.
    assert max_abs(host(lse_m), host(lse_full)) <= 2.0 ** -10
    o_ref, lse_ref = oracle.partial_attention(q, k, v)
    assert_close(o_m_heads, o_ref, what="merged vs oracle")
    assert_close(host(lse_m), lse_ref, what="merged lse vs oracle")


def test_merge_ignores_empty_parts_and_handles_all_empty():
    say("merge with empty parts")
    h, sq, d = 2, 40, 128
    rng = np.random.default_rng(9)
    o_parts = rng.standard_normal((3, h, sq, d)).astype(np.float32)
    lse_parts = rng.standard_normal((3, h, sq)).astype(np.float32)
    lse_parts[1] = -np.inf
    o_out = torch.empty((sq, h * d), dtype=torch.float32, device="cuda")
    lse_out = torch.empty((h, sq), dtype=torch.float32, device="cuda")
    B.attn_merge_lse(3, h, d, sq, dev(o_parts), dev(lse_parts), o_out, torch.float32, lse_out)
    o_ref, lse_ref = oracle.merge_partials(o_parts, lse_parts)
    got = host(o_out).reshape(sq, h, d).transpose(1, 0, 2)
    assert rel_l2(got, o_ref) <= 1e-6
    assert rel_l2(host(lse_out), lse_ref) <= 1e-6
    lse_parts[:] = -np.inf
    B.attn_merge_lse(3, h, d, sq, dev(o_parts), dev(lse_parts), o_out, torch.float32, lse_out)
    assert np.all(host(o_out) == 0.0) and np.all(np.isneginf(host(lse_out)))


@pytest.mark.parametrize("a,b", [(256, 512), (100, 357), (999, 1000)])
def test_row_chunk_is_bit_exact(a, b):
    # Rows [a, b) run alone against the full K/V equal rows [a, b) of the full run.
    # Below 1024 keys no launch plan splits keys, so both runs are plain launches
    # and every row's arithmetic is the kernel's alone (with a split tail, rows
    # in it are summed in another order, and which rows fall there depends on sq).
    say(f"row chunk [{a},{b}) bit-exact")
    h, sq, skv, d = 2, 1000, 1000, 128
    q, k, v = attention_inputs(h, sq, skv, d, seed=7)
    kd, vt = dev(k), to_vt(v)
    vtd = dev(vt)
    o_full, lse_full = partial(dev(q), kd, vtd, sq, skv, vt.shape[2])
    qc = dev(np.ascontiguousarray(q[:, a:b]))
    o_c, lse_c = partial(qc, kd, vtd, b - a, skv, vt.shape[2])
    assert torch.equal(o_c, o_full[:, a:b])
    assert torch.equal(lse_c, lse_full[:, a:b])


def test_whole_key_tail_in_256_row_workgroups_vs_oracle():
    # 40 heads of 3100 rows over 1000 keys (too few to split): the launch plan
    # runs rows [0, 2304) in 384-row workgroups (240, one round of 256 CUs) and
    # the 796 rows after them over all keys in 256-row workgroups (160, one
    # more round) straight into the outputs. Against the oracle on three heads,
    # and row for row against runs of parts of the rows alone: [0, 1000) alone
    # takes 256-row workgroups, yet its bits equal those the 384-row workgroups
    # gave the same rows (no row's arithmetic depends on the rows beside it).
    h, sq, skv, d = 40, 3100, 1000, 128
    say(f"main launch + whole-key tail of the other workgroup size: H={h} sq={sq} skv={skv}")
    q, k, v = attention_inputs(h, sq, skv, d, seed=16)
    kd, vt = dev(k), to_vt(v)
    vtd = dev(vt)
    o, lse = partial(dev(q), kd, vtd, sq, skv, vt.shape[2])
    heads = [0, 21, h - 1]
    o_ref, lse_ref = oracle.partial_attention(q[heads], k[heads], v[heads])
    assert_close(host(o)[heads], o_ref, what="o_part (main rows and whole-key tail)")
    assert_close(host(lse)[heads], lse_ref, what="lse_part (main rows and whole-key tail)")
    for a, b in [(0, 1000), (2304, 3100), (2200, 2400)]:
        o_c, lse_c = partial(dev(np.ascontiguousarray(q[:, a:b])), kd, vtd, b - a, skv, vt.shape[2])
        assert torch.equal(o_c, o[:, a:b]) and torch.equal(lse_c, lse[:, a:b]), f"rows [{a},{b}) alone differ"


def test_two_runs_are_bit_identical():
    say("determinism")
    h, sq, skv, d = 4, 1024, 2048, 128
    q, k, v = attention_inputs(h, sq, skv, d, seed=8)
    vt = to_vt(v)
    args = (dev(q), dev(k), dev(vt), sq, skv, vt.shape[2])
    o1, l1 = partial(*args)
    o2, l2 = partial(*args)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_partials_on_two_streams_match_one_stream():
    """attn_partial_forward keeps no state between calls, so block partials
    enqueued alternately on two streams (each into its own output) equal the
    same calls on one stream bit for bit, and so does their merge."""
    say("block partials on two streams")
    h, sq, skv, d, n = 4, 512, 4096, 128, 4
    q, k, v = attention_inputs(h, sq, skv, d, seed=12)
    qd, kd = dev(q), dev(k)
    vt = dev(to_vt(v))
    ld, blk = vt.shape[2], skv // n

    def run(streams):
        o = torch.empty((n, h, sq, d), dtype=torch.float32, device="cuda")
        lse = torch.empty((n, h, sq), dtype=torch.float32, device="cuda")
        main = torch.cuda.current_stream()
        fork = torch.cuda.Event()
        fork.record(main)
        for st in streams:
            st.wait_event(fork)
        for b in range(n):
            st = streams[b % len(streams)]
            B.attn_partial_forward_vt(h, d, qd, sq, qd.stride(0), kd[:, b * blk:], blk, kd.stride(0), vt[:, :, b * blk:],
                                   vt.stride(0), ld, o[b], lse[b], stream=st.cuda_stream)
        for st in streams:
            join = torch.cuda.Event()
            join.record(st)
            main.wait_event(join)
        out = torch.empty((sq, h * d), dtype=torch.float16, device="cuda")
        B.attn_merge_lse(n, h, d, sq, o, lse, out, torch.float16)
        torch.cuda.synchronize()
        return o, lse, out

    one = run([torch.cuda.current_stream()])
    two = run([torch.cuda.current_stream(), torch.cuda.Stream()])
    for a, b2 in zip(one, two):
        assert torch.equal(a, b2)


@pytest.mark.parametrize("d", [64, 128])
def test_partial_f32_vs_oracle(d):
    say(f"partial f32 d={d}")
    (q, k, v), o, lse = _run(4, 256, 300, d=d, dtype=np.float32, seed=10)
    o_ref, lse_ref = oracle.partial_attention(q, k, v)
    assert_close(o, o_ref, rel=REL_L2_F32, mabs=1e-5, what="o f32")
    assert_close(lse, lse_ref, rel=REL_L2_F32, mabs=1e-5, what="lse f32")


def test_tiny_config_split_into_four_chunks_fp32():
    # Tiny configuration: 4 heads of 64, 256 keys split into 4 chunks of 64,
    # partials merged by LSE, against the oracle and the unsplit GPU result.
    say("tiny fp32 4-chunk split")
    h, s, d = 4, 256, 64
    q, k, v = attention_inputs(h, s, s, d, dtype=np.float32, seed=0)
    qd = dev(q)
    vt_full = to_vt(v)
    o_full, lse_full = partial(qd, dev(k), dev(vt_full), s, s, vt_full.shape[2], dtype=torch.float32)
    o_parts = torch.empty((4, h, s, d), dtype=torch.float32, device="cuda")
    lse_parts = torch.empty((4, h, s), dtype=torch.float32, device="cuda")
    for b in range(4):
        kb = np.ascontiguousarray(k[:, 64 * b:64 * (b + 1)])
        vtb = to_vt(np.ascontiguousarray(v[:, 64 * b:64 * (b + 1)]))
        ob, lb = partial(qd, dev(kb), dev(vtb), s, 64, vtb.shape[2], dtype=torch.float32)
        o_parts[b].copy_(ob)
        lse_parts[b].copy_(lb)
    o_m = torch.empty((s, h * d), dtype=torch.float32, device="cuda")
    lse_m = torch.empty((h, s), dtype=torch.float32, device="cuda")
    B.attn_merge_lse(4, h, d, s, o_parts, lse_parts, o_m, torch.float32, lse_m)
    got = host(o_m).reshape(s, h, d).transpose(1, 0, 2)
    o_ref, lse_ref = oracle.partial_attention(q, k, v)
    assert_close(got, o_ref, rel=REL_L2_F32, mabs=1e-5, what="tiny merged vs oracle")
    assert_close(host(lse_m), lse_ref, rel=REL_L2_F32, mabs=1e-5, what="tiny merged lse")
    assert rel_l2(got, host(o_full)) <= REL_L2_SPLIT


# ------------------------------------------------ attn_partial_forward, V row-major
@pytest.mark.parametrize("h,sq,skv,d,dt", [(2, 300, 1, 128, np.float16), (3, 257, 63, 128, np.float16),
                                           (1, 64, 65, 128, np.float16), (2, 500, 1000, 128, np.float16),
                                           (4, 256, 4100, 128, np.float16), (4, 256, 300, 64, np.float32),
                                           (2, 100, 77, 128, np.float32)])
def test_partial_rows_vs_oracle_and_vt(h, sq, skv, d, dt):
    """V given row-major [H,skv,d]: within the gates of the oracle, and bit for
    bit the V^T entry point on the same values (the staging transpose moves
    data only; the attention kernel is the same)."""
    say(f"partial rows H={h} sq={sq} skv={skv} d={d} {np.dtype(dt).name}")
    q, k, v = attention_inputs(h, sq, skv, d, dtype=dt, seed=20 + skv)
    tdt = torch.float16 if dt == np.float16 else torch.float32
    qd, kd, vd = dev(q), dev(k), dev(v)
    o, lse = partial_rows(qd, kd, vd, sq, skv, dtype=tdt)
    vt = to_vt(v)
    o_t, lse_t = partial(qd, kd, dev(vt), sq, skv, vt.shape[2], dtype=tdt)
    assert torch.equal(o, o_t) and torch.equal(lse, lse_t), "row-major V differs from V^T"
    o_ref, lse_ref = oracle.partial_attention(q, k, v)
    rel, mabs = (REL_L2_F16, 2e-2) if dt == np.float16 else (REL_L2_F32, 1e-5)
    assert_close(host(o), o_ref, rel=rel, mabs=mabs, what="o_part (V rows)")
    assert_close(host(lse), lse_ref, rel=rel, mabs=mabs, what="lse_part (V rows)")


def test_partial_rows_strided_heads_and_empty_block():
    """K/V as views into a longer sequence (head stride > skv*d, as for one
    block of a gathered K/V), and a block with no keys."""
    say("partial rows: strided head views, empty block")
    h, sq, s_all, d = 3, 200, 1500, 128
    q, k, v = attention_inputs(h, sq, s_all, d, seed=31)
    qd, kd, vd = dev(q), dev(k), dev(v)
    a, b = 448, 1203
    o, lse = partial_rows(qd, kd[:, a:], vd[:, a:], sq, b - a)
    o_ref, lse_ref = oracle.partial_attention(q, k[:, a:b], v[:, a:b])
    assert_close(host(o), o_ref, what="o_part strided")
    assert_close(host(lse), lse_ref, what="lse strided")
    o0 = torch.full((h, sq, d), 7.0, dtype=torch.float32, device="cuda")
    l0 = torch.zeros((h, sq), dtype=torch.float32, device="cuda")
    B.attn_partial_forward(h, d, qd, sq, qd.stride(0), None, None, 0, 0, o0, l0)
    assert torch.all(o0 == 0) and torch.all(torch.isneginf(l0))


def test_partial_rows_on_two_streams_match_one_stream():
    """Each call's V^T staging is taken from and returned to a stream-ordered
    pool, so row-major partials enqueued alternately on two streams equal the
    same calls on one stream bit for bit."""
    say("row-major partials on two streams")
    h, sq, skv, d, n = 4, 512, 4096, 128, 4
    q, k, v = attention_inputs(h, sq, skv, d, seed=13)
    qd, kd, vd = dev(q), dev(k), dev(v)
    blk = skv // n

    def run(streams):
        o = torch.empty((n, h, sq, d), dtype=torch.float32, device="cuda")
        lse = torch.empty((n, h, sq), dtype=torch.float32, device="cuda")
        main = torch.cuda.current_stream()
        fork = torch.cuda.Event()
        fork.record(main)
        for st in streams:
            st.wait_event(fork)
        for b in range(n):
            st = streams[b % len(streams)]
            B.attn_partial_forward(h, d, qd, sq, qd.stride(0), kd[:, b * blk:], vd[:, b * blk:], blk, kd.stride(0),
                                   o[b], lse[b], stream=st.cuda_stream)
        for st in streams:
            join = torch.cuda.Event()
            join.record(st)
            main.wait_event(join)
        torch.cuda.synchronize()
        return o, lse

    one = run([torch.cuda.current_stream()])
    two = run([torch.cuda.current_stream(), torch.cuda.Stream()])
    for a, b2 in zip(one, two):
        assert torch.equal(a, b2)
    o_ref, lse_ref = oracle.partial_attention(q, k[:, :blk], v[:, :blk])
    assert_close(host(one[0][0]), o_ref, what="block 0 o_part")
