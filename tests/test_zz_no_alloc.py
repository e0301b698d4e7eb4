"""GPU check of attn_partial_forward_noalloc, the entry point that allocates
nothing (its V^T staging is a fixed device array): through the C ABI its
output equals attn_partial_forward's bit for bit, on two calls in a row (the
second smaller, so stale contents of the array would show), at the array's
maximum size, and within the gates of the fp64 oracle."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from long_context_self_amd import binding as B
from long_context_self_amd.synthetic import attention_inputs

from .gpu_util import REL_L2_F32, assert_close, dev, host, say

pytestmark = pytest.mark.gpu


def _both(h, sq, skv, d, dt, seed):
    q, k, v = attention_inputs(h, sq, skv, d, dtype=dt, seed=seed)
    tdt = torch.float16 if dt == np.float16 else torch.float32
    qd, kd, vd = dev(q), dev(k), dev(v)
    outs = []
    for fn in (B.attn_partial_forward, B.attn_partial_forward_noalloc):
        o = torch.full((h, sq, d), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((h, sq), float("nan"), dtype=torch.float32, device="cuda")
        fn(h, d, qd, sq, qd.stride(0), kd, vd, skv, kd.stride(0), o, lse, dtype=tdt)
        outs.append((o, lse))
    torch.cuda.synchronize()
    return (q, k, v), outs


@pytest.mark.parametrize("dt", [np.float16, np.float32])
def test_noalloc_equals_allocating_entry_point_two_calls(dt):
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    d = 128
    # first call large, second call smaller: the second must not see the first's staging
    h0 = 32 if dt == np.float16 else 16  # the first call's staging stays within the 64 MiB array
    for i, (h, sq, skv) in enumerate([(h0, 300, 4100), (3, 77, 65)]):
        say(f"noalloc call {i}: H={h} sq={sq} skv={skv} {np.dtype(dt).name}")
        (q, k, v), ((o1, l1), (o2, l2)) = _both(h, sq, skv, d, dt, seed=40 + i)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), "no-alloc output differs from attn_partial_forward"
        o_ref, lse_ref = oracle.partial_attention(q[:2], k[:2], v[:2])
        rel, mabs = (5e-3, 2e-2) if dt == np.float16 else (REL_L2_F32, 1e-5)
        assert_close(host(o2[:2]), o_ref, rel=rel, mabs=mabs, what="no-alloc o_part vs oracle")
        assert_close(host(l2[:2]), lse_ref, rel=rel, mabs=mabs, what="no-alloc lse vs oracle")


def test_noalloc_at_maximum_size_and_above():
    # 32 heads x 128 x ATTN_VT_LD(8192) fp16 = 64 MiB: the largest accepted staging
    say("noalloc at the 64 MiB limit")
    (_, _, _), ((o1, l1), (o2, l2)) = _both(32, 128, 8192, 128, np.float16, seed=50)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    q = torch.zeros((32, 128, 128), dtype=torch.float16, device="cuda")
    kv = torch.zeros((32, 8193, 128), dtype=torch.float16, device="cuda")
    o = torch.zeros((32, 128, 128), dtype=torch.float32, device="cuda")
    lse = torch.zeros((32, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(B.AttnError) as ei:
        B.attn_partial_forward_noalloc(32, 128, q, 128, q.stride(0), kv, kv, 8193, kv.stride(0), o, lse)
    assert ei.value.status == B.ATTN_E_UNSUPPORTED
    assert torch.all(o == 0)
