"""Pins of the Ulysses and tensor-parallel share oracle (oracle/shares.py).

Each ``pin_*`` takes the shares module (real, or a copy with a planted
mistake) and returns ``(ok, detail)``. What they rest on:

* library     -- torch.nn.functional.scaled_dot_product_attention over all
                 heads in float64: every rank's Ulysses share is its heads'
                 slice; torch.nn.MultiheadAttention (bias off, float64): the
                 TP partial outputs of all ranks sum to its output (the
                 all-reduce of "Tensor Parallelism: Sharding Weights for
                 Parallel Layer Execution", section 3, step 4);
* brute force -- pure-Python index loops for the all-to-all blocks, and a
                 loop implementation of one rank's TP partial output;
* round trips -- gathering what a rank receives gives back its heads of the
                 head-major tensors; the second all-to-all plus unpacking
                 rebuilds each rank's rows of the full attention output.
"""

from __future__ import annotations

import math

import numpy as np

from . import brute


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _qkv(rng, hh, s, d):
    q = rng.standard_normal((hh, s, d)) / math.sqrt(d) * 1.5
    return q, rng.standard_normal((hh, s, d)), rng.standard_normal((hh, s, d))


def pin_ulysses_share_torch(sh, tol=1e-10):
    import torch
    import torch.nn.functional as F

    worst = 0.0
    for seed, (hh, s, d, n) in enumerate([(4, 16, 8, 2), (8, 24, 4, 4), (6, 12, 6, 3)]):
        rng = np.random.default_rng(500 + seed)
        q, k, v = _qkv(rng, hh, s, d)
        # scale 1 because q is already q_scaled
        ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                             scale=1.0).numpy()
        for r in range(n):
            o, lse = sh.ulysses_share(q, k, v, n, r)
            hl = hh // n
            want = ref[r * hl:(r + 1) * hl].transpose(1, 0, 2).reshape(s, hl * d)
            worst = max(worst, _rel(o, want))
            qs = q[r * hl:(r + 1) * hl]
            sc = np.einsum("hid,hjd->hij", qs, k[r * hl:(r + 1) * hl])
            worst = max(worst, _rel(lse, np.log(np.exp(sc).sum(-1))))
    return worst <= tol, f"Ulysses share vs torch SDPA head slices: {worst:.3e}"


def pin_ulysses_layouts_bruteforce(sh, tol=0.0):
    bad = []
    for seed, (hh, s, d, n) in enumerate([(4, 8, 2, 2), (6, 9, 3, 3), (8, 8, 1, 4)]):
        rng = np.random.default_rng(520 + seed)
        t = rng.standard_normal((hh, s, d))
        vt = rng.standard_normal((hh, d, s))
        for r in range(n):
            if not np.array_equal(sh.ulysses_recv_qk(t, n, r), np.array(brute.ulysses_recv_blocks(t.tolist(), n, r))):
                bad.append(("qk", hh, s, d, n, r))
            got = sh.ulysses_recv_vt(vt, n, r)
            if not np.array_equal(got, np.array(brute.ulysses_recv_blocks(vt.tolist(), n, r, keys_last=True))):
                bad.append(("vt", hh, s, d, n, r))
    return not bad, f"all-to-all blocks differing from brute force: {bad}"


def pin_ulysses_round_trips(sh, tol=0.0):
    bad = []
    rng = np.random.default_rng(540)
    hh, s, d, n = 8, 16, 4, 4
    t = rng.standard_normal((hh, s, d))
    vt = rng.standard_normal((hh, d, s))
    hl, c = hh // n, s // n
    for r in range(n):
        if not np.array_equal(sh.ulysses_gather_qk(sh.ulysses_recv_qk(t, n, r)), t[r * hl:(r + 1) * hl]):
            bad.append(("gather_qk", r))
        if not np.array_equal(sh.ulysses_gather_vt(sh.ulysses_recv_vt(vt, n, r)), vt[r * hl:(r + 1) * hl]):
            bad.append(("gather_vt", r))
    # second all-to-all: every rank gets its rows of the concatenated full output
    full = rng.standard_normal((s, hh * d))
    shares = [full[:, r * hl * d:(r + 1) * hl * d] for r in range(n)]
    for p in range(n):
        if not np.array_equal(sh.ulysses_unpack_o(sh.ulysses_return_o(shares, n, p)), full[p * c:(p + 1) * c]):
            bad.append(("return_o", p))
    return not bad, f"round trips failing: {bad}"


def pin_tp_allreduce_torch(sh, tol=1e-10):
    import torch

    worst = 0.0
    for seed, (s, h, nh, n) in enumerate([(32, 64, 4, 2), (20, 48, 6, 3), (40, 64, 8, 8)]):
        rng = np.random.default_rng(560 + seed)
        x = rng.standard_normal((s, h))
        wq, wk, wv, wo = (rng.standard_normal((h, h)) / math.sqrt(h) for _ in range(4))
        mha = torch.nn.MultiheadAttention(h, nh, bias=False, batch_first=True, dtype=torch.float64)
        with torch.no_grad():
            mha.in_proj_weight.copy_(torch.from_numpy(np.concatenate([wq.T, wk.T, wv.T], 0)))
            mha.out_proj.weight.copy_(torch.from_numpy(wo.T.copy()))
            xt = torch.from_numpy(x)[None]
            ref, _ = mha(xt, xt, xt, need_weights=False)
        total = sum(sh.tp_share(x, wq, wk, wv, wo, nh, n, r) for r in range(n))
        worst = max(worst, _rel(total, ref[0].numpy()))
        rows = [s - 1, 0, 3]
        total_rows = sum(sh.tp_share(x, wq, wk, wv, wo, nh, n, r, rows=rows) for r in range(n))
        worst = max(worst, _rel(total_rows, ref[0].numpy()[rows]))
    return worst <= tol, f"sum of TP partial outputs vs torch MultiheadAttention: {worst:.3e}"


def pin_tp_share_bruteforce(sh, tol=1e-12):
    worst = 0.0
    for seed, (s, h, nh, n) in enumerate([(5, 8, 2, 2), (6, 12, 4, 2), (4, 6, 3, 3)]):
        rng = np.random.default_rng(580 + seed)
        x = rng.standard_normal((s, h)) * 1.5
        ws = [rng.standard_normal((h, h)) / math.sqrt(h) for _ in range(4)]
        for r in range(n):
            worst = max(worst, _rel(sh.tp_share(x, *ws, nh, n, r), brute.tp_share(x, *ws, nh, n, r)))
    return worst <= tol, f"TP partial output vs brute force: {worst:.3e}"


SHARE_PINS = [pin_ulysses_share_torch, pin_ulysses_layouts_bruteforce, pin_ulysses_round_trips,
              pin_tp_allreduce_torch, pin_tp_share_bruteforce]
