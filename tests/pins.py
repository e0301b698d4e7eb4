"""Pins of the fp64 oracle against things other than itself.

Each ``pin_*`` takes an oracle module (the real one, or a copy with a planted
mistake) and returns ``(ok, detail)``. ``test_oracle_pins.py`` asserts every
pin holds for the real oracle, and that each planted mistake trips at least one
pin. What each pin rests on:

* brute force    -- a pure-Python loop implementation written from the block
                    definition ("Tensor Parallelism: Sharding Weights for
                    Parallel Layer Execution", section 3), tiny shapes;
* closed forms   -- hand-derived worked examples in tests/golden/;
* library        -- torch.nn.MultiheadAttention (bias off) and
                    torch.nn.functional.scaled_dot_product_attention in float64
                    on the CPU, whose default scale is 1/sqrt(head_dim);
* invariants     -- zero query -> mean of V; V = I exposes the softmax rows,
                    which are >= 0 and sum to 1; equal keys -> mean of V; one
                    key -> that key's V row; a dominant key -> its V row;
                    symmetries in the keys, queries and values;
* merge          -- log-sum-exp merging of any key split equals the unsplit
                    result (online softmax, as Ring Attention streams K/V);
* linearity      -- y is linear in W_O; W_V A pairs with A W_O.
* RMSNorm        -- brute force; torch.nn.functional.rms_norm in float64 (and a
                    torch pre-norm + MultiheadAttention block); closed forms of
                    constant rows; invariants (unit mean square, scale and sign).
* stacking       -- the multi-layer model ("TensorRT Multi-Device (multi-GPU)
                    support", "Validation (TRT 11.0)", multi-layer model) as
                    plain composition: the brute-force block, and torch's
                    MultiheadAttention, applied layer after layer, each layer
                    fed the previous layer's output (with and without
                    pre-norm); weights sharp enough that the layers' order and
                    their chaining both change the result.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

from . import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_cases.json")


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = max(np.linalg.norm(b), 1e-300)
    return float(np.linalg.norm(a - b) / den)


def _rng(seed):
    return np.random.default_rng(1000 + seed)


def _rand_block(rng, s, h):
    x = rng.standard_normal((s, h))
    ws = [rng.standard_normal((h, h)) / math.sqrt(h) for _ in range(4)]
    return x, ws


# ---------------------------------------------------------------- brute force
def pin_bruteforce(orc, tol=1e-12):
    worst = 0.0
    for seed, (s, h, nh) in enumerate([(5, 4, 1), (7, 8, 2), (9, 8, 4), (12, 6, 3)]):
        rng = _rng(seed)
        x, (wq, wk, wv, wo) = _rand_block(rng, s, h)
        x = x * 1.7  # sharper softmax than unit scores
        t = orc.block_forward(x, wq, wk, wv, wo, nh, taps=True)
        y_b, o_b, lse_b = brute.block(x, wq, wk, wv, wo, nh)
        worst = max(worst, _rel(t["y"], y_b), _rel(t["o"], o_b), _rel(t["lse"], lse_b))
        rows = [s - 1, 0, s // 2]
        y_rows = orc.block_forward(x, wq, wk, wv, wo, nh, rows=rows)
        worst = max(worst, _rel(y_rows, np.asarray(y_b)[rows]))
    return worst <= tol, f"max rel err vs brute force {worst:.3e}"


def pin_bruteforce_attention(orc, tol=1e-12):
    rng = _rng(50)
    worst = 0.0
    for sq, skv, d in [(3, 5, 4), (6, 1, 3), (4, 11, 8)]:
        q = rng.standard_normal((sq, d))
        k = rng.standard_normal((skv, d))
        v = rng.standard_normal((skv, d))
        o, lse = orc.attention(q, k, v)
        o_b, lse_b = brute.attention_one_head(q, k, v)
        worst = max(worst, _rel(o, o_b), _rel(lse, lse_b))
    return worst <= tol, f"max rel err vs brute-force attention {worst:.3e}"


# --------------------------------------------------------------- closed forms
def pin_closed_forms(orc, tol=1e-14):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    sigma = 1.0 / (1.0 + math.exp(-1.0 / math.sqrt(2.0)))
    worst = 0.0
    names = []
    for c in cases:
        want = np.array([[c0 + c1 * sigma for (c0, c1) in row] for row in c["y"]])
        got = orc.block_forward(np.array(c["x"], float), np.array(c["wq"], float),
                                np.array(c["wk"], float), np.array(c["wv"], float),
                                np.array(c["wo"], float), c["num_heads"])
        err = float(np.max(np.abs(got - want)))
        if err > tol:
            names.append(c["name"])
        worst = max(worst, err)
    return worst <= tol, f"closed-form max abs err {worst:.3e} failing={names}"


# -------------------------------------------------------------------- library
def pin_torch_mha(orc, tol=1e-10):
    import torch

    worst = 0.0
    for seed, (s, h, nh) in enumerate([(64, 64, 4), (33, 48, 3), (256, 256, 4)]):
        rng = _rng(100 + seed)
        x, (wq, wk, wv, wo) = _rand_block(rng, s, h)
        mha = torch.nn.MultiheadAttention(h, nh, bias=False, batch_first=True,
                                          dtype=torch.float64)
        with torch.no_grad():
            # torch applies x @ weight.T, so weight = W^T for Y = X W.
            mha.in_proj_weight.copy_(torch.from_numpy(np.concatenate([wq.T, wk.T, wv.T], 0)))
            mha.out_proj.weight.copy_(torch.from_numpy(wo.T.copy()))
            xt = torch.from_numpy(x)[None]
            ref, _ = mha(xt, xt, xt, need_weights=False)
        got = orc.block_forward(x, wq, wk, wv, wo, nh)
        worst = max(worst, _rel(got, ref[0].numpy()))
    return worst <= tol, f"max rel err vs torch MultiheadAttention {worst:.3e}"


def pin_torch_sdpa(orc, tol=1e-10):
    import torch
    import torch.nn.functional as F

    rng = _rng(200)
    worst = 0.0
    for nh, sq, skv, d in [(2, 17, 40, 8), (3, 64, 64, 64), (1, 5, 300, 128)]:
        q = rng.standard_normal((nh, sq, d))
        k = rng.standard_normal((nh, skv, d))
        v = rng.standard_normal((nh, skv, d))
        ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k),
                                             torch.from_numpy(v)).numpy()
        # sdpa scales by 1/sqrt(d) internally; the oracle takes q_scaled.
        o, _ = orc.partial_attention(orc.scale_query(q, d), k, v)
        worst = max(worst, _rel(o, ref))
    return worst <= tol, f"max rel err vs torch sdpa {worst:.3e}"


# ----------------------------------------------------------------- invariants
def pin_invariants(orc, tol=1e-12):
    rng = _rng(300)
    errs = {}
    d, skv = 8, 13
    k = rng.standard_normal((skv, d))
    v = rng.standard_normal((skv, d))
    # zero query: uniform scores -> column mean of V, lse = ln(skv)
    o, lse = orc.attention(np.zeros((2, d)), k, v)
    errs["zero_query"] = max(np.max(np.abs(o - v.mean(0))), abs(lse[0] - math.log(skv)))
    # V = identity (skv = d): O rows are the softmax rows: >= 0, sum to 1
    kk = rng.standard_normal((d, d))
    q = rng.standard_normal((5, d)) * 2
    o, lse = orc.attention(q, kk, np.eye(d))
    errs["rows_sum_to_one"] = float(np.max(np.abs(o.sum(1) - 1.0)))
    errs["rows_nonneg"] = float(max(0.0, -o.min()))
    s = q @ kk.T
    errs["softmax_row"] = float(np.max(np.abs(o - np.exp(s - lse[:, None]))))
    # all keys equal: any query -> mean of V
    keq = np.tile(rng.standard_normal((1, d)), (skv, 1))
    o, _ = orc.attention(rng.standard_normal((4, d)), keq, v)
    errs["equal_keys"] = float(np.max(np.abs(o - v.mean(0))))
    # one key: O = that V row, lse = the score
    q1 = rng.standard_normal((3, d))
    o, lse = orc.attention(q1, k[:1], v[:1])
    errs["one_key"] = float(max(np.max(np.abs(o - v[0])), np.max(np.abs(lse - q1 @ k[0]))))
    # dominant key: k_j = c q makes key j win by a margin > 40 nats
    qd = rng.standard_normal((1, d))
    kd = rng.standard_normal((skv, d)) * 0.01
    kd[4] = qd[0] * (60.0 / float(qd[0] @ qd[0]))
    o, _ = orc.attention(qd, kd, v)
    errs["dominant_key"] = float(np.max(np.abs(o[0] - v[4])))
    bad = {n: e for n, e in errs.items() if e > tol}
    return not bad, f"invariant errors {errs}"


def pin_symmetries(orc, tol=1e-12):
    rng = _rng(400)
    sq, skv, d = 9, 21, 8
    q = rng.standard_normal((sq, d))
    k = rng.standard_normal((skv, d))
    v = rng.standard_normal((skv, d))
    o, lse = orc.attention(q, k, v)
    errs = {}
    pk = rng.permutation(skv)
    o2, lse2 = orc.attention(q, k[pk], v[pk])
    errs["perm_kv"] = max(_rel(o2, o), _rel(lse2, lse))
    pq = rng.permutation(sq)
    o3, lse3 = orc.attention(q[pq], k, v)
    errs["perm_q"] = max(_rel(o3, o[pq]), _rel(lse3, lse[pq]))
    u = rng.standard_normal(d)
    o4, lse4 = orc.attention(q, k + u[None], v)
    errs["key_shift"] = max(_rel(o4, o), _rel(lse4, lse + q @ u))
    w = rng.standard_normal(d)
    o5, _ = orc.attention(q, k, v + w[None])
    errs["value_shift"] = _rel(o5, o + w[None])
    bad = {n: e for n, e in errs.items() if e > tol}
    return not bad, f"symmetry errors {errs}"


# ---------------------------------------------------------------------- merge
def pin_merge(orc, tol=1e-12):
    rng = _rng(500)
    nh, sq, skv, d = 3, 10, 37, 8
    q = rng.standard_normal((nh, sq, d))
    k = rng.standard_normal((nh, skv, d))
    v = rng.standard_normal((nh, skv, d))
    o_ref, lse_ref = orc.partial_attention(q, k, v)
    errs = {}
    splits = {
        "equal": [0, 12, 24, 37],  # near-equal blocks
        "uneven": [0, 3, 30, 37],
        "size_one": [0, 1, 2, 36, 37],
        "whole": [0, 37],
    }
    for name, cuts in splits.items():
        parts = [orc.partial_attention(q, k[:, a:b], v[:, a:b]) for a, b in zip(cuts[:-1], cuts[1:])]
        o, lse = orc.merge_partials([p[0] for p in parts], [p[1] for p in parts])
        errs[name] = max(_rel(o, o_ref), _rel(lse, lse_ref))
        if name == "uneven":
            rev = parts[::-1]
            o, lse = orc.merge_partials([p[0] for p in rev], [p[1] for p in rev])
            errs["reversed"] = max(_rel(o, o_ref), _rel(lse, lse_ref))
            # an empty block carries lse = -inf and must not change the result
            e_o, e_l = orc.partial_attention(q, k[:, :0], v[:, :0])
            o, lse = orc.merge_partials([p[0] for p in parts] + [e_o], [p[1] for p in parts] + [e_l])
            errs["with_empty"] = max(_rel(o, o_ref), _rel(lse, lse_ref))
    bad = {n: e for n, e in errs.items() if e > tol}
    return not bad, f"merge errors {errs}"


def pin_merge_rows(orc, tol=1e-12):
    """The rank share: rows [a, b) of the full result equal the block run on
    that Q chunk alone against the full K/V."""
    rng = _rng(600)
    s, h, nh = 24, 16, 2
    x, (wq, wk, wv, wo) = _rand_block(rng, s, h)
    full = orc.block_forward(x, wq, wk, wv, wo, nh)
    worst = 0.0
    for r in range(4):
        rows = np.arange(r * s // 4, (r + 1) * s // 4)
        worst = max(worst, _rel(orc.block_forward(x, wq, wk, wv, wo, nh, rows=rows), full[rows]))
    return worst <= tol, f"row-chunk err {worst:.3e}"


# ------------------------------------------------------------------ linearity
def pin_linearity(orc, tol=1e-12):
    rng = _rng(700)
    s, h, nh = 11, 12, 3
    x, (wq, wk, wv, wo) = _rand_block(rng, s, h)
    y = orc.block_forward(x, wq, wk, wv, wo, nh)
    errs = {"scale_wo": _rel(orc.block_forward(x, wq, wk, wv, 2.0 * wo, nh), 2.0 * y)}
    # A block-diagonal per head keeps every head's value inside its own columns.
    d = h // nh
    a = np.zeros((h, h))
    for j in range(nh):
        a[j * d:(j + 1) * d, j * d:(j + 1) * d] = rng.standard_normal((d, d))
    errs["wv_a_wo"] = _rel(orc.block_forward(x, wq, wk, wv @ a, wo, nh),
                           orc.block_forward(x, wq, wk, wv, a @ wo, nh))
    bad = {n: e for n, e in errs.items() if e > tol}
    return not bad, f"linearity errors {errs}"


# -------------------------------------------------------------------- RMSNorm
def pin_rmsnorm_bruteforce(orc, tol=1e-12):
    worst = 0.0
    for seed, (s, h, nh) in enumerate([(5, 4, 1), (7, 8, 2), (6, 6, 3)]):
        rng = _rng(300 + seed)
        x, (wq, wk, wv, wo) = _rand_block(rng, s, h)
        x = x * rng.uniform(0.01, 3.0, size=(s, 1))  # rows of different magnitudes
        g = rng.uniform(0.5, 1.5, size=h)
        eps = [1e-6, 1e-3, 0.25][seed]
        xn_b = brute.rms_norm(x, g, eps)
        worst = max(worst, _rel(orc.rms_norm(x, g, eps), xn_b), _rel(orc.rms_norm(x, None, eps),
                                                                     brute.rms_norm(x, None, eps)))
        y_b, _, _ = brute.block(xn_b, wq, wk, wv, wo, nh)
        worst = max(worst, _rel(orc.block_forward(x, wq, wk, wv, wo, nh, norm=(g, eps)), y_b))
    return worst <= tol, f"max rel err vs brute-force RMSNorm {worst:.3e}"


def pin_rmsnorm_torch(orc, tol=1e-10):
    import torch
    import torch.nn.functional as F

    worst = 0.0
    for seed, (s, h, nh) in enumerate([(64, 64, 4), (40, 96, 3)]):
        rng = _rng(320 + seed)
        x, (wq, wk, wv, wo) = _rand_block(rng, s, h)
        g = rng.uniform(0.5, 1.5, size=h)
        xt = torch.from_numpy(x)
        ref_n = F.rms_norm(xt, (h,), weight=torch.from_numpy(g), eps=1e-6).numpy()
        worst = max(worst, _rel(orc.rms_norm(x, g, 1e-6), ref_n))
        mha = torch.nn.MultiheadAttention(h, nh, bias=False, batch_first=True, dtype=torch.float64)
        with torch.no_grad():
            mha.in_proj_weight.copy_(torch.from_numpy(np.concatenate([wq.T, wk.T, wv.T], 0)))
            mha.out_proj.weight.copy_(torch.from_numpy(wo.T.copy()))
            xn = torch.from_numpy(ref_n)[None]
            ref, _ = mha(xn, xn, xn, need_weights=False)
        worst = max(worst, _rel(orc.block_forward(x, wq, wk, wv, wo, nh, norm=(g, 1e-6)), ref[0].numpy()))
    return worst <= tol, f"max rel err vs torch rms_norm (+ MultiheadAttention) {worst:.3e}"


def pin_rmsnorm_closed_forms(orc, tol=1e-14):
    # a constant row c*1 has mean square c^2: every entry becomes c / sqrt(c^2 + eps) * g_j
    errs = []
    g = np.array([1.0, 2.0, 0.5, -1.0])
    for c, eps in [(3.0, 1e-6), (1e-3, 1e-6), (-2.0, 0.0), (0.5, 0.25)]:
        x = np.full((1, 4), c)
        want = c / math.sqrt(c * c + eps) * g
        errs.append(float(np.max(np.abs(orc.rms_norm(x, g, eps)[0] - want))))
    # alternating row (a, -a, a, -a): the same mean square a^2
    a, eps = 2.0, 0.5
    x = np.array([[a, -a, a, -a]])
    want = np.array([a, -a, a, -a]) / math.sqrt(a * a + eps)
    errs.append(float(np.max(np.abs(orc.rms_norm(x, None, eps)[0] - want))))
    return max(errs) <= tol, f"RMSNorm closed-form errors {errs}"


def pin_rmsnorm_invariants(orc, tol=1e-12):
    rng = _rng(340)
    x = rng.standard_normal((6, 10)) * rng.uniform(0.1, 5.0, size=(6, 1))
    g = rng.uniform(0.5, 1.5, size=10)
    errs = {}
    y = orc.rms_norm(x, None, 0.0)
    errs["unit_mean_square"] = float(np.max(np.abs((y * y).mean(axis=1) - 1.0)))
    errs["scale"] = _rel(orc.rms_norm(3.7 * x, None, 0.0), y)
    errs["sign"] = _rel(orc.rms_norm(-x, g, 1e-6), -orc.rms_norm(x, g, 1e-6))
    errs["gain"] = _rel(orc.rms_norm(x, g, 1e-6), orc.rms_norm(x, None, 1e-6) * g)
    # with eps = 0 a pre-normed block does not see the scale of its input rows
    s, h, nh = 7, 8, 2
    xb, (wq, wk, wv, wo) = _rand_block(rng, s, h)
    lam = rng.uniform(0.2, 5.0, size=(s, 1))
    gb = rng.uniform(0.5, 1.5, size=h)
    errs["block_row_scale"] = _rel(orc.block_forward(lam * xb, wq, wk, wv, wo, nh, norm=(gb, 0.0)),
                                   orc.block_forward(xb, wq, wk, wv, wo, nh, norm=(gb, 0.0)))
    errs["block_norm_changes_output"] = 0.0 if _rel(
        orc.block_forward(lam * xb, wq, wk, wv, wo, nh, norm=(gb, 0.0)),
        orc.block_forward(lam * xb, wq, wk, wv, wo, nh)) > 1e-3 else 1.0
    bad = {n: e for n, e in errs.items() if e > tol}
    return not bad, f"RMSNorm invariant errors {errs}"


# ------------------------------------------------------------------- stacking
def _stack_case(rng, s, h, n_layers, use_norm):
    """Input and n_layers independent weight sets. W_Q and W_K with std
    3/sqrt(h) keep every layer's softmax sharp, so the rows stay distinct
    (relative row spread above 0.18 after every layer of these cases) instead
    of collapsing to one vector, and the layers do not commute; W_V and W_O
    have std 1.5/sqrt(h)."""
    x = rng.standard_normal((s, h)) * 1.5
    layers = [tuple(rng.standard_normal((h, h)) * (f / math.sqrt(h)) for f in (3.0, 3.0, 1.5, 1.5))
              for _ in range(n_layers)]
    norms = None
    if use_norm:
        norms = [(rng.uniform(0.5, 1.5, size=h), [1e-6, 1e-3, 0.05][i % 3]) for i in range(n_layers)]
    return x, layers, norms


def pin_stack_bruteforce(orc, tol=1e-12):
    """stack_forward against the brute-force block applied layer by layer,
    layer l fed layer l-1's output (1 layer: the block itself)."""
    worst = 0.0
    cases = [(5, 4, 1, 1, False), (6, 8, 2, 2, False), (7, 6, 3, 3, False), (6, 8, 2, 3, True),
             (5, 4, 2, 2, True)]
    for seed, (s, h, nh, n_layers, use_norm) in enumerate(cases):
        rng = _rng(800 + seed)
        x, layers, norms = _stack_case(rng, s, h, n_layers, use_norm)
        cur = x
        for i, (wq, wk, wv, wo) in enumerate(layers):
            if norms is not None:
                cur = brute.rms_norm(cur, norms[i][0], norms[i][1])
            cur, _, _ = brute.block(cur, wq, wk, wv, wo, nh)
        worst = max(worst, _rel(orc.stack_forward(x, layers, nh, norms=norms), cur))
    return worst <= tol, f"max rel err vs brute-force layer-by-layer stack {worst:.3e}"


def pin_stack_torch(orc, tol=1e-10):
    """stack_forward against torch.nn.MultiheadAttention (bias off, float64)
    applied layer after layer, with and without torch's rms_norm before each
    layer."""
    import torch
    import torch.nn.functional as F

    worst = 0.0
    for seed, (s, h, nh, n_layers, use_norm) in enumerate([(40, 64, 4, 3, False), (33, 48, 3, 4, True)]):
        rng = _rng(850 + seed)
        x, layers, norms = _stack_case(rng, s, h, n_layers, use_norm)
        cur = torch.from_numpy(x)[None]
        with torch.no_grad():
            for i, (wq, wk, wv, wo) in enumerate(layers):
                mha = torch.nn.MultiheadAttention(h, nh, bias=False, batch_first=True, dtype=torch.float64)
                mha.in_proj_weight.copy_(torch.from_numpy(np.concatenate([wq.T, wk.T, wv.T], 0)))
                mha.out_proj.weight.copy_(torch.from_numpy(wo.T.copy()))
                if norms is not None:
                    cur = F.rms_norm(cur, (h,), weight=torch.from_numpy(norms[i][0]), eps=norms[i][1])
                cur, _ = mha(cur, cur, cur, need_weights=False)
        worst = max(worst, _rel(orc.stack_forward(x, layers, nh, norms=norms), cur[0].numpy()))
    return worst <= tol, f"max rel err vs torch MultiheadAttention layer by layer {worst:.3e}"


ALL_PINS = [
    pin_bruteforce, pin_bruteforce_attention, pin_closed_forms, pin_torch_mha,
    pin_torch_sdpa, pin_invariants, pin_symmetries, pin_merge, pin_merge_rows,
    pin_linearity, pin_rmsnorm_bruteforce, pin_rmsnorm_torch, pin_rmsnorm_closed_forms,
    pin_rmsnorm_invariants, pin_stack_bruteforce, pin_stack_torch,
]
