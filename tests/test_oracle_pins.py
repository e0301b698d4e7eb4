"""CPU tests: the fp64 oracle against its pins, and the pins against planted
mistakes in a copy of the oracle (a pin set that no mistake can trip pins
nothing)."""

from __future__ import annotations

import importlib.util
import os

import numpy as np
import pytest

import oracle
from oracle import mha as oracle_attention

from . import pins

ORACLE_SRC = oracle_attention.__file__


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    ok, detail = pin(oracle_attention)
    assert ok, detail


# (name, [(old, new), ...]) -- each replacement must match exactly once.
MUTANTS = [
    ("projection_transposed", [("return as_f64(x) @ as_f64(w)", "return as_f64(x) @ as_f64(w).T")]),
    ("output_projection_transposed", [("y = project(o, wo)", "y = project(o, as_f64(wo).T)")]),
    ("scale_1_over_d", [("(1.0 / np.sqrt(head_dim))", "(1.0 / head_dim)")]),
    ("scale_missing", [("return as_f64(q) * (1.0 / np.sqrt(head_dim))", "return as_f64(q)")]),
    ("heads_interleaved", [
        ("t.reshape(s, num_heads, d).transpose(1, 0, 2)", "t.reshape(s, d, num_heads).transpose(2, 0, 1)"),
        ("t.transpose(1, 0, 2).reshape(s, hh * d)", "t.transpose(1, 2, 0).reshape(s, hh * d)"),
    ]),
    ("lse_without_log", [("m[:, 0] + np.log(l[:, 0])", "m[:, 0] + l[:, 0]")]),
    ("softmax_not_normalised", [("o[r0:r1] = (p / l) @ v", "o[r0:r1] = p @ v")]),
    ("score_sign", [("s = q[r0:r1] @ k.T", "s = -(q[r0:r1] @ k.T)")]),
    ("keys_from_wv", [("k = split_heads(project(x, wk), num_heads)", "k = split_heads(project(x, wv), num_heads)")]),
    ("query_from_wk", [("project(x[rows], wq)", "project(x[rows], wk)")]),
    ("query_rows_ignored", [("project(x[rows], wq)", "project(x, wq)[: len(rows)]")]),
    ("merge_weight_sign", [("wn = np.exp(lse_parts - lse_safe[None])", "wn = np.exp(lse_safe[None] - lse_parts)")]),
    ("merge_lse_drops_max", [("m_safe + np.log(np.where(empty, 1.0, total))", "np.log(np.where(empty, 1.0, total))")]),
    ("merge_unnormalised", [("wn = np.exp(lse_parts - lse_safe[None])", "wn = np.exp(lse_parts - m_safe[None])")]),
    ("rms_sum_not_mean", [("mean_sq = (x * x).mean(axis=-1, keepdims=True)",
                           "mean_sq = (x * x).sum(axis=-1, keepdims=True)")]),
    ("rms_no_square", [("mean_sq = (x * x).mean(axis=-1, keepdims=True)",
                        "mean_sq = np.abs(x).mean(axis=-1, keepdims=True)")]),
    ("rms_eps_outside_sqrt", [("y = x / np.sqrt(mean_sq + eps)", "y = x / (np.sqrt(mean_sq) + eps)")]),
    ("rms_gain_dropped", [("y = y * as_f64(gain)", "y = y")]),
    ("rms_norm_skipped", [("x = rms_norm(x, norm[0], norm[1])", "x = x")]),
    ("rms_norm_after_projection", [("x = rms_norm(x, norm[0], norm[1])", "x = x * 1.0"),
                                   ("y = project(o, wo)", "y = project(o, wo) if norm is None else rms_norm(project(o, wo), norm[0], norm[1])")]),
    ("stack_unchained", [("y = block_forward(y, wq, wk, wv, wo, num_heads,", "y = block_forward(as_f64(x), wq, wk, wv, wo, num_heads,")]),
    ("stack_reversed", [("in enumerate(layers):", "in enumerate(layers[::-1]):")]),
    ("stack_drops_last_layer", [("in enumerate(layers):", "in enumerate(layers[:-1]):")]),
    ("stack_first_norm_only", [("else norms[i])", "else norms[0])")]),
]


def _load_mutant(name, edits):
    with open(ORACLE_SRC) as f:
        src = f.read()
    for old, new in edits:
        assert src.count(old) == 1, f"{name}: pattern {old!r} matches {src.count(old)} times"
        src = src.replace(old, new)
    spec = importlib.util.spec_from_loader(f"oracle_mutant_{name}", loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__file__ = os.path.join(os.path.dirname(ORACLE_SRC), f"mutant_{name}.py")
    exec(compile(src, mod.__file__, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, edits):
    mod = _load_mutant(name, edits)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            ok, _ = pin(mod)
        except Exception:  # a crash also counts as the pin catching it
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name} passed every pin"


def test_oracle_package_exports():
    assert oracle.block_forward is oracle_attention.block_forward
    x = np.zeros((3, 4))
    w = np.eye(4)
    assert oracle.block_forward(x, w, w, w, w, 2).shape == (3, 4)
