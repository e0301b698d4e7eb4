"""CPU tests of the Ulysses / tensor-parallel share oracle against its pins,
and of the pins against planted mistakes in a copy of oracle/shares.py."""

from __future__ import annotations

import importlib.util
import os
import sys

import pytest

from oracle import shares as oracle_shares

from . import pins_shares

SRC = oracle_shares.__file__


@pytest.mark.parametrize("pin", pins_shares.SHARE_PINS, ids=lambda p: p.__name__)
def test_shares_pin(pin):
    ok, detail = pin(oracle_shares)
    assert ok, detail


MUTANTS = [
    ("head_range_shifted", [("return slice(rank * hl, (rank + 1) * hl)", "return slice(rank * hl + 1, (rank + 1) * hl + 1)")]),
    ("recv_qk_own_rows", [("np.stack([t[hs, row_range(s, n_ranks, p)] for p in range(n_ranks)])",
                           "np.stack([t[hs, row_range(s, n_ranks, rank)] for p in range(n_ranks)])")]),
    ("recv_vt_rows_not_keys", [("np.stack([vt[hs, :, row_range(s, n_ranks, p)] for p in range(n_ranks)])",
                                "np.stack([vt[hs, row_range(vt.shape[1], n_ranks, p), :] for p in range(n_ranks)])")]),
    ("gather_reversed", [("np.concatenate([recv[p] for p in range(n)], axis=1)",
                          "np.concatenate([recv[n - 1 - p] for p in range(n)], axis=1)")]),
    ("unpack_rows_not_cols", [("np.concatenate([recv[r] for r in range(recv.shape[0])], axis=1)",
                               "np.concatenate([recv[r] for r in range(recv.shape[0])], axis=0)")]),
    ("share_all_heads", [("o, lse = partial_attention(as_f64(q_scaled)[hs], as_f64(k)[hs], as_f64(v)[hs])",
                          "o, lse = partial_attention(as_f64(q_scaled), as_f64(k), as_f64(v))")]),
    ("tp_wo_column_shard", [("return project(merge_heads(o), as_f64(wo)[cols, :])",
                             "return project(merge_heads(o), as_f64(wo)[:, cols].T)")]),
    ("tp_no_query_scale", [("q = split_heads(scale_query(project(x[rows], as_f64(wq)[:, cols]), d), hl)",
                            "q = split_heads(project(x[rows], as_f64(wq)[:, cols]), hl)")]),
    ("tp_keys_from_wq", [("k = split_heads(project(x, as_f64(wk)[:, cols]), hl)",
                          "k = split_heads(project(x, as_f64(wq)[:, cols]), hl)")]),
]


def _load_mutant(name, edits):
    with open(SRC) as f:
        src = f.read()
    for old, new in edits:
        assert src.count(old) == 1, f"{name}: pattern {old!r} matches {src.count(old)} times"
        src = src.replace(old, new)
    modname = f"oracle._mutant_shares_{name}"
    spec = importlib.util.spec_from_loader(modname, loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__file__ = os.path.join(os.path.dirname(SRC), f"_mutant_shares_{name}.py")
    mod.__package__ = "oracle"
    sys.modules[modname] = mod
    try:
        exec(compile(src, mod.__file__, "exec"), mod.__dict__)
    finally:
        sys.modules.pop(modname, None)
    return mod


@pytest.mark.parametrize("name,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, edits):
    mod = _load_mutant(name, edits)
    failed = []
    for pin in pins_shares.SHARE_PINS:
        try:
            ok, _ = pin(mod)
        except Exception:
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name} passed every pin"
