"""Seeded synthetic inputs for the self-attention block and its rank share.

This module only draws random numbers with a fixed recipe; it holds none of the
method's arithmetic, so both the fp64 oracle's tests and the HIP path's tests can
take their inputs from it.

Recipe (the pages print no data, so the workloads are stood in for by draws of
the shapes they name: an activation of shape (sequence_length, batch_size,
hidden) in fp16 with hidden 4096 / 32 heads of 128 ["Multi-Device Attention
Inference with TensorRT", "Generating the ONNX Models", Step 1], sequences of
8K-64K tokens ["TensorRT Multi-Device (multi-GPU) support", "Validation (TRT
11.0)"]):

* generator: ``numpy.random.default_rng(seed)`` (PCG64), seed 0 by default;
* draw order: X [S, h] first, then for each layer W_Q, W_K, W_V, W_O, each
  [h, h], each as ``standard_normal(dtype=float32)``;
* X ~ N(0, 1); every weight ~ N(0, 1/h) (variance 1/h, so each projection keeps
  unit variance);
* the draws are then cast to the configuration's dtype (fp16, or fp32 for the
  tiny configuration). The cast arrays are what both sides receive.

Attention-only inputs (for the rank-share calls) draw q_scaled ~ N(0, 1/d) and
K, V ~ N(0, 1), which is the distribution the block itself produces after the
projections and the 1/sqrt(d) pre-scale; ``score_std`` scales q to make the
softmax more peaked for edge-case tests.
"""

from __future__ import annotations

import numpy as np

__all__ = ["block_inputs", "attention_inputs", "sample_rows"]


def _cast(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a.astype(dtype))


def block_inputs(seq: int, hidden: int, layers: int = 1, dtype=np.float16, seed: int = 0):
    """Return ``(x, [(wq, wk, wv, wo), ...])`` for ``layers`` blocks.

    x is [seq, hidden] (batch 1 folded away), each weight is [hidden, hidden]
    applied as Y = X W (input features along rows).
    """
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((seq, hidden), dtype=np.float32)
    std = np.float32(1.0 / np.sqrt(hidden))
    weights = []
    for _ in range(layers):
        ws = []
        for _name in ("wq", "wk", "wv", "wo"):
            w = rng.standard_normal((hidden, hidden), dtype=np.float32)
            w *= std
            ws.append(_cast(w, dtype))
        weights.append(tuple(ws))
    return _cast(x, dtype), weights


def norm_gain(hidden: int, dtype=np.float16, seed: int = 0):
    """RMSNorm gain [hidden] ~ U(0.5, 1.5) from its own seeded stream (the
    default reading is unit gain; tests also use a non-trivial one)."""
    rng = np.random.default_rng(seed + 7919)
    return _cast(rng.uniform(0.5, 1.5, size=hidden).astype(np.float32), dtype)


def attention_inputs(num_heads: int, sq: int, skv: int, head_dim: int, dtype=np.float16,
                     seed: int = 0, score_std: float = 1.0):
    """Return head-major ``(q_scaled [H,sq,d], k [H,skv,d], v [H,skv,d])``.

    q_scaled ~ N(0, score_std^2 / d), K, V ~ N(0, 1), so the scores have
    standard deviation about ``score_std``.
    """
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((num_heads, sq, head_dim), dtype=np.float32)
    q *= np.float32(score_std / np.sqrt(head_dim))
    k = rng.standard_normal((num_heads, skv, head_dim), dtype=np.float32)
    v = rng.standard_normal((num_heads, skv, head_dim), dtype=np.float32)
    return _cast(q, dtype), _cast(k, dtype), _cast(v, dtype)


def sample_rows(seq: int, count: int = 256, seed: int = 0, must=()):
    """Sorted unique row indices in [0, seq): ``count`` seeded draws plus the
    first row, the last row and every index in ``must`` (e.g. chunk borders)."""
    rng = np.random.default_rng(seed + 7919)
    picks = set(int(i) for i in rng.choice(seq, size=min(count, seq), replace=False))
    picks.update({0, seq - 1})
    picks.update(int(i) for i in must if 0 <= int(i) < seq)
    return np.array(sorted(picks), dtype=np.int64)
