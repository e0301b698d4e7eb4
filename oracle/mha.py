"""CPU fp64 oracle of the non-causal multi-head self-attention block.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it, to check and to time against.

It is a plain, slow, obviously correct restatement of what the pages define,
in float64 numpy, sharing no code with the HIP library. Every query row does one
full, unsplit softmax over all of its keys; nothing is blocked across keys,
fused or reordered beyond the definition. Inputs are taken exactly as given
(the fp16 or fp32 values the GPU receives, upcast to float64).

Sources, by page title and section:

* MHA operations: project X to Q, K, V; split them into heads; scaled
  dot-product attention per head; concatenate the head outputs and multiply by
  W_O -- "Tensor Parallelism: Sharding Weights for Parallel Layer Execution",
  section 3 "Parallelizing the Multi-Head Attention Block". A linear layer is
  Y = X A (section 1 of the same page), so each W is [h_in, h_out].
* Block contents (Q/K/V projections, scaled dot-product attention, output
  projection; 32 heads of 128 at hidden 4096; tensor (sequence, batch, hidden))
  and the pre-scaled query tensor ``q_scaled`` that feeds the QK^T product --
  "Multi-Device Attention Inference with TensorRT", "What is hint.json?" and
  "Generating the ONNX Models", Step 1.
* Non-causal (bidirectional, no mask) attention -- the news summary of
  "Scaling AI Inference Across Multiple GPUs Using NVIDIA TensorRT with
  Multi-Device Inference Support", section on context parallelism.
* Rank share: a rank keeps its own Q slice and attends to the gathered full
  K/V (AllGather KV); or K/V stream in blocks and the per-block results are
  combined by online softmax (Ring Attention) -- same summary, section on the
  three context-parallel implementations.
* Stacked blocks -- "TensorRT Multi-Device (multi-GPU) support", "Validation
  (TRT 11.0)", multi-layer model.

Readings where the pages are silent (each listed in the design notes):
softmax scale 1/sqrt(d) applied to Q before QK^T; no biases; head j owns
columns [j*d, (j+1)*d); a KV block's partial output is normalised within the
block and carries its natural-log LSE; stacking is plain composition.
RMSNorm, which the sample lists among the model's operations without placement
or parameters, is optional here: when asked for, it normalises each token row
of the block input (pre-norm) with eps 1e-6 and unit gain unless one is given.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "as_f64", "project", "scale_query", "split_heads", "merge_heads",
    "attention", "partial_attention", "merge_partials", "rms_norm", "block_forward",
    "stack_forward",
]

RMS_EPS = 1e-6  # reading: the sample gives no epsilon

ROW_BLOCK = 256  # query rows per softmax batch; memory only, no effect on values


def as_f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def project(x, w) -> np.ndarray:
    """Linear layer Y = X W with W stored [h_in, h_out] (MHA step 1; section 1's
    Y = X A)."""
    return as_f64(x) @ as_f64(w)


def scale_query(q, head_dim: int) -> np.ndarray:
    """q_scaled = Q / sqrt(d): the query tensor that feeds the QK^T matmul."""
    return as_f64(q) * (1.0 / np.sqrt(head_dim))


def split_heads(t, num_heads: int) -> np.ndarray:
    """[S, h] -> [H, S, d]; head j takes columns [j*d, (j+1)*d) (MHA step 2)."""
    t = as_f64(t)
    s, h = t.shape
    d = h // num_heads
    return t.reshape(s, num_heads, d).transpose(1, 0, 2).copy()


def merge_heads(t) -> np.ndarray:
    """[H, S, d] -> [S, h]: concatenation of the head outputs (MHA step 4)."""
    t = as_f64(t)
    hh, s, d = t.shape
    return t.transpose(1, 0, 2).reshape(s, hh * d).copy()


def attention(q_scaled, k, v):
    """Scaled dot-product attention of one head, no mask (MHA step 3).

    q_scaled [Sq, d], k [Skv, d], v [Skv, d] -> (o [Sq, d], lse [Sq]).
    For each query row i: s = q_i K^T over all Skv keys, m = max s,
    p = exp(s - m), l = sum p, o_i = (p / l) V, lse_i = m + ln l.
    Skv = 0 has no softmax; it returns o = 0 and lse = -inf, the values that
    give such a block zero weight in a merge.
    """
    q = as_f64(q_scaled)
    k = as_f64(k)
    v = as_f64(v)
    sq, d = q.shape
    skv = k.shape[0]
    o = np.zeros((sq, v.shape[1]), dtype=np.float64)
    lse = np.full((sq,), -np.inf, dtype=np.float64)
    if skv == 0:
        return o, lse
    for r0 in range(0, sq, ROW_BLOCK):
        r1 = min(sq, r0 + ROW_BLOCK)
        s = q[r0:r1] @ k.T
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        l = p.sum(axis=1, keepdims=True)
        o[r0:r1] = (p / l) @ v
        lse[r0:r1] = m[:, 0] + np.log(l[:, 0])
    return o, lse


def partial_attention(q_scaled, k_block, v_block):
    """One KV block's share for a rank's Q chunk, all heads.

    q_scaled [H, Sq, d]; k_block, v_block [H, Skv_b, d] -> (o_b [H, Sq, d]
    normalised within the block, lse_b [H, Sq]). This is `attention` applied to
    the keys of one block only.
    """
    q = as_f64(q_scaled)
    hh = q.shape[0]
    o = np.empty((hh, q.shape[1], as_f64(v_block).shape[2]), dtype=np.float64)
    lse = np.empty((hh, q.shape[1]), dtype=np.float64)
    for j in range(hh):
        o[j], lse[j] = attention(q[j], k_block[j], v_block[j])
    return o, lse


def merge_partials(o_parts, lse_parts):
    """Combine per-block partial results by log-sum-exp (online softmax).

    o_parts [n, ..., d] (each normalised within its block), lse_parts [n, ...].
    With M = max_b lse_b: lse = M + ln sum_b exp(lse_b - M) and
    o = sum_b exp(lse_b - lse) o_b. Rows whose blocks are all empty
    (every lse_b = -inf) get o = 0 and lse = -inf.
    """
    o_parts = as_f64(o_parts)
    lse_parts = as_f64(lse_parts)
    m = lse_parts.max(axis=0)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(lse_parts - m_safe[None])
    total = w.sum(axis=0)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, total)))
    lse_safe = np.where(empty, 0.0, lse)
    wn = np.exp(lse_parts - lse_safe[None])
    wn = np.where(empty[None], 0.0, wn)
    o = (wn[..., None] * o_parts).sum(axis=0)
    return o, lse


def rms_norm(x, gain=None, eps: float = RMS_EPS) -> np.ndarray:
    """RMSNorm of every token row: x / sqrt(mean_j x_j^2 + eps), times gain.

    The sample's self-attention model lists RMSNorm among its operations
    ("Multi-Device Attention Inference with TensorRT", "Generating the ONNX
    Models", Step 1), and the same page's introduction has each GPU normalise
    its own tokens, i.e. the operation is local to a token. gain [h] defaults
    to ones.
    """
    x = as_f64(x)
    mean_sq = (x * x).mean(axis=-1, keepdims=True)
    y = x / np.sqrt(mean_sq + eps)
    if gain is not None:
        y = y * as_f64(gain)
    return y


def block_forward(x, wq, wk, wv, wo, num_heads: int, rows=None, taps: bool = False, norm=None):
    """Forward pass of one block: y = Concat_j(attn_j) W_O.

    x [S, h]; rows selects the query rows to compute (all when None). K and V
    always come from all S rows; the result for a selected row is exact, not
    an approximation. norm = (gain or None, eps) applies RMSNorm to x first
    (pre-norm); None leaves x as is. Returns y [len(rows), h], or with
    ``taps`` a dict with q_scaled [H, R, d], k [H, S, d], v [H, S, d],
    o [R, h] (pre-projection), lse [H, R] and y.
    """
    x = as_f64(x)
    if norm is not None:
        x = rms_norm(x, norm[0], norm[1])
    s, h = x.shape
    d = h // num_heads
    if rows is None:
        rows = np.arange(s)
    rows = np.asarray(rows, dtype=np.int64)
    k = split_heads(project(x, wk), num_heads)
    v = split_heads(project(x, wv), num_heads)
    q = split_heads(scale_query(project(x[rows], wq), d), num_heads)
    o_heads, lse = partial_attention(q, k, v)
    o = merge_heads(o_heads)
    y = project(o, wo)
    if taps:
        return {"q_scaled": q, "k": k, "v": v, "o": o, "lse": lse, "y": y}
    return y


def stack_forward(x, layers, num_heads: int, norms=None):
    """Plain composition of blocks: x_{l+1} = Block_l(x_l) (multi-layer model).
    norms: None, or one (gain or None, eps) per layer for its pre-norm."""
    y = as_f64(x)
    for i, (wq, wk, wv, wo) in enumerate(layers):
        y = block_forward(y, wq, wk, wv, wo, num_heads, norm=None if norms is None else norms[i])
    return y
