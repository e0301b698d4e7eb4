"""CPU fp64 oracle of one GPU's share under Ulysses context parallelism and
under tensor parallelism -- TEST INFRASTRUCTURE ONLY (same rules as
oracle/mha.py: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may use it; the HIP library never does).

Sources, by page title and section:

* Ulysses: the sequence is split across the GPUs; before attention an
  all-to-all on Q, K and V gives every GPU the whole sequence for a subset of
  the attention heads; a second all-to-all puts the head and sequence
  dimensions back -- news summary of "Scaling AI Inference Across Multiple
  GPUs Using NVIDIA TensorRT with Multi-Device Inference Support", the three
  context-parallel implementations (DeepSpeed Ulysses).
* Tensor parallelism of the attention block: W_Q, W_K, W_V split by columns
  (each GPU owns a subset of heads), attention local to the GPU, W_O split by
  rows, each GPU's product is a partial output and an all-reduce sums them --
  "Tensor Parallelism: Sharding Weights for Parallel Layer Execution",
  section 1 (column- and row-wise splits of Y = X A) and section 3, steps 1-4.

Readings (pages silent): N ranks own equal, contiguous head ranges (rank r
owns heads [r*H/N, (r+1)*H/N)) and equal, contiguous sequence chunks (rank p
owns rows [p*S/N, (p+1)*S/N)); all-to-all block p on the receiving side is
the one rank p sent, in rank order.

The layout functions below are the index rearrangements the two all-to-alls
perform, written as plain numpy slicing; attention itself is oracle.mha's.
"""

from __future__ import annotations

import numpy as np

from .mha import as_f64, merge_heads, partial_attention, project, scale_query, split_heads

__all__ = [
    "head_range", "row_range", "ulysses_recv_qk", "ulysses_recv_vt", "ulysses_gather_qk",
    "ulysses_gather_vt", "ulysses_share", "ulysses_return_o", "ulysses_unpack_o", "tp_share",
]


def head_range(num_heads: int, n_ranks: int, rank: int) -> slice:
    """Heads owned by `rank` (Ulysses after the first all-to-all; TP)."""
    hl = num_heads // n_ranks
    return slice(rank * hl, (rank + 1) * hl)


def row_range(seq: int, n_ranks: int, rank: int) -> slice:
    """Sequence rows owned by `rank` before the first all-to-all."""
    c = seq // n_ranks
    return slice(rank * c, (rank + 1) * c)


def ulysses_recv_qk(t, n_ranks: int, rank: int) -> np.ndarray:
    """First all-to-all, Q or K: t is the head-major [H][S][d] tensor whose row
    chunk p lives on rank p; rank `rank` receives block p = t[its heads][rows
    of p], i.e. [N][H/N][S/N][d]."""
    t = np.asarray(t)
    s = t.shape[1]
    hs = head_range(t.shape[0], n_ranks, rank)
    return np.stack([t[hs, row_range(s, n_ranks, p)] for p in range(n_ranks)])


def ulysses_recv_vt(vt, n_ranks: int, rank: int) -> np.ndarray:
    """First all-to-all, V^T [H][d][S] (keys last): blocks [N][H/N][d][S/N]."""
    vt = np.asarray(vt)
    s = vt.shape[2]
    hs = head_range(vt.shape[0], n_ranks, rank)
    return np.stack([vt[hs, :, row_range(s, n_ranks, p)] for p in range(n_ranks)])


def ulysses_gather_qk(recv) -> np.ndarray:
    """The receiving rank's full-sequence layout [H/N][S][d] from its blocks
    [N][H/N][S/N][d]: block p supplies rows [p*S/N, (p+1)*S/N)."""
    recv = np.asarray(recv)
    n, hl, c, d = recv.shape
    return np.concatenate([recv[p] for p in range(n)], axis=1).reshape(hl, n * c, d)


def ulysses_gather_vt(recv) -> np.ndarray:
    """[N][H/N][d][S/N] -> [H/N][d][S]."""
    recv = np.asarray(recv)
    return np.concatenate([recv[p] for p in range(recv.shape[0])], axis=2)


def ulysses_share(q_scaled, k, v, n_ranks: int, rank: int):
    """Rank `rank`'s Ulysses attention: its heads over the FULL sequence.

    q_scaled, k, v [H][S][d] -> (o [S][(H/N)*d] token-major, the concatenation
    of those heads' outputs; lse [H/N][S])."""
    hs = head_range(as_f64(q_scaled).shape[0], n_ranks, rank)
    o, lse = partial_attention(as_f64(q_scaled)[hs], as_f64(k)[hs], as_f64(v)[hs])
    return merge_heads(o), lse


def ulysses_return_o(o_shares, n_ranks: int, rank: int) -> np.ndarray:
    """Second all-to-all: rank `rank` receives, from every rank r, r's share
    o_shares[r] [S][h/N] restricted to its own rows: [N][S/N][h/N]."""
    s = np.asarray(o_shares[0]).shape[0]
    rows = row_range(s, n_ranks, rank)
    return np.stack([np.asarray(o_shares[r])[rows] for r in range(n_ranks)])


def ulysses_unpack_o(recv) -> np.ndarray:
    """[N][S/N][h/N] -> [S/N][h]: block r holds the columns of r's heads."""
    recv = np.asarray(recv)
    return np.concatenate([recv[r] for r in range(recv.shape[0])], axis=1)


def tp_share(x, wq, wk, wv, wo, num_heads: int, n_ranks: int, rank: int, rows=None) -> np.ndarray:
    """Rank `rank`'s tensor-parallel partial output Y_r = O_r W_O[rows of its
    heads] (before the all-reduce), where O_r is the attention of its heads and
    their Q/K/V come from the matching column shards of W_Q, W_K, W_V.
    x [S][h] (replicated); rows selects query rows (K/V always over all rows).
    sum_r Y_r = Y of the unsharded block."""
    x = as_f64(x)
    s, h = x.shape
    d = h // num_heads
    hl = num_heads // n_ranks
    cols = slice(rank * hl * d, (rank + 1) * hl * d)
    if rows is None:
        rows = np.arange(s)
    rows = np.asarray(rows, dtype=np.int64)
    k = split_heads(project(x, as_f64(wk)[:, cols]), hl)
    v = split_heads(project(x, as_f64(wv)[:, cols]), hl)
    q = split_heads(scale_query(project(x[rows], as_f64(wq)[:, cols]), d), hl)
    o, _ = partial_attention(q, k, v)
    return project(merge_heads(o), as_f64(wo)[cols, :])
