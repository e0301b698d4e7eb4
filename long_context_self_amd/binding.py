"""Thin Python binding of libattnblock.so (C ABI in include/attn_block.h).

Argument marshalling only: every step runs in the library's HIP kernels.
torch supplies device memory and the stream (``torch.cuda.current_stream()``
unless one is passed). The functions keep the C names:

* ``attn_block_create`` / ``attn_block_set_prenorm`` / ``attn_block_forward`` /
  ``attn_block_destroy`` (wrapped by the ``AttnBlock`` class),
* ``attn_block_create_shard`` (tensor-parallel share, ``AttnBlock(..., n_ranks=, rank=)``),
* ``attn_partial_forward`` (V row-major), ``attn_partial_forward_vt`` (V^T),
  ``attn_partial_forward_noalloc`` (V row-major, fixed staging, no allocation),
  ``attn_merge_lse``, ``attn_heads_forward``,
* ``attn_ulysses_gather``, ``attn_ulysses_unpack_o``,
* ``attn_ring_create`` / ``attn_ring_forward`` / ``attn_ring_destroy`` (the ``AttnRing`` class).

There is no fallback: if the library is missing or fails to load, ``lib()``
raises, and every call raises ``AttnError`` on a non-OK status.
"""

from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattnblock.so")

ATTN_OK, ATTN_E_INVALID_ARG, ATTN_E_UNSUPPORTED, ATTN_E_OOM, ATTN_E_HIP = range(5)
ATTN_F16, ATTN_F32 = 0, 1
STATUS_NAMES = {0: "ATTN_OK", 1: "ATTN_E_INVALID_ARG", 2: "ATTN_E_UNSUPPORTED", 3: "ATTN_E_OOM",
                4: "ATTN_E_HIP"}

EXPORTS = ("attn_block_create", "attn_block_create_shard", "attn_block_set_prenorm", "attn_block_forward",
           "attn_partial_forward", "attn_partial_forward_vt", "attn_partial_forward_noalloc", "attn_merge_lse", "attn_heads_forward", "attn_ulysses_gather",
           "attn_ulysses_unpack_o", "attn_ring_create", "attn_ring_forward", "attn_ring_destroy",
           "attn_block_destroy", "attn_last_error")


def vt_ld(seq: int) -> int:
    """Row stride of a head-major V^T tensor for ``seq`` keys (ATTN_VT_LD)."""
    return (seq + 7) // 8 * 8


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class Taps(ctypes.Structure):
    _fields_ = [("q_scaled", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v_t", ctypes.c_void_p),
                ("attn_out", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("qkv_only", ctypes.c_int),
                ("events", ctypes.c_void_p), ("v", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libattnblock.so (once). Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m long_context_self_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    L.attn_block_create.argtypes = [ctypes.POINTER(vp), i32, i32, i32, vp, vp, vp, vp, i64, vp]
    L.attn_block_create.restype = i32
    L.attn_block_create_shard.argtypes = [ctypes.POINTER(vp), i32, i32, i32, i32, i32, vp, vp, vp, vp, i64, vp]
    L.attn_block_create_shard.restype = i32
    L.attn_heads_forward.argtypes = [i32, i32, i32, vp, vp, vp, i64, vp, i64, vp, vp]
    L.attn_heads_forward.restype = i32
    L.attn_ulysses_gather.argtypes = [i32, i32, i32, i32, i64, vp, vp, vp, vp, vp, vp, vp]
    L.attn_ulysses_gather.restype = i32
    L.attn_ulysses_unpack_o.argtypes = [i32, i32, i32, i32, i64, vp, vp, vp]
    L.attn_ulysses_unpack_o.restype = i32
    L.attn_ring_create.argtypes = [ctypes.POINTER(vp), i32, i32, i32, i32, i64, i64]
    L.attn_ring_create.restype = i32
    L.attn_ring_forward.argtypes = [vp, vp, i64, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(i64), vp, vp,
                                    vp]
    L.attn_ring_forward.restype = i32
    L.attn_ring_destroy.argtypes = [vp]
    L.attn_ring_destroy.restype = None
    L.attn_block_set_prenorm.argtypes = [vp, vp, ctypes.c_float, vp]
    L.attn_block_set_prenorm.restype = i32
    L.attn_block_forward.argtypes = [vp, vp, vp, i64, i64, ctypes.POINTER(Taps), vp]
    L.attn_block_forward.restype = i32
    L.attn_partial_forward.argtypes = [i32, i32, i32, vp, i64, i64, vp, vp, i64, i64, vp, vp, vp]
    L.attn_partial_forward.restype = i32
    L.attn_partial_forward_noalloc.argtypes = [i32, i32, i32, vp, i64, i64, vp, vp, i64, i64, vp, vp, vp]
    L.attn_partial_forward_noalloc.restype = i32
    L.attn_partial_forward_vt.argtypes = [i32, i32, i32, vp, i64, i64, vp, i64, i64, vp, i64, i64, vp, vp, vp]
    L.attn_partial_forward_vt.restype = i32
    L.attn_merge_lse.argtypes = [i32, i32, i32, i64, vp, vp, vp, i32, vp, vp]
    L.attn_merge_lse.restype = i32
    L.attn_block_destroy.argtypes = [vp]
    L.attn_block_destroy.restype = None
    L.attn_last_error.argtypes = []
    L.attn_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int) -> None:
    if status != ATTN_OK:
        raise AttnError(status, lib().attn_last_error().decode(errors="replace"))


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float16:
        return ATTN_F16
    if dt == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {dt}")


def attn_block_create(hidden: int, num_heads: int, wq, wk, wv, wo, max_tokens: int, stream=None) -> int:
    handle = ctypes.c_void_p()
    _check(lib().attn_block_create(ctypes.byref(handle), hidden, num_heads, _dtype_code(wq.dtype),
                                   _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wo), max_tokens, _stream(stream)))
    return handle.value


def attn_block_create_shard(hidden: int, num_heads: int, n_ranks: int, rank: int, wq, wk, wv, wo,
                            max_tokens: int, stream=None) -> int:
    handle = ctypes.c_void_p()
    _check(lib().attn_block_create_shard(ctypes.byref(handle), hidden, num_heads, n_ranks, rank,
                                         _dtype_code(wq.dtype), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wo), max_tokens,
                                         _stream(stream)))
    return handle.value


def attn_heads_forward(num_heads: int, head_dim: int, q_scaled, k, v_t, seq: int, o, o_ld: int, lse=None,
                       dtype: torch.dtype = torch.float16, stream=None) -> None:
    _check(lib().attn_heads_forward(num_heads, head_dim, _dtype_code(dtype), _ptr(q_scaled), _ptr(k), _ptr(v_t), seq,
                                    _ptr(o), o_ld, _ptr(lse), _stream(stream)))


def attn_ulysses_gather(n_ranks: int, num_heads_local: int, head_dim: int, seq: int, recv_q, recv_k, recv_vt,
                        q_scaled, k, v_t, dtype: torch.dtype = torch.float16, stream=None) -> None:
    _check(lib().attn_ulysses_gather(n_ranks, num_heads_local, head_dim, _dtype_code(dtype), seq, _ptr(recv_q),
                                     _ptr(recv_k), _ptr(recv_vt), _ptr(q_scaled), _ptr(k), _ptr(v_t),
                                     _stream(stream)))


def attn_ulysses_unpack_o(n_ranks: int, num_heads: int, head_dim: int, rows: int, recv_o, o,
                          dtype: torch.dtype = torch.float16, stream=None) -> None:
    _check(lib().attn_ulysses_unpack_o(n_ranks, num_heads, head_dim, _dtype_code(dtype), rows, _ptr(recv_o), _ptr(o),
                                       _stream(stream)))


def attn_block_set_prenorm(handle: int, gain=None, eps: float = 1e-6, stream=None) -> None:
    _check(lib().attn_block_set_prenorm(handle, _ptr(gain), eps, _stream(stream)))


def attn_block_forward(handle: int, x, y, seq: int, batch: int = 1, taps: Taps | None = None,
                       stream=None) -> None:
    _check(lib().attn_block_forward(handle, _ptr(x), _ptr(y), seq, batch,
                                    ctypes.byref(taps) if taps is not None else None, _stream(stream)))


def attn_block_destroy(handle: int) -> None:
    if handle:
        lib().attn_block_destroy(handle)


def attn_partial_forward(num_heads: int, head_dim: int, q_scaled, sq: int, q_head_stride: int,
                         k, v, skv: int, kv_head_stride: int, o_part, lse_part,
                         dtype: torch.dtype = torch.float16, stream=None) -> None:
    _check(lib().attn_partial_forward(num_heads, head_dim, _dtype_code(dtype), _ptr(q_scaled), sq,
                                      q_head_stride, _ptr(k), _ptr(v), skv, kv_head_stride, _ptr(o_part),
                                      _ptr(lse_part), _stream(stream)))


def attn_partial_forward_noalloc(num_heads: int, head_dim: int, q_scaled, sq: int, q_head_stride: int,
                                 k, v, skv: int, kv_head_stride: int, o_part, lse_part,
                                 dtype: torch.dtype = torch.float16, stream=None) -> None:
    _check(lib().attn_partial_forward_noalloc(num_heads, head_dim, _dtype_code(dtype), _ptr(q_scaled), sq,
                                              q_head_stride, _ptr(k), _ptr(v), skv, kv_head_stride, _ptr(o_part),
                                              _ptr(lse_part), _stream(stream)))


def attn_partial_forward_vt(num_heads: int, head_dim: int, q_scaled, sq: int, q_head_stride: int,
                            k, skv: int, k_head_stride: int, v_t, v_head_stride: int, v_row_stride: int,
                            o_part, lse_part, dtype: torch.dtype = torch.float16, stream=None) -> None:
    _check(lib().attn_partial_forward_vt(num_heads, head_dim, _dtype_code(dtype), _ptr(q_scaled), sq,
                                         q_head_stride, _ptr(k), skv, k_head_stride, _ptr(v_t), v_head_stride,
                                         v_row_stride, _ptr(o_part), _ptr(lse_part), _stream(stream)))


def attn_merge_lse(n_parts: int, num_heads: int, head_dim: int, sq: int, o_parts, lse_parts, o_out,
                   out_dtype: torch.dtype = torch.float16, lse_out=None, stream=None) -> None:
    _check(lib().attn_merge_lse(n_parts, num_heads, head_dim, sq, _ptr(o_parts), _ptr(lse_parts),
                                _ptr(o_out), _dtype_code(out_dtype), _ptr(lse_out), _stream(stream)))


class AttnRing:
    """Ring-style K/V streaming (attn_ring_*): blocks copied on the ring's copy
    stream while earlier blocks' attention runs, merged by log-sum-exp."""

    def __init__(self, num_heads: int, head_dim: int, n_blocks: int, max_sq: int, max_block_len: int,
                 dtype: torch.dtype = torch.float16):
        self.n_blocks = n_blocks
        self.dtype = dtype
        handle = ctypes.c_void_p()
        _check(lib().attn_ring_create(ctypes.byref(handle), num_heads, head_dim, _dtype_code(dtype), n_blocks,
                                      max_sq, max_block_len))
        self.handle = handle.value

    def forward(self, q_scaled, sq: int, k_blocks, vt_blocks, block_lens, o_out, lse_out=None, stream=None) -> None:
        n = self.n_blocks
        kb = (ctypes.c_void_p * n)(*[_ptr(t) for t in k_blocks])
        vb = (ctypes.c_void_p * n)(*[_ptr(t) for t in vt_blocks])
        lens = (ctypes.c_int64 * n)(*block_lens)
        _check(lib().attn_ring_forward(self.handle, _ptr(q_scaled), sq, kb, vb, lens, _ptr(o_out), _ptr(lse_out),
                                       _stream(stream)))

    def close(self) -> None:
        if getattr(self, "handle", None):
            lib().attn_ring_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class AttnBlock:
    """One self-attention block: packed weights + workspace in the library."""

    def __init__(self, wq, wk, wv, wo, num_heads: int, max_tokens: int, stream=None, n_ranks: int = 1,
                 rank: int = 0):
        """With n_ranks > 1 the block is rank `rank`'s tensor-parallel share
        (attn_block_create_shard): its forward returns the partial output."""
        for w in (wq, wk, wv, wo):
            if not (w.is_cuda and w.is_contiguous() and w.dim() == 2 and w.shape[0] == w.shape[1]):
                raise ValueError("weights must be contiguous square device tensors [h, h]")
        self.hidden = wq.shape[0]
        self.num_heads = num_heads
        self.head_dim = self.hidden // num_heads
        self.dtype = wq.dtype
        self.max_tokens = max_tokens
        self.n_ranks, self.rank = n_ranks, rank
        if n_ranks == 1 and rank == 0:
            self.handle = attn_block_create(self.hidden, num_heads, wq, wk, wv, wo, max_tokens, stream)
        else:
            self.handle = attn_block_create_shard(self.hidden, num_heads, n_ranks, rank, wq, wk, wv, wo, max_tokens,
                                                  stream)

    def set_prenorm(self, gain=None, eps: float = 1e-6, stream=None) -> None:
        """Enable RMSNorm of the input rows (pre-norm) for later forwards."""
        if gain is not None and not (gain.is_cuda and gain.is_contiguous() and gain.dtype == self.dtype
                                     and gain.numel() == self.hidden):
            raise ValueError("gain must be a contiguous device tensor [h] of the block's dtype")
        attn_block_set_prenorm(self.handle, gain, eps, stream)

    def forward(self, x, y=None, taps: Taps | None = None, stream=None):
        """x: [seq, 1, h] or [seq, h] device tensor; returns y of the same shape."""
        if not (x.is_cuda and x.is_contiguous()):
            raise ValueError("x must be a contiguous device tensor")
        seq = x.shape[0]
        batch = x.shape[1] if x.dim() == 3 else 1
        if y is None and not (taps is not None and taps.qkv_only):
            y = torch.empty_like(x)
        attn_block_forward(self.handle, x, y, seq, batch, taps, stream)
        return y

    __call__ = forward

    def close(self) -> None:
        if getattr(self, "handle", None):
            attn_block_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
