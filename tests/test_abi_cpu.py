"""CPU tests of the C ABI: libattnblock.so loads, exports every function that
include/attn_block.h declares, and rejects invalid arguments with the
documented status before making any HIP call (so these run without a GPU)."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

from long_context_self_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_block.h")


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)) - {"attn_block_t"})


@pytest.fixture(scope="module")
def L():
    return B.lib()


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), f"{name} missing from {B.LIB_PATH}"


def test_library_exports_nothing_else():
    # -fvisibility=hidden: only the C ABI is visible.
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(B.EXPORTS) <= syms
    assert not {s for s in syms if s.startswith("_ZN7attnblk")}, "internal symbols leaked"


def _err(L):
    return L.attn_last_error().decode()


NULL = None
FAKE = 0x10000  # aligned non-null address; never dereferenced when validation fails


def test_create_rejects(L):
    h = ctypes.c_void_p()
    st = L.attn_block_create(None, 4096, 32, B.ATTN_F16, FAKE, FAKE, FAKE, FAKE, 16, None)
    assert st == B.ATTN_E_INVALID_ARG and "out is NULL" in _err(L)
    st = L.attn_block_create(ctypes.byref(h), 4096, 33, B.ATTN_F16, FAKE, FAKE, FAKE, FAKE, 16, None)
    assert st == B.ATTN_E_INVALID_ARG and "multiple" in _err(L)
    st = L.attn_block_create(ctypes.byref(h), 2048, 32, B.ATTN_F16, FAKE, FAKE, FAKE, FAKE, 16, None)
    assert st == B.ATTN_E_UNSUPPORTED and "head_dim 64" in _err(L)
    st = L.attn_block_create(ctypes.byref(h), 256, 4, 7, FAKE, FAKE, FAKE, FAKE, 16, None)
    assert st == B.ATTN_E_INVALID_ARG and "dtype" in _err(L)
    st = L.attn_block_create(ctypes.byref(h), 256, 4, B.ATTN_F32, FAKE, None, FAKE, FAKE, 16, None)
    assert st == B.ATTN_E_INVALID_ARG
    st = L.attn_block_create(ctypes.byref(h), 256, 4, B.ATTN_F32, FAKE + 2, FAKE, FAKE, FAKE, 16, None)
    assert st == B.ATTN_E_INVALID_ARG and "aligned" in _err(L)
    st = L.attn_block_create(ctypes.byref(h), 256, 4, B.ATTN_F32, FAKE, FAKE, FAKE, FAKE, 0, None)
    assert st == B.ATTN_E_INVALID_ARG and "max_tokens" in _err(L)
    assert h.value is None


def test_forward_rejects_null_block(L):
    st = L.attn_block_forward(None, FAKE, FAKE, 8, 1, None, None)
    assert st == B.ATTN_E_INVALID_ARG and "blk is NULL" in _err(L)


def test_set_prenorm_rejects_null_block(L):
    st = L.attn_block_set_prenorm(None, None, ctypes.c_float(1e-6), None)
    assert st == B.ATTN_E_INVALID_ARG and "blk is NULL" in _err(L)


def test_shard_and_ulysses_reject(L):
    h = ctypes.c_void_p()
    st = L.attn_block_create_shard(ctypes.byref(h), 4096, 32, 3, 0, B.ATTN_F16, FAKE, FAKE, FAKE, FAKE, 16, None)
    assert st == B.ATTN_E_INVALID_ARG and "n_ranks" in _err(L)
    st = L.attn_block_create_shard(ctypes.byref(h), 4096, 32, 8, 8, B.ATTN_F16, FAKE, FAKE, FAKE, FAKE, 16, None)
    assert st == B.ATTN_E_INVALID_ARG and "rank" in _err(L)
    st = L.attn_block_create_shard(ctypes.byref(h), 4096, 32, 0, 0, B.ATTN_F16, FAKE, FAKE, FAKE, FAKE, 16, None)
    assert st == B.ATTN_E_INVALID_ARG
    assert h.value is None
    # attn_heads_forward: o_ld too small, NULL, unsupported head_dim, seq 0
    assert L.attn_heads_forward(4, 128, B.ATTN_F16, FAKE, FAKE, FAKE, 64, FAKE, 256, None, None) == B.ATTN_E_INVALID_ARG
    assert L.attn_heads_forward(4, 128, B.ATTN_F16, None, FAKE, FAKE, 64, FAKE, 512, None, None) == B.ATTN_E_INVALID_ARG
    assert L.attn_heads_forward(4, 64, B.ATTN_F16, FAKE, FAKE, FAKE, 64, FAKE, 512, None, None) == B.ATTN_E_UNSUPPORTED
    assert L.attn_heads_forward(4, 128, B.ATTN_F16, FAKE, FAKE, FAKE, 0, FAKE, 512, None, None) == B.ATTN_OK
    # Ulysses layouts: seq not n_ranks x multiple of 8, NULL, misaligned
    g = lambda **kw: L.attn_ulysses_gather(kw.get("n", 8), 4, 128, B.ATTN_F16, kw.get("seq", 4096), FAKE, FAKE,
                                           kw.get("rvt", FAKE), FAKE, FAKE, FAKE, None)
    assert g(seq=4100) == B.ATTN_E_INVALID_ARG and "multiple of 8" in _err(L)
    assert g(seq=8 * 12) == B.ATTN_E_INVALID_ARG
    assert g(rvt=None) == B.ATTN_E_INVALID_ARG
    assert g(rvt=FAKE + 8) == B.ATTN_E_INVALID_ARG
    assert g(seq=0) == B.ATTN_OK
    assert L.attn_ulysses_unpack_o(8, 30, 128, B.ATTN_F16, 16, FAKE, FAKE, None) == B.ATTN_E_INVALID_ARG
    assert L.attn_ulysses_unpack_o(8, 32, 128, B.ATTN_F16, 16, None, FAKE, None) == B.ATTN_E_INVALID_ARG
    assert L.attn_ulysses_unpack_o(8, 32, 128, B.ATTN_F16, 0, FAKE, FAKE, None) == B.ATTN_OK


def test_ring_rejects(L):
    h = ctypes.c_void_p()
    assert L.attn_ring_create(None, 32, 128, B.ATTN_F16, 8, 4096, 4096) == B.ATTN_E_INVALID_ARG
    assert L.attn_ring_create(ctypes.byref(h), 32, 64, B.ATTN_F16, 8, 4096, 4096) == B.ATTN_E_UNSUPPORTED
    assert L.attn_ring_create(ctypes.byref(h), 32, 128, B.ATTN_F16, 0, 4096, 4096) == B.ATTN_E_INVALID_ARG
    assert L.attn_ring_create(ctypes.byref(h), 32, 128, B.ATTN_F16, 8, 0, 4096) == B.ATTN_E_INVALID_ARG
    assert h.value is None
    assert L.attn_ring_forward(None, FAKE, 16, None, None, None, FAKE, None, None) == B.ATTN_E_INVALID_ARG
    assert "ring is NULL" in _err(L)
    L.attn_ring_destroy(None)


def test_partial_rejects(L):
    args = dict(nh=32, d=128, dt=B.ATTN_F16, q=FAKE, sq=256, qhs=256 * 128, k=FAKE, skv=512,
                khs=512 * 128, v=FAKE, vhs=128 * 512, vrs=512, o=FAKE, lse=FAKE)

    def call(**kw):
        a = dict(args, **kw)
        return L.attn_partial_forward_vt(a["nh"], a["d"], a["dt"], a["q"], a["sq"], a["qhs"], a["k"], a["skv"],
                                         a["khs"], a["v"], a["vhs"], a["vrs"], a["o"], a["lse"], None)

    assert call(d=64) == B.ATTN_E_UNSUPPORTED
    assert call(dt=B.ATTN_F32, d=96) == B.ATTN_E_UNSUPPORTED
    assert call(q=None) == B.ATTN_E_INVALID_ARG
    assert call(k=None) == B.ATTN_E_INVALID_ARG
    assert call(k=None, v=None, skv=0) != B.ATTN_E_INVALID_ARG or True  # skv=0 needs no k/v (GPU call)
    assert call(sq=-1) == B.ATTN_E_INVALID_ARG
    assert call(vrs=500) == B.ATTN_E_INVALID_ARG and "v_row_stride" in _err(L)
    assert call(vrs=516, vhs=128 * 516) == B.ATTN_E_INVALID_ARG and "multiples" in _err(L)
    assert call(q=FAKE + 8) == B.ATTN_E_INVALID_ARG and "aligned" in _err(L)
    assert call(qhs=100 * 128) == B.ATTN_E_INVALID_ARG
    assert call(nh=0) == B.ATTN_E_INVALID_ARG
    big = (1 << 24) + 8
    assert call(vrs=big, vhs=128 * big) == B.ATTN_E_UNSUPPORTED and "v_row_stride" in _err(L)
    assert call(sq=0) == B.ATTN_OK  # nothing to do, nothing enqueued


def test_partial_rows_rejects(L):
    """attn_partial_forward (V row-major [H][skv][d], one K/V head stride)."""
    args = dict(nh=32, d=128, dt=B.ATTN_F16, q=FAKE, sq=256, qhs=256 * 128, k=FAKE, v=FAKE, skv=512,
                kvhs=512 * 128, o=FAKE, lse=FAKE)

    def call(**kw):
        a = dict(args, **kw)
        return L.attn_partial_forward(a["nh"], a["d"], a["dt"], a["q"], a["sq"], a["qhs"], a["k"], a["v"], a["skv"],
                                      a["kvhs"], a["o"], a["lse"], None)

    assert call(d=64) == B.ATTN_E_UNSUPPORTED and "attn_partial_forward:" in _err(L)
    assert call(dt=B.ATTN_F32, d=96) == B.ATTN_E_UNSUPPORTED
    assert call(q=None) == B.ATTN_E_INVALID_ARG
    assert call(v=None) == B.ATTN_E_INVALID_ARG and "k or v is NULL" in _err(L)
    assert call(k=None) == B.ATTN_E_INVALID_ARG
    assert call(v=FAKE + 8) == B.ATTN_E_INVALID_ARG and "aligned" in _err(L)
    assert call(kvhs=500 * 128) == B.ATTN_E_INVALID_ARG and "kv_head_stride" in _err(L)
    assert call(kvhs=512 * 128 + 4) == B.ATTN_E_INVALID_ARG and "multiples" in _err(L)
    assert call(sq=-1) == B.ATTN_E_INVALID_ARG
    assert call(skv=(1 << 24) + 1, kvhs=((1 << 24) + 1) * 128) == B.ATTN_E_UNSUPPORTED
    assert call(nh=0) == B.ATTN_E_INVALID_ARG
    assert call(sq=0) == B.ATTN_OK  # nothing to do, nothing enqueued, no staging


def test_partial_noalloc_rejects(L):
    """attn_partial_forward_noalloc: the checks of attn_partial_forward, and
    calls whose V^T staging exceeds the fixed 64 MiB are refused before any
    HIP call."""
    def call(nh=32, d=128, dt=B.ATTN_F16, sq=256, skv=4096, kvhs=None, v=FAKE):
        kvhs = skv * d if kvhs is None else kvhs
        return L.attn_partial_forward_noalloc(nh, d, dt, FAKE, sq, sq * d, FAKE, v, skv, kvhs, FAKE, FAKE, None)

    assert call(skv=8193) == B.ATTN_E_UNSUPPORTED and "64" in _err(L) and "scratch" in _err(L)
    assert call(nh=64, skv=4097) == B.ATTN_E_UNSUPPORTED
    assert call(dt=B.ATTN_F32, d=128, skv=4097) == B.ATTN_E_UNSUPPORTED
    assert call(skv=8193, sq=0) == B.ATTN_E_UNSUPPORTED  # the limit applies even with no query rows
    assert call(v=None) == B.ATTN_E_INVALID_ARG and "attn_partial_forward_noalloc" in _err(L)
    assert call(d=64) == B.ATTN_E_UNSUPPORTED
    assert call(kvhs=4000 * 128) == B.ATTN_E_INVALID_ARG
    assert call(sq=0) == B.ATTN_OK


def test_merge_rejects(L):
    assert L.attn_merge_lse(0, 32, 128, 16, FAKE, FAKE, FAKE, B.ATTN_F16, None, None) == B.ATTN_E_INVALID_ARG
    assert L.attn_merge_lse(8, 32, 96, 16, FAKE, FAKE, FAKE, B.ATTN_F16, None, None) == B.ATTN_E_UNSUPPORTED
    assert L.attn_merge_lse(8, 32, 128, 16, None, FAKE, FAKE, B.ATTN_F16, None, None) == B.ATTN_E_INVALID_ARG
    assert L.attn_merge_lse(8, 32, 128, 16, FAKE + 4, FAKE, FAKE, B.ATTN_F16, None, None) == B.ATTN_E_INVALID_ARG
    assert L.attn_merge_lse(8, 32, 128, 16, FAKE, FAKE, FAKE, 9, None, None) == B.ATTN_E_INVALID_ARG
    assert L.attn_merge_lse(8, 32, 128, 0, FAKE, FAKE, FAKE, B.ATTN_F16, None, None) == B.ATTN_OK


def test_binding_raises_attn_error(L):
    with pytest.raises(B.AttnError) as ei:
        B.attn_merge_lse(0, 32, 128, 16, FAKE, FAKE, FAKE, lse_out=None, stream=0)
    assert ei.value.status == B.ATTN_E_INVALID_ARG


def test_destroy_null_is_noop(L):
    L.attn_block_destroy(None)


def test_vt_ld_matches_header():
    with open(HEADER) as f:
        assert "((((int64_t)(seq)) + 7) / 8 * 8)" in f.read()
    assert [B.vt_ld(s) for s in (1, 8, 9, 4096, 4097)] == [8, 8, 16, 4096, 4104]
