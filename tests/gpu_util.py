"""Helpers for the GPU parity tests: moving seeded numpy inputs to the device,
reading results back, and the comparison metrics the gates are stated in."""

from __future__ import annotations

import sys

import numpy as np
import torch

from long_context_self_amd import binding as B

# Gates for fp16 results against the fp64 oracle, and for a split-and-merge
# result against the unsplit result on the GPU.
REL_L2_F16 = 5e-3
MAX_ABS_F16 = 2e-2
REL_L2_SPLIT = 1e-3
# fp32 path: fp32 arithmetic throughout; relative error of a length-K fp32
# dot product is O(sqrt(K) * 2^-24) ~ 1e-6 at K = 256, so 1e-5 leaves margin.
REL_L2_F32 = 1e-5


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().to(torch.float64).cpu().numpy()


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def max_abs(got, ref) -> float:
    return float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))))


def assert_close(got, ref, rel=REL_L2_F16, mabs=MAX_ABS_F16, what=""):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    r, m = rel_l2(got, ref), max_abs(got, ref)
    say(f"  {what}: rel_l2={r:.3e} max_abs={m:.3e}")
    assert r <= rel, f"{what}: rel-L2 {r:.3e} > {rel:.1e}"
    assert m <= mabs, f"{what}: max-abs {m:.3e} > {mabs:.1e}"


def to_vt(v: np.ndarray) -> np.ndarray:
    """[H, S, d] -> [H, d, vt_ld(S)] with zero padding (the V^T layout)."""
    hh, s, d = v.shape
    out = np.zeros((hh, d, B.vt_ld(s)), dtype=v.dtype)
    out[:, :, :s] = v.transpose(0, 2, 1)
    return out


def partial(q, k, vt, sq, skv, ld, dtype=torch.float16):
    """attn_partial_forward_vt on contiguous [H,sq,d] q, [H,skv,d] k and
    [H,d,ld] v_t device tensors -> (o [H,sq,d] fp32, lse [H,sq] fp32)."""
    hh, _, d = q.shape
    o = torch.empty((hh, sq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((hh, sq), dtype=torch.float32, device="cuda")
    B.attn_partial_forward_vt(hh, d, q, sq, q.stride(0), k, skv, k.stride(0), vt, vt.stride(0), ld, o, lse,
                           dtype=dtype)
    return o, lse


def partial_rows(q, k, v, sq, skv, dtype=torch.float16, stream=None):
    """attn_partial_forward (V row-major) on [H,sq,d] q and [H,*,d] k, v device
    tensors sharing one head stride -> (o [H,sq,d] fp32, lse [H,sq] fp32)."""
    hh, _, d = q.shape
    assert k.stride() == v.stride()
    o = torch.empty((hh, sq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((hh, sq), dtype=torch.float32, device="cuda")
    B.attn_partial_forward(hh, d, q, sq, q.stride(0), k, v, skv, k.stride(0), o, lse, dtype=dtype, stream=stream)
    return o, lse
