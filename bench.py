#!/usr/bin/env python3
"""Benchmark of the MI355X self-attention block forward (one GPU).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick] [--seq S] [--no-cpu]

A step is one forward of the block -- QKV projection (with the head split and
the q_scaled pre-scale fused into its epilogue), attention over the full
sequence, output projection -- on the headline workload: seq 65536, batch 1,
hidden 4096, 32 heads of 128, fp16, non-causal, seeded synthetic inputs
already resident in HBM (the largest single-block configuration, where
attention is 89% of the block's FLOPs). W untimed steps, then K timed steps
bracketed by torch.cuda.synchronize(); HIP events recorded by the library
between its kernels (the ``events`` tap) give per-kernel durations inside the
timed region, on the stream the kernels run on.

The same run also times, with the same K and W, the other workloads: seq 8192 /
16384 / 32768 at hidden 4096, seq 8192 at hidden 8192 (64 heads), the block with
RMSNorm pre-norm, the context-parallel rank share (a 4096-row query chunk of
seq 32768 against K/V in 8 blocks of 4096, per-block partials alternating over
two streams, then the LSE merge; with V row-major as attn_partial_forward takes
it, and with V^T), the Ulysses and tensor-parallel one-GPU shares, Ring-style
streaming, and 6 stacked blocks at seq 32768.

The CPU baseline is the fp64 oracle in a child process that never touches the
GPU, run before the GPU work: K and V over all rows and a seeded sample of
query rows, heads spread over a process pool, at the headline workload (and at
the other single-block sizes, reported beside it).

Prints one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

PEAK_F16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12  # 2516.6: MI355X dense fp16 MFMA (published 2.5 PFLOP/s)
PEAK_HBM_GBS = 8000.0                         # MI355X HBM3E, 8 TB/s

METRIC = "ms/forward + attention TFLOP/s (frac of fp16 MFMA peak), 1 MI355X"

# Latencies the pages report for TensorRT on one B200 (context, not a target).
B200_CONTEXT = {
    "hardware": "1x NVIDIA B200, TensorRT 11.0 via Triton, batch 1, end-to-end request latency (+-10%)",
    "seq16384_h4096_ms": "480-724", "seq32768_h4096_ms": "1160", "seq65536_h4096_ms": "2224",
    "seq8192_h8192_ms": "593-728", "six_stack_seq32768_ms": "1187-1388",
}


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


class Hip:
    """HIP events through the runtime torch already loaded (one runtime per process)."""

    def __init__(self):
        self.L = ctypes.CDLL("libamdhip64.so.7")
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def events(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            if self.L.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            arr[i] = ev.value
        return arr

    def record(self, ev, stream):
        if self.L.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b) -> float:
        out = ctypes.c_float()
        if self.L.hipEventElapsedTime(ctypes.byref(out), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def destroy(self, arr):
        for e in arr:
            self.L.hipEventDestroy(e)


def block_flops(seq, h):
    return {"qkv": 6.0 * seq * h * h, "attn": 4.0 * seq * seq * h, "oproj": 2.0 * seq * h * h}


def stats(xs):
    xs = np.asarray(xs, dtype=np.float64)
    return {"median": float(np.median(xs)), "min": float(xs.min()), "p90": float(np.percentile(xs, 90)),
            "mean": float(xs.mean())}


def run_block(torch, B, hip, seq, h, nh, layers, warmup, steps, seed=0, prenorm=False):
    """Time `steps` forwards of a stack of `layers` blocks; per-kernel times from the events tap.
    With `prenorm`, every block applies RMSNorm (unit gain, eps 1e-6) to its input; the row-norm
    kernel then falls inside the "qkv" interval."""
    from long_context_self_amd.synthetic import block_inputs

    x, ws = block_inputs(seq, h, layers, dtype=np.float16, seed=seed)
    blocks = [B.AttnBlock(*(torch.from_numpy(w).cuda() for w in lw), num_heads=nh, max_tokens=seq) for lw in ws]
    if prenorm:
        for blk in blocks:
            blk.set_prenorm(None, 1e-6)
    del ws
    xd = torch.from_numpy(x).cuda()
    del x
    bufs = [torch.empty_like(xd), torch.empty_like(xd)]
    stream = torch.cuda.current_stream().cuda_stream
    evs = hip.events(4 * layers * steps)
    tot = hip.events(2)

    def one(step_events):
        cur = xd
        for li, blk in enumerate(blocks):
            taps = None
            if step_events is not None:
                base = ctypes.addressof(evs) + (step_events + 4 * li) * ctypes.sizeof(ctypes.c_void_p)
                taps = B.Taps(None, None, None, None, None, 0, base)
            out = bufs[li % 2]
            blk.forward(cur, out, taps=taps)
            cur = out
        return cur

    for _ in range(warmup):
        one(None)
    torch.cuda.synchronize()
    hip.record(tot[0], stream)
    for s in range(steps):
        one(4 * layers * s)
    hip.record(tot[1], stream)
    torch.cuda.synchronize()
    total_ms = hip.ms(tot[0], tot[1])
    k = {"qkv": [], "attn": [], "oproj": [], "step": []}
    for s in range(steps):
        e = [evs[4 * layers * s + i] for i in range(4 * layers)]
        k["step"].append(hip.ms(e[0], e[4 * layers - 1]))
        for li in range(layers):
            b = 4 * li
            k["qkv"].append(hip.ms(e[b], e[b + 1]))
            k["attn"].append(hip.ms(e[b + 1], e[b + 2]))
            k["oproj"].append(hip.ms(e[b + 2], e[b + 3]))
    hip.destroy(evs)
    hip.destroy(tot)
    for blk in blocks:
        blk.close()
    del bufs, xd
    torch.cuda.empty_cache()
    return total_ms / steps, {n: stats(v) for n, v in k.items()}


def run_rank_share(torch, B, hip, warmup, steps, seq=32768, h=4096, nh=32, ranks=8, seed=0):
    """Rank 0's share: its seq/8 query chunk against K/V streamed in 8 blocks
    (partial + LSE per block, then one merge), inputs from the block's QKV taps.
    Timed with V row-major [H][keys][d] as attn_partial_forward takes it (its
    V^T staging transpose included), and with V^T (attn_partial_forward_vt)."""
    from long_context_self_amd.synthetic import block_inputs

    d = h // nh
    x, [ws] = block_inputs(seq, h, 1, dtype=np.float16, seed=seed)
    blk = B.AttnBlock(*(torch.from_numpy(w).cuda() for w in ws), num_heads=nh, max_tokens=seq)
    ld = B.vt_ld(seq)
    q = torch.empty((nh, seq, d), dtype=torch.float16, device="cuda")
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    vt = torch.zeros((nh, d, ld), dtype=torch.float16, device="cuda")
    blk.forward(torch.from_numpy(x).cuda(), taps=B.Taps(q.data_ptr(), k.data_ptr(), vt.data_ptr(), None, None, 1,
                                                           None, v.data_ptr()))
    torch.cuda.synchronize()
    blk.close()
    chunk = seq // ranks
    o_parts = torch.empty((ranks, nh, chunk, d), dtype=torch.float32, device="cuda")
    lse_parts = torch.empty((ranks, nh, chunk), dtype=torch.float32, device="cuda")
    o = torch.empty((chunk, h), dtype=torch.float16, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    evs = hip.events(3 * steps)

    def timed(partials):
        """Stats of `partials()` and of the merge that follows it."""
        def one(s):
            if s is not None:
                hip.record(evs[3 * s], stream)
            partials()
            if s is not None:
                hip.record(evs[3 * s + 1], stream)
            B.attn_merge_lse(ranks, nh, d, chunk, o_parts, lse_parts, o, torch.float16)
            if s is not None:
                hip.record(evs[3 * s + 2], stream)

        for _ in range(warmup):
            one(None)
        torch.cuda.synchronize()
        for s in range(steps):
            one(s)
        torch.cuda.synchronize()
        return (stats([hip.ms(evs[3 * s], evs[3 * s + 1]) for s in range(steps)]),
                stats([hip.ms(evs[3 * s + 1], evs[3 * s + 2]) for s in range(steps)]))

    # the 8 block partials, one call per block. They are independent (each
    # writes its own part), so they alternate over the caller's stream and a
    # second one; the tail of one launch then overlaps the start of the next.
    # The merge waits for both.
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()

    def per_block(rows_v):
        def run():
            fork = torch.cuda.Event()
            fork.record(main)
            side.wait_event(fork)
            for b in range(ranks):
                st = main if b % 2 == 0 else side
                if rows_v:
                    B.attn_partial_forward(nh, d, q, chunk, seq * d, k[:, b * chunk:], v[:, b * chunk:], chunk,
                                           seq * d, o_parts[b], lse_parts[b], stream=st.cuda_stream)
                else:
                    B.attn_partial_forward_vt(nh, d, q, chunk, seq * d, k[:, b * chunk:], chunk, seq * d,
                                              vt[:, :, b * chunk:], d * ld, ld, o_parts[b], lse_parts[b],
                                              stream=st.cuda_stream)
            join = torch.cuda.Event()
            join.record(side)
            main.wait_event(join)
        return run

    ps, ms_ = timed(per_block(True))
    ps_t, ms_t = timed(per_block(False))
    # comparison: the same chunk against all 32768 keys in one launch (no blocks, no merge)
    for s in range(warmup + steps):
        if s >= warmup:
            hip.record(evs[3 * (s - warmup)], stream)
        B.attn_partial_forward_vt(nh, d, q, chunk, seq * d, k, seq, seq * d, vt, d * ld, ld, o_parts[0],
                                  lse_parts[0])
        if s >= warmup:
            hip.record(evs[3 * (s - warmup) + 1], stream)
    torch.cuda.synchronize()
    one_shot = stats([hip.ms(evs[3 * s], evs[3 * s + 1]) for s in range(steps)])
    hip.destroy(evs)
    flops = 4.0 * chunk * seq * h
    merge_bytes = ranks * chunk * h * 4 + ranks * nh * chunk * 4 + chunk * h * 2
    transpose_bytes = 2 * seq * h * 2  # every block's V read once and written once as V^T
    del q, k, v, vt, o_parts, lse_parts, o
    torch.cuda.empty_cache()
    return {
        "workload": "rank share: 4096-row query chunk of seq 32768 vs K/V in 8 blocks of 4096, hidden 4096, 32 heads "
                    "(block partials alternating over two streams, V row-major [H][keys][d])",
        "ms": ps["median"] + ms_["median"], "partials_ms": ps, "merge_ms": ms_,
        "attention_tflops": flops / (ps["median"] * 1e-3) / 1e12,
        "attention_frac_of_peak": flops / (ps["median"] * 1e-3) / 1e12 / PEAK_F16_TFLOPS,
        "v_transpose_bytes": transpose_bytes,
        "ms_vt": ps_t["median"] + ms_t["median"], "partials_vt_ms": ps_t, "merge_vt_ms": ms_t,
        "attention_tflops_vt": flops / (ps_t["median"] * 1e-3) / 1e12,
        "merge_gbs": merge_bytes / (ms_["median"] * 1e-3) / 1e9,
        "merge_frac_of_hbm": merge_bytes / (ms_["median"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "merge_bytes": merge_bytes,
        "one_shot_ms": one_shot["median"], "one_shot": one_shot,
        "one_shot_attention_tflops": flops / (one_shot["median"] * 1e-3) / 1e12,
    }


def run_ulysses_share(torch, B, hip, warmup, steps, seq=32768, h=4096, nh=32, ranks=8, seed=0):
    """Rank 0's Ulysses share: receive-side layout of the first all-to-all (its 4 heads' blocks from all 8
    ranks -> full-sequence head-major), attention of those heads over all 32768 rows, receive-side layout of
    the second all-to-all (8 blocks of its rows -> concatenated heads). Q/K/V are the block's own projection
    (taps); the all-to-all blocks are slices of them, as the ranks' projections would send them."""
    from long_context_self_amd.synthetic import block_inputs

    d = h // nh
    hl, ch = nh // ranks, seq // ranks
    x, [ws] = block_inputs(seq, h, 1, dtype=np.float16, seed=seed)
    blk = B.AttnBlock(*(torch.from_numpy(w).cuda() for w in ws), num_heads=nh, max_tokens=seq)
    q = torch.empty((nh, seq, d), dtype=torch.float16, device="cuda")
    k = torch.empty_like(q)
    vt = torch.zeros((nh, d, B.vt_ld(seq)), dtype=torch.float16, device="cuda")
    blk.forward(torch.from_numpy(x).cuda(), taps=B.Taps(q.data_ptr(), k.data_ptr(), vt.data_ptr(), None, None, 1,
                                                           None))
    torch.cuda.synchronize()
    blk.close()
    # what rank 0 receives from rank p: rows of chunk p for heads 0..hl-1
    rq = torch.stack([q[:hl, p * ch:(p + 1) * ch] for p in range(ranks)]).contiguous()
    rk = torch.stack([k[:hl, p * ch:(p + 1) * ch] for p in range(ranks)]).contiguous()
    rvt = torch.stack([vt[:hl, :, p * ch:(p + 1) * ch] for p in range(ranks)]).contiguous()
    del q, k, vt
    gq = torch.empty((hl, seq, d), dtype=torch.float16, device="cuda")
    gk = torch.empty_like(gq)
    gvt = torch.empty((hl, d, B.vt_ld(seq)), dtype=torch.float16, device="cuda")
    o = torch.empty((seq, hl * d), dtype=torch.float16, device="cuda")
    recv_o = torch.randn((ranks, ch, hl * d), device="cuda").half()
    o_full = torch.empty((ch, h), dtype=torch.float16, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    evs = hip.events(4 * steps)

    def one(s):
        if s is not None:
            hip.record(evs[4 * s], stream)
        B.attn_ulysses_gather(ranks, hl, d, seq, rq, rk, rvt, gq, gk, gvt)
        if s is not None:
            hip.record(evs[4 * s + 1], stream)
        B.attn_heads_forward(hl, d, gq, gk, gvt, seq, o, hl * d)
        if s is not None:
            hip.record(evs[4 * s + 2], stream)
        B.attn_ulysses_unpack_o(ranks, nh, d, ch, recv_o, o_full)
        if s is not None:
            hip.record(evs[4 * s + 3], stream)

    for _ in range(warmup):
        one(None)
    torch.cuda.synchronize()
    for s in range(steps):
        one(s)
    torch.cuda.synchronize()
    g = stats([hip.ms(evs[4 * s], evs[4 * s + 1]) for s in range(steps)])
    a = stats([hip.ms(evs[4 * s + 1], evs[4 * s + 2]) for s in range(steps)])
    u = stats([hip.ms(evs[4 * s + 2], evs[4 * s + 3]) for s in range(steps)])
    hip.destroy(evs)
    flops = 4.0 * seq * seq * hl * d
    gather_bytes = 2 * 3 * hl * seq * d * 2
    unpack_bytes = 2 * ch * h * 2
    del rq, rk, rvt, gq, gk, gvt, o, recv_o, o_full
    torch.cuda.empty_cache()
    return {
        "workload": f"Ulysses share: rank 0 of {ranks}, {hl} of {nh} heads over seq {seq}, hidden {h}",
        "ms": g["median"] + a["median"] + u["median"], "gather_ms": g, "attention_ms": a, "unpack_ms": u,
        "attention_tflops": flops / (a["median"] * 1e-3) / 1e12,
        "attention_frac_of_peak": flops / (a["median"] * 1e-3) / 1e12 / PEAK_F16_TFLOPS,
        "gather_gbs": gather_bytes / (g["median"] * 1e-3) / 1e9, "gather_bytes": gather_bytes,
        "unpack_gbs": unpack_bytes / (u["median"] * 1e-3) / 1e9, "unpack_bytes": unpack_bytes,
    }


def run_tp_share(torch, B, hip, warmup, steps, seq=8192, h=4096, nh=32, ranks=8, seed=0):
    """Rank 0's tensor-parallel share: Q/K/V for its 4 heads (column shard), their attention, and the
    partial output through its row shard of W_O."""
    from long_context_self_amd.synthetic import block_inputs

    x, [ws] = block_inputs(seq, h, 1, dtype=np.float16, seed=seed)
    blk = B.AttnBlock(*(torch.from_numpy(w).cuda() for w in ws), num_heads=nh, max_tokens=seq, n_ranks=ranks,
                      rank=0)
    del ws
    xd = torch.from_numpy(x).cuda()
    y = torch.empty_like(xd)
    stream = torch.cuda.current_stream().cuda_stream
    evs = hip.events(4 * steps)

    def one(s):
        taps = None
        if s is not None:
            taps = B.Taps(None, None, None, None, None, 0,
                          ctypes.addressof(evs) + 4 * s * ctypes.sizeof(ctypes.c_void_p))
        blk.forward(xd, y, taps=taps)

    for _ in range(warmup):
        one(None)
    torch.cuda.synchronize()
    for s in range(steps):
        one(s)
    torch.cuda.synchronize()
    st = {n: stats([hip.ms(evs[4 * s + i], evs[4 * s + i + 1]) for s in range(steps)])
          for i, n in enumerate(("qkv", "attn", "oproj"))}
    step = stats([hip.ms(evs[4 * s], evs[4 * s + 3]) for s in range(steps)])
    hip.destroy(evs)
    blk.close()
    del xd, y
    torch.cuda.empty_cache()
    w = h // ranks
    fl = {"qkv": 6.0 * seq * h * w, "attn": 4.0 * seq * seq * w, "oproj": 2.0 * seq * w * h}
    return {
        "workload": f"tensor-parallel share: rank 0 of {ranks} ({nh // ranks} heads), seq {seq}, hidden {h}, "
                    "partial output before the all-reduce",
        "ms_per_forward": step["median"], "kernels_ms": st,
        "kernels_tflops": {n: fl[n] / (st[n]["median"] * 1e-3) / 1e12 for n in fl},
        "share_tflops": sum(fl.values()) / (step["median"] * 1e-3) / 1e12,
    }

def run_ring_share(torch, B, hip, warmup, steps, seq=32768, h=4096, nh=32, ranks=8, seed=0):
    """Rank 0 of 8 with Ring-style streaming: its 4096-row query chunk against 8 K/V blocks of 4096 keys that
    arrive by copy from pinned host memory (a stand-in for a peer's link) on the ring's copy stream while the
    earlier blocks' attention runs. Reported beside the same blocks already in device memory (the ring then
    computes every block's partial in one launch), the per-block partial calls and merge with K/V resident
    (compute only), and the copies alone (transfer only)."""
    from long_context_self_amd.synthetic import block_inputs

    d, ch = h // nh, seq // ranks
    x, [ws] = block_inputs(seq, h, 1, dtype=np.float16, seed=seed)
    blk = B.AttnBlock(*(torch.from_numpy(w).cuda() for w in ws), num_heads=nh, max_tokens=seq)
    q = torch.empty((nh, seq, d), dtype=torch.float16, device="cuda")
    k = torch.empty_like(q)
    vt = torch.zeros((nh, d, B.vt_ld(seq)), dtype=torch.float16, device="cuda")
    blk.forward(torch.from_numpy(x).cuda(), taps=B.Taps(q.data_ptr(), k.data_ptr(), vt.data_ptr(), None, None, 1,
                                                           None))
    torch.cuda.synchronize()
    blk.close()
    q0 = q[:, :ch].contiguous()
    kd = [k[:, b * ch:(b + 1) * ch].contiguous() for b in range(ranks)]
    vd = [vt[:, :, b * ch:(b + 1) * ch].contiguous() for b in range(ranks)]
    kh = [t.cpu().pin_memory() for t in kd]
    vh = [t.cpu().pin_memory() for t in vd]
    del q, k, vt
    lens = [ch] * ranks
    ring = B.AttnRing(nh, d, ranks, ch, ch)
    o = torch.empty((ch, h), dtype=torch.float16, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    slot = [torch.empty_like(kd[0]), torch.empty_like(vd[0])]

    def timed(fn):
        evs = hip.events(2 * steps)
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        for s_ in range(steps):
            hip.record(evs[2 * s_], stream)
            fn()
            hip.record(evs[2 * s_ + 1], stream)
        torch.cuda.synchronize()
        r = stats([hip.ms(evs[2 * s_], evs[2 * s_ + 1]) for s_ in range(steps)])
        hip.destroy(evs)
        return r

    t_host = timed(lambda: ring.forward(q0, ch, kh, vh, lens, o))
    t_dev = timed(lambda: ring.forward(q0, ch, kd, vd, lens, o))

    def copies():
        for b in range(ranks):
            slot[0].copy_(kh[b], non_blocking=True)
            slot[1].copy_(vh[b], non_blocking=True)

    t_copy = timed(copies)
    o_parts = torch.empty((ranks, nh, ch, d), dtype=torch.float32, device="cuda")
    lse_parts = torch.empty((ranks, nh, ch), dtype=torch.float32, device="cuda")

    def compute():
        for b in range(ranks):
            B.attn_partial_forward_vt(nh, d, q0, ch, ch * d, kd[b], ch, ch * d, vd[b], d * ch, ch, o_parts[b],
                                   lse_parts[b])
        B.attn_merge_lse(ranks, nh, d, ch, o_parts, lse_parts, o, torch.float16)

    t_comp = timed(compute)
    ring.close()
    kv_bytes = 2 * ranks * nh * ch * d * 2
    tc, tx, tr = t_comp["median"], t_copy["median"], t_host["median"]
    del kd, vd, kh, vh, q0, o, o_parts, lse_parts, slot
    torch.cuda.empty_cache()
    return {
        "workload": f"ring streaming: rank 0 of {ranks} at seq {seq} (query chunk {ch}) vs {ranks} K/V blocks of {ch} "
                    f"keys copied from pinned host memory while earlier blocks compute, hidden {h}",
        "ms": tr, "ring_host_blocks_ms": t_host, "ring_device_blocks_ms": t_dev,
        "compute_only_ms": t_comp, "transfer_only_ms": t_copy,
        "transfer_gbs": kv_bytes / (tx * 1e-3) / 1e9,
        "overlap_efficiency": (tc + tx - tr) / min(tc, tx),
        "attention_tflops_device_blocks": 4.0 * ch * seq * h / (t_dev["median"] * 1e-3) / 1e12,
    }

PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "long_context_self_amd", "csrc")
# the sources that decide the attention step's launches and kernels (its HBM counters go stale with them)
ATTN_SOURCES = ("flash_fwd.hip", "common.hpp", "lse_merge.hip", "launch_plan.hpp")


def hbm_traffic(kernel: str, sources: tuple[str, ...], counters: str):
    """HBM bytes per launch of `kernel` from the committed FETCH_SIZE /
    WRITE_SIZE counter readings in profiles/`counters`, each scaled by what
    the same counter reads for a plain device copy of known size; None when
    the file is missing or the kernel's sources changed since the counters
    were taken."""
    import hashlib

    try:
        vals = {}
        with open(os.path.join(PROFILES, counters)) as f:
            for line in f:
                if line.strip() and not line.startswith("#"):
                    k, v = line.split()
                    vals[k] = v
        digest = "+".join(hashlib.sha256(open(os.path.join(CSRC, s), "rb").read()).hexdigest() for s in sources)
        if vals.get(f"{kernel}.kernel_source_sha256") != digest:
            return None
        cb = float(vals["copy_bytes"])
        f_fetch = cb / (float(vals["copy_fetch_size_kib"]) * 1024)
        f_write = cb / (float(vals["copy_write_size_kib"]) * 1024)
        return (float(vals[f"{kernel}.fetch_size_kib"]) * 1024 * f_fetch
                + float(vals[f"{kernel}.write_size_kib"]) * 1024 * f_write)
    except (OSError, KeyError, ValueError):
        return None


# ------------------------------------------------------------------ CPU baseline
_POOL_STATE = {}


def _pool_init():
    try:
        from threadpoolctl import threadpool_limits
        _POOL_STATE["limit"] = threadpool_limits(1)  # one BLAS thread per worker process
    except Exception:
        pass


def _pool_head(j):
    import oracle
    st = _POOL_STATE
    return oracle.attention(st["q"][j], st["k"][j], st["v"][j])


def oracle_sampled(seq, h, nh, rows, seed, workers):
    """One sampled-row oracle forward: the oracle's own steps in its order --
    K and V over all seq rows (BLAS on every core), q_scaled for the sampled
    rows, attention head by head (heads spread over `workers` forked
    processes), concatenation and W_O. Returns seconds and FLOPs."""
    import multiprocessing as mp

    import oracle
    from long_context_self_amd.synthetic import block_inputs, sample_rows

    x, [(wq, wk, wv, wo)] = block_inputs(seq, h, 1, dtype=np.float16, seed=seed)
    r = sample_rows(seq, rows, seed=seed, must=[seq // 8 * i for i in range(9)])
    d = h // nh
    t0 = time.perf_counter()
    xf = oracle.as_f64(x)
    _POOL_STATE["k"] = oracle.split_heads(oracle.project(xf, wk), nh)
    _POOL_STATE["v"] = oracle.split_heads(oracle.project(xf, wv), nh)
    _POOL_STATE["q"] = oracle.split_heads(oracle.scale_query(oracle.project(xf[r], wq), d), nh)
    t1 = time.perf_counter()
    with mp.get_context("fork").Pool(workers, initializer=_pool_init) as pool:
        t1b = time.perf_counter()  # workers forked (they inherit K, V and q_scaled)
        res = pool.map(_pool_head, range(nh), chunksize=1)
        o = oracle.merge_heads(np.stack([a[0] for a in res]))
        y = oracle.project(o, wo)
        t2 = time.perf_counter()
    assert np.isfinite(y).all()
    _POOL_STATE.clear()
    flops_kv = 4.0 * seq * h * h
    flops_rows = len(r) * (2.0 * h * h + 4.0 * seq * h + 2.0 * h * h)
    return {"seconds": t2 - t0, "seconds_kv": t1 - t0, "seconds_pool_start": t1b - t1, "seconds_rows": t2 - t1b,
            "rows": int(len(r)), "flops": flops_kv + flops_rows, "flops_kv": flops_kv, "flops_rows": flops_rows}


def cpu_baseline_child(workloads) -> dict:
    """Run in a child process (no torch, no GPU): the sampled-row oracle at
    each (seq, h, nh, rows); the first entry is the headline."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("internal_api") == "openblas"]
                   or [1])
    except Exception:
        blas = None
    workers = len(os.sched_getaffinity(0))
    out = []
    for seq, h, nh, rows in workloads:
        m = oracle_sampled(seq, h, nh, rows, 0, workers)
        per_row = m["seconds_rows"] / m["rows"]
        # every query row at the measured per-row cost (pool start counted once)
        full_s = m["seconds_kv"] + m["seconds_pool_start"] + per_row * seq
        blk_flops = 8.0 * seq * h * h + 4.0 * seq * seq * h
        out.append({"seq": seq, "hidden": h, "heads": nh, "rows_sampled": m["rows"],
                    "seconds": m["seconds"], "seconds_kv_all_rows": m["seconds_kv"],
                    "seconds_pool_start": m["seconds_pool_start"], "seconds_sampled_rows": m["seconds_rows"],
                    "value": m["flops"] / m["seconds"] / 1e12, "unit": "TFLOP/s",
                    "extrapolated_ms_per_forward": full_s * 1e3,
                    "extrapolated_block_tflops": blk_flops / full_s / 1e12})
    return {"blas_threads": blas, "pool_workers": workers, "results": out}


def cpu_baseline(workloads):
    """Start the CPU baseline child (this script with --cpu-child) and parse its JSON."""
    import subprocess

    spec = ";".join(",".join(str(v) for v in w) for w in workloads)
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-child", spec], capture_output=True,
                       text=True)
    if r.returncode != 0:
        raise RuntimeError(f"CPU baseline child failed ({r.returncode}): {r.stderr[-2000:]}")
    return json.loads(r.stdout.strip().splitlines()[-1])


def trace_summary(path: str) -> str:
    """Per (kernel, grid size) dispatch count and mean/min/max duration from a
    rocprofv3 --kernel-trace CSV, as a markdown table."""
    import csv
    import collections

    groups = collections.defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            short = name.replace("attnblk::(anonymous namespace)::", "").split("(")[0]
            key = (short, int(r["Grid_Size_X"]) * int(r.get("Grid_Size_Y", 1) or 1) * int(r.get("Grid_Size_Z", 1) or 1),
                   int(r["Workgroup_Size_X"]))
            groups[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6)
    lines = ["| kernel | grid threads | workgroup | dispatches | mean ms | min ms | max ms |",
             "|---|---|---|---|---|---|---|"]
    for (k, g, w), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| {k} | {g} | {w} | {len(v)} | {np.mean(v):.4f} | {np.min(v):.4f} | {np.max(v):.4f} |")
    return "\n".join(lines)


def block_entry(name, seq, h, nh, ms, kern, layers=1):
    f = block_flops(seq, h)
    tfl = {n: f[n] / (kern[n]["mean"] * 1e-3) / 1e12 for n in ("qkv", "attn", "oproj")}
    return {"workload": name, "seq": seq, "hidden": h, "heads": nh, "layers": layers, "ms_per_forward": ms,
            "ms_per_forward_stats": kern["step"], "kernels_ms": {n: kern[n] for n in ("qkv", "attn", "oproj")},
            "attention_tflops": tfl["attn"], "attention_frac_of_peak": tfl["attn"] / PEAK_F16_TFLOPS,
            "qkv_tflops": tfl["qkv"], "oproj_tflops": tfl["oproj"],
            "block_tflops": layers * sum(f.values()) / (ms * 1e-3) / 1e12}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--seq", type=int, default=65536, help="headline sequence length (hidden 4096, 32 heads)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (for HBM counter calibration)")
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="print a per-(kernel, grid) summary of a rocprofv3 kernel-trace CSV and exit")
    ap.add_argument("--cpu-child", metavar="SPEC", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.trace_summary:
        print(trace_summary(args.trace_summary))
        return 0
    if args.cpu_child:
        wl = [tuple(int(v) for v in w.split(",")) for w in args.cpu_child.split(";")]
        print(json.dumps(cpu_baseline_child(wl)), flush=True)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the library builds no "
              f"multi-GPU path)", file=sys.stderr)
        return 2
    seq, h, nh = args.seq, 4096, 32
    steps, warmup = args.steps, args.warmup

    # CPU baseline first, in a child process, before this process touches the GPU.
    cpu = cpu_other = None
    if not args.no_cpu:
        wl = [(seq, h, nh, 2048)]
        if not args.quick:
            wl += [(s2, 4096, 32, 256) for s2 in (8192, 16384, 32768) if s2 != seq] + [(8192, 8192, 64, 256)]
        log(f"cpu baseline: fp64 oracle, sampled rows, {len(wl)} workloads (child process)")
        res = cpu_baseline(wl)
        head = res["results"][0]
        cpu = {"value": head["value"], "unit": "TFLOP/s", "cores": res["pool_workers"], "kind": "oracle",
               "blas_threads": res["blas_threads"], "pool_workers": res["pool_workers"],
               "seconds": head["seconds"], "rows_sampled": head["rows_sampled"],
               "seconds_kv_all_rows": head["seconds_kv_all_rows"],
               "seconds_sampled_rows": head["seconds_sampled_rows"],
               "extrapolated_ms_per_forward": head["extrapolated_ms_per_forward"],
               "sample": f"fp64 numpy oracle at seq {seq}, hidden {h}, {nh} heads: K and V over all {seq} rows "
                         f"({res['blas_threads']} BLAS threads), then {head['rows_sampled']} seeded query rows "
                         f"(first, last, the 1/8 borders) through q_scaled, attention (heads over "
                         f"{res['pool_workers']} processes) and W_O, measured once ({head['seconds']:.1f} s); "
                         f"value = algorithmic FLOPs of that sample / wall time. extrapolated_ms_per_forward "
                         f"(all {seq} rows at the measured per-row cost) is an extrapolation, not a measurement"}
        cpu_other = res["results"][1:]
        log(f"  {head['seconds']:.1f} s at seq {seq} ({head['value'] * 1e3:.0f} GFLOP/s; full forward "
            f"extrapolated {head['extrapolated_ms_per_forward'] / 1e3:.0f} s)")

    import torch

    from long_context_self_amd import binding as B

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    B.lib()
    hip = Hip()

    if args.copy_calibration:
        a = torch.empty(1 << 29, dtype=torch.float16, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    log(f"headline: seq {seq} hidden {h} heads {nh}, warmup {warmup}, steps {steps}")
    ms, kern = run_block(torch, B, hip, seq, h, nh, 1, warmup, steps)
    head = block_entry(f"block forward seq {seq} hidden {h} heads {nh} fp16", seq, h, nh, ms, kern)
    fl = block_flops(seq, h)
    total_flops = sum(fl.values())
    kernel_tflops = {n: fl[n] / (kern[n]["mean"] * 1e-3) / 1e12 for n in ("qkv", "attn", "oproj")}
    dom = max(("qkv", "attn", "oproj"), key=lambda n: kern[n]["mean"])
    names = {"qkv": "gemm_f16_nt (QKV projection, fused layout epilogue)",
             "attn": "attention step: flash_fwd_f16_d128 over the whole-key query blocks (384 rows each), then over "
                     "the tail rows in 256-row workgroups, split over key ranges and merged by lse_merge, or over "
                     "all keys (as the launch plan picks for the shape)",
             "oproj": "gemm_f16_nt (output projection)"}
    counters = f"hbm_counters_seq{seq}_h{h}.txt"
    roofline = {"bound": "mfma", "kernel": names[dom], "achieved": kernel_tflops[dom], "peak": PEAK_F16_TFLOPS,
                "unit": "TFLOP/s", "frac": kernel_tflops[dom] / PEAK_F16_TFLOPS,
                "traffic": hbm_traffic("attention", ATTN_SOURCES, counters) if dom == "attn" else None,
                "flops_per_launch": fl[dom], "avg_launch_ms": kern[dom]["mean"],
                "traffic_unit": "HBM bytes per launch (FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0, copy-calibrated, "
                                f"profiles/{counters})",
                "algorithmic_bytes": 4 * seq * h * 2 if dom == "attn" else None}
    log(f"  {ms:.3f} ms/forward; kernels ms: " + ", ".join(f"{n} {kern[n]['mean']:.3f}" for n in fl)
        + f"; attention {kernel_tflops['attn']:.0f} TFLOP/s ({kernel_tflops['attn'] / PEAK_F16_TFLOPS:.3f})")

    extra = []
    if not args.quick:
        for s2, h2, nh2 in ((8192, 4096, 32), (16384, 4096, 32), (32768, 4096, 32), (8192, 8192, 64)):
            if (s2, h2) == (seq, h):
                continue
            log(f"block seq {s2} hidden {h2}")
            m2, k2 = run_block(torch, B, hip, s2, h2, nh2, 1, warmup, steps)
            extra.append(block_entry(f"block forward seq {s2} hidden {h2} heads {nh2} fp16", s2, h2, nh2, m2, k2))
            log(f"  {m2:.3f} ms/forward, attention {extra[-1]['attention_tflops']:.0f} TFLOP/s "
                f"({extra[-1]['attention_frac_of_peak']:.3f})")
        log("block seq 8192 hidden 4096 with RMSNorm pre-norm")
        # the same block without the norm is timed right before it, so both see the same clock state
        m0, k0 = run_block(torch, B, hip, 8192, h, nh, 1, warmup, steps)
        mn, kn = run_block(torch, B, hip, 8192, h, nh, 1, warmup, steps, prenorm=True)
        norm_bytes = 8192 * h * 2 + 8192 * 4
        extra.append({"workload": "block forward with RMSNorm pre-norm (unit gain, eps 1e-6), seq 8192 hidden 4096 "
                                  "heads 32 fp16", "ms_per_forward": mn, "ms_per_forward_without_norm": m0,
                      "qkv_with_norm_ms": kn["qkv"]["median"], "qkv_without_norm_ms": k0["qkv"]["median"],
                      "norm_overhead_ms": kn["qkv"]["median"] - k0["qkv"]["median"],
                      "norm_algorithmic_bytes": norm_bytes,
                      "block_tflops": sum(block_flops(8192, h).values()) / (mn * 1e-3) / 1e12})
        log(f"  {mn:.3f} ms/forward, norm overhead {extra[-1]['norm_overhead_ms'] * 1e3:.1f} us")
        log("rank share")
        extra.append(run_rank_share(torch, B, hip, warmup, steps))
        log(f"  {extra[-1]['ms']:.3f} ms (V^T: {extra[-1]['ms_vt']:.3f}), attention {extra[-1]['attention_tflops']:.0f}"
            f" TFLOP/s, merge {extra[-1]['merge_gbs']:.0f} GB/s; one launch over all keys "
            f"{extra[-1]['one_shot_ms']:.3f} ms")
        log("Ulysses share (rank 0 of 8), seq 32768")
        extra.append(run_ulysses_share(torch, B, hip, warmup, steps))
        log(f"  {extra[-1]['ms']:.3f} ms: gather {extra[-1]['gather_gbs']:.0f} GB/s, attention "
            f"{extra[-1]['attention_tflops']:.0f} TFLOP/s, unpack {extra[-1]['unpack_gbs']:.0f} GB/s")
        log("tensor-parallel share (rank 0 of 8), seq 8192")
        extra.append(run_tp_share(torch, B, hip, warmup, steps))
        log(f"  {extra[-1]['ms_per_forward']:.3f} ms/forward, {extra[-1]['share_tflops']:.0f} TFLOP/s")
        log("ring streaming (rank 0 of 8), seq 32768, K/V blocks from pinned host memory")
        extra.append(run_ring_share(torch, B, hip, warmup, steps))
        log(f"  {extra[-1]['ms']:.3f} ms (compute only {extra[-1]['compute_only_ms']['median']:.3f}, device blocks "
            f"in one launch "
            f"{extra[-1]['ring_device_blocks_ms']['median']:.3f}, transfer only "
            f"{extra[-1]['transfer_only_ms']['median']:.3f} at {extra[-1]['transfer_gbs']:.0f} GB/s), overlap "
            f"efficiency {extra[-1]['overlap_efficiency']:.2f}")
        log("6 stacked blocks seq 32768")
        m6, k6 = run_block(torch, B, hip, 32768, 4096, 32, 6, warmup, steps)
        extra.append(block_entry("6 stacked blocks seq 32768 hidden 4096 heads 32 fp16", 32768, 4096, 32, m6, k6,
                                 layers=6))
        log(f"  {m6:.3f} ms per 6-block forward")

    out = {
        "metric": METRIC,
        "value": total_flops / (ms * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "self-attention block forward, non-causal: QKV projection + q_scaled + "
                               "attention + output projection", "seq_len": seq, "batch": 1, "hidden": h,
                   "heads": nh, "head_dim": h // nh, "dtype": "fp16", "seed": 0},
        "value_definition": "block TFLOP/s = (8 S h^2 + 4 S^2 h) / ms_per_step",
        "ms_per_forward": kern["step"],
        "attention": {"ms": kern["attn"]["mean"], "tflops": kernel_tflops["attn"],
                      "frac_of_peak": kernel_tflops["attn"] / PEAK_F16_TFLOPS},
        "kernels_ms": {n: kern[n] for n in ("qkv", "attn", "oproj")},
        "kernels_tflops": kernel_tflops,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "cpu_baseline_other_workloads": cpu_other,
        "other_workloads": extra,
        "context_b200": B200_CONTEXT,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
