#!/usr/bin/env python3
"""Benchmark of the ring-cache chunk-attention path on one MI355X.

Workload: one streaming chunk of the 57B video DiT served by Runway
Characters (abstract): 4 denoising passes x 60 layers = 240 attention calls,
each over a 5,788-slot FP8 ring cache in which 757 tokens are new; 40 heads,
head_dim 128, RoPE base 10000, cache bias 0.  A step is one chunk: for every
pass and layer one rc_cache_write (757 tokens) and one rc_chunk_attention
(757 queries over all 5,788 slots), then rc_ring_advance on all 60 layers.
Each layer has its own ring (60 x 61 MB, far beyond the last-level cache) and
Q/K/V come from a pool of 16 synthetic N(0,1) bf16 sets (372 MB).

Prints ONE JSON line on stdout.  ``value`` is chunk-attention TFLOP/s over the
whole step (240 x 89.73 GFLOP / wall time per chunk); ``ms_per_step`` is
ms per chunk.  ``roofline`` covers the attention kernel, timed with HIP events
on the stream it runs on, around layer 0's launches of every pass in the timed
chunks; the write and rerotate kernels' bandwidths are reported beside it.
``roofline.traffic`` is the attention kernel's HBM bytes per launch from
recorded rocprofv3 counter runs, or null if the kernel changed since.
``cpu_baseline`` times the float64 oracle on the host cores on a bounded sample
of the same workload (layer calls, about ten seconds).  ``joint_av`` times the
six paths of a joint audio-video block (StreamLTX project page, Training:
one-second blocks of 1,152 video and 25 audio tokens, 10 blocks cached, 32
heads, bf16, block-causal; Data: each block sees only its own segment's
prompt, here three prompts of 96-160 tokens), each with the last block's
queries and with all ten blocks' queries, and video self-attention with the
first block one latent frame longer (1,536 tokens).  ``qkv_projection`` times
the fused QKV projection + cache write (FP8 GEMM 757 x 5120 x 15360 with the
write in its epilogue) beside the unfused bf16 library GEMM + rc_cache_write.

``--longrun K`` instead runs K chunks of the long-run schedule (a position
reset every 300 chunks by a delta rotation of all 60 rings, ten cache-bias
ramps 0, -2, -4, -2, 0) and prints one JSON line with the sustained ms/chunk
(median and p99).  ``--anchor A`` makes those rings anchored: the first A
tokens (A = 757: the first chunk) stay pinned and the other slots slide;
``--memory M`` adds a scored content memory of M slots: the last pass of
every chunk also computes each layer's key mass for the next write's
candidates (rc_key_mass_slots over the occupied memory slots and the slots
that write overwrites, from that pass's queries and lse), and the next
chunk's first write keeps the best tokens in the memory
(rc_cache_write_scored, diversity ``--diversity``).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "chunk-attention TFLOP/s + ms/chunk (757 new × 5788-slot fp8 ring cache)"
H, D, N, NEW, HIST = 40, 128, 5788, 757, 5031
LAYERS, PASSES, POOL = 60, 4, 16
ATTN_FLOP = 4.0 * H * D * NEW * N            # every slot visible to every query
WRITE_BYTES = (2 * NEW * H * D * 2            # K and V in, bf16
               + 2 * NEW * H * D              # K and V codes out
               + 2 * NEW * H * 4              # K and V scales out
               + 2 * NEW * 4)                 # slot_pos, slot_block
REROT_BYTES = 2 * (H * N * D + H * N * 4) + N * 4 + 2 * N * 4  # codes+scales in/out, block read, pos rw
PEAK_FP8_TFLOPS = 5000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
AV_H, AV_BLOCKS, AV_VIDEO, AV_AUDIO = 32, 10, 1152, 25
RESET_EVERY, RAMPS, RAMP_FIRST, RAMP_SPACING, RAMP_DEPTH = 300, 10, 150, 200, 4.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(min_seconds: float = 10.0, max_calls: int = 12) -> dict:
    """The oracle as it stands on the host cores, on a bounded sample of the
    same workload: layer calls (write 757 tokens into a full 5,788-slot FP8
    ring, then attend 757 queries over it, 40 heads), repeated until about
    ten seconds of work have been timed."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle.attention import ring_attention
    from oracle.ring import Ring as OracleRing
    from synthetic_inputs import normal_bf16

    cores = len(os.sched_getaffinity(0))
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 0x7E, size=(H, N, D), dtype=np.uint8)  # finite codes
    codes |= (rng.integers(0, 2, size=codes.shape, dtype=np.uint8) << 7)
    vcodes = rng.integers(0, 0x7E, size=(H, N, D), dtype=np.uint8)
    scale = (rng.uniform(0.5, 1.5, size=(H, N)) / 100).astype(np.float32)
    _, k = normal_bf16(rng, (NEW, H, D))
    _, v = normal_bf16(rng, (NEW, H, D))
    _, q = normal_bf16(rng, (NEW, H, D))
    calls, dt = 0, 0.0
    with threadpool_limits(limits=cores):
        used = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        while calls < max_calls and (dt < min_seconds or calls == 0):
            ring = OracleRing.from_arrays(kv_dtype="fp8", rope_base=10000.0, k=codes, v=vcodes, k_scale=scale,
                                          v_scale=scale.copy(), slot_pos=np.arange(N),
                                          slot_block=np.zeros(N, np.int64), state=(HIST, HIST, 0, 0, 0))
            t0 = time.perf_counter()
            ring.write(k, v, NEW, HIST, 1)
            ring_attention(ring, q, HIST, 1, NEW, 0.0)
            dt += time.perf_counter() - t0
            calls += 1
        # the position reset: the oracle's delta rotation of the full ring (every slot occupied)
        t0 = time.perf_counter()
        ring.rerotate(-3000)
        rot_s = time.perf_counter() - t0
    per_call = dt / calls
    return {"value": ATTN_FLOP / per_call / 1e12, "unit": "TFLOP/s", "cores": int(used), "kind": "oracle",
            "sample": f"{calls} layer calls (each: write {NEW} tokens + attention {NEW} x {N}, {H} heads, "
                      f"d {D}), {dt:.1f} s on {used} threads, then one rerotate(-3000) of the full ring "
                      f"({rot_s:.2f} s); host has {cores} cores available",
            "seconds": dt, "ms_per_chunk_extrapolated": per_call * 1e3 * PASSES * LAYERS,
            "rerotate_seconds": round(rot_s, 3), "rerotate_gb_per_s": round(REROT_BYTES / rot_s / 1e9, 3)}


# HBM traffic of the attention kernel per launch, from rocprofv3 FETCH_SIZE
# and WRITE_SIZE counter runs (scaled by the same counters on a plain 1 GiB
# copy), recorded with a hash of the kernel source they were taken on.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fp8_757x5788_traffic.txt")
KERNEL_SOURCE = os.path.join(ROOT, "autoregressive_video_diffusion_ring_amd", "csrc", "attn_fp8.hip")


def timed_us(fn, stream, reps: int = 20, warm: int = 3) -> float:
    """Median of `reps` launches of fn, each bracketed by HIP events on `stream`."""
    import torch
    for _ in range(warm):
        fn()
    evs = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    return t[len(t) // 2]


def joint_av(dev, stream) -> dict:
    """The four attention paths of one joint audio-video block: bf16 rings of
    ten one-second blocks (video 1,152 tokens per block, audio 25), 32 heads,
    d 128, no RoPE, bias 0.  Work per path is 4*H*d per visible (query, slot)
    pair; bytes are the ring's K and V once plus Q in and O out."""
    import torch

    from autoregressive_video_diffusion_ring_amd import Ring
    gen = torch.Generator(device=dev)
    gen.manual_seed(3)
    rnd = lambda n: torch.randn((n, AV_H, D), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    rings, qs = {}, {}
    for name, blen in (("video", AV_VIDEO), ("audio", AV_AUDIO)):
        r = Ring(blen * AV_BLOCKS, AV_H, D, "bf16", 0.0, device=dev)
        for b in range(AV_BLOCKS):
            r.write(rnd(blen), rnd(blen), blen * b, b)
            if b < AV_BLOCKS - 1:
                r.advance(blen)
        rings[name] = (r, blen)
        qs[name] = rnd(blen * AV_BLOCKS)
    res = {}
    # text cross-attention: three prompt segments (blocks 0-3, 4-6, 7-9; 128,
    # 96 and 160 tokens), each block sees only its own segment's prompt
    seg_of_block = [0, 0, 0, 0, 1, 1, 1, 2, 2, 2]
    prompts = [128, 96, 160]
    text = Ring(sum(prompts), AV_H, D, "bf16", 0.0, device=dev)
    for sg, n in enumerate(prompts):
        text.write(rnd(n), rnd(n), 0, sg)
        if sg < len(prompts) - 1:
            text.advance(n)
    for qn in ("video", "audio"):
        qblen = rings[qn][1]
        for mode in ("last_block", "all_blocks"):
            q = qs[qn][(AV_BLOCKS - 1) * qblen:].contiguous() if mode == "last_block" else qs[qn]
            blocks = [AV_BLOCKS - 1] if mode == "last_block" else list(range(AV_BLOCKS))
            ids = torch.tensor([seg_of_block[b] for b in blocks for _ in range(qblen)], dtype=torch.int32,
                               device=dev)
            out = torch.empty_like(q)
            us = timed_us(lambda: text.attention(q, 0, 0, None, 0.0, out=out, q_block=ids, same_block=True,
                                                 stream=stream), stream)
            pairs = sum(qblen * prompts[seg_of_block[b]] for b in blocks)
            flop = 4.0 * AV_H * D * pairs
            nbytes = 2 * AV_H * text.N * D * 2 + 2 * q.shape[0] * AV_H * D * 2
            res[f"{qn[0]}->t {mode}"] = {
                "queries": q.shape[0], "slots": text.N, "us": round(us, 2), "gflop": round(flop / 1e9, 3),
                "tflops": round(flop / (us * 1e-6) / 1e12, 2), "mbytes": round(nbytes / 1e6, 2),
                "gbs": round(nbytes / (us * 1e-6) / 1e9, 1)}
    # the first block of a take: one latent frame more (1,536 video tokens)
    first = Ring(1536 + (AV_BLOCKS - 1) * AV_VIDEO, AV_H, D, "bf16", 0.0, device=dev)
    lens = [1536] + [AV_VIDEO] * (AV_BLOCKS - 1)
    for b, n in enumerate(lens):
        first.write(rnd(n), rnd(n), 0, b)
        if b < AV_BLOCKS - 1:
            first.advance(n)
    qf = rnd(first.N)
    ids = torch.repeat_interleave(torch.arange(AV_BLOCKS, device=dev, dtype=torch.int32),
                                  torch.tensor(lens, device=dev))
    out = torch.empty_like(qf)
    need = first.workspace_bytes(first.N)
    ws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    us = timed_us(lambda: first.attention(qf, 0, 0, None, 0.0, out=out, workspace=ws, q_block=ids, stream=stream),
                  stream)
    csum = [sum(lens[:b + 1]) for b in range(AV_BLOCKS)]
    flop = 4.0 * AV_H * D * sum(lens[b] * csum[b] for b in range(AV_BLOCKS))
    res["v->v all_blocks first_block_shape"] = {
        "queries": first.N, "slots": first.N, "us": round(us, 2), "gflop": round(flop / 1e9, 3),
        "tflops": round(flop / (us * 1e-6) / 1e12, 2),
        "frac_bf16_peak": round(flop / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    for qn, kn in (("video", "video"), ("audio", "audio"), ("video", "audio"), ("audio", "video")):
        ring, kblen = rings[kn]
        qblen = rings[qn][1]
        for mode in ("last_block", "all_blocks"):
            q = qs[qn][(AV_BLOCKS - 1) * qblen:].contiguous() if mode == "last_block" else qs[qn]
            qb0 = AV_BLOCKS - 1 if mode == "last_block" else 0
            n_q = q.shape[0]
            out = torch.empty_like(q)
            need = ring.workspace_bytes(n_q)
            ws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
            us = timed_us(lambda: ring.attention(q, 0, qb0, qblen, 0.0, out=out, workspace=ws, stream=stream), stream)
            blocks = [AV_BLOCKS - 1] if mode == "last_block" else list(range(AV_BLOCKS))
            pairs = sum(qblen * (b + 1) * kblen for b in blocks)
            flop = 4.0 * AV_H * D * pairs
            nbytes = 2 * AV_H * ring.N * D * 2 + 2 * n_q * AV_H * D * 2
            tf, gbs = flop / (us * 1e-6) / 1e12, nbytes / (us * 1e-6) / 1e9
            res[f"{qn[0]}->{kn[0]} {mode}"] = {
                "queries": n_q, "slots": ring.N, "us": round(us, 2), "gflop": round(flop / 1e9, 3),
                "tflops": round(tf, 2), "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                "mbytes": round(nbytes / 1e6, 2), "gbs": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
    return res


def qkv_projection(dev, stream) -> dict:
    """The fused QKV projection + cache write of one streaming layer call
    (757 tokens, width C = H d = 5,120, FP8 operands, 40 heads of 128):
    2 * 757 * 5120 * 15360 = 119.1 GFLOP per call.  Beside it, the unfused
    path a caller would otherwise run: a library bf16 GEMM (torch.matmul,
    hipBLASLt) producing q, k, v, then rc_cache_write of k and v."""
    import torch

    from autoregressive_video_diffusion_ring_amd import Ring, rc_qkv_workspace_bytes
    C = H * D
    gen = torch.Generator(device=dev)
    gen.manual_seed(6)
    ring = Ring(N, H, D, "fp8", 10000.0, device=dev)
    hist = torch.randn((HIST, H, D), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    ring.write(hist, hist, 0, 0)
    ring.advance(HIST)
    x = torch.randn((NEW, C), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    mag = torch.randint(0, 0x7F, (3 * C, C), generator=gen, device=dev, dtype=torch.int32)
    sign = torch.randint(0, 2, (3 * C, C), generator=gen, device=dev, dtype=torch.int32) << 7
    w = (mag | sign).to(torch.uint8)
    w_scale = torch.full((3 * C,), 1.0 / (64.0 * C ** 0.5), dtype=torch.float32, device=dev)
    q = torch.empty((NEW, H, D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(rc_qkv_workspace_bytes(NEW, C), dtype=torch.uint8, device=dev)
    us = timed_us(lambda: ring.project_write(x, w, w_scale, HIST, 1, q_out=q, workspace=ws, stream=stream), stream)
    flop = 2.0 * NEW * C * 3 * C
    wb = torch.randn((3 * C, C), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    out = torch.empty((NEW, 3 * C), dtype=torch.bfloat16, device=dev)

    def unfused():
        torch.matmul(x, wb.t(), out=out)
        k = out[:, C:2 * C].view(NEW, H, D)
        v = out[:, 2 * C:].view(NEW, H, D)
        ring.write(k.contiguous(), v.contiguous(), HIST, 1, stream=stream)
    us_gemm = timed_us(lambda: torch.matmul(x, wb.t(), out=out), stream)
    us_unfused = timed_us(unfused, stream)
    tf = flop / (us * 1e-6) / 1e12
    return {"us": round(us, 2), "gflop": round(flop / 1e9, 2), "tflops": round(tf, 1),
            "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4),
            "unfused_bf16_gemm_us": round(us_gemm, 2), "unfused_gemm_plus_write_us": round(us_unfused, 2)}


def chunk_pos0(t: int) -> int:
    """First position of chunk t; every reset rebases the cache to 0..N-1."""
    return NEW * t if t < RESET_EVERY else N + NEW * (t % RESET_EVERY)


def bias_at(t: int) -> float:
    shape = (0.0, -RAMP_DEPTH / 2, -RAMP_DEPTH, -RAMP_DEPTH / 2, 0.0)
    for k in range(RAMPS):
        s0 = RAMP_FIRST + k * RAMP_SPACING
        if s0 <= t < s0 + len(shape):
            return shape[t - s0]
    return 0.0


def longrun(n_chunks: int, anchor: int = 0, memory: int = 0, diversity: float = 0.9) -> dict:
    """Sustained chunks of the long-run schedule from an empty cache: each
    chunk is 4 passes x 60 layers of write + attention, then 60 advances;
    before every 300th chunk all 60 rings are rerotated so that the most
    recent N cached positions become 0..N-1 (the oldest cached position of a
    plain ring; an anchor, older still, moves below 0 with them); the cache
    bias follows ten ramps.  With anchor > 0 every ring pins its first
    `anchor` tokens; with memory > 0 every ring has a scored content memory
    of that many slots, scored by the key mass of each chunk's last pass
    (computed for the next scored write's candidates only: the occupied
    memory slots and the slots that write overwrites)."""
    import torch

    from autoregressive_video_diffusion_ring_amd import (Ring, rc_cache_write, rc_cache_write_scored,
                                                         rc_cache_write_scored_workspace_bytes, rc_chunk_attention,
                                                         rc_key_mass_slots, rc_key_mass_workspace_bytes,
                                                         rc_ring_advance)
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    gen = torch.Generator(device=dev)
    gen.manual_seed(4)
    rings = [Ring(N, H, D, "fp8", 10000.0, n_anchor=anchor, n_memory=memory, device=dev) for _ in range(LAYERS)]
    pool = [[torch.randn((NEW, H, D), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
             for _ in range(3)] for _ in range(POOL)]
    out = torch.empty((NEW, H, D), dtype=torch.bfloat16, device=dev)
    structs = [r.struct for r in rings]
    if memory:
        v_ld = rings[0].v_ld
        masses = torch.zeros((LAYERS, H, v_ld), dtype=torch.float32, device=dev)
        lse = torch.empty((H, NEW), dtype=torch.float32, device=dev)
        nb_m = rc_key_mass_workspace_bytes(structs[0], NEW)
        ws_m = torch.empty(nb_m, dtype=torch.uint8, device=dev)
        nb_w = rc_cache_write_scored_workspace_bytes(structs[0], NEW)
        ws_w = torch.empty(nb_w, dtype=torch.uint8, device=dev)
    ev_mass, ev_scored = [], []
    torch.cuda.synchronize()
    evs, resets = [], []
    for t in range(n_chunks):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        if t > 0 and t % RESET_EVERY == 0:
            delta = -(chunk_pos0(t - 1) + NEW - N)  # oldest cached position -> 0 (the ring is full)
            for r in rings:
                r.rerotate(delta)
            resets.append(t)
        pos0, bias = chunk_pos0(t), bias_at(t)
        for p in range(PASSES):
            score = memory and p == PASSES - 1
            if score:
                masses.zero_()
                # the next scored write's candidates: the occupied memory slots
                # and the slots that write overwrites (all rings move together)
                s0 = structs[0]
                E = N - memory
                nh = s0.head + NEW
                nh = nh if nh < E else anchor + nh - E
                ranges = [(nh, min(nh + NEW, E))]
                if nh + NEW > E:
                    ranges.append((anchor, anchor + nh + NEW - E))
                if s0.n_mem > 0:
                    ranges.append((E, E + s0.n_mem))
            for layer in range(LAYERS):
                q, k, v = pool[(240 * t + 60 * p + layer) % POOL]
                sample = layer == 0 and t >= 8
                if memory and p == 0:
                    if sample:
                        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                        a0.record(stream)
                    rc_cache_write_scored(structs[layer], k, v, NEW, pos0, t, masses[layer], diversity, ws_w, nb_w,
                                          sptr)
                    if sample:
                        a1.record(stream)
                        ev_scored.append((a0, a1))
                else:
                    rc_cache_write(structs[layer], k, v, NEW, pos0, t, sptr)
                rc_chunk_attention(structs[layer], q, NEW, pos0, t, NEW, bias, 0.0, out, lse if score else None,
                                   None, 0, sptr)
                if score:
                    if sample:
                        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                        b0.record(stream)
                    rc_key_mass_slots(structs[layer], q, NEW, pos0, t, NEW, bias, 0.0, lse, ranges, masses[layer],
                                      ws_m, nb_m, sptr)
                    if sample:
                        b1.record(stream)
                        ev_mass.append((b0, b1))
        for s in structs:
            rc_ring_advance(s, NEW)
        e1.record(stream)
        evs.append((e0, e1))
        if t % 100 == 99:
            torch.cuda.synchronize()
            log(f"[longrun] {t + 1} chunks")
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    steady = sorted(m for i, m in enumerate(ms) if i >= 8 and i not in resets)
    full = sorted(ms[8:])
    pick = lambda v, f: v[min(len(v) - 1, int(f * len(v)))]
    kind = f"anchored fp8 ring, first {anchor} tokens pinned" if anchor else "fp8 ring"
    if memory:
        kind += f", scored memory of {memory} slots (diversity {diversity})"
    med = lambda evl: (sorted(a.elapsed_time(b) for a, b in evl)[len(evl) // 2] * 1e3) if evl else None
    return {"metric": f"sustained ms/chunk, long-run schedule (757 new x 5788-slot {kind}, 60 layers)",
            "value": round(pick(full, 0.5), 4), "unit": "ms", "higher_is_better": False,
            "n_anchor": anchor, "n_memory": memory, "final_state": list(rings[0].state()),
            "key_mass_us": med(ev_mass), "scored_write_us": med(ev_scored),
            "chunks": n_chunks, "p99_ms": round(pick(full, 0.99), 4), "mean_ms": round(sum(full) / len(full), 4),
            "steady_median_ms": round(pick(steady, 0.5), 4),
            "reset_chunk_ms": [round(ms[i], 3) for i in resets],
            "fill_chunks_ms": [round(m, 3) for m in ms[:8]],
            "dtype": "fp8", "data": "synthetic", "n_gpus": 1}


def kernel_source_hash() -> str:
    import hashlib
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def recorded_traffic():
    """Bytes per launch from the recorded counter runs, or None when there is
    no record or the kernel source changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            fields = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith("#"))
    except OSError:
        return None
    fields = {k.strip(): v.strip() for k, v in fields.items()}
    if fields.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10, help="timed chunks")
    ap.add_argument("--warmup", type=int, default=2, help="untimed chunks")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (for scaling HBM counters)")
    ap.add_argument("--no-joint-av", action="store_true", help="skip the joint audio-video paths")
    ap.add_argument("--joint-av-only", action="store_true",
                    help="time only the joint audio-video paths and print their line")
    ap.add_argument("--longrun", type=int, default=0, metavar="K",
                    help="run K chunks of the long-run schedule instead and print that line")
    ap.add_argument("--anchor", type=int, default=0, metavar="A",
                    help="with --longrun: pin the first A tokens of every ring (757 = the first chunk)")
    ap.add_argument("--memory", type=int, default=0, metavar="M",
                    help="with --longrun: a scored content memory of M slots in every ring")
    ap.add_argument("--diversity", type=float, default=0.9, help="with --memory: gamma in (0, 1]")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"this path runs on one GPU; --gpus {args.gpus} (WORLD_SIZE {world}) is not supported: "
              "the attention heads of a layer shard across GPUs with no communication, "
              "so per-GPU throughput is the one-GPU figure", file=sys.stderr)
        return 2

    import torch

    from autoregressive_video_diffusion_ring_amd import Ring, rc_cache_write, rc_chunk_attention, rc_ring_advance

    if args.longrun > 0:
        torch.cuda.set_device(0)
        print(json.dumps(longrun(args.longrun, args.anchor, args.memory, args.diversity)), flush=True)
        return 0

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    if args.joint_av_only:
        print(json.dumps({"joint_av": joint_av(dev, stream)}), flush=True)
        return 0
    sptr = stream.cuda_stream
    gen = torch.Generator(device=dev)
    gen.manual_seed(1)

    log(f"[bench] allocating {LAYERS} rings of {N} slots x {H} heads x d {D} (fp8)")
    rings = [Ring(N, H, D, "fp8", 10000.0, device=dev) for _ in range(LAYERS)]
    pool = [[torch.randn((NEW, H, D), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
             for _ in range(3)] for _ in range(POOL)]
    hist = torch.randn((HIST, H, D), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    for r in rings:
        r.write(hist, hist, 0, 0)
        r.advance(HIST)
    out = torch.empty((NEW, H, D), dtype=torch.bfloat16, device=dev)
    structs = [r.struct for r in rings]
    torch.cuda.synchronize()

    n_chunks = args.warmup + args.steps
    chunk = 0
    ev_attn = []
    ev_write = []

    def run_chunk(t, timed):
        pos0 = HIST + NEW * t
        blk = 1 + t
        for p in range(PASSES):
            for layer in range(LAYERS):
                q, k, v = pool[(240 * t + 60 * p + layer) % POOL]
                s = structs[layer]
                # kernel durations: HIP events around layer 0's two launches
                # of every pass (sampling keeps their cost out of the step)
                ev = timed and layer == 0
                if ev:
                    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
                    e0.record(stream)
                rc_cache_write(s, k, v, NEW, pos0, blk, sptr)
                if ev:
                    e1.record(stream)
                rc_chunk_attention(s, q, NEW, pos0, blk, NEW, 0.0, 0.0, out, None, None, 0, sptr)
                if ev:
                    e2.record(stream)
                    ev_write.append((e0, e1))
                    ev_attn.append((e1, e2))
        for s in structs:
            rc_ring_advance(s, NEW)

    log(f"[bench] warmup {args.warmup} chunks")
    for _ in range(args.warmup):
        run_chunk(chunk, False)
        chunk += 1
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} chunks")
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        run_chunk(chunk, True)
        chunk += 1
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_chunk = total_ms / args.steps
    attn_us = sum(a.elapsed_time(b) for a, b in ev_attn) / len(ev_attn) * 1e3
    write_us = sum(a.elapsed_time(b) for a, b in ev_write) / len(ev_write) * 1e3
    log(f"[bench] {ms_chunk:.3f} ms/chunk; attention {attn_us:.2f} us/call; write {write_us:.2f} us/call")

    # Kernel durations of the write and the rerotate: one batch of back-to-back
    # launches (the next chunk's write, then a position reset, on all 60
    # rings) between two events, so that no event sits between launches; the
    # C calls are made directly, so that the host issues faster than the GPU
    # runs them (rocprofv3 of the same command agrees, see profiles/).
    from autoregressive_video_diffusion_ring_amd import _lib
    L = _lib.lib()
    q, k, v = pool[0]
    kp, vp = k.data_ptr(), v.data_ptr()
    pos_w, blk_w = HIST + NEW * chunk, 1 + chunk
    torch.cuda.synchronize()
    b0, b1, b2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    b0.record(stream)
    for s in structs:
        _lib.check(L.rc_cache_write(ctypes.byref(s), kp, vp, NEW, pos_w, blk_w, sptr))
    b1.record(stream)
    for s in structs:
        _lib.check(L.rc_cache_rerotate(ctypes.byref(s), -3000, sptr))
    b2.record(stream)
    torch.cuda.synchronize()
    write_batch_us = b0.elapsed_time(b1) * 1e3 / len(structs)
    rot_us = b1.elapsed_time(b2) * 1e3 / len(structs)
    # the write's practical ceiling: plain device copies moving the same HBM
    # traffic (half of WRITE_BYTES read, half written), timed the same way
    half = WRITE_BYTES // 2 // 16 * 16
    bufs = [(torch.empty(half, dtype=torch.uint8, device=dev), torch.empty(half, dtype=torch.uint8, device=dev))
            for _ in range(8)]
    for src, dst in bufs:
        dst.copy_(src)
    torch.cuda.synchronize()
    b0.record(stream)
    for i in range(len(structs)):
        src, dst = bufs[i % len(bufs)]
        dst.copy_(src)
    b1.record(stream)
    torch.cuda.synchronize()
    copy_us = b0.elapsed_time(b1) * 1e3 / len(structs)
    del bufs

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 1 GiB read + 1 GiB written")

    attn_tflops = ATTN_FLOP / (attn_us * 1e-6) / 1e12
    value = PASSES * LAYERS * ATTN_FLOP / (ms_chunk * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_chunk, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": "streaming chunk: 4 passes x 60 layers of write(757) + attention "
                               "757 x 5788 fp8 ring, 40 heads, d 128, RoPE 10000, bias 0",
                   "heads": H, "head_dim": D, "slots": N, "new_tokens": NEW, "layers": LAYERS,
                   "passes": PASSES, "calls_per_chunk": PASSES * LAYERS},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_FP8_TFLOPS, 4),
                     "traffic": recorded_traffic(),
                     "kernel": "attn_fp8_kernel<128,false,false>", "us_per_launch": round(attn_us, 2),
                     "flop_per_launch": ATTN_FLOP},
        "write": {"bound": "hbm", "us_per_launch": round(write_batch_us, 2), "bytes_per_launch": WRITE_BYTES,
                  "achieved": round(WRITE_BYTES / (write_batch_us * 1e-6) / 1e9, 1), "peak": PEAK_HBM_GBS,
                  "unit": "GB/s", "frac": round(WRITE_BYTES / (write_batch_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                  "timing": "60 back-to-back launches between two events",
                  "us_per_launch_in_chunk_events": round(write_us, 2),
                  "copy_same_traffic_us": round(copy_us, 2), "vs_copy": round(write_batch_us / copy_us, 3)},
        "rerotate": {"bound": "hbm", "us_per_launch": round(rot_us, 2), "bytes_per_launch": REROT_BYTES,
                     "timing": "60 back-to-back launches between two events",
                     "achieved": round(REROT_BYTES / (rot_us * 1e-6) / 1e9, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(REROT_BYTES / (rot_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
        "cpu_baseline": None,
        "joint_av": None,
        "qkv_projection": None,
    }
    if not args.no_joint_av:
        log("[bench] joint audio-video paths")
        result["joint_av"] = joint_av(dev, stream)
    if not args.no_joint_av:
        log("[bench] fused QKV projection + cache write")
        result["qkv_projection"] = qkv_projection(dev, stream)
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host (one layer call)")
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
