#!/usr/bin/env python3
"""Benchmark of the block-scaled FP8 hot path on one MI355X.

Headline step (the workload the metric is quoted on): the dense decode GEMM
M=64, N=7168, K=18432 -- per-token 1x128 quant + UE8M0 pack of A (bf16, N(0,1)
with 1% x50 outliers) followed by the block-scaled NT GEMM against e4m3 weights
with 128x128 UE8M0 block scales, bf16 out.  Weights are quantized once, outside
the timed region (as the DeepGEMM benchmark post does, section 4.1).  The inputs
are the GPU parity tests' own seeded tensors; several weight copies (128-row-block
rotations of the one weight set) are rotated so that every step streams its
weights from HBM rather than from the 256 MB last-level cache.

Prints one JSON line on stdout: the headline, then sub-objects for the prefill
sweep, the masked MoE gate_up GEMM and the fused SiLU-quant + masked down GEMM (all
on weights pre-shuffled offline, each also timed on the plain layout), each per call:
mean and p10/median/p90 over batches, TFLOPS, GB/s, roofline fraction; then the
oracle timed on the host cores, and a check of the timed call's output against
the oracle's.  --sweep also times the other layouts and entry
points and prints a table on stderr (and JSON lines to --sweep-out).

Metric definitions follow the benchmark post (section 4.3): TFLOPS = 2*M*N*K/t,
GB/s = (M*K + N*K + 2*M*N)/t (FP8 inputs 1 byte/element, bf16 output 2 bytes;
scale bytes not counted).  For masked GEMMs only valid rows count: flops
2*S*N*K and bytes S*K + E_active*N*K + 2*S*N.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense FP8 MFMA, published
H100_DEEPGEMM_DECODE_TFLOPS = 243.6  # benchmark post, section 3.2, m=64 n=7168 k=18432 (context)
GRAPH_RUN_STEPS = 40          # steps per captured graph (rounded to whole weight rotations)
SETTLE_MS = 40.0              # GPU time run before timing a long launch (clock settling)
SHORT_LAUNCH_MS = 0.05        # launches shorter than this are timed behind a spin kernel
SETTLE_MAX_LAUNCHES = 400


# ----------------------------------------------------------------------------- metrics

def gemm_flops(M, N, K):
    return 2.0 * M * N * K


def gemm_bytes(M, N, K):
    return float(M * K + N * K + 2 * M * N)


def masked_flops(S, N, K):
    return 2.0 * S * N * K


def masked_bytes(S, E_active, N, K):
    return float(S * K + E_active * N * K + 2 * S * N)


def quant_bytes(M, K):
    W = (K // 128 + 3) // 4
    return float(2 * M * K + M * K + 4 * W * M)


def silu_bytes(S, H):
    W = (H // 128 + 3) // 4
    return float(4 * H * S + H * S + 4 * W * S)


# ----------------------------------------------------------------------------- inputs (device)

def _gen(seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return g


def randn_bf16(shape, std=1.0, seed=0):
    return (torch.randn(shape, generator=_gen(seed), device="cuda", dtype=torch.float32) * std).to(torch.bfloat16)


def randn_bf16_outliers(shape, seed=0, frac=0.01, factor=50.0):
    v = torch.randn(shape, generator=_gen(seed), device="cuda", dtype=torch.float32)
    mask = torch.rand(shape, generator=_gen(seed + 7919), device="cuda") < frac
    return torch.where(mask, v * factor, v).to(torch.bfloat16)


def quantized_weights(F, n_copies, N, K, seed, experts=1):
    """Weight copies quantized on the GPU with the 128x128 block quant kernel."""
    out = []
    for c in range(n_copies):
        qs, ss = [], []
        for e in range(experts):
            w = randn_bf16((N, K), std=0.02, seed=seed + 1000 * c + e)
            q, s = F.fp8_block_quant_128x128(w)
            del w
            qs.append(q)
            ss.append(s)
        if experts == 1:
            out.append((qs[0], ss[0]))
        else:
            out.append((torch.stack(qs), torch.stack(ss)))
        del qs, ss
    torch.cuda.synchronize()
    return out


def n_copies_for(bytes_per_copy, cache_bytes=256 << 20, floor=1):
    """Enough rotating copies that the working set exceeds the last-level cache twice."""
    n = int(np.ceil(2 * cache_bytes / max(bytes_per_copy, 1)))
    return max(floor, min(n, 16))


# ----------------------------------------------------------------------------- timing

def kernel_times(stream, launches, steps, settle_ms=SETTLE_MS):
    """Average GPU duration of each launch type, in ms: `steps` back-to-back calls of
    one launch between two HIP events recorded on the launch stream.

    Launches shorter than SHORT_LAUNCH_MS are queued behind a spin kernel, so that
    they run back to back although the host enqueues them more slowly than they run.
    Longer launches (the prefill and MoE GEMMs, which the host easily stays ahead of)
    first run back to back for at least `settle_ms` of GPU time, queued together with
    the timed calls: the clock of a GPU that starts from idle boosts, then drops under
    the power limit for a few launches of an MFMA-bound kernel before it settles, and
    the figure wanted is the settled one."""
    out = []
    for fn in launches:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for s in range(3):
                fn(s)
            e1.record(stream)
        stream.synchronize()
        t_est = e0.elapsed_time(e1) / 3
        with torch.cuda.stream(stream):
            if t_est < SHORT_LAUNCH_MS:
                torch.cuda._sleep(int(2e7))
            else:
                for s in range(int(min(SETTLE_MAX_LAUNCHES, np.ceil(settle_ms / t_est)))):
                    fn(s)
            e0.record(stream)
            for s in range(steps):
                fn(s)
            e1.record(stream)
        stream.synchronize()
        out.append(e0.elapsed_time(e1) / steps)
    return out


def kernel_time_stats(stream, fn, batches=11, per_batch=10, settle_ms=SETTLE_MS):
    """Per-call GPU time of one launch type as (mean, p10, median, p90) in ms: `batches`
    batches of `per_batch` back-to-back calls, each batch between two HIP events on the
    launch stream, queued behind a spin kernel (short calls) or after >= settle_ms of the
    same call (long ones, so that the clock has settled), as kernel_times does; the
    percentiles are over the batch means."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for s in range(3):
            fn(s)
        e1.record(stream)
    stream.synchronize()
    t_est = e0.elapsed_time(e1) / 3
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(batches + 1)]
    with torch.cuda.stream(stream):
        if t_est < SHORT_LAUNCH_MS:
            torch.cuda._sleep(int(2e7))
        else:
            for s in range(int(min(SETTLE_MAX_LAUNCHES, np.ceil(settle_ms / t_est)))):
                fn(s)
        evs[0].record(stream)
        for b in range(batches):
            for s in range(per_batch):
                fn(b * per_batch + s)
            evs[b + 1].record(stream)
    stream.synchronize()
    per = np.array([evs[b].elapsed_time(evs[b + 1]) / per_batch for b in range(batches)])
    total = evs[0].elapsed_time(evs[batches]) / (batches * per_batch)
    return total, float(np.percentile(per, 10)), float(np.median(per)), float(np.percentile(per, 90))


def graph_step_time(stream, step_fn, n_variants, steps, warmup):
    """Wall ms per step over exactly `steps` steps, with synchronizations on both
    sides of the timed loop.  Steps are replayed from HIP graphs that each hold a run
    of consecutive steps over the rotating input variants (one graph of `per_graph`
    steps -- whole rotations, about 40 steps -- replayed steps // per_graph times, plus
    one graph holding the remaining steps), so the host cost of a graph launch (about
    13 us between two replays, measured) is paid once per run of steps rather than
    once per step, as in a serving loop that queues many steps."""
    per_graph = n_variants * max(1, GRAPH_RUN_STEPS // n_variants)
    with torch.cuda.stream(stream):
        for _ in range(2):
            for v in range(n_variants):
                step_fn(v)
    stream.synchronize()

    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for v in range(n):
                step_fn(v)
        return g

    full = capture(per_graph)
    rest = steps % per_graph
    tail = capture(rest) if rest else None
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        full.replay()
        e1.record(stream)
    stream.synchronize()
    n_warm = max(1, warmup // per_graph, int(np.ceil(SETTLE_MS / max(e0.elapsed_time(e1), 1e-3))))
    with torch.cuda.stream(stream):
        for i in range(min(n_warm, SETTLE_MAX_LAUNCHES)):
            full.replay()
        if tail is not None:
            tail.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for i in range(steps // per_graph):
            full.replay()
        if tail is not None:
            tail.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) * 1e3 / steps


# ----------------------------------------------------------------------------- workloads

def setup_dense(F, M, N, K, outliers, seed=0):
    a = randn_bf16_outliers((M, K), seed=seed) if outliers else randn_bf16((M, K), seed=seed)
    copies = quantized_weights(F, n_copies_for(N * K), N, K, seed + 1)
    qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sfa = torch.empty(((K // 128 + 3) // 4, max(4, (M + 3) // 4 * 4)), dtype=torch.int32, device="cuda")
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    return a, copies, qa, sfa, c


def bf16_dev(bits):
    """numpy uint16 bf16 bit patterns -> device bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def rotated_copies(qb0, sfb0, n, dim=0):
    """n weight copies for HBM-cold timing: copy 0 is the weight itself, copy c its 128-row
    blocks rotated by 11c blocks along `dim` (the same quantized weight set in another row
    order, scales rotated with their blocks)."""
    nb = sfb0.shape[dim]
    out = [(qb0, sfb0)]
    for c in range(1, n):
        sh = (11 * c) % nb if nb > 1 else 0
        out.append((torch.roll(qb0, 128 * sh, dim) if sh else qb0.clone(),
                    torch.roll(sfb0, sh, dim) if sh else sfb0.clone()))
    torch.cuda.synchronize()
    return out


def setup_dense_parity(F, host, shape):
    """The dense workload on the parity tests' own tensors: A and B as the seeded input
    generators draw them (host = (A bits, B bits), seed 0: the tensors the GPU parity tests
    compare with the oracle), B block-quantized on the GPU (bit-exact with the oracle's block
    quant), and rotated copies of it (rotated_copies) that keep every timed call HBM-cold."""
    M, N, K = shape.M, shape.N, shape.K
    a_np, b_np = host
    a = bf16_dev(a_np)
    b = bf16_dev(b_np)
    qb0, sfb0 = F.fp8_block_quant_128x128(b)
    del b
    copies = rotated_copies(qb0, sfb0, n_copies_for(N * K))
    qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sfa = torch.empty(((K // 128 + 3) // 4, max(4, (M + 3) // 4 * 4)), dtype=torch.int32, device="cuda")
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    return a, copies, qa, sfa, c


def bench_dense(F, stream, shape, steps, warmup, preshuffled=False, hot=False, host=None, stats=False,
                keep_out=True):
    """The dense step: quant/pack of A, then the GEMM.  preshuffled: the weight copies
    are put into the pre-shuffled layout once, outside timing (offline weight
    preparation, like the quantization), and fp8_block_gemm_nt_preshuffled runs.
    host: (A bits, B bits) from the seeded generators, to time the parity tests' own
    tensors; the result then carries the output of one step on weight copy 0."""
    M, N, K = shape.M, shape.N, shape.K
    if host is not None:
        a, copies, qa, sfa, c = setup_dense_parity(F, host, shape)
    else:
        a, copies, qa, sfa, c = setup_dense(F, M, N, K, shape.outliers)
    if preshuffled:
        copies = [(F.fp8_weight_preshuffle(qb), sfb) for qb, sfb in copies]
        torch.cuda.synchronize()
    nv = len(copies)
    gemm_fn = F.fp8_block_gemm_nt_preshuffled if preshuffled else F.fp8_block_gemm_nt

    def quant(s):
        F.fp8_quant_group_pack(a, q=qa, sf=sfa, stream=stream)

    def gemm(s):
        qb, sfb = copies[s % nv]
        gemm_fn(qa, sfa, qb, sfb, c=c, stream=stream)

    def step(v):
        quant(v)
        gemm(v)

    def gemm_hot(s):  # one weight copy every call: served from the last-level cache
        qb, sfb = copies[0]
        gemm_fn(qa, sfa, qb, sfb, c=c, stream=stream)

    with torch.cuda.stream(stream):
        for i in range(warmup):
            step(i)
    t_quant, t_gemm = kernel_times(stream, [quant, gemm], steps)
    t_hot = kernel_times(stream, [gemm_hot], steps)[0] if hot else None
    st = kernel_time_stats(stream, gemm, per_batch=max(2, steps // 10)) if stats else None
    ms = graph_step_time(stream, step, nv, steps, warmup)
    out0 = None
    if host is not None and keep_out:
        with torch.cuda.stream(stream):
            quant(0)
            gemm(0)
        stream.synchronize()
        out0 = c.view(torch.int16).cpu().numpy().view(np.uint16).copy()
    r = {
        "workload": shape.name + ("_preshuffled" if preshuffled else ""), "M": M, "N": N, "K": K,
        "ms_per_step": ms,
        "step_tflops": gemm_flops(M, N, K) / (ms * 1e-3) / 1e12,
        "quant_us": t_quant * 1e3, "gemm_us": t_gemm * 1e3, "gemm_us_hot": None if t_hot is None else t_hot * 1e3,
        "gemm_tflops": gemm_flops(M, N, K) / (t_gemm * 1e-3) / 1e12,
        "gemm_gbs": gemm_bytes(M, N, K) / (t_gemm * 1e-3) / 1e9,
        "quant_gbs": quant_bytes(M, K) / (t_quant * 1e-3) / 1e9,
        "config": F.gemm_config(F.LAYOUT_DENSE_PRESHUFFLED if preshuffled else F.LAYOUT_DENSE, M, N, K),
        "weight_copies": nv,
    }
    r["frac_hbm"] = r["gemm_gbs"] / HBM_PEAK_GBS
    r["frac_mfma"] = r["gemm_tflops"] / FP8_PEAK_TFLOPS
    if st is not None:
        r["gemm_us_p10"], r["gemm_us_median"], r["gemm_us_p90"] = st[1] * 1e3, st[2] * 1e3, st[3] * 1e3
    if out0 is not None:
        r["_out0"] = out0
    del a, copies, qa, sfa, c
    return r


def bench_dense_float(F, stream, shape, steps, warmup, preshuffled=False):
    """The dense step in the float-scale (non-UE8M0) format: activation quant with fp32
    group scales, weights block-quantized with fp32 scales, the float-scale GEMM."""
    M, N, K = shape.M, shape.N, shape.K
    a = randn_bf16_outliers((M, K), seed=0) if shape.outliers else randn_bf16((M, K), seed=0)
    copies = []
    for c in range(n_copies_for(N * K)):
        w = randn_bf16((N, K), std=0.02, seed=1 + 1000 * c)
        copies.append(F.fp8_block_quant_128x128_float(w))
        del w
    torch.cuda.synchronize()
    if preshuffled:
        copies = [(F.fp8_weight_preshuffle(qb), sfb) for qb, sfb in copies]
        torch.cuda.synchronize()
    nv = len(copies)
    qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sfa = torch.empty((K // 128, max(4, (M + 3) // 4 * 4)), dtype=torch.float32, device="cuda")
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def quant(s):
        F.fp8_quant_group_float(a, q=qa, sf=sfa, stream=stream)

    def gemm(s):
        qb, sfb = copies[s % nv]
        F.fp8_block_gemm_nt_float_scales(qa, sfa, qb, sfb, c=c, stream=stream, preshuffled=preshuffled)

    with torch.cuda.stream(stream):
        for i in range(warmup):
            quant(i)
            gemm(i)
    t_quant, t_gemm = kernel_times(stream, [quant, gemm], steps)
    r = {"workload": shape.name.replace("dense_", "dense_float_scales_") + ("_preshuffled" if preshuffled else ""),
         "M": M, "N": N, "K": K,
         "quant_us": t_quant * 1e3, "gemm_us": t_gemm * 1e3,
         "gemm_tflops": gemm_flops(M, N, K) / (t_gemm * 1e-3) / 1e12,
         "gemm_gbs": gemm_bytes(M, N, K) / (t_gemm * 1e-3) / 1e9,
         "config": F.gemm_config(F.LAYOUT_DENSE_FLOAT_PRESHUFFLED if preshuffled else F.LAYOUT_DENSE_FLOAT, M, N, K),
         "weight_copies": nv}
    r["frac_hbm"] = r["gemm_gbs"] / HBM_PEAK_GBS
    r["frac_mfma"] = r["gemm_tflops"] / FP8_PEAK_TFLOPS
    del a, copies, qa, sfa, c
    return r


def _preshuffle_copies(F, copies):
    """Weight copies in the pre-shuffled layout (offline, outside timing)."""
    out = [(F.fp8_weight_preshuffle(qb), sfb) for qb, sfb in copies]
    torch.cuda.synchronize()
    return out


def expert_weights(F, W, E, N, K):
    """Per-expert weights [E, N, K] from N(0, 0.02) (seed 0, tensor id T_B: the masked
    parity tests' weights), block-quantized on the GPU one expert at a time."""
    w = W.normal_bf16((E * N, K), std=0.02, seed=0, tensor_id=W.T_B)
    qb = torch.empty((E, N, K), dtype=torch.uint8, device="cuda")
    sfb = torch.empty((E, (N + 127) // 128, K // 128), dtype=torch.float32, device="cuda")
    for e in range(E):
        q, s = F.fp8_block_quant_128x128(bf16_dev(w[e * N:(e + 1) * N]))
        qb[e].copy_(q)
        sfb[e].copy_(s)
    del w
    torch.cuda.synchronize()
    return qb, sfb


def bench_masked_gate_up(F, W, stream, steps, warmup, preshuffled=False):
    E, M_max, N, K = W.MOE_E, W.MOE_M_MAX, W.MOE_GATE_UP["N"], W.MOE_GATE_UP["K"]
    counts = torch.from_numpy(W.zipf_counts()).to("cuda")
    S = int(counts.clamp(0, M_max).sum())
    E_active = int((counts > 0).sum())
    # the masked parity test's tensors: x and w from the seeded generators (seed 0)
    x = bf16_dev(W.normal_bf16((E * M_max, K), seed=0))
    qa, sfa_flat = F.fp8_quant_group_pack(x, ld_sf=E * M_max)
    Wd = (K // 128 + 3) // 4
    a = qa.view(E, M_max, K)
    sfa = sfa_flat.view(Wd, E, M_max).permute(1, 0, 2).contiguous()
    del x
    copies = rotated_copies(*expert_weights(F, W, E, N, K), n_copies_for(E * N * K, floor=1), dim=1)
    if preshuffled:
        copies = _preshuffle_copies(F, copies)
    nv = len(copies)
    c = torch.empty((E, M_max, N), dtype=torch.bfloat16, device="cuda")

    def gemm(s):
        qb, sfb = copies[s % nv]
        F.fp8_block_gemm_grouped_masked(a, sfa, qb, sfb, counts, c=c, stream=stream, preshuffled=preshuffled)

    with torch.cuda.stream(stream):
        for i in range(warmup):
            gemm(i)
    (t,) = kernel_times(stream, [gemm], steps)
    st = kernel_time_stats(stream, gemm, per_batch=max(2, steps // 10))
    r = {"workload": "moe_gate_up_masked_E32_Mmax256_N4096_K7168" + ("_preshuffled" if preshuffled else ""),
         "gemm_us_p10": st[1] * 1e3, "gemm_us_median": st[2] * 1e3, "gemm_us_p90": st[3] * 1e3,
         "S": S, "E_active": E_active,
         "gemm_us": t * 1e3, "gemm_tflops": masked_flops(S, N, K) / (t * 1e-3) / 1e12,
         "gemm_gbs": masked_bytes(S, E_active, N, K) / (t * 1e-3) / 1e9, "weight_copies": nv,
         "config": F.gemm_config(F.LAYOUT_MASKED_PRESHUFFLED if preshuffled else F.LAYOUT_MASKED, M_max, N, K)}
    r["frac_hbm"] = r["gemm_gbs"] / HBM_PEAK_GBS
    r["frac_mfma"] = r["gemm_tflops"] / FP8_PEAK_TFLOPS
    del copies, a, sfa, c
    return r


def bench_contiguous_gate_up(F, W, stream, steps, warmup):
    """The gate_up workload in the contiguous grouped layout: the Zipf counts' rows in
    128-row runs per expert (padding rows included in the launch, skipped blocks none)."""
    E, N, K = W.MOE_E, W.MOE_GATE_UP["N"], W.MOE_GATE_UP["K"]
    counts_np = W.zipf_counts()
    S = int(counts_np.sum())
    E_active = int((counts_np > 0).sum())
    mi_np = W.contiguous_layout(counts_np)
    M = len(mi_np)
    m_indices = torch.from_numpy(mi_np).to("cuda")
    x = randn_bf16((M, K), seed=13)
    qa, sfa = F.fp8_quant_group_pack(x)
    del x
    copies = quantized_weights(F, n_copies_for(E * N * K, floor=1), N, K, 23, experts=E)
    nv = len(copies)
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def gemm(s):
        qb, sfb = copies[s % nv]
        F.fp8_block_gemm_grouped_contiguous(qa, sfa, qb, sfb, m_indices, c=c, stream=stream)

    with torch.cuda.stream(stream):
        for i in range(warmup):
            gemm(i)
    (t,) = kernel_times(stream, [gemm], steps)
    r = {"workload": "moe_gate_up_contiguous_E32_N4096_K7168", "S": S, "M_rows": M, "E_active": E_active,
         "gemm_us": t * 1e3, "gemm_tflops": masked_flops(S, N, K) / (t * 1e-3) / 1e12,
         "gemm_gbs": masked_bytes(S, E_active, N, K) / (t * 1e-3) / 1e9, "weight_copies": nv,
         "config": F.gemm_config(2, M, N, K)}
    r["frac_hbm"] = r["gemm_gbs"] / HBM_PEAK_GBS
    r["frac_mfma"] = r["gemm_tflops"] / FP8_PEAK_TFLOPS
    del copies, qa, sfa, c, m_indices
    return r


def bench_dispatch_quant(F, W, stream, steps, warmup):
    """Per-token quant into the masked expert layout of routed tokens: 512 tokens x
    top-8 of 32 experts (Zipf(1.1) weights), capacity 256, K = 7168."""
    E, M_max, K = W.MOE_E, W.MOE_M_MAX, W.MOE_GATE_UP["K"]
    ids_np = W.topk_routing()
    T, topk = ids_np.shape
    ids = torch.from_numpy(ids_np).to("cuda")
    x = randn_bf16((T, K), seed=17)
    Wd = (K // 128 + 3) // 4
    q = torch.empty((E, M_max, K), dtype=torch.uint8, device="cuda")
    sf = torch.empty((E, Wd, M_max), dtype=torch.int32, device="cuda")
    mm = torch.empty((E,), dtype=torch.int32, device="cuda")
    slot = torch.empty((T, topk), dtype=torch.int32, device="cuda")

    def op(s):
        F.fp8_quant_group_pack_to_experts(x, ids, E, M_max, q=q, sf=sf, masked_m=mm, slot_of=slot, stream=stream)

    with torch.cuda.stream(stream):
        for i in range(warmup):
            op(i)
    (t,) = kernel_times(stream, [op], steps)
    rows = int(mm.clamp(0, M_max).sum())
    # algorithmic bytes: bf16 tokens read once, e4m3 rows + scale words written per routed
    # pair, ids read and slots written
    nbytes = 2 * T * K + rows * (K + 4 * Wd) + 8 * T * topk + 4 * E
    r = {"workload": "moe_dispatch_quant_T512_top8_E32_Mmax256_K7168", "rows_written": rows,
         "op_us": t * 1e3, "op_gbs": nbytes / (t * 1e-3) / 1e9}
    r["frac_hbm"] = r["op_gbs"] / HBM_PEAK_GBS
    r["frac_mfma"] = 0.0
    del x, q, sf, mm, slot, ids
    return r


def bench_silu_down(F, W, stream, steps, warmup, preshuffled=False):
    E, M_max, H, N = W.MOE_E, W.MOE_M_MAX, W.MOE_DOWN["H"], W.MOE_DOWN["N"]
    K = H
    counts = torch.from_numpy(W.zipf_counts()).to("cuda")
    S = int(counts.clamp(0, M_max).sum())
    E_active = int((counts > 0).sum())
    # the SiLU -> down parity test's tensors (seed 0)
    x = bf16_dev(W.normal_bf16((E, M_max, 2 * H), seed=0, tensor_id=W.T_X))
    copies = rotated_copies(*expert_weights(F, W, E, N, K), n_copies_for(E * N * K, floor=1), dim=1)
    if preshuffled:
        copies = _preshuffle_copies(F, copies)
    nv = len(copies)
    q = torch.empty((E, M_max, H), dtype=torch.uint8, device="cuda")
    sf = torch.empty((E, (H // 128 + 3) // 4, M_max), dtype=torch.int32, device="cuda")
    c = torch.empty((E, M_max, N), dtype=torch.bfloat16, device="cuda")

    def silu(s):
        F.silu_mul_quant_group_pack(x, counts, q=q, sf=sf, stream=stream)

    def gemm(s):
        qb, sfb = copies[s % nv]
        F.fp8_block_gemm_grouped_masked(q, sf, qb, sfb, counts, c=c, stream=stream, preshuffled=preshuffled)

    with torch.cuda.stream(stream):
        for i in range(warmup):
            silu(i)
            gemm(i)
    t_silu, t_gemm = kernel_times(stream, [silu, gemm], steps)
    st_s = kernel_time_stats(stream, silu, per_batch=max(2, steps // 10))
    st_g = kernel_time_stats(stream, gemm, per_batch=max(2, steps // 10))
    r = {"workload": "moe_silu_quant_then_down_masked_E32_Mmax256_H2048_N7168" + ("_preshuffled" if preshuffled else ""),
         "silu_us_p10": st_s[1] * 1e3, "silu_us_median": st_s[2] * 1e3, "silu_us_p90": st_s[3] * 1e3,
         "gemm_us_p10": st_g[1] * 1e3, "gemm_us_median": st_g[2] * 1e3, "gemm_us_p90": st_g[3] * 1e3,
         "S": S, "config": F.gemm_config(F.LAYOUT_MASKED_PRESHUFFLED if preshuffled else F.LAYOUT_MASKED, M_max, N, K),
         "silu_us": t_silu * 1e3, "silu_gbs": silu_bytes(S, H) / (t_silu * 1e-3) / 1e9,
         "gemm_us": t_gemm * 1e3, "gemm_tflops": masked_flops(S, N, K) / (t_gemm * 1e-3) / 1e12,
         "gemm_gbs": masked_bytes(S, E_active, N, K) / (t_gemm * 1e-3) / 1e9, "weight_copies": nv}
    r["frac_hbm"] = r["gemm_gbs"] / HBM_PEAK_GBS
    r["frac_mfma"] = r["gemm_tflops"] / FP8_PEAK_TFLOPS
    del copies, x, q, sf, c
    return r


# ----------------------------------------------------------------------------- CPU baseline

def cpu_model():
    """The host CPU's model name, as /proc/cpuinfo (and lscpu) report it."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def _timed_reps(fn, budget_s, max_reps):
    """Run fn at least once and until budget_s of its own time has passed; (reps, seconds,
    last result)."""
    reps, t, out = 0, 0.0, None
    while reps == 0 or (t < budget_s and reps < max_reps):
        t0 = time.perf_counter()
        out = fn()
        t += time.perf_counter() - t0
        reps += 1
    return reps, t, out


def cpu_baseline(W, shape, host, budget_s):
    """The oracle (as it stands) running the headline step -- quant/pack of all M rows of
    A, then the block-scaled GEMM accumulated in double -- on the same host tensors the GPU
    step timed, the whole step repeated for about budget_s; plus single-thread figures for
    the small dense case and for the SiLU-mul-quant kernel.  Returns the baseline object
    and the oracle's output of the step (for the parity check of the timed GPU call)."""
    import oracle as O
    M, N, K = shape.M, shape.N, shape.K
    a, b = host
    qb, sfb = O.block_quant_128x128(b)  # offline weight step, as on the GPU: not timed

    def step():
        qa, sfa = O.quant_group_pack(a)
        return O.gemm_nt(qa, sfa, qb, sfb)

    cores = O.num_threads()
    reps, t, ref = _timed_reps(step, budget_s, 64)
    res = {"value": reps * gemm_flops(M, N, K) / t / 1e12, "unit": "TFLOPS", "cores": cores, "kind": "oracle",
           "cpu_model": cpu_model(), "step_ms": t / reps * 1e3,
           "sample": "the whole %dx%dx%d step (quant/pack of all %d rows + double-accumulated block GEMM, "
                     "%d distinct outputs) run %d times on the timed tensors; %.1f s"
                     % (M, N, K, M, M * N, reps, t)}
    single = {}
    O.set_num_threads(1)
    try:
        s1 = W.DENSE_SMALL
        a1, b1 = W.dense_inputs(s1)
        qb1, sfb1 = O.block_quant_128x128(b1)

        def small():
            qa1, sfa1 = O.quant_group_pack(a1)
            return O.gemm_nt(qa1, sfa1, qb1, sfb1)

        n1, t1, _ = _timed_reps(small, 2.0, 10000)
        single[s1.name + "_step"] = {"us": t1 / n1 * 1e6, "tflops": n1 * gemm_flops(s1.M, s1.N, s1.K) / t1 / 1e12,
                                     "reps": n1}
        E, M_max, H = W.MOE_E, W.MOE_M_MAX, W.MOE_DOWN["H"]
        x = W.normal_bf16((E, M_max, 2 * H), seed=0, tensor_id=W.T_X)
        counts = W.zipf_counts()
        S = int(np.minimum(np.maximum(counts, 0), M_max).sum())
        n2, t2, _ = _timed_reps(lambda: O.silu_mul_quant_group_pack(x, counts), 3.0, 100)
        single["silu_mul_quant_group_pack_E%d_Mmax%d_H%d" % (E, M_max, H)] = {
            "us": t2 / n2 * 1e6, "gbs": silu_bytes(S, H) / (t2 / n2) / 1e9, "valid_rows": S, "reps": n2}
    finally:
        O.set_num_threads(cores)
    res["single_thread"] = single
    return res, ref


def parity_check(c_bits, ref):
    """The timed GPU call's output against the oracle's, element by element:
    |c - ref| <= 1e-2 |ref| + 1e-2 rms(ref), and calc_diff (1 - 2 sum(c ref) / sum(c^2 + ref^2))."""
    import oracle as O
    import workloads as W
    c = W.bf16_bits_to_f32(c_bits).astype(np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    bound = 1e-2 * np.abs(ref) + 1e-2 * rms
    err = np.abs(c - ref)
    ok = bool(np.all(err <= bound))
    return {"elements": int(ref.size), "within_tolerance": ok,
            "outside": int(np.sum(~(err <= bound))),
            "max_err_over_bound": float(np.max(err / bound)), "calc_diff": float(O.calc_diff(c, ref)),
            "against": "oracle output of the same step on weight copy 0 (cpu_baseline leg)"}


# ----------------------------------------------------------------------------- main

KERNEL_NAMES = {56: "wsd_kernel: pre-shuffled weight streaming, split-K partials summed in the kernel by the "
                    "last-arriving workgroup of each split group, one launch"}


RIDGE_FLOP_PER_BYTE = FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)  # 625: MFMA-bound above


def sub_object(r, bound_flops=None):
    """Per-workload figures for the JSON line: mean and p10/median/p90 per call, TFLOPS,
    GB/s and the roofline fraction, against the FP8 MFMA peak when the workload's
    arithmetic intensity (algorithmic flops per algorithmic HBM byte) is above the ridge
    point, else against HBM bandwidth (bound_flops forces one)."""
    if bound_flops is None:
        bound_flops = r["gemm_tflops"] * 1e3 / r["gemm_gbs"] > RIDGE_FLOP_PER_BYTE
    o = {"gemm_us": round(r["gemm_us"], 2)}
    for q in ("p10", "median", "p90"):
        if "gemm_us_" + q in r:
            o["gemm_us_" + q] = round(r["gemm_us_" + q], 2)
    o["gemm_tflops"] = round(r["gemm_tflops"], 1)
    o["gemm_gbs"] = round(r["gemm_gbs"], 1)
    if bound_flops:
        o["roofline"] = {"bound": "mfma", "achieved": round(r["gemm_tflops"], 1), "peak": FP8_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(r["gemm_tflops"] / FP8_PEAK_TFLOPS, 4)}
    else:
        o["roofline"] = {"bound": "hbm", "achieved": round(r["gemm_gbs"], 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(r["gemm_gbs"] / HBM_PEAK_GBS, 4)}
    o["frac_mfma"] = round(r["frac_mfma"], 4)
    o["frac_hbm"] = round(r["frac_hbm"], 4)
    o["tile"] = r["config"]
    o["weight_copies"] = r["weight_copies"]
    return o


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sweep", action="store_true", help="also time every other workload, table on stderr")
    ap.add_argument("--sweep-out", default=None, help="file for per-workload JSON lines")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-targets", action="store_true",
                    help="skip the prefill and MoE sub-objects (headline only)")
    ap.add_argument("--no-hot", action="store_true",
                    help="skip the warm-cache GEMM timing (kernel traces then hold cold-cache calls only)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic_decode_gemm.json"),
                    help="HBM traffic per GEMM launch measured with rocprofv3 counters")
    ap.add_argument("--counters", action="store_true",
                    help="workload for rocprofv3 --pmc passes: a 256 MiB torch copy (counter calibration), "
                         "then --steps eager steps of --counters-shape; no timing")
    ap.add_argument("--counters-shape", default="decode",
                    help="decode: M=64 N=7168 K=18432 with pre-shuffled weights (the headline step); "
                         "decode_plain: the same with weights [N][K]; prefill: M=4096 N=4096 K=7168 "
                         "(pre-shuffled weights, as for every prefill shape name); "
                         "masked: the MoE gate_up GEMM; scale_ablation: UE8M0 in the MFMA against "
                         "unscaled MFMA + VALU scale at 1024x4096x7168; or a prefill shape name such as "
                         "dense_prefill_2048x4096x7168")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print("bench.py measures one GPU: this library runs on a single MI355X (no sharding, no "
                  "collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import block_scaled_fp8_token_amd as F
    import workloads as W

    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    shape = W.DENSE_DECODE
    if args.counters:
        named = {s.name: s for s in W.DENSE_PREFILL}
        if args.counters_shape == "masked":
            counters_masked_workload(F, W, args.steps)
        elif args.counters_shape == "scale_ablation":
            counters_scale_ablation_workload(F, W, args.steps)
        elif args.counters_shape == "prefill":
            counters_workload(F, W.DENSE_PREFILL[2], args.steps, preshuffled=True)
        elif args.counters_shape in named:
            counters_workload(F, named[args.counters_shape], args.steps, preshuffled=True)
        elif args.counters_shape in ("decode", "decode_plain"):
            counters_workload(F, shape, args.steps, preshuffled=args.counters_shape == "decode")
        else:
            ap.error("unknown --counters-shape %s" % args.counters_shape)
        return
    host = W.dense_inputs(shape)
    r = bench_dense(F, stream, shape, args.steps, args.warmup, preshuffled=True, hot=not args.no_hot, host=host,
                    stats=True)
    out0 = r.pop("_out0")
    print("[bench] %s" % json.dumps(r), file=sys.stderr, flush=True)
    plain = bench_dense(F, stream, shape, args.steps, args.warmup, hot=not args.no_hot, host=host, stats=True)
    plain.pop("_out0", None)
    print("[bench] %s" % json.dumps(plain), file=sys.stderr, flush=True)

    traffic = None
    if args.traffic_json and os.path.exists(args.traffic_json):
        try:
            t = json.load(open(args.traffic_json))
            if t.get("kernel_source_hash") == _kernel_hash():
                traffic = t.get("bytes_per_launch")
        except (OSError, ValueError):
            traffic = None

    gb = gemm_bytes(shape.M, shape.N, shape.K)
    kname = KERNEL_NAMES.get(r["config"]["kernel"], "table entry %d" % r["config"]["kernel"])
    line = {
        "metric": "TFLOPS and HBM GB/s per (M,N,K) shape; % of FP8 MFMA / HBM roofline",
        "value": round(r["step_tflops"], 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(r["step_tflops"] / H100_DEEPGEMM_DECODE_TFLOPS, 3),
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": "dense_decode_gemm_M64_N7168_K18432", "M": shape.M, "N": shape.N,
                   "K": shape.K, "step": "fp8_quant_group_pack(A) + fp8_block_gemm_nt_preshuffled",
                   "inputs": "the parity tests' seeded tensors (A N(0,1) with 1% x50 outliers, B N(0,0.02)), "
                             "seed 0",
                   "weights": "e4m3 + 128x128 UE8M0 block scales, pre-shuffled offline (byte permutation, "
                              "outside timing like the quantization), %d rotating copies (row-block rotations "
                              "of the one weight set, HBM-cold)" % r["weight_copies"],
                   "tile": r["config"]},
        "gemm_us": round(r["gemm_us"], 2),
        "gemm_us_p10": round(r["gemm_us_p10"], 2),
        "gemm_us_median": round(r["gemm_us_median"], 2),
        "gemm_us_p90": round(r["gemm_us_p90"], 2),
        "gemm_gbs": round(r["gemm_gbs"], 1),
        "gemm_tflops": round(r["gemm_tflops"], 2),
        "quant_us": round(r["quant_us"], 2),
        "gemm_us_hot": None if r["gemm_us_hot"] is None else round(r["gemm_us_hot"], 2),
        "roofline": {"bound": "hbm",
                     "kernel": "fp8_block_gemm_nt_preshuffled (%s)" % kname,
                     "achieved": round(r["gemm_gbs"], 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(r["gemm_gbs"] / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes_per_launch": gb, "traffic": traffic},
        "plain_layout": {"step": "fp8_quant_group_pack(A) + fp8_block_gemm_nt (weights [N][K] as quantized)",
                         "ms_per_step": round(plain["ms_per_step"], 5),
                         "step_tflops": round(plain["step_tflops"], 2),
                         "gemm_us_hot": None if plain["gemm_us_hot"] is None else round(plain["gemm_us_hot"], 2),
                         **sub_object(plain, bound_flops=False)},
    }
    target_rows = []
    if not args.no_targets:
        pre_steps = max(10, args.steps // 4)
        # prefill: weights pre-shuffled offline, as for the headline step (the ring tiles
        # then move one contiguous kilobyte per weight DMA instruction); the plain layout
        # timed beside it
        prefill = {}
        for s in W.DENSE_PREFILL:
            host_s = W.dense_inputs(s)
            x = bench_dense(F, stream, s, pre_steps, args.warmup, preshuffled=True, host=host_s, stats=True,
                            keep_out=False)
            xp = bench_dense(F, stream, s, pre_steps, args.warmup, host=host_s, keep_out=False)
            target_rows += [x, xp]
            print("[bench] %s" % json.dumps(x), file=sys.stderr, flush=True)
            print("[bench] %s" % json.dumps(xp), file=sys.stderr, flush=True)
            o = {"weights": "pre-shuffled", **sub_object(x)}
            o["target_us_60pct_mfma"] = round(gemm_flops(s.M, s.N, s.K) / (0.6 * FP8_PEAK_TFLOPS * 1e12) * 1e6, 1)
            o["plain_layout"] = {"gemm_us": round(xp["gemm_us"], 2), "gemm_tflops": round(xp["gemm_tflops"], 1),
                                 "frac_mfma": round(xp["frac_mfma"], 4), "tile": xp["config"]}
            prefill[s.name] = o
        line["prefill"] = prefill
        # MoE: both expert weight sets pre-shuffled offline (as for the dense GEMMs), the
        # plain layout timed beside them
        x = bench_masked_gate_up(F, W, stream, pre_steps, args.warmup, preshuffled=True)
        xp = bench_masked_gate_up(F, W, stream, pre_steps, args.warmup)
        target_rows += [x, xp]
        print("[bench] %s" % json.dumps(x), file=sys.stderr, flush=True)
        print("[bench] %s" % json.dumps(xp), file=sys.stderr, flush=True)
        line["moe_gate_up_masked"] = dict(workload=x["workload"], weights="pre-shuffled", valid_rows=x["S"],
                                          experts_active=x["E_active"], **sub_object(x),
                                          plain_layout={"gemm_us": round(xp["gemm_us"], 2), "tile": xp["config"]})
        x = bench_silu_down(F, W, stream, pre_steps, args.warmup, preshuffled=True)
        xp = bench_silu_down(F, W, stream, pre_steps, args.warmup)
        target_rows += [x, xp]
        print("[bench] %s" % json.dumps(x), file=sys.stderr, flush=True)
        print("[bench] %s" % json.dumps(xp), file=sys.stderr, flush=True)
        o = dict(workload=x["workload"], weights="pre-shuffled", valid_rows=x["S"], **sub_object(x),
                 plain_layout={"gemm_us": round(xp["gemm_us"], 2), "tile": xp["config"]})
        o["silu_us"] = round(x["silu_us"], 2)
        for q in ("p10", "median", "p90"):
            o["silu_us_" + q] = round(x["silu_us_" + q], 2)
        o["silu_gbs"] = round(x["silu_gbs"], 1)
        o["silu_frac_hbm"] = round(x["silu_gbs"] / HBM_PEAK_GBS, 4)
        line["moe_silu_then_down_masked"] = o
    if not args.no_cpu_baseline:
        line["cpu_baseline"], ref = cpu_baseline(W, shape, host, args.cpu_seconds)
        line["parity_check"] = parity_check(out0, ref)

    if args.sweep:
        rows = [r, plain] + target_rows
        rows.append(bench_dense(F, stream, W.DENSE_SMALL, args.steps, args.warmup, host=W.dense_inputs(W.DENSE_SMALL)))
        rows[-1].pop("_out0", None)
        if not target_rows:  # (--no-targets) every prefill and MoE row on both weight layouts
            for s in W.DENSE_PREFILL:
                for pre in (True, False):
                    rows.append(bench_dense(F, stream, s, max(10, args.steps // 4), args.warmup, preshuffled=pre,
                                            host=W.dense_inputs(s), keep_out=False))
                    print("[bench] %s" % json.dumps(rows[-1]), file=sys.stderr, flush=True)
            for pre in (True, False):
                rows.append(bench_masked_gate_up(F, W, stream, max(10, args.steps // 4), args.warmup,
                                                 preshuffled=pre))
                print("[bench] %s" % json.dumps(rows[-1]), file=sys.stderr, flush=True)
                rows.append(bench_silu_down(F, W, stream, max(10, args.steps // 4), args.warmup, preshuffled=pre))
                print("[bench] %s" % json.dumps(rows[-1]), file=sys.stderr, flush=True)
        rows.append(bench_contiguous_gate_up(F, W, stream, max(10, args.steps // 4), args.warmup))
        print("[bench] %s" % json.dumps(rows[-1]), file=sys.stderr, flush=True)
        rows.append(bench_dispatch_quant(F, W, stream, args.steps, args.warmup))
        print("[bench] %s" % json.dumps(rows[-1]), file=sys.stderr, flush=True)
        for fs, pre in ((W.DENSE_DECODE, False), (W.DENSE_DECODE, True), (W.DENSE_PREFILL[0], False),
                        (W.DENSE_PREFILL[1], False), (W.DENSE_PREFILL[2], False), (W.DENSE_PREFILL[4], False)):
            rows.append(bench_dense_float(F, stream, fs, max(10, args.steps // 4), args.warmup, preshuffled=pre))
            print("[bench] %s" % json.dumps(rows[-1]), file=sys.stderr, flush=True)
        print("%-58s %10s %10s %10s %8s %8s" % ("workload", "us", "TFLOPS", "GB/s", "%MFMA", "%HBM"),
              file=sys.stderr)
        for x in rows:
            print("%-58s %10.2f %10.1f %10.1f %8.1f %8.1f" % (x["workload"], x.get("gemm_us", x.get("op_us")),
                                                             x.get("gemm_tflops", 0.0),
                                                             x.get("gemm_gbs", x.get("op_gbs")),
                                                             100 * x["frac_mfma"], 100 * x["frac_hbm"]),
                  file=sys.stderr)
        if args.sweep_out:
            with open(args.sweep_out, "w") as f:
                for x in rows:
                    f.write(json.dumps(x) + "\n")
    print(json.dumps(line), flush=True)
    if "parity_check" in line and not line["parity_check"]["within_tolerance"]:
        print("[bench] the timed call's output is outside the oracle tolerance", file=sys.stderr, flush=True)
        sys.exit(1)


def counters_workload(F, shape, steps, preshuffled=False):
    """Kernels for the counter passes: three copies of 256 MiB (a plain copy kernel of
    known size, to calibrate FETCH_SIZE / WRITE_SIZE), then eager dense steps on the
    timed tensors (pre-shuffled weights, as the headline decode step and the prefill
    sub-objects time them; decode_plain: the plain layout)."""
    x = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    import workloads as W
    a, copies, qa, sfa, c = setup_dense_parity(F, W.dense_inputs(shape), shape)
    if preshuffled:
        copies = [(F.fp8_weight_preshuffle(qb), sfb) for qb, sfb in copies]
    gemm_fn = F.fp8_block_gemm_nt_preshuffled if preshuffled else F.fp8_block_gemm_nt
    for i in range(steps):
        F.fp8_quant_group_pack(a, q=qa, sf=sfa)
        qb, sfb = copies[i % len(copies)]
        gemm_fn(qa, sfa, qb, sfb, c=c)
    torch.cuda.synchronize()
    layout = F.LAYOUT_DENSE_PRESHUFFLED if preshuffled else F.LAYOUT_DENSE
    print(json.dumps({"copy_bytes_each_way": 256 << 20, "steps": steps, "preshuffled": preshuffled,
                      "config": F.gemm_config(layout, shape.M, shape.N, shape.K)}))


def counters_scale_ablation_workload(F, W, steps):
    """Kernels for counter passes on the scale ablation at 1024x4096x7168, where both
    automatic choices are 128x128 full-row ring tiles: --steps calls with UE8M0 scales
    applied inside the MFMA, then --steps calls on the same codes with the same scales
    as fp32 powers of two (float-scale format: unscaled MFMAs, the scale FMA on the
    VALU).  The two outputs are compared bit for bit."""
    x = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    del x, y
    shape = W.DENSE_PREFILL[0]
    M, N, K = shape.M, shape.N, shape.K
    KB = K // 128
    a, copies, qa, sfa, c = setup_dense_parity(F, W.dense_inputs(shape), shape)
    qb, sfb = copies[0]
    F.fp8_quant_group_pack(a, q=qa, sf=sfa)
    wd = sfa.shape[0]
    by = sfa.contiguous().view(torch.uint8).view(wd, sfa.shape[1], 4).permute(0, 2, 1).reshape(4 * wd, sfa.shape[1])[:KB]
    sfa_f = torch.ldexp(torch.ones_like(by, dtype=torch.float32), by.int() - 127).contiguous()
    c2 = torch.empty_like(c)
    for i in range(steps):
        F.fp8_block_gemm_nt(qa, sfa, qb, sfb, c=c)
    torch.cuda.synchronize()
    for i in range(steps):
        F.fp8_block_gemm_nt_float_scales(qa, sfa_f, qb, sfb, c=c2)
    torch.cuda.synchronize()
    same = bool(torch.equal(c.view(torch.int16), c2.view(torch.int16)))
    print(json.dumps({"copy_bytes_each_way": 256 << 20, "steps_per_variant": steps, "outputs_equal": same,
                      "ue8m0_config": F.gemm_config(F.LAYOUT_DENSE, M, N, K),
                      "float_config": F.gemm_config(F.LAYOUT_DENSE_FLOAT, M, N, K)}))


def counters_masked_workload(F, W, steps):
    """Kernels for counter passes on the masked gate_up GEMM on pre-shuffled weights (as
    the bench line times it): the calibration copies, then --steps calls with the Zipf
    counts, --steps with every count halved and --steps with all counts zero (HBM bytes
    should follow the valid rows)."""
    x = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    del x, y
    E, M_max, N, K = W.MOE_E, W.MOE_M_MAX, W.MOE_GATE_UP["N"], W.MOE_GATE_UP["K"]
    zipf = torch.from_numpy(W.zipf_counts()).to("cuda")
    xa = randn_bf16((E * M_max, K), seed=11)
    qa, sfa_flat = F.fp8_quant_group_pack(xa, ld_sf=E * M_max)
    Wd = (K // 128 + 3) // 4
    a = qa.view(E, M_max, K)
    sfa = sfa_flat.view(Wd, E, M_max).permute(1, 0, 2).contiguous()
    del xa
    (qb, sfb), = quantized_weights(F, 1, N, K, 21, experts=E)
    qb = F.fp8_weight_preshuffle(qb)
    c = torch.empty((E, M_max, N), dtype=torch.bfloat16, device="cuda")
    sets = [("zipf", zipf), ("halved", (zipf + 1) // 2), ("zero", torch.zeros_like(zipf))]
    for name, counts in sets:
        for i in range(steps):
            F.fp8_block_gemm_grouped_masked(a, sfa, qb, sfb, counts, c=c, preshuffled=True)
        torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": 256 << 20, "steps_per_set": steps,
                      "sets": {n: {"S": int(cn.sum()), "E_active": int((cn > 0).sum())} for n, cn in sets},
                      "config": F.gemm_config(F.LAYOUT_MASKED_PRESHUFFLED, M_max, N, K)}))


def _kernel_hash():
    """Hash of the code the decode GEMM kernel is built from (the GEMM kernels and the two
    headers they include, without their // comments and blank lines): stored traffic
    counters stay valid until the code changes."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_scaled_fp8_token_amd", "csrc")
    for name in ("fp8bs_device.hpp", "fp8bs_launch.hpp", "gemm_kernels.hip"):
        for line in open(os.path.join(csrc, name), encoding="utf-8"):
            code = line.split("//", 1)[0].strip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
