"""Benchmark: one HSA global iteration on one MI355X.

Workload: Wan-1.3B-shaped stack of 30 bf16 blocks (D 1536, 12 heads x 128,
MLP 8960, C 16 latent channels) over N = 32760 tokens (21 x 30 x 52), three
groups with budgets {40, 20, 10} and 25/25/50% shares.  A step is one call of
hsa_step at an odd iteration (i = 11: only G_1 is active, |A_i| = 8190 = 25%)
with regrouping switched on, so every stage of the hot path runs: select,
active set, gather + embed, 30 x (LN, QKV + K/V scatter, active-query
attention over all 32760 cached rows, out-projection, LN, GELU MLP), unembed,
cached Euler + score.  Inputs (random-init weights, mid-run K/V caches and
sampler state) are generated on the device before timing.

Also measured in the same run: the attention kernel alone (HIP events on its
stream), also at other active fractions, at the 14B-shaped layer and on
all-zero operands (the clock it runs at depends on the operand values), the full
T = 40 sampling loop from fresh latents (also under other schedules and
against dense sampling), iteration time
against the active fraction, the Euler pass on a working set past the
Infinity Cache and over growing working sets, selection over a batch of up
to 8192 videos, the block's four GEMMs alone at three active fractions, one
block's stages (gathered QKV + scatter, attention,
out-projection) at four active fractions and two active-set patterns, the
iteration with the Wan-style block features on (and with
cross-attention and guidance batch 2), attainable peaks (an MFMA-only probe
kernel and a 256 MiB device copy) and the CPU oracle on a bounded sample.

Prints one JSON line.  `value` is HSA iterations per second.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "active-query attn TFLOP/s + HSA iterations/s at N=32760, 25% active (1 GPU)"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
MALL_BYTES = 256 << 20          # Infinity Cache: passes below 4x this are partly cache-resident
# copy probe launch shapes: (16-byte loads per thread in flight, workgroup cap; 0 = uncapped)
COPY_VARIANTS = ((4, 8192), (4, 0), (8, 0), (16, 0), (8, 2048))
ITER = 11


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--blocks", type=int, default=30, help="number of blocks (the workload uses 30)")
    p.add_argument("--attn-reps", type=int, default=50)
    p.add_argument("--no-loop", action="store_true", help="skip the full T=40 sampling loop")
    p.add_argument("--no-peaks", action="store_true", help="skip the attainable-peak probes")
    p.add_argument("--no-graph", action="store_true", help="skip the graph-replay timing of the step")
    p.add_argument("--no-presets", action="store_true",
                   help="skip the sampler under other schedules and the dense reference loop")
    p.add_argument("--no-sweep", action="store_true",
                   help="skip the attention sweep over active fractions and the 14B-shaped layer")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-features", action="store_true",
                   help="skip the iteration with the Wan-style block features switched on")
    p.add_argument("--no-stages", action="store_true",
                   help="skip the per-stage timing of one block at four active fractions")
    p.add_argument("--no-wan14b", action="store_true",
                   help="skip the whole 14B-shaped iteration (40 blocks, N=75600; ~155 GB of HBM)")
    p.add_argument("--no-scaling", action="store_true", help="skip the iteration-time vs active-fraction sweep")
    p.add_argument("--no-hbm-sweep", action="store_true",
                   help="skip the Euler and batched-select bandwidth sweeps")
    p.add_argument("--cpu-rows", type=int, default=2048)
    p.add_argument("--euler-tokens", type=int, default=1 << 24,
                   help="tokens for the Euler-pass bandwidth measurement (>= 1 GiB working set)")
    return p.parse_args()


ATTN_SRC = os.path.join(ROOT, "token_sparse_attention_compact_amd", "csrc", "attention.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_d128_n32760_a25_hbm_traffic.json")


def source_hash(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per attention launch from the committed FETCH_SIZE/WRITE_SIZE
    passes, only while the kernel source is the one those counters measured."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("attention_source_sha256_16") != source_hash(ATTN_SRC):
        return None
    return rec.get("bytes_per_launch")


def calibration_copy():
    """A plain device copy of exactly 256 MiB, run once before the timed region:
    the reference dispatch for scaling HBM byte counters (FETCH_SIZE, WRITE_SIZE)."""
    src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()


def attainable_peaks(reps: int = 3):
    """What this GPU delivers under load: an MFMA-only probe kernel (bf16
    32x32x16, operands in registers, lib/libhsa_probe.so) and a 1 GiB
    streaming copy kernel (same library; read + write bytes)."""
    import ctypes as ct
    lib = ct.CDLL(os.path.join(ROOT, "token_sparse_attention_compact_amd", "lib", "libhsa_probe.so"))
    n_wg, iters = 1024, 4000
    out = torch.empty(n_wg * 512, dtype=torch.float32, device="cuda")
    stream = ct.c_void_p(torch.cuda.current_stream().cuda_stream)
    call = lambda: lib.hsa_probe_mfma_peak(n_wg, iters, ct.c_void_p(out.data_ptr()), stream)
    assert call() == 0
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        assert call() == 0
    e.record()
    torch.cuda.synchronize()
    t = s.elapsed_time(e) / 1e3 / reps
    mfma_tflops = n_wg * 8 * 16 * iters * 32768.0 / t / 1e12
    rcall = lambda: lib.hsa_probe_mfma_peak_random(n_wg, iters, ct.c_void_p(out.data_ptr()), stream)
    assert rcall() == 0
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        assert rcall() == 0
    e.record()
    torch.cuda.synchronize()
    t = s.elapsed_time(e) / 1e3 / reps
    mfma_random_tflops = n_wg * 8 * 16 * iters * 32768.0 / t / 1e12
    src = torch.ones(256 << 20, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    nbytes = src.numel() * 4
    best = None
    for per_thread, max_blocks in COPY_VARIANTS:
        copy = lambda: lib.hsa_probe_copy(ct.c_void_p(src.data_ptr()), ct.c_void_p(dst.data_ptr()),
                                          ct.c_int64(nbytes), per_thread, max_blocks, stream)
        assert copy() == 0
        torch.cuda.synchronize()
        s.record()
        for _ in range(reps):
            assert copy() == 0
        e.record()
        torch.cuda.synchronize()
        t = s.elapsed_time(e) / 1e3 / reps
        assert torch.equal(src[:1024], dst[:1024]) and torch.equal(src[-1024:], dst[-1024:])
        gbs = 2 * nbytes / t / 1e9
        if best is None or gbs > best[0]:
            best = (gbs, per_thread, max_blocks)
    del src, dst, out
    return {"mfma_bf16_tflops": round(mfma_tflops, 1),
            "mfma_bf16_random_operands_tflops": round(mfma_random_tflops, 1),
            "copy_gbs": round(best[0], 1),
            "copy_variant": {"loads_per_thread": best[1], "max_blocks": best[2] or "uncapped"},
            "probe": "MFMA-only loop, 1024 workgroups x 8 waves x 64000 MFMAs, on one repeated operand pair "
                     "and on four random operand pairs per lane in turn; 1 GiB streaming copy "
                     "(16-byte non-temporal accesses, read + write bytes), best of "
                     f"{len(COPY_VARIANTS)} launch shapes"}


def time_euler(H, n_tokens: int, C: int = 16, frac: float = 0.25, reps: int = 10):
    """The fused Euler + v_hat + score kernel on a working set well past the
    256 MB Infinity Cache: GB/s of algorithmic bytes."""
    dev = "cuda"
    nA = int(n_tokens * frac)
    x = torch.randn((n_tokens, C), device=dev)
    vh = torch.randn((n_tokens, C), device=dev)
    sc = torch.rand((n_tokens,), device=dev)
    vn = torch.randn((nA, C), device=dev)
    pos = torch.full((n_tokens,), -1, dtype=torch.int32, device=dev)
    act = torch.randperm(n_tokens, device=dev)[:nA].sort().values
    pos[act] = torch.arange(nA, dtype=torch.int32, device=dev)
    for _ in range(2):
        H.hsa_euler(x, vh, sc, vn, pos, -0.025, True)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        H.hsa_euler(x, vh, sc, vn, pos, -0.025, True)
    e.record()
    torch.cuda.synchronize()
    t = s.elapsed_time(e) / 1e3 / reps
    nbytes = n_tokens * (4 + 3 * 4 * C) + nA * (2 * 4 * C + 4)
    del x, vh, sc, vn, pos, act
    return {"tokens": n_tokens, "active_frac": frac, "bytes": nbytes, "us": round(t * 1e6, 1),
            "gbs": round(nbytes / t / 1e9, 1), "frac_of_hbm_peak": round(nbytes / t / 1e9 / PEAK_HBM_GBS, 4)}


def time_select_batch(H, B: int, N: int = 32760, counts=(8190, 8190, 16380), reps: int = 5):
    """hsa_select_batch over B independent score rows of N tokens (one
    selection per video): GB/s of algorithmic bytes, each score read once and
    each group written once (5 B per token)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(B)
    score = torch.rand((B, N), generator=g, device="cuda")
    out = torch.empty((B, N), dtype=torch.uint8, device="cuda")
    for _ in range(2):
        H.hsa_select_batch(score, list(counts), out)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        H.hsa_select_batch(score, list(counts), out)
    e.record()
    torch.cuda.synchronize()
    t = s.elapsed_time(e) / 1e3 / reps
    nbytes = B * N * 5
    del score, out
    return {"rows": B, "tokens_per_row": N, "bytes": nbytes, "us": round(t * 1e6, 1),
            "gbs": round(nbytes / t / 1e9, 1), "frac_of_hbm_peak": round(nbytes / t / 1e9 / PEAK_HBM_GBS, 4)}


def hbm_sweep(H, copy_gbs=None):
    """The two HBM-bound passes over growing working sets, up to past 1 GiB:
    the Euler + v_hat + score kernel over more tokens, and selection over a
    batch of videos of the workload's 32760 tokens (the working set of one
    video, 0.16 MB, is latency-bound and cache-resident)."""
    out = {"euler": [time_euler(H, n) for n in (32760, 1 << 20, 1 << 22, 1 << 24, 24 << 20)],
           "select_batch": [time_select_batch(H, b) for b in (1, 64, 512, 2048, 8192)]}
    for r in out["euler"] + out["select_batch"]:
        # HBM fractions only where the working set is >= 4x the Infinity Cache
        if r["bytes"] < 4 * MALL_BYTES:
            r["cache_resident_part"] = True
            del r["frac_of_hbm_peak"]
        elif copy_gbs:
            r["frac_of_attainable_copy"] = round(r["gbs"] / copy_gbs, 4)
    return out


def device_inputs(c, H, seed_base):
    """Random-init weights N(0, 1/fan_in) and a mid-run state, generated on the device."""
    dev = "cuda"
    g = torch.Generator(device=dev)
    dt = torch.bfloat16

    def randn(shape, std, sub):
        g.manual_seed(seed_base * 1000 + sub)
        return (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * std).to(dt)

    D, F, N, C = c.D, c.F, c.N, c.C
    blocks = []
    for l in range(c.L):
        s = 100 * (l + 1)
        blocks.append({
            "w_qkv": randn((3 * D, D), D ** -0.5, s + 1),
            "w_o": randn((D, D), D ** -0.5, s + 2),
            "w_1": randn((F, D), D ** -0.5, s + 3),
            "w_2": randn((D, F), F ** -0.5, s + 4),
            "k_cache": randn((N, D), 1.0, s + 5),
            "v_cache": randn((N, D), 1.0, s + 6),
        })
    dims = H.make_dims(N, C, D, c.H, c.Dh, F, c.L, 0, dt)
    model = H.DeviceModel(dims, randn((D, C), C ** -0.5, 1), randn((C, D), D ** -0.5, 2), blocks)
    g.manual_seed(seed_base * 1000 + 3)
    x = torch.randn((N, C), generator=g, device=dev)
    v_hat = torch.randn((N, C), generator=g, device=dev)
    score = torch.rand((N,), generator=g, device=dev)
    group = torch.from_numpy(synth.group0(c)).to(dev)
    state = H.DeviceState(dims, x, group, v_hat, score)
    return model, state


def timed_steps(H, model, sched, state, sigma, steps, warmup):
    for _ in range(warmup):
        H.hsa_step(model, sched, state, ITER, float(sigma[ITER]), float(sigma[ITER + 1]), True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        H.hsa_step(model, sched, state, ITER, float(sigma[ITER]), float(sigma[ITER + 1]), True)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def graph_steps(H, model, sched, state, sigma, steps: int):
    """The timed step captured once in a HIP graph (torch.cuda.graph over the
    library's stream-ordered launches) and replayed: iterations/s without
    per-launch host overhead."""
    g = torch.cuda.CUDAGraph()
    H.hsa_step(model, sched, state, ITER, float(sigma[ITER]), float(sigma[ITER + 1]), True)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        H.hsa_step(model, sched, state, ITER, float(sigma[ITER]), float(sigma[ITER + 1]), True)
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    t = (time.perf_counter() - t0) / steps
    return {"ms_per_step": round(t * 1e3, 3), "iter_per_s": round(1.0 / t, 4), "steps": steps}


def time_attention(H, model, c, n_active, reps, warmup: int = 10):
    """Average duration of the attention kernel at the step's launch configuration,
    with HIP events on the stream the kernel runs on.  Layers' caches rotate so
    K/V come from HBM as in the stack."""
    q = torch.randn((n_active, c.D), device="cuda").to(torch.bfloat16)
    o = torch.empty_like(q)
    ws = torch.empty(max(1, H.hsa_attn_workspace_size(n_active, c.N, c.H, c.Dh)), dtype=torch.uint8,
                     device="cuda")
    L = len(model.blocks)
    for r in range(warmup):
        b = model.blocks[r % L]
        H.hsa_attn_active(q, b["k_cache"], b["v_cache"], o, c.H, c.Dh, ws=ws)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for r in range(reps):
        b = model.blocks[(warmup + r) % L]
        H.hsa_attn_active(q, b["k_cache"], b["v_cache"], o, c.H, c.Dh, ws=ws)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3 / reps


def attention_sweep(H, model, c, fracs=(1.0, 0.5, 0.25, 0.125, 0.0625, 0.05), reps: int = 10):
    """Attention alone at other active fractions of the same stack (K/V of the
    stack's layers, rotating), at the 14B-shaped layer: N = 75600 cached
    rows, |A| = 18900 (25%), 40 heads x 128, and with 64-wide heads: N =
    32760, 32 heads x 64, |A| = 8190 and 2048."""
    out = {"N": c.N, "heads": c.H, "frac": list(fracs), "n_active": [], "tflops": []}
    for f in fracs:
        nA = synth.n_active_for_fraction(c.N, f)
        t = time_attention(H, model, c, nA, reps, warmup=3)
        out["n_active"].append(nA)
        out["tflops"].append(round(4.0 * nA * c.N * c.D / t / 1e12, 1))
    c4 = synth.CONFIGS[4]
    nA = c4.counts()[0]
    g = torch.Generator(device="cuda")
    g.manual_seed(4 * 1000 + 5)
    kc = torch.randn((c4.N, c4.D), generator=g, device="cuda").to(torch.bfloat16)
    vc = torch.randn((c4.N, c4.D), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((nA, c4.D), generator=g, device="cuda").to(torch.bfloat16)
    o = torch.empty_like(q)
    ws = torch.empty(max(1, H.hsa_attn_workspace_size(nA, c4.N, c4.H, c4.Dh)), dtype=torch.uint8,
                     device="cuda")
    for _ in range(2):
        H.hsa_attn_active(q, kc, vc, o, c4.H, c4.Dh, ws=ws)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(5):
        H.hsa_attn_active(q, kc, vc, o, c4.H, c4.Dh, ws=ws)
    e.record()
    torch.cuda.synchronize()
    t = s.elapsed_time(e) / 1e3 / 5
    out["wan14b_shape"] = {"N": c4.N, "n_active": nA, "heads": c4.H, "head_dim": c4.Dh,
                           "ms": round(t * 1e3, 2), "tflops": round(4.0 * nA * c4.N * c4.D / t / 1e12, 1)}
    del kc, vc, q, o, ws
    # 64-wide heads (the LTX-style head layout): N = 32760, 32 x 64, 25% and 1/16 active
    Hh, Dh = 32, 64
    D = Hh * Dh
    kc = torch.randn((c.N, D), generator=g, device="cuda").to(torch.bfloat16)
    vc = torch.randn((c.N, D), generator=g, device="cuda").to(torch.bfloat16)
    rows = []
    for nA in (8190, 2048):
        q = torch.randn((nA, D), generator=g, device="cuda").to(torch.bfloat16)
        o = torch.empty_like(q)
        ws = torch.empty(max(1, H.hsa_attn_workspace_size(nA, c.N, Hh, Dh)), dtype=torch.uint8,
                         device="cuda")
        t = _event_time(lambda: H.hsa_attn_active(q, kc, vc, o, Hh, Dh, ws=ws), 5)
        rows.append({"n_active": nA, "ms": round(t * 1e3, 3), "tflops": round(4.0 * nA * c.N * D / t / 1e12, 1)})
    out["heads_64_wide"] = {"N": c.N, "heads": Hh, "head_dim": Dh, "runs": rows}
    del kc, vc
    return out


def attention_operand_data(H, c, n_active: int, reps: int = 10, rounds: int = 3):
    """The attention launch of the step (|A| queries over N cached rows, the
    stack's heads) on two inputs of the same shapes: N(0,1) caches and
    queries, as in the workload, and all-zero ones.  Same kernel, grid and
    instruction stream; only the operand values differ, and with them the
    switching power of the matrix cores and so the clock the chip holds.
    Interleaved rounds, HIP events; the fastest round of each is kept."""
    g = torch.Generator(device="cuda")
    g.manual_seed(7 * 1000 + 11)
    bf = torch.bfloat16
    data = {"normal": [torch.randn((c.N, c.D), generator=g, device="cuda").to(bf) for _ in range(2)]
                      + [torch.randn((n_active, c.D), generator=g, device="cuda").to(bf)],
            "zero": [torch.zeros((c.N, c.D), dtype=bf, device="cuda") for _ in range(2)]
                    + [torch.zeros((n_active, c.D), dtype=bf, device="cuda")]}
    o = torch.empty((n_active, c.D), dtype=bf, device="cuda")
    ws = torch.empty(max(1, H.hsa_attn_workspace_size(n_active, c.N, c.H, c.Dh)), dtype=torch.uint8,
                     device="cuda")
    best = {}
    for _ in range(rounds):
        for name, (kc, vc, q) in data.items():
            t = _event_time(lambda: H.hsa_attn_active(q, kc, vc, o, c.H, c.Dh, ws=ws), reps)
            best[name] = min(best.get(name, t), t)
    flop = 4.0 * n_active * c.N * c.D
    out = {"n_active": n_active, "N": c.N}
    for name, t in best.items():
        out[name] = {"us": round(t * 1e6, 1), "tflops": round(flop / t / 1e12, 1)}
    out["zero_over_normal_speed"] = round(best["normal"] / best["zero"], 3)
    del data, o, ws
    torch.cuda.empty_cache()
    return out


def sampling_loop(H, model, c, sigma, budgets=None, counts=None, regroup_at=None):
    """The whole sampler: iterations 0..T-1 of hsa_step from fresh latents
    (every group active at i = 0), regrouping at the start of the iterations in
    regroup_at, one device synchronisation at the end.  Defaults: the stack's
    schedule (budgets 40/20/10 at 25/25/50%, regrouping at 10, 20, 30)."""
    dev = "cuda"
    budgets = c.budgets if budgets is None else budgets
    counts = c.counts() if counts is None else counts
    regroup_at = set(c.regroup if regroup_at is None else regroup_at)
    g = torch.Generator(device=dev)
    g.manual_seed(3 * 1000 + 9)
    x0 = torch.randn((c.N, c.C), generator=g, device=dev)
    group0 = torch.from_numpy(synth.group0(c.with_(budgets=tuple(budgets),
                                                   shares=tuple(n / c.N for n in counts)))).to(dev)
    state = H.DeviceState(model.dims, x0, group0)
    sched = H.make_schedule(c.T, budgets, counts)
    n_act = [H.hsa_n_active(sched, i) for i in range(c.T)]
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(c.T):
        H.hsa_step(model, sched, state, i, float(sigma[i]), float(sigma[i + 1]), i in regroup_at)
    e.record()
    torch.cuda.synchronize()
    t = s.elapsed_time(e) / 1e3
    ok = bool(torch.isfinite(state.x).all().item())
    del state
    return {"iterations": c.T, "s": round(t, 3), "iter_per_s": round(c.T / t, 3),
            "mean_active_frac": round(sum(n_act) / (c.T * c.N), 4), "regroup_at": sorted(regroup_at),
            "budgets": list(budgets), "counts": list(counts), "finite": ok}


def schedule_presets(H, model, c, sigma, moderate):
    """The sampler under other schedules, against dense sampling (every token
    every step): runtime of each relative to the dense 40-step loop."""
    N = c.N
    c5 = synth.CONFIGS[5]                      # budgets 40/10/5 at 12.5/37.5/50%
    assert c5.N == N and c5.T == c.T
    runs = {
        "dense": sampling_loop(H, model, c, sigma, (c.T,), [N], ()),
        "moderate_dynamic": moderate,
        "moderate_static": sampling_loop(H, model, c, sigma, c.budgets, c.counts(), ()),
        "aggressive_dynamic": sampling_loop(H, model, c, sigma, c5.budgets, c5.counts(), c5.regroup),
    }
    dense = runs["dense"]["s"]
    for r in runs.values():
        r["runtime_vs_dense"] = round(r["s"] / dense, 4)
    return runs


def step_scaling(H, model, state, c, sigma, reps: int = 5):
    """Iteration time against the active fraction: hsa_step (no regroup) at
    |A|/N = 1, 0.5, 0.25 (iterations 0, 2, 1 of the 25/25/50 schedule) and
    0.0625 (a schedule whose full-budget group holds 2048 tokens, odd
    iteration); least-squares fit t(f) = t0 + b f."""
    N = c.N
    cases = [(1.0, c.counts(), 0), (0.5, c.counts(), 2), (0.25, c.counts(), 1),
             (0.0625, [2048, 10240, N - 12288], 1)]
    fr, ms = [], []
    for f, counts, it in cases:
        sched = H.make_schedule(c.T, c.budgets, counts)
        assert H.hsa_n_active(sched, it) == round(f * N)
        for _ in range(2):
            H.hsa_step(model, sched, state, it, float(sigma[it]), float(sigma[it + 1]), False)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            H.hsa_step(model, sched, state, it, float(sigma[it]), float(sigma[it + 1]), False)
        e.record()
        torch.cuda.synchronize()
        fr.append(f)
        ms.append(s.elapsed_time(e) / reps)
    b, t0 = np.polyfit(np.array(fr), np.array(ms), 1)
    pred = t0 + b * np.array(fr)
    return {"active_frac": fr, "ms_per_step": [round(x, 2) for x in ms], "fit_t0_ms": round(float(t0), 2),
            "fit_slope_ms": round(float(b), 2),
            "fit_max_rel_residual": round(float(np.max(np.abs(pred - ms) / np.array(ms))), 4)}


def featured_model(H, model, c, features, n_text: int = 0, seed: int = 77):
    """The bench stack with Wan-style block features switched on, sharing its
    weights and caches: float32 gains 1 + N(0, 0.1^2), modulation tables
    N(0, 0.1^2) with unit-centred gates, a timestep MLP, and with guidance
    (needs n_text text rows) random cross-attention weights, text K/V for
    both branches and a copy of every cache for the unconditional branch."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    D, N = c.D, c.N
    bf = torch.bfloat16

    def randn(shape, std, dtype=torch.float32):
        return (torch.randn(shape, generator=g, device="cuda") * std).to(dtype)

    blocks = []
    for b in model.blocks:
        nb = dict(b)
        nb["q_gain"], nb["k_gain"] = 1 + randn((D,), 0.1), 1 + randn((D,), 0.1)
        mod = randn((6, D), 0.1)
        mod[2] += 1
        mod[5] += 1
        nb["mod"] = mod
        if n_text:
            for k in ("w_qx", "w_ox"):
                nb[k] = randn((D, D), D ** -0.5, bf)
            for k in ("k_text", "v_text", "k_text_u", "v_text_u"):
                nb[k] = randn((n_text, D), 1.0, bf)
        if "cfg" in features:
            nb["k_cache_u"], nb["v_cache_u"] = b["k_cache"].clone(), b["v_cache"].clone()
        blocks.append(nb)
    time_w = {"t_w1": randn((D, H.T_FREQ), H.T_FREQ ** -0.5), "t_b1": randn((D,), 0.01),
              "t_w2": randn((D, D), D ** -0.5), "t_b2": randn((D,), 0.01),
              "t_w3": randn((6 * D, D), 0.3 * D ** -0.5), "t_b3": randn((6 * D,), 0.01),
              "head_mod": randn((2, D), 0.1)}
    dims = H.make_dims(N, c.C, D, c.H, c.Dh, c.F, c.L, n_text, bf, features=features, grid=c.grid)
    return H.DeviceModel(dims, model.w_in, model.w_out, blocks, time_w, cfg_scale=5.0)


def wan_features(H, model, state, c, sigma, plain_ms: float, steps: int = 5, reps: int = 20):
    """The timed iteration with the Wan-style block features on: (a) qk-RMSNorm
    + 3D rotary embedding + adaLN timestep modulation on the bench stack; (b)
    additionally 512-token cross-attention and classifier-free guidance with
    batch 2 (two block stacks per iteration on the same active rows).  Plus
    the fused qk-norm + rotation pass alone (HIP events on its stream) against
    HBM peak: it reads and writes the |A| fresh q rows and |A| K-cache rows,
    8 |A| D bytes per launch in bf16."""
    out = {"plain_ms": round(plain_ms, 3)}
    sched = H.make_schedule(c.T, c.budgets, c.counts())
    for name, feats, n_text in (("qk_rope_adaln", ("qk_norm", "rope3d", "adaln"), 0),
                                ("qk_rope_adaln_xattn512_cfg", ("qk_norm", "rope3d", "adaln", "cfg"), 512)):
        fm = featured_model(H, model, c, feats, n_text)
        fs = H.DeviceState(fm.dims, state.x, state.group, state.v_hat, state.score)
        t = timed_steps(H, fm, sched, fs, sigma, steps, 2) / steps * 1e3
        out[name + "_ms"] = round(t, 3)
        out[name + "_vs_plain"] = round(t / plain_ms, 4)
        del fm, fs
        torch.cuda.empty_cache()
    # the fused qk-norm + rotation pass alone, at the step's |A_i|
    nA = H.hsa_n_active(sched, ITER)
    idx = torch.from_numpy(synth.active_random(c, nA)).to("cuda")
    q = torch.randn((nA, c.D), device="cuda").to(torch.bfloat16)
    kc = torch.randn((c.N, c.D), device="cuda").to(torch.bfloat16)
    gq, gk = torch.ones(c.D, device="cuda"), torch.ones(c.D, device="cuda")
    dims = H.make_dims(c.N, c.C, c.D, c.H, c.Dh, c.F, 1, 0, torch.bfloat16,
                       features=("qk_norm", "rope3d"), grid=c.grid)
    for _ in range(3):
        H.hsa_qk_norm_rope(q, kc, idx, nA, dims, gq, gk)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        H.hsa_qk_norm_rope(q, kc, idx, nA, dims, gq, gk)
    end.record()
    torch.cuda.synchronize()
    t = start.elapsed_time(end) / 1e3 / reps
    nbytes = 8.0 * nA * c.D
    out["qk_norm_rope"] = {"n_active": nA, "avg_launch_us": round(t * 1e6, 2),
                           "bytes_per_launch": int(nbytes), "gbs": round(nbytes / t / 1e9, 1),
                           "frac_of_hbm_peak": round(nbytes / t / 1e9 / PEAK_HBM_GBS, 4)}
    return out


def _event_time(fn, reps: int, warmup: int = 2) -> float:
    """Mean seconds per call of fn() under HIP events on the current stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / 1e3 / reps


def stage_bench(H, model, c, reps: int = 10):
    """One Wan-1.3B-shaped block's stages (the single-block workload: D 1536,
    12 x 128 heads, N = 32760 cached rows) at |A| in {32760, 16380, 8190,
    2048}, active rows uniform random or contiguous spatial blobs: QKV with
    the K/V scatter reading the active rows straight from the [N][D]
    per-token LayerNorm output (gather mode) and from a compact copy,
    attention over all N cached rows, out-projection with the residual add.
    Layer 0's weights, fresh caches; HIP events, mean over reps."""
    b = model.blocks[0]
    N, D = c.N, c.D
    bf = torch.bfloat16
    hidden = torch.randn(N, D, device="cuda").to(bf)
    kc = torch.randn(N, D, device="cuda").to(bf)
    vc = torch.randn(N, D, device="cuda").to(bf)
    rows = []
    for nA in (32760, 16380, 8190, 2048):
        for pattern in ("random", "blob"):
            idx_np = synth.active_random(c, nA) if pattern == "random" else synth.active_blob(c, nA)
            idx = torch.from_numpy(idx_np).to("cuda")
            q = torch.empty(nA, D, dtype=bf, device="cuda")
            o = torch.empty(nA, D, dtype=bf, device="cuda")
            hres = torch.zeros(nA, D, device="cuda")
            compact = hidden[idx.long()].contiguous()
            ws = torch.empty(max(1, H.hsa_attn_workspace_size(nA, N, c.H, c.Dh)), dtype=torch.uint8,
                             device="cuda")
            t_g = _event_time(lambda: H.hsa_qkv_scatter(hidden, idx, nA, b["w_qkv"], q, kc, vc, gather=True), reps)
            t_c = _event_time(lambda: H.hsa_qkv_scatter(compact, idx, nA, b["w_qkv"], q, kc, vc), reps)
            t_a = _event_time(lambda: H.hsa_attn_active(q, kc, vc, o, c.H, c.Dh, ws=ws), reps)
            t_o = _event_time(lambda: H.hsa_linear_residual(o, b["w_o"], hres), reps)
            qkv_f, attn_f, out_f = 2.0 * nA * D * 3 * D, 4.0 * nA * N * D, 2.0 * nA * D * D
            rows.append({"n_active": nA, "pattern": pattern,
                         "qkv_scatter_gather_us": round(t_g * 1e6, 1),
                         "qkv_scatter_gather_tflops": round(qkv_f / t_g / 1e12, 1),
                         "qkv_scatter_compact_us": round(t_c * 1e6, 1),
                         "attention_us": round(t_a * 1e6, 1), "attention_tflops": round(attn_f / t_a / 1e12, 1),
                         "out_proj_us": round(t_o * 1e6, 1), "out_proj_tflops": round(out_f / t_o / 1e12, 1)})
    del hidden, kc, vc
    torch.cuda.empty_cache()
    return rows


def gemm_bench(H, model, c, fracs=(1.0, 0.25, 0.0625)):
    """The block's four GEMMs with their fused epilogues, alone: QKV with the
    K/V scatter, out-projection + residual, MLP up + GELU, MLP down +
    residual, at |A|/N in fracs. Each call uses the next layer's weights (30
    rotating sets, read cold from HBM as in the iteration); HIP events, mean
    over two passes of the 30 layers."""
    N, D, F = c.N, c.D, c.F
    bf = torch.bfloat16
    out = []
    for f in fracs:
        nA = synth.n_active_for_fraction(N, f)
        a = torch.randn(nA, D, device="cuda").to(bf)
        u = torch.randn(nA, F, device="cuda").to(bf)
        q = torch.empty(nA, D, dtype=bf, device="cuda")
        hid = torch.empty(nA, F, dtype=bf, device="cuda")
        hres = torch.zeros(nA, D, device="cuda")
        idx = torch.arange(nA, dtype=torch.int32, device="cuda")
        kc = torch.empty(N, D, dtype=bf, device="cuda")      # scatter targets (not the model's caches)
        vc = torch.empty(N, D, dtype=bf, device="cuda")
        L = len(model.blocks)
        cnt = [0]

        def nxt():
            b = model.blocks[cnt[0] % L]
            cnt[0] += 1
            return b
        calls = {
            "qkv_scatter": (2.0 * nA * D * 3 * D,
                            lambda: H.hsa_qkv_scatter(a, idx, nA, nxt()["w_qkv"], q, kc, vc)),
            "out_proj_residual": (2.0 * nA * D * D, lambda: H.hsa_linear_residual(a, nxt()["w_o"], hres)),
            "mlp_up_gelu": (2.0 * nA * D * F, lambda: H.hsa_linear(a, nxt()["w_1"], hid, act=1)),
            "mlp_down_residual": (2.0 * nA * F * D, lambda: H.hsa_linear_residual(u, nxt()["w_2"], hres)),
        }
        row = {"n_active": nA}
        for name, (flop, fn) in calls.items():
            t = _event_time(fn, 2 * L, warmup=L)
            row[name + "_us"] = round(t * 1e6, 1)
            row[name + "_tflops"] = round(flop / t / 1e12, 1)
        out.append(row)
        del a, u, q, hid, hres, kc, vc
    torch.cuda.empty_cache()
    return out


def wan14b_iteration(H, steps: int = 2):
    """The whole 14B-shaped iteration (--no-wan14b skips it): 40 blocks, N = 75600
    (21 x 45 x 80), D 5120, 40 x 128 heads, F 13824, 512-token cross-attention,
    iteration 11 of the {40, 20, 10} schedule (|A| = 18900, 25%), regroup on;
    (a) the plain block with cross-attention, (b) with qk-RMSNorm, 3D RoPE,
    adaLN modulation and guidance batch 2 (a second cache set: ~155 GB of HBM
    in all)."""
    c = synth.CONFIGS[4]
    sched = H.make_schedule(c.T, c.budgets, c.counts())
    sigma = synth.sigma_schedule(c.T)
    base, state = device_inputs(c, H, seed_base=5)
    nA = H.hsa_n_active(sched, ITER)
    # model FLOPs of one block stack: self-attention over all N cached rows, the
    # block's GEMMs and the cross-attention (q and out projections, 512 text rows)
    flop = c.L * (4.0 * nA * c.N * c.D + 2.0 * nA * c.D * (3 * c.D + c.D + 2 * c.F)
                  + 2.0 * nA * c.D * 2 * c.D + 4.0 * nA * c.n_text * c.D)
    out = {"workload": "wan14b-shaped 40-block stack, N=75600 (21x45x80), 25% active, 512 text tokens",
           "n_active": nA, "model_tflop_per_iter": round(flop / 1e12, 1)}
    for name, feats in (("xattn", ()), ("xattn_qk_rope_adaln_cfg", ("qk_norm", "rope3d", "adaln", "cfg"))):
        fm = featured_model(H, base, c, feats, c.n_text)
        fs = H.DeviceState(fm.dims, state.x, state.group, state.v_hat, state.score)
        t = timed_steps(H, fm, sched, fs, sigma, steps, 1) / steps
        out[name + "_s_per_iter"] = round(t, 3)
        out[name + "_model_tflops"] = round(flop * (2 if "cfg" in feats else 1) / t / 1e12, 1)
        del fm, fs
        torch.cuda.empty_cache()
    return out


def cpu_baseline(c, rows: int):
    """The oracle on a bounded sample of the same iteration: one block with `rows`
    active tokens over all N cached rows (its cost is linear in the number of
    active rows), scaled to 8190 rows x 30 blocks, plus the oracle's Euler +
    select over all N tokens."""
    from oracle import hsa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    cs = c.with_(L=1)
    dims = O.Dims(N=cs.N, C=cs.C, D=cs.D, H=cs.H, Dh=cs.Dh, F=cs.F, L=1, bf16=True)
    om = O.make_model(dims, synth.io_weights(cs), [synth.block_weights(cs, 0)])
    kc, vc = synth.kv_cache(cs)
    kc, vc = kc.astype(np.float64), vc.astype(np.float64)
    idx = synth.active_random(cs, rows)
    h = synth.hidden_states(cs, rows)
    t0 = time.perf_counter()
    O.block_forward(om, 0, h, idx, kc, vc)
    t_block = time.perf_counter() - t0
    st = synth.mid_run_state(cs.with_(L=1))
    t0 = time.perf_counter()
    grp = O.select_groups(st["score"], cs.counts())
    aidx, _ = O.active_set(grp, cs.budgets, cs.T, ITER)
    O.euler_update(st["x"], st["v_hat"], st["score"], st["v_hat"][aidx], aidx, -0.025, True)
    t_tail = time.perf_counter() - t0
    n_active = O.n_active_closed_form(cs.counts(), cs.budgets, cs.T, ITER)
    t_iter = t_block * (n_active / rows) * c.L + t_tail
    return {"value": 1.0 / t_iter, "unit": "iter/s", "cores": int(threads), "kind": "oracle",
            "sample": f"1 block with {rows} of {n_active} active rows over N={cs.N} cached rows "
                      f"({t_block:.2f} s), scaled x{n_active / rows:.1f} rows x {c.L} blocks, "
                      f"+ select/active-set/Euler over all N ({t_tail:.2f} s); projected "
                      f"{t_iter:.1f} s per iteration",
            "dit_lite_full_run": oracle_dit_lite_run()}


def oracle_dit_lite_run():
    """The oracle's whole 8-iteration float32 DiT-lite run (N = 256 on the 4x8x8
    grid, budgets {8, 4}, regrouping from i = 3 on), with the BLAS thread pool
    as it is and with one thread."""
    from oracle import hsa_oracle as O
    c = synth.CONFIGS[1]
    dims = O.Dims(N=c.N, C=c.C, D=c.D, H=c.H, Dh=c.Dh, F=c.F, L=c.L, bf16=False)
    om = O.make_model(dims, synth.io_weights(c), [synth.block_weights(c, l) for l in range(c.L)])
    sched = O.Schedule(c.T, list(c.budgets), c.counts(), regroup=c.regroup)
    sigma = synth.sigma_schedule(c.T)

    def run():
        st = O.init_state(dims, synth.x0(c), synth.group0(c))
        t0 = time.perf_counter()
        O.sample(om, sched, st, sigma)
        return time.perf_counter() - t0

    out = {"iterations": c.T, "s": round(run(), 4)}
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            out["s_single_thread"] = round(run(), 4)
    except Exception:  # pragma: no cover
        pass
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): the library has no "
              f"multi-GPU path; the per-GPU kernel is what is measured.", file=sys.stderr)
        sys.exit(2)
    from token_sparse_attention_compact_amd import hsa as H
    H.load()
    c = synth.CONFIGS[3].with_(L=args.blocks)
    sched = H.make_schedule(c.T, c.budgets, c.counts())
    n_active = H.hsa_n_active(sched, ITER)
    sigma = synth.sigma_schedule(c.T)
    model, state = device_inputs(c, H, seed_base=3)
    calibration_copy()
    torch.cuda.synchronize()

    elapsed = timed_steps(H, model, sched, state, sigma, args.steps, args.warmup)
    ms = elapsed / args.steps * 1e3
    it_s = args.steps / elapsed

    t_attn = time_attention(H, model, c, n_active, args.attn_reps)
    attn_flop = 4.0 * n_active * c.N * c.D
    attn_tflops = attn_flop / t_attn / 1e12
    gemm_flop = 2.0 * n_active * c.D * (3 * c.D + c.D + 2 * c.F) * c.L
    iter_flop = attn_flop * c.L + gemm_flop

    out = {
        "metric": METRIC,
        "value": round(it_s, 4),
        "unit": "iter/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (random-init weights N(0,1/fan_in), N(0,1) caches and latents)",
        "config": {"workload": f"wan1.3b-shaped {c.L}-block stack, N=32760 (21x30x52), 25% active "
                               f"(iteration {ITER} of T=40, budgets 40/20/10, regroup on)",
                   "N": c.N, "n_active": n_active, "blocks": c.L, "D": c.D, "heads": c.H,
                   "head_dim": c.Dh, "F": c.F, "C": c.C},
        "attn_tflops": round(attn_tflops, 2),
        "iter_tflops": round(iter_flop * it_s / 1e12, 2),
        "roofline": {"bound": "mfma", "kernel": "attn_bf16_d128_kernel",
                     "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "avg_launch_us": round(t_attn * 1e6, 2),
                     "traffic": recorded_traffic()},
    }
    if not args.no_graph:
        out["graph_replay"] = graph_steps(H, model, sched, state, sigma, args.steps)
    if not args.no_peaks:
        peaks = attainable_peaks()
        out["attainable"] = peaks
        out["roofline"]["frac_of_attainable"] = round(attn_tflops / peaks["mfma_bf16_tflops"], 4)
        out["roofline"]["frac_of_attainable_random_operands"] = round(
            attn_tflops / peaks["mfma_bf16_random_operands_tflops"], 4)
    if not args.no_sweep:
        out["attention_sweep"] = attention_sweep(H, model, c)
        out["attention_operand_data"] = attention_operand_data(H, c, n_active)
    if not args.no_loop:
        out["sampling_loop"] = sampling_loop(H, model, c, sigma)
        if not args.no_presets:
            out["schedule_presets"] = schedule_presets(H, model, c, sigma, out["sampling_loop"])
    if args.euler_tokens > 0:
        out["euler_hbm"] = time_euler(H, args.euler_tokens)
        if "attainable" in out:
            out["euler_hbm"]["frac_of_attainable_copy"] = round(
                out["euler_hbm"]["gbs"] / out["attainable"]["copy_gbs"], 4)
    if not args.no_hbm_sweep:
        out["hbm_sweep"] = hbm_sweep(H, out.get("attainable", {}).get("copy_gbs"))
    if not args.no_scaling:
        out["scaling_with_active_fraction"] = step_scaling(H, model, state, c, sigma)
    if not args.no_stages:
        out["stage_bench"] = stage_bench(H, model, c)
        out["gemm_bench"] = gemm_bench(H, model, c)
    if not args.no_features:
        out["wan_features"] = wan_features(H, model, state, c, sigma, ms)
        if "attainable" in out:
            out["wan_features"]["qk_norm_rope"]["frac_of_attainable_copy"] = round(
                out["wan_features"]["qk_norm_rope"]["gbs"] / out["attainable"]["copy_gbs"], 4)
    if not args.no_wan14b:
        del model, state
        torch.cuda.empty_cache()
        try:
            out["wan14b_iteration"] = wan14b_iteration(H)
        except (RuntimeError, torch.cuda.OutOfMemoryError) as e:   # keep the rest of the line
            out["wan14b_iteration"] = {"error": str(e)[:200]}
            torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(c, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
