"""Benchmark of the gated delta rule on one MI355X.

A step is one gdn_chunk_fwd (chunkwise prefill) over one batch of the Qwen3.6-27B-shaped GDN
workload, the largest single-GPU configuration: B=1, T=65536, 16 query/key heads, 48 value heads,
head dim 128, chunk 64, bf16 inputs, float32 state.  `value` is prefill tokens/s with the inputs
resident in HBM (one input set of 2.2 GB, larger than the 256 MB Infinity Cache).

The same JSON line carries
  roofline      -- the prefill call's achieved algorithmic bytes/s against 8 TB/s (its binding
                   roofline: 188 flop/B is below the bf16-MFMA/HBM ridge of 315), the call's
                   average duration from HIP events on its own stream (every kernel the call
                   launches), its bf16-MFMA fraction (algorithmic flops / time / 2.5166 PFLOP/s),
                   and the HBM traffic measured with rocprofv3 counters when a record taken on the
                   current kernel sources exists;
  cpu_baseline  -- the float64 oracle timed on the host cores on the same 48-chain batch;
  decode        -- the 64-step fused decode workload (B=256, Hv=32, d=128, fp32 state 512 MiB):
                   steps/s and its own HBM roofline object;
  prefill_configs -- the batched (B=8, T=8192, S0 != 0) and Qwen3-Next-shaped (B=1, T=4096)
                   prefill workloads, each with its own roofline object, and the Qwen3-Next shape
                   with float32 inputs (the float32 kernel, against the float32 peak);
  layer_ops     -- the layer steps either side of the recurrence at the Qwen3-Next shape (short
                   conv + SiLU + q/k L2 norm; gated RMSNorm): time and achieved HBM bandwidth;
  gated_prefill -- gdn_chunk_fwd_gated (prefill with the output's gated RMSNorm in the same
                   call) on the Qwen3-Next and the batched workloads;
  backward      -- gdn_chunk_bwd (gradients of q, k, v, g, beta, S0) at the Qwen3-Next shape:
                   tokens/s and its roofline fraction (the time the work would take with each
                   part at the peak of the unit that runs it: float16 matrix cores for the bf16
                   route's passes and three gradient products, float32 for the rest, over the
                   measured time), for the method's own work and for the work as computed
                   (which recomputes the states);
  kda           -- gdn_kda_chunk_fwd (Kimi Delta Attention, per-key-channel decay) on the KDA
                   workload (B1 T4096, 32/32 heads, d128, chunk 64 on the float16 matrix cores):
                   tokens/s and its fraction of the 16-bit matrix-core peak;
  varlen        -- gdn_chunk_fwd_varlen on 64 packed sequences of 64..2048 tokens;
  scan          -- gdn_chunk_fwd_scan (the affine chunk scan) against gdn_chunk_fwd on the 64K-token
                   workload and on one GPU's share of it under an 8-way head split.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--quick] [--no-cpu-baseline]
                       [--leg layer_ops|backward|kda|varlen|scan|decode]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # B/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5166e15  # flop/s, MI355X dense bf16 matrix cores
CSRC = os.path.join(ROOT, "gated_deltanet_linear_delta_amd", "csrc")


def prefill_alg_bytes(B, T, Hqk, Hv, dk, dv, es, with_s0, with_sf):
    """Algorithmic HBM bytes of one prefill: q, k once per query/key head, v and o once, g and
    beta in float32, initial and final state in float32."""
    n = B * T
    b = n * Hqk * dk * es * 2 + n * Hv * dv * es * 2 + n * Hv * 4 * 2
    st = B * Hv * dk * dv * 4
    return b + (st if with_s0 else 0) + (st if with_sf else 0)


def prefill_alg_flops(B, T, Hqk, Hv, dk, dv, C):
    """Algorithmic flops of the chunkwise method per token and value head (masked halves
    excluded): 6 dk dv (W h, Q h, K^T Delta) + C dk (W) + 2 C dv (U, Aqk Delta)
    + 2 C dk / G (K K^T, Q K^T shared by the G value heads of a group) + C^2 / 3 (the solve)."""
    G = Hv // Hqk
    per = 6 * dk * dv + C * dk + 2 * C * dv + 2 * C * dk / G + C * C / 3
    return per * B * T * Hv


FP32_VALU_PEAK = 157.3e12   # flop/s, MI355X float32 vector units


def backward_alg_flops(B, T, Hqk, Hv, dk, dv, C=32, recompute=True):
    """Flops of the chunkwise backward (chunks of C = 32), per token and value head: the reverse
    state pass 6 dk dv + 2 C (dk + dv); the per-chunk gradients 12 dk dv + 6 C dv + 9 C dk
    + 7 C^2 / 3 (T, and dT's two triangular products).  With `recompute`, also the forward state
    recompute the kernels run because the states are not kept from the forward,
    4 dk dv + C (dk + dv); without it, the method's own work."""
    per = 18 * dk * dv + 8 * C * dv + 11 * C * dk + 7 * C * C / 3
    if recompute:
        per += 4 * dk * dv + C * (dk + dv)
    return per * B * T * Hv


def backward_f16_flops(B, T, Hqk, Hv, dk, dv, C=32, recompute=True):
    """The part of backward_alg_flops that the bf16 route runs on the float16 matrix cores: the
    reverse state pass, 6 dk dv + 2 C (dk + dv) (and the state recompute beside it), and the
    gradient kernel's three products that contract over a tile's value columns (dDelta h^T,
    Delta dh'^T, dO h^T), 6 dk dv.  The rest runs on the float32 matrix cores."""
    per = 12 * dk * dv + 2 * C * (dk + dv)
    if recompute:
        per += 4 * dk * dv + C * (dk + dv)
    return per * B * T * Hv


def kda_alg_flops(B, T, Hqk, Hv, dk, dv, C=32):
    """Flops of the chunkwise KDA forward per token and value head: the state products
    (e^gc K) h0, (e^gc Q) h0 and the state update, 6 dk dv; the decay-weighted K K^T and Q K^T
    over the lower triangle, 2 C dk multiply-adds plus C dk exponentials (each counted once);
    the solve and the output product, 2 C dv."""
    per = 6 * dk * dv + 3 * C * dk + 2 * C * dv
    return per * B * T * Hv


def decode_alg_bytes(B, Hqk, Hv, dk, dv, es):
    """Per step: the float32 state read and written once, q and k per query/key head, v and o per
    value head, g and beta in float32."""
    return B * Hv * dk * dv * 4 * 2 + B * Hqk * dk * es * 2 + B * Hv * dv * es * 2 + B * Hv * 4 * 2


# What one gdn_chunk_fwd launches, per kernel family; the roofline is taken over the whole call
# (HIP events around it on its stream), i.e. over both kernels of the split path.
KERNELS = {"mfma": "chunk_mfma_kernel",
           "mfma (gated epilogue)": "chunk_mfma_kernel with the gated RMSNorm",
           "mfma_pipe": "chunk_pipe_kernel",
           "mfma_split": "chunk_prep_kernel + chunk_state_kernel (rows of 256 chunks or more: in pieces, "
                         "chunk_overlap_kernel)",
           "mfma_f32": "chunk_simt_kernel (float32 matrix-core products)"}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def prefill_roofline(r, traffic):
    """The roofline object of one prefill workload: its binding roofline is HBM (the chunkwise
    method's intensity, 167-188 flop/B, is below the bf16-MFMA/HBM ridge); `achieved` is the
    algorithmic bytes of one call over the call's average duration (HIP events on its stream,
    every kernel the call launches); the bf16-MFMA fraction of the algorithmic flops rides along."""
    achieved = r["bytes"] / r["kern"]
    return {"bound": "hbm", "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
            "frac": achieved / HBM_PEAK, "traffic": traffic,
            "kernel": f"chunk_fwd ({KERNELS.get(r['kernel'], r['kernel'])})", "kernel_ms": r["kern"] * 1e3,
            "workspace_bytes": r["workspace"], "alg_bytes": r["bytes"], "alg_flops": r["flops"],
            "mfma_achieved_TFLOPs": r["flops"] / r["kern"] / 1e12,
            "mfma_frac": r["flops"] / r["kern"] / MFMA_BF16_PEAK,
            "cold_kernel_ms": None if r.get("kern_cold") is None else r["kern_cold"] * 1e3}


def measured_traffic(workload: str, op: str = "chunk_fwd"):
    """HBM bytes per call from the committed rocprofv3 counter record, if it was taken on the
    current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{op}_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_hash:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_b or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_b.group(1))


def time_launches(fn, n_sets, steps, warmup, torch):
    """Warm up, then time exactly `steps` launches: one (start, end) HIP event pair per launch on
    the current stream (the one the library launches on), sync-bracketed wall clock around all."""
    for i in range(warmup):
        fn(i % n_sets)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        evs[i][0].record(st)
        fn(i % n_sets)
        evs[i][1].record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern = [a.elapsed_time(b) * 1e-3 for a, b in evs]
    return wall, sum(kern) / len(kern)


def time_cold(fn, steps, torch, flush_bytes=512 << 20):
    """Average of `steps` launches, each after a 512 MiB device write that evicts the 256 MB
    Infinity Cache (the write itself is outside the timed events)."""
    flush = torch.empty(flush_bytes // 4, dtype=torch.float32, device="cuda:0")
    st = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        flush.fill_(float(i))
        evs[i][0].record(st)
        fn(0)
        evs[i][1].record(st)
    torch.cuda.synchronize()
    del flush
    return sum(a.elapsed_time(b) for a, b in evs) / steps * 1e-3


def bench_prefill(cfg, steps, warmup, torch, gdn, gi, min_bytes=640 << 20, gated=False, cold_steps=5):
    """gdn_chunk_fwd (or, gated, gdn_chunk_fwd_gated: the output's gated RMSNorm in the same call,
    whose algorithmic bytes add the gate z read once and the norm weight)."""
    dev = "cuda:0"
    base = gi.generate_torch(cfg, dev)
    es = 2 if cfg.dtype == "bf16" else 4
    per_set = prefill_alg_bytes(cfg.B, cfg.T, cfg.Hqk, cfg.Hv, cfg.dk, cfg.dv, es, cfg.s0_std > 0, True)
    if gated:
        per_set += cfg.B * cfg.T * cfg.Hv * cfg.dv * es + cfg.dv * 4
        g = torch.Generator(device=dev)
        g.manual_seed(cfg.seed + 29)
        base["z"] = torch.randn((cfg.B, cfg.T, cfg.Hv, cfg.dv), generator=g, device=dev).to(base["q"].dtype)
        nw = 1.0 + 0.1 * torch.randn(cfg.dv, generator=g, device=dev)
    n_sets = max(1, min(8, -(-min_bytes // per_set)))
    sets = [base]
    for s in range(1, n_sets):
        sets.append({n: (None if t is None else t.clone()) for n, t in base.items()})
    outs = [torch.empty((cfg.B, cfg.T, cfg.Hv, cfg.dv), dtype=base["q"].dtype, device=dev) for _ in range(n_sets)]
    sfs = [torch.empty((cfg.B, cfg.Hv, cfg.dk, cfg.dv), dtype=torch.float32, device=dev) for _ in range(n_sets)]
    dt = gdn.GDN_BF16 if es == 2 else gdn.GDN_F32
    wsf = gdn.gdn_chunk_fwd_gated_workspace_bytes if gated else gdn.gdn_chunk_fwd_workspace_bytes
    need = wsf(cfg.B, cfg.T, cfg.Hqk, cfg.Hv, cfg.dk, cfg.dv, cfg.chunk, dt)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev) if need else None

    def fn(i):
        x = sets[i]
        if gated:
            gdn.gdn_chunk_fwd_gated(x["q"], x["k"], x["v"], x["g"], x["beta"], x["z"], nw, x["s0"],
                                    chunk=cfg.chunk, y=outs[i], final_state=sfs[i], workspace=ws)
        else:
            gdn.gdn_chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], chunk=cfg.chunk,
                              o=outs[i], final_state=sfs[i], workspace=ws)

    wall, kern = time_launches(fn, n_sets, steps, warmup, torch)
    kern_cold = time_cold(fn, cold_steps, torch) if cold_steps else None
    flops = prefill_alg_flops(cfg.B, cfg.T, cfg.Hqk, cfg.Hv, cfg.dk, cfg.dv, cfg.chunk)
    del sets, outs, sfs, ws
    torch.cuda.empty_cache()
    kernel = gdn.gdn_chunk_fwd_kernel_name(cfg.B, cfg.T, cfg.Hqk, cfg.Hv, cfg.dk, cfg.dv, cfg.chunk, dt)
    if gated:
        # the norm inside the fused kernel when it holds whole heads (no workspace), else a second kernel
        kernel = "mfma (gated epilogue)" if need == 0 and es == 2 else kernel + " + gated_rmsnorm"
    return dict(wall=wall, kern=kern, kern_cold=kern_cold, bytes=per_set, flops=flops, n_sets=n_sets,
                workspace=need, kernel=kernel)


def bench_scan(torch, gdn, gi, steps=5, warmup=2):
    """gdn_chunk_fwd_scan (each chain cut into segments: per-segment state maps, their
    composition, then every segment from its entry state) against the unsegmented gdn_chunk_fwd,
    on one GPU's share of the 64K-token workload under an 8-way head split (6 value heads) and
    on the whole 64K-token workload (48 value heads)."""
    dev = "cuda:0"
    out = {}
    for name, seg_list in (("qwen36_long_prefill_tp8", (2, 3, 4, 6, 8, 12)), ("qwen36_long_prefill", (2, 3, 4))):
        cfg = gi.CONFIGS[name]
        x = gi.generate_torch(cfg, dev)
        o = torch.empty((cfg.B, cfg.T, cfg.Hv, cfg.dv), dtype=x["q"].dtype, device=dev)
        sf = torch.empty((cfg.B, cfg.Hv, cfg.dk, cfg.dv), dtype=torch.float32, device=dev)
        need = max(gdn.gdn_chunk_fwd_scan_workspace_bytes(cfg.B, cfg.T, cfg.Hqk, cfg.Hv, cfg.dk, cfg.dv, cfg.chunk,
                                                          gdn.GDN_BF16, p) for p in seg_list)
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        es = 2
        alg_bytes = prefill_alg_bytes(cfg.B, cfg.T, cfg.Hqk, cfg.Hv, cfg.dk, cfg.dv, es, cfg.s0_std > 0, True)
        flops = prefill_alg_flops(cfg.B, cfg.T, cfg.Hqk, cfg.Hv, cfg.dk, cfg.dv, cfg.chunk)

        def plain(i):
            gdn.gdn_chunk_fwd_scan(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], chunk=cfg.chunk,
                                   segments=1, o=o, final_state=sf, workspace=ws)

        _, kp = time_launches(plain, 1, steps, warmup, torch)
        auto = gdn.gdn_chunk_fwd_kernel_name(cfg.B, cfg.T, cfg.Hqk, cfg.Hv, cfg.dk, cfg.dv, cfg.chunk, gdn.GDN_BF16)
        r = {"unsegmented_ms": kp * 1e3, "unsegmented_tokens_per_s": cfg.B * cfg.T / kp,
             "gdn_chunk_fwd_route": auto}
        best = None
        for p in seg_list:
            def scan(i, p=p):
                gdn.gdn_chunk_fwd_scan(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], chunk=cfg.chunk,
                                       segments=p, o=o, final_state=sf, workspace=ws)
            _, ks = time_launches(scan, 1, steps, warmup, torch)
            r[f"segments_{p}_ms"] = ks * 1e3
            if best is None or ks < best[1]:
                best = (p, ks)
        p, ks = best
        r.update({"best_segments": p, "best_ms": ks * 1e3, "best_tokens_per_s": cfg.B * cfg.T / ks,
                  "speedup": kp / ks, "mfma_frac": flops / ks / MFMA_BF16_PEAK, "hbm_frac": alg_bytes / ks / HBM_PEAK})
        out[name] = r
        del x, o, sf, ws
        torch.cuda.empty_cache()
    return out


def bench_decode(cfg, torch, gdn, gi, repeats=3):
    dev = "cuda:0"
    x = gi.generate_torch(cfg, dev, decode_steps=cfg.steps)
    state = torch.empty_like(x["s0"])
    o = torch.empty((cfg.steps, cfg.B, cfg.Hv, cfg.dv), dtype=x["q"].dtype, device=dev)
    st = torch.cuda.current_stream()
    best = None
    kern_all = []
    for r in range(repeats + 1):  # first round is warm-up
        state.copy_(x["s0"])
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(cfg.steps)]
        t0 = time.perf_counter()
        for s in range(cfg.steps):
            evs[s][0].record(st)
            gdn.gdn_recurrent_step(x["q"][s], x["k"][s], x["v"][s], x["g"][s], x["beta"][s], state, o=o[s])
            evs[s][1].record(st)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        if r == 0:
            continue
        kern_all += [a.elapsed_time(b) * 1e-3 for a, b in evs]
        best = wall if best is None else min(best, wall)
    es = 2 if cfg.dtype == "bf16" else 4
    per_step = decode_alg_bytes(cfg.B, cfg.Hqk, cfg.Hv, cfg.dk, cfg.dv, es)
    kern = sum(kern_all) / len(kern_all)
    del x, state, o
    torch.cuda.empty_cache()
    return dict(wall64=best, kern=kern, bytes=per_step)


def bench_layer_ops(cfg, torch, gdn, W=4, steps=20, warmup=3, min_bytes=640 << 20):
    """The layer steps either side of the recurrence at the workload's shape: the q/k/v prologue
    (short conv width W, SiLU, q/k L2 norm, conv state in and out) and the gated RMSNorm of the
    output.  Both are memory-bound: algorithmic bytes = each input read once + each output written
    once; rotating input sets larger than the Infinity Cache keep the reads cold."""
    dev = "cuda:0"
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    es = 2 if cfg.dtype == "bf16" else 4
    B, T, Hqk, Hv, dk, dv = cfg.B, cfg.T, cfg.Hqk, cfg.Hv, cfg.dk, cfg.dv
    C = 2 * Hqk * dk + Hv * dv
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed + 17)
    rnd = lambda *shape: torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
    wq, wk, wv = rnd(Hqk * dk, W) / W ** 0.5, rnd(Hqk * dk, W) / W ** 0.5, rnd(Hv * dv, W) / W ** 0.5
    pro_bytes = 2 * B * T * C * es + C * W * 4 + 2 * B * C * (W - 1) * 4
    n_sets = max(1, min(8, -(-min_bytes // pro_bytes)))
    sets = [dict(q=rnd(B, T, Hqk, dk).to(dt), k=rnd(B, T, Hqk, dk).to(dt), v=rnd(B, T, Hv, dv).to(dt),
                 st=rnd(B, C, W - 1), so=torch.empty(B, C, W - 1, device=dev),
                 oq=torch.empty(B, T, Hqk, dk, dtype=dt, device=dev), ok=torch.empty(B, T, Hqk, dk, dtype=dt, device=dev),
                 ov=torch.empty(B, T, Hv, dv, dtype=dt, device=dev)) for _ in range(n_sets)]

    def pro(i):
        x = sets[i]
        gdn.gdn_qkv_prologue(x["q"], x["k"], x["v"], wq, wk, wv, x["st"], conv_state_out=x["so"],
                             q=x["oq"], k=x["ok"], v=x["ov"])

    _, kp = time_launches(pro, n_sets, steps, warmup, torch)
    del sets
    rms_bytes = 3 * B * T * Hv * dv * es + dv * 4
    n_sets = max(1, min(8, -(-min_bytes // rms_bytes)))
    w = 1.0 + 0.1 * rnd(dv)
    sets = [dict(o=rnd(B, T, Hv, dv).to(dt), z=rnd(B, T, Hv, dv).to(dt), y=torch.empty(B, T, Hv, dv, dtype=dt, device=dev))
            for _ in range(n_sets)]

    def rms(i):
        x = sets[i]
        gdn.gdn_gated_rmsnorm(x["o"], x["z"], w, y=x["y"])

    _, kr = time_launches(rms, n_sets, steps, warmup, torch)
    del sets
    torch.cuda.empty_cache()
    return {"workload": cfg.name, "conv_width": W,
            "qkv_prologue": {"kernel_us": kp * 1e6, "alg_bytes": pro_bytes, "hbm_GBps": pro_bytes / kp / 1e9,
                             "hbm_frac": pro_bytes / kp / HBM_PEAK},
            "gated_rmsnorm": {"kernel_us": kr * 1e6, "alg_bytes": rms_bytes, "hbm_GBps": rms_bytes / kr / 1e9,
                              "hbm_frac": rms_bytes / kr / HBM_PEAK}}


def bench_backward(cfg, torch, gdn, steps=10, warmup=2):
    """gdn_chunk_bwd at the workload's shape: dL/dO ~ N(0,1), dL/dS_final ~ 0.1 N(0,1)."""
    import gdn_inputs as gi
    dev = "cuda:0"
    x = gi.generate_torch(cfg, dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed + 41)
    do = torch.randn((cfg.B, cfg.T, cfg.Hv, cfg.dv), generator=gen, device=dev).to(x["q"].dtype)
    dsf = 0.1 * torch.randn((cfg.B, cfg.Hv, cfg.dk, cfg.dv), generator=gen, device=dev)
    dt = gdn.GDN_BF16 if cfg.dtype == "bf16" else gdn.GDN_F32
    ws = torch.empty(gdn.gdn_chunk_bwd_workspace_bytes(cfg.B, cfg.T, cfg.Hqk, cfg.Hv, cfg.dk, cfg.dv, dt),
                     dtype=torch.uint8, device=dev)

    def fn(i):
        gdn.gdn_chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], do, x["s0"], dsf, workspace=ws)

    _, kern = time_launches(fn, 1, steps, warmup, torch)
    flops = backward_alg_flops(cfg.B, cfg.T, cfg.Hqk, cfg.Hv, cfg.dk, cfg.dv, recompute=False)
    flops_rc = backward_alg_flops(cfg.B, cfg.T, cfg.Hqk, cfg.Hv, cfg.dk, cfg.dv, recompute=True)
    del x, do, dsf, ws
    torch.cuda.empty_cache()
    # bf16 inputs: the two sequential passes and three of the gradient kernel's products run on
    # the float16 matrix cores, the chunk matrices and the other gradient products on the float32
    # matrix cores (whose peak equals the float32 vector peak).  The roofline is then the time the
    # work would take with each part at its own unit's peak, over the measured time; float32
    # inputs run everything in float32.
    f16 = cfg.dtype == "bf16" and cfg.dk in (64, 128) and cfg.dv in (32, 64, 128)
    passes = ("bwd_pass16_kernel (state recompute and reverse state pass, float16 matrix cores)" if f16 else
              "bwd_pass_kernel (state recompute beside the reverse state pass, float32)")
    grad = ("bwd_chunk_kernel (float32 matrix cores; dDelta h^T, Delta dh^T, dO h^T on the float16 ones)" if f16 else
            "bwd_chunk_kernel (float32 matrix cores)")

    def t_min(total, recompute):
        h = backward_f16_flops(cfg.B, cfg.T, cfg.Hqk, cfg.Hv, cfg.dk, cfg.dv, recompute=recompute) if f16 else 0.0
        return h / MFMA_BF16_PEAK + (total - h) / FP32_VALU_PEAK, h

    tm, h16 = t_min(flops, False)
    tm_rc, _ = t_min(flops_rc, True)
    return {"workload": cfg.name, "tokens_per_s": cfg.B * cfg.T / kern, "kernel_ms": kern * 1e3,
            "alg_flops": flops, "alg_flops_f16_matrix_cores": h16, "bound": "mfma", "unit": "TFLOP/s",
            "achieved_TFLOPs": flops / kern / 1e12, "peak_TFLOPs": flops / tm / 1e12, "frac": tm / kern,
            "peak_note": "each part of the work at the peak of the unit that runs it (float16 matrix cores "
                         "2516.6, float32 157.3 TFLOP/s): peak = work / that time",
            "frac_of_bf16_mfma_peak": flops / kern / MFMA_BF16_PEAK,
            "frac_of_fp32_peak": flops / kern / FP32_VALU_PEAK,
            "flops_with_state_recompute": flops_rc, "frac_with_state_recompute": tm_rc / kern,
            "kernels": f"bwd_gram_kernel + {passes} + {grad}"}


def bench_kda(cfg, torch, gdn, steps=10, warmup=2):
    """gdn_kda_chunk_fwd on the KDA workload (inputs drawn on the device with the recipe of
    gdn_inputs.generate_kda: per-channel log gates logsigmoid(N(mu + offset, 1)))."""
    dev = "cuda:0"
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    B, T, Hqk, Hv, dk, dv = cfg.B, cfg.T, cfg.Hqk, cfg.Hv, cfg.dk, cfg.dv
    rnd = lambda *shape: torch.randn(shape, generator=gen, device=dev)
    q = torch.nn.functional.normalize(rnd(B, T, Hqk, dk), dim=-1).to(dt)
    k = torch.nn.functional.normalize(rnd(B, T, Hqk, dk), dim=-1).to(dt)
    v = rnd(B, T, Hv, dv).to(dt)
    beta = torch.sigmoid(rnd(B, T, Hv))
    g = torch.nn.functional.logsigmoid(rnd(B, T, Hv, dk) + cfg.mu + rnd(1, 1, Hv, dk))
    o = torch.empty((B, T, Hv, dv), dtype=dt, device=dev)
    sf = torch.empty((B, Hv, dk, dv), device=dev)

    def fn(i):
        gdn.gdn_kda_chunk_fwd(q, k, v, g, beta, None, chunk=cfg.chunk, o=o, final_state=sf)

    _, kern = time_launches(fn, 1, steps, warmup, torch)
    flops = kda_alg_flops(B, T, Hqk, Hv, dk, dv, cfg.chunk)
    del q, k, v, beta, g, o, sf
    torch.cuda.empty_cache()
    # chunk 64 runs its products on the float16 matrix cores (the bf16 rate); chunks 16 and 32
    # run the float32 vector kernel
    mfma = cfg.chunk == 64
    peak = MFMA_BF16_PEAK if mfma else FP32_VALU_PEAK
    return {"workload": cfg.name, "chunk": cfg.chunk, "tokens_per_s": B * T / kern, "kernel_ms": kern * 1e3,
            "alg_flops": flops, "bound": "mfma" if mfma else "alu", "unit": "TFLOP/s",
            "achieved_TFLOPs": flops / kern / 1e12, "peak_TFLOPs": peak / 1e12, "frac": flops / kern / peak,
            "kernels": "kda_prep_kernel + kda_state_kernel" if mfma else "kda_chunk_kernel"}


def bench_varlen(torch, gdn, gi, steps=10, warmup=2):
    """gdn_chunk_fwd_varlen on a packed batch: 64 sequences with lengths uniform in [64, 2048]
    (gdn_inputs.varlen_lengths), Qwen3-Next heads (16 query/key, 32 value, d 128), bf16, zero
    initial states; inputs drawn on the device with the recipe of gdn_inputs.generate."""
    import numpy as np
    dev = "cuda:0"
    lengths = gi.varlen_lengths()
    total, N, Hqk, Hv, d = int(lengths.sum()), len(lengths), 16, 32, 128
    cfg = gi.Config("varlen", B=1, T=total, Hqk=Hqk, Hv=Hv, dk=d, dv=d, chunk=64, dtype="bf16", mu=3.0,
                    s0_std=0.0, seed=5002)
    x = gi.generate_torch(cfg, dev)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)).to(dev)
    o = torch.empty((total, Hv, d), dtype=torch.bfloat16, device=dev)
    sf = torch.empty((N, Hv, d, d), device=dev)
    need = gdn.gdn_chunk_fwd_varlen_workspace_bytes(N, int(lengths.max()), Hqk, Hv, d, d, 64, gdn.GDN_BF16)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev) if need else None
    q, k, v, g, b = (x[n][0] for n in ("q", "k", "v", "g", "beta"))

    def fn(i):
        gdn.gdn_chunk_fwd_varlen(q, k, v, g, b, cu, int(lengths.max()), None, o=o, final_state=sf, workspace=ws)

    _, kern = time_launches(fn, 1, steps, warmup, torch)
    nbytes = prefill_alg_bytes(1, total, Hqk, Hv, d, d, 2, False, False) + N * Hv * d * d * 4
    flops = prefill_alg_flops(1, total, Hqk, Hv, d, d, 64)
    del x, o, sf, ws
    torch.cuda.empty_cache()
    return {"workload": f"{N} packed sequences, lengths {int(lengths.min())}..{int(lengths.max())}, {total} tokens",
            "tokens_per_s": total / kern, "kernel_ms": kern * 1e3, "hbm_frac": nbytes / kern / HBM_PEAK,
            "mfma_frac": flops / kern / MFMA_BF16_PEAK,
            "kernel": gdn.gdn_chunk_fwd_kernel_name(N, int(lengths.max()), Hqk, Hv, d, d, 64, gdn.GDN_BF16)}


def cpu_baseline(cfg, gi, min_seconds=10.0, max_repeats=30):
    """The float64 oracle on the same workload (whole batch), repeated until about min_seconds."""
    import numpy as np
    import oracle
    d = gi.generate(cfg)
    f = lambda a: gi.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)
    q, k, v = f(d["q"]), f(d["k"]), f(d["v"])
    threads = len(os.sched_getaffinity(0))
    reps, t_total = 0, 0.0
    while reps < max_repeats and t_total < min_seconds:
        t0 = time.perf_counter()
        oracle.recurrent(q, k, v, d["g"], d["beta"], d["s0"], threads=threads)
        t_total += time.perf_counter() - t0
        reps += 1
    tokens = cfg.B * cfg.T * reps
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    return {"value": tokens / t_total, "unit": "tokens/s", "cores": threads, "kind": "oracle", "cpu_model": model,
            "sample": f"whole {cfg.name} batch (B={cfg.B}, T={cfg.T}, Hv={cfg.Hv}) x {reps} runs, "
                      f"{t_total:.1f} s, float64 token-by-token recurrence, OpenMP over {cfg.B * cfg.Hv} chains"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen36_long_prefill")
    ap.add_argument("--quick", action="store_true",
                    help="headline workload only, warm calls only (no cold-cache timing): for profiler runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--gated", action="store_true",
                    help="time gdn_chunk_fwd_gated (prefill with the output's gated RMSNorm) instead")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--leg", choices=("layer_ops", "backward", "kda", "varlen", "scan", "decode"),
                    help="run only this secondary leg and print its result (for profiling)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the gated delta rule shards by (batch, head) with no "
              "exchange, so only --gpus 1 is run here", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": src.numel() * 4, "copies": 3}))
        return
    import gdn_inputs as gi
    import gated_deltanet_linear_delta_amd as gdn

    gdn.load_library()
    cfg = gi.CONFIGS[args.workload]
    if args.leg:
        # the layer steps and the backward run at the Qwen3-Next shape unless a workload is named
        lcfg = cfg if args.workload != ap.get_default("workload") else gi.CONFIGS["qwen3next_prefill"]
        legs = {"layer_ops": lambda: bench_layer_ops(lcfg, torch, gdn),
                "backward": lambda: bench_backward(lcfg, torch, gdn),
                "kda": lambda: bench_kda(gi.CONFIGS["kda_prefill"], torch, gdn),
                "varlen": lambda: bench_varlen(torch, gdn, gi),
                "scan": lambda: bench_scan(torch, gdn, gi),
                "decode": lambda: bench_decode(gi.CONFIGS["decode"], torch, gdn, gi)}
        print(json.dumps({"leg": args.leg, **legs[args.leg]()}), flush=True)
        return
    print(f"bench: prefill {cfg}{' (gated)' if args.gated else ''}", file=sys.stderr, flush=True)
    r = bench_prefill(cfg, args.steps, args.warmup, torch, gdn, gi, gated=args.gated, cold_steps=0 if args.quick else 5)
    tokens = cfg.B * cfg.T
    ms = r["wall"] / args.steps * 1e3
    line = {
        "metric": "GDN prefill tokens/sec + % MFMA peak; decode steps/sec + HBM GB/s, 1 MI355X",
        "value": tokens * args.steps / r["wall"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "T": cfg.T, "Hqk": cfg.Hqk, "Hv": cfg.Hv,
                   "dk": cfg.dk, "dv": cfg.dv, "chunk": cfg.chunk, "state": "float32",
                   "initial_state": cfg.s0_std > 0, "input_sets": r["n_sets"]},
        "roofline": prefill_roofline(r, measured_traffic(cfg.name, "chunk_fwd_gated" if args.gated else "chunk_fwd")),
    }
    if args.gated:
        line["config"]["gated_output_norm"] = True
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(cfg, gi)
    if not args.quick:
        dcfg = gi.CONFIGS["decode"]
        print(f"bench: decode {dcfg}", file=sys.stderr, flush=True)
        dr = bench_decode(dcfg, torch, gdn, gi)
        bw = dr["bytes"] / dr["kern"]
        line["decode"] = {"workload": dcfg.name, "B": dcfg.B, "Hv": dcfg.Hv, "d": dcfg.dk, "steps": dcfg.steps,
                          "steps_per_s": dcfg.steps / dr["wall64"], "ms_64_steps": dr["wall64"] * 1e3,
                          "tokens_per_s": dcfg.steps * dcfg.B / dr["wall64"],
                          "roofline": {"bound": "hbm", "achieved": bw / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                                       "frac": bw / HBM_PEAK, "traffic": measured_traffic("decode", "recurrent_step"),
                                       "kernel": "recurrent_step_kernel", "kernel_us": dr["kern"] * 1e6,
                                       "alg_bytes": dr["bytes"]}}
        pc = {}
        for name in ("batched_prefill", "qwen3next_prefill"):
            if name == cfg.name:
                continue
            c = gi.CONFIGS[name]
            print(f"bench: prefill {c}", file=sys.stderr, flush=True)
            rr = bench_prefill(c, 10, 3, torch, gdn, gi)
            pc[name] = {"tokens_per_s": c.B * c.T / rr["kern"], "kernel_ms": rr["kern"] * 1e3,
                        "roofline": prefill_roofline(rr, measured_traffic(name))}
        # the Qwen3-Next shape with float32 q, k, v, o: the float32 kernel (float32 matrix-core
        # products), bound by its per-chunk chain; fraction of the float32 peak
        c32 = dataclasses.replace(gi.CONFIGS["qwen3next_prefill"], name="qwen3next_prefill_f32", dtype="f32")
        print(f"bench: prefill {c32}", file=sys.stderr, flush=True)
        rr = bench_prefill(c32, 5, 2, torch, gdn, gi)
        pc[c32.name] = {"tokens_per_s": c32.B * c32.T / rr["kern"], "kernel_ms": rr["kern"] * 1e3,
                        "roofline": {"bound": "mfma", "achieved": rr["flops"] / rr["kern"] / 1e12,
                                     "peak": FP32_VALU_PEAK / 1e12, "unit": "TFLOP/s",
                                     "frac": rr["flops"] / rr["kern"] / FP32_VALU_PEAK,
                                     "hbm_frac": rr["bytes"] / rr["kern"] / HBM_PEAK, "kernel": rr["kernel"]}}
        line["prefill_configs"] = pc
        print("bench: layer steps (prologue, gated RMSNorm)", file=sys.stderr, flush=True)
        line["layer_ops"] = bench_layer_ops(gi.CONFIGS["qwen3next_prefill"], torch, gdn)
        gp = {}
        for name in ("qwen3next_prefill", "batched_prefill"):
            c = gi.CONFIGS[name]
            print(f"bench: gated prefill {c}", file=sys.stderr, flush=True)
            rr = bench_prefill(c, 5, 2, torch, gdn, gi, gated=True)
            fused = gdn.gdn_chunk_fwd_gated_workspace_bytes(c.B, c.T, c.Hqk, c.Hv, c.dk, c.dv, c.chunk,
                                                            gdn.GDN_BF16 if c.dtype == "bf16" else gdn.GDN_F32) == 0
            gp[name] = {"tokens_per_s": c.B * c.T / rr["kern"], "kernel_ms": rr["kern"] * 1e3,
                        "alg_bytes": rr["bytes"], "hbm_frac": rr["bytes"] / rr["kern"] / HBM_PEAK,
                        "route": "norm fused into the prefill kernel" if fused
                        else "O through the workspace, then the norm kernel"}
        line["gated_prefill"] = gp
        bcfg = gi.CONFIGS["qwen3next_prefill"]
        print(f"bench: backward {bcfg}", file=sys.stderr, flush=True)
        line["backward"] = bench_backward(bcfg, torch, gdn)
        kcfg = gi.CONFIGS["kda_prefill"]
        print(f"bench: kda {kcfg}", file=sys.stderr, flush=True)
        line["kda"] = bench_kda(kcfg, torch, gdn)
        print("bench: packed variable-length prefill", file=sys.stderr, flush=True)
        line["varlen"] = bench_varlen(torch, gdn, gi)
        print("bench: affine chunk scan on the 64K-token workloads", file=sys.stderr, flush=True)
        line["scan"] = bench_scan(torch, gdn, gi)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
