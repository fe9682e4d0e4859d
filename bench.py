#!/usr/bin/env python3
"""Benchmark of the Sol-Attn forward pass on one MI355X (one process, one GPU).

A step is one pass of the whole hot path over the workload: sol_attn_fwd (K/V pooling, pooled-key
mean, fused routing + pooled-token + exact-attention kernel) and sol_dense_fwd, the dense
reference the speedup is measured against, on the same resident tensors.  The timed region runs
the K sparse passes back to back and then the K dense passes, each after warm-up passes of its
own, so that each is timed in its own steady state: right after a dense pass the chip is still at
the lower clock that the dense kernel's power draw sets, and a sparse pass started there runs
about 10% slower (the work and the step count are the same either way).

Printed: one JSON line.  value = effective TFLOP/s of the sparse forward: kept-block FLOPs
F = 4*d*sum over query tiles t of sum over kept blocks j of rows_t*n_j, divided by its latency.
Extra fields give the dense latency, the speedup, densities, per-kernel times, the roofline of the
fused kernel (live HIP events on the launch stream) and the fp64 CPU oracle timed on a bounded
sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload wan] [--beta B] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse attn fwd ms + eff. TFLOPS & speedup vs own dense, N=75600 h40 d128"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


def calibrate_beta(sol, q, k, v, block, target, ws, out, per_row=False):
    """Bisection on beta so that the kept-block density hits target (density is non-increasing in
    beta): at query-tile granularity (rho_tile), or per row (rho_row) when per_row is set."""
    import torch
    N = q.shape[2]
    M = sol.n_blocks(N, block)

    def density(beta):
        _, dbg = sol.attn_fwd(q, k, v, beta, block, out=out, workspace=ws, debug=True)
        if per_row:
            mask = dbg["mask"].view(torch.int32)
            bits = sum(int(torch.bitwise_and(torch.bitwise_right_shift(mask, s), 1).sum().item())
                       for s in range(32))
            return bits / (q.shape[0] * q.shape[1] * N * M)
        tk = dbg["tile_kept"]
        return float(tk.sum().item()) / (tk.numel() * M)

    lo, hi = 0.0, 4.0
    d_hi = density(hi)
    while d_hi > target and hi < 16:
        lo, hi = hi, hi * 2
        d_hi = density(hi)
    if density(lo) < target:
        lo = -8.0
    for _ in range(20):
        mid = 0.5 * (lo + hi)
        dm = density(mid)
        if dm > target:
            lo = mid
        else:
            hi = mid
        if abs(dm - target) < 2e-4:
            return mid
    torch.cuda.synchronize()
    return 0.5 * (lo + hi)


def mfma_probe_tflops(sol, workgroups=2048, iters=1000, reps=3):
    """bf16 MFMA rate of the library's matrix-core probe (best of reps), TFLOP/s."""
    import torch
    sink, flops = sol.mfma_probe(workgroups, iters)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        sol.mfma_probe(workgroups, iters, sink=sink)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    return best


def cpu_model() -> str:
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, q, k, v, beta, F_tile, seconds=12.0):
    """The fp64 oracle on a bounded, seeded sample of query rows spread over every head, scaled to
    the same effective-TFLOP/s unit as the GPU value (F_tile x sampled fraction / oracle seconds).

    Two probes on head 0 size the sample to about ``seconds`` of oracle time; the sample then
    takes the same number of uniformly drawn rows from each head of batch 0 (each head's call also
    pools that head's K and V, as the method does)."""
    import numpy as np
    from oracle import oracle
    B, H, N = w.B, w.H, w.N
    total_rows = B * H * N
    rng = np.random.default_rng(0)

    def head(h):
        return tuple(t[0, h].float().cpu().numpy() for t in (q, k, v))

    # two probes on head 0 split the oracle's cost into a per-call part (pooling K and V over the
    # head) and a per-row part, to size the sample to about `seconds` of oracle time
    qh, kh, vh = head(0)
    cost = []
    for r in (128, 512):
        rows = np.sort(rng.choice(N, size=r, replace=False))
        t0 = time.perf_counter()
        oracle.attn_rows(qh, kh, vh, beta, w.block, rows=rows)
        cost.append(time.perf_counter() - t0)
    per_row = max((cost[1] - cost[0]) / 384, 1e-9)
    per_call = max(cost[0] - 128 * per_row, 0.0)
    per_head = int(min(N, max(16, (seconds / H - per_call) / per_row)))
    dt = 0.0
    n = 0
    for h in range(H):
        qh, kh, vh = head(h)
        rows = np.sort(rng.choice(N, size=per_head, replace=False))
        t0 = time.perf_counter()
        oracle.attn_rows(qh, kh, vh, beta, w.block, rows=rows)
        dt += time.perf_counter() - t0
        n += per_head
    frac = n / total_rows
    return {
        "value": F_tile * frac / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.threads(),
        "cpu_model": cpu_model(),
        "host_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": f"{n} of {total_rows} query rows ({per_head} seeded-uniform rows in each of the "
                  f"{H} heads of batch 0), full method per row incl. per-head K/V pooling, "
                  f"{dt:.1f} s of oracle time; value = kept-block FLOPs x {frac:.3e} / seconds",
    }


def ablation(sol, w, q, k, v, ws, betas, rows_per_head=48, steps=5):
    """Drop-vs-approximate ablation: for each beta, the output of the method (unselected blocks as
    pooled tokens) and of the same selection with unselected blocks dropped, both against exact
    dense softmax attention computed by the fp64 oracle on seeded sampled rows of every head;
    plus the fused kernel's time in each mode."""
    import numpy as np
    import torch
    from oracle import oracle
    B, H, N, d = q.shape
    rng = np.random.default_rng(1)
    rows = [np.sort(rng.choice(N, size=min(rows_per_head, N), replace=False)) for _ in range(B * H)]
    ref = []
    t0 = time.perf_counter()
    for bh in range(B * H):
        b, h = divmod(bh, H)
        qh, kh, vh = (t[b, h].float().cpu().numpy() for t in (q, k, v))
        ref.append(oracle.dense_rows(qh, kh, vh, rows=rows[bh])["out"])
    log(f"oracle dense reference on {sum(len(r) for r in rows)} rows: {time.perf_counter() - t0:.1f} s")
    idx = [torch.from_numpy(r).to(q.device) for r in rows]
    out = torch.empty_like(q)
    ev = sol.HipEvents(4)
    results = []
    for beta in betas:
        entry = {"beta": beta}
        for mode, drop in (("pooled", False), ("dropped", True)):
            _, dbg = sol.attn_fwd(q, k, v, beta, w.block, out=out, workspace=ws, debug=True,
                                  drop_unselected=drop)
            o32 = dbg["out_f32"].view(B * H, N, d)
            num = den = 0.0
            max_abs = 0.0
            for bh in range(B * H):
                g = o32[bh].index_select(0, idx[bh]).double().cpu().numpy()
                diff = g - ref[bh]
                num += float((diff ** 2).sum())
                den += float((ref[bh] ** 2).sum())
                max_abs = max(max_abs, float(np.abs(diff).max()))
            ms = []
            for i in range(steps + 2):
                sol.attn_fwd(q, k, v, beta, w.block, out=out, workspace=ws, drop_unselected=drop,
                             events=ev.handles)
                torch.cuda.synchronize()
                if i >= 2:
                    ms.append(ev.elapsed_ms(2, 3))
            entry[mode] = {"rel_l2_vs_dense": math.sqrt(num / den), "max_abs_vs_dense": max_abs,
                           "fused_ms": sum(ms) / len(ms)}
            if not drop:
                M = sol.n_blocks(N, w.block)
                tk = dbg["tile_kept"]
                entry["rho_tile"] = float(tk.sum().item()) / (tk.numel() * M)
                units = sol.union_units(dbg["mask"], N, w.block, heights=(1,))
                entry["row_kept_key_fraction"] = units[1] / (B * H * N * N)
            del dbg
        log(f"beta {beta}: pooled rel-L2 {entry['pooled']['rel_l2_vs_dense']:.3e}, dropped "
            f"{entry['dropped']['rel_l2_vs_dense']:.3e}, rho_tile {entry['rho_tile']:.4f}")
        results.append(entry)
    return {"ablation": "unselected blocks pooled (the method) vs dropped", "workload": w.name,
            "rows_sampled": sum(len(r) for r in rows), "reference": "fp64 oracle dense attention",
            "results": results}


def routing_comparison(sol, w, q, k, v, ws, spec, steps=5, warmup=2):
    """The prior-art pipeline the fused pass replaces: full proxy map in memory, top-k or top-p
    selection from it, then attention with that selection (pooled unselected blocks, as in the
    method, so that only the routing differs).  Each stage is timed with events; the fused
    Sol-Attn forward is timed at the beta whose kept-block density (128-row tiles) matches."""
    import torch
    mode, prm = spec.split(":")
    prm = int(prm) if mode == "topk" else float(prm)
    B, H, N, d = q.shape
    M = sol.n_blocks(N, w.block)
    smap = torch.empty((B, H, N, M), dtype=torch.float32, device=q.device)
    sel = torch.empty((B, H, N, (M + 31) // 32), dtype=torch.int32, device=q.device)
    out = torch.empty_like(q)

    def timed(fn):
        ts = []
        for i in range(warmup + steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            if i >= warmup:
                ts.append(e0.elapsed_time(e1))
        return sum(ts) / len(ts)

    t_map = timed(lambda: sol.proxy_map(q, k, w.block, s_map=smap, workspace=ws))
    if mode == "topk":
        t_sel = timed(lambda: sol.select_topk(smap, tuple(q.shape), w.block, prm, mask=sel))
    else:
        t_sel = timed(lambda: sol.select_topp(smap, tuple(q.shape), w.block, prm, mask=sel))
    t_attn = timed(lambda: sol.attn_fwd_masked(q, k, v, sel, w.block, out=out, workspace=ws))
    units = sol.union_units(sel, N, w.block, heights=(1, 128))
    F_tile = 4.0 * d * units[128]
    # union density at 128-row tiles, counted in blocks
    shifts = torch.arange(32, device=q.device, dtype=torch.int32)
    kept_tiles = 0
    T = (N + 127) // 128
    for b in range(B):
        for h in range(H):
            bits = ((sel[b, h].unsqueeze(-1) >> shifts) & 1).to(torch.uint8).reshape(N, -1)[:, :M]
            bits = torch.nn.functional.pad(bits, (0, 0, 0, T * 128 - N))
            kept_tiles += int(bits.view(T, 128, M).amax(dim=1).sum().item())
    rho_tile = kept_tiles / (B * H * T * M)
    log(f"{spec}: map {t_map:.2f} ms, select {t_sel:.2f} ms, attention {t_attn:.2f} ms, "
        f"rho_tile {rho_tile:.4f}")
    beta = calibrate_beta(sol, q, k, v, w.block, rho_tile, ws, out)
    t_sol = timed(lambda: sol.attn_fwd(q, k, v, beta, w.block, out=out, workspace=ws))
    t_dense = timed(lambda: sol.dense_fwd(q, k, v, out=out), ) if N <= 131072 else None
    map_bytes = 4.0 * B * H * M * N
    passes = 1  # the selection reads the map once
    return {
        "routing_comparison": spec, "workload": w.name,
        "prior_art_ms": {"proxy_map": t_map, "select": t_sel, "attention": t_attn,
                         "total": t_map + t_sel + t_attn},
        "prior_art_rho_tile": rho_tile,
        "prior_art_rho_row_keys": units[1] / (B * H * N * N),
        "prior_art_tflops_on_tile_flops": F_tile / ((t_map + t_sel + t_attn) * 1e-3) / 1e12,
        "proxy_map_bytes": map_bytes,
        "proxy_map_round_trip_bytes": map_bytes * (1 + passes),
        "sol_attn_beta_at_same_rho_tile": beta,
        "sol_attn_ms": t_sol,
        "sol_attn_speedup_over_prior_art": (t_map + t_sel + t_attn) / t_sol,
        "dense_ms": t_dense,
    }


# the fused kernels' sources: a counter record stays valid while these are unchanged
FUSED_SOURCES = ("attn.hip", "tiles.hpp", "common.hpp", "kernels.hpp")


def recorded_traffic(kernel_sources, workload, beta, grid):
    """HBM bytes per launch of the fused kernel, as recorded from rocprofv3 FETCH_SIZE/WRITE_SIZE
    counters (scaled by a plain-copy calibration) in profiles/sol_attn_wan_hbm_traffic.md, or
    None when the record is missing, is for another workload, beta or row grouping (latent grid
    or not), or the kernel's sources have changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "sol_attn_wan_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    rec = None
    for line in open(path):
        if line.startswith("traffic-record:"):
            rec = json.loads(line.split(":", 1)[1])
    if rec is None or rec.get("workload") != workload or abs(rec.get("beta", 1e9) - beta) > 1e-3:
        return None
    if bool(rec.get("grid", False)) != grid:
        return None
    h = hashlib.sha256()
    for f in kernel_sources:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return rec["traffic_bytes"] if h.hexdigest() == rec.get("source_sha256") else None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wan")
    ap.add_argument("--beta", type=float, default=None)
    ap.add_argument("--target", type=float, default=None,
                    help="kept-block density (at 128-row query tiles) to calibrate beta to, instead "
                         "of the workload's own target")
    ap.add_argument("--row-target", type=float, default=None,
                    help="calibrate beta to this per-row kept density instead (the secondary "
                         "operating point)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--interleave", action="store_true",
                    help="time each step as a sparse pass followed by a dense pass (the chip then "
                         "starts every sparse pass at the dense kernel's lower clock)")
    ap.add_argument("--no-grid", action="store_true",
                    help="call the fused pass without the workload's latent grid (query rows in "
                         "contiguous 128-row workgroups) instead of sol_attn_fwd_grid")
    ap.add_argument("--ablation", default=None, metavar="BETAS",
                    help="comma-separated betas: run the drop-vs-approximate ablation instead of the "
                         "benchmark and print its JSON line")
    ap.add_argument("--routing", default=None, metavar="topk:K|topp:P",
                    help="time the prior-art pipeline (materialised proxy map, top-k/top-p "
                         "selection, attention) against the fused pass at matched density and "
                         "print its JSON line instead of the benchmark")
    ap.add_argument("--cache", default=None, metavar="DIR",
                    help="keep the generated inputs in DIR (torch.save) and reuse them on later runs")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (calibrates the HBM "
                         "byte counters of a profiler run) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the Sol-Attn forward is measured per GPU (heads "
              "shard with no communication); --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_sparse_attention_sol_amd import solattn as sol
    from block_sparse_attention_sol_amd import synth

    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)
        return

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    sol.load_library()
    w = synth.WORKLOADS[args.workload]
    target = w.target_density[0] if w.target_density else None
    if args.target is not None:
        target = args.target
    log(f"workload {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} block={w.block}; generating")
    t0 = time.perf_counter()

    def gen_progress(b, h):
        if (h + 1) % 8 == 0 or h + 1 == w.H:
            log(f"  generated head {h + 1}/{w.H} ({time.perf_counter() - t0:.0f} s)")

    cache = os.path.join(args.cache, f"{w.name}_seed0.pt") if args.cache else None
    if cache and os.path.exists(cache):
        q, k, v = (t.cuda() for t in torch.load(cache, weights_only=True))
        log(f"  loaded inputs from {cache}")
    else:
        qkv = synth.generate(w, progress=gen_progress)
        if cache:
            os.makedirs(args.cache, exist_ok=True)
            torch.save(list(qkv), cache)
        q, k, v = (t.cuda() for t in qkv)
        del qkv
    B, H, N, d = q.shape
    out = torch.empty_like(q)
    dout = torch.empty_like(q)
    ws = sol.new_workspace(q.shape, w.block)

    if args.routing:
        print(json.dumps(routing_comparison(sol, w, q, k, v, ws, args.routing)), flush=True)
        return

    if args.ablation:
        betas = [float(x) for x in args.ablation.split(",")]
        print(json.dumps(ablation(sol, w, q, k, v, ws, betas)), flush=True)
        return

    if args.beta is not None:
        beta = args.beta
    elif args.row_target is not None:
        beta = calibrate_beta(sol, q, k, v, w.block, args.row_target, ws, out, per_row=True)
    elif target is not None:
        beta = calibrate_beta(sol, q, k, v, w.block, target, ws, out)
    else:
        beta = w.betas[0]
    # the workload's latent grid: the fused kernel groups query rows by it (same results)
    grid = None if args.no_grid else w.grid
    _, dbg = sol.attn_fwd(q, k, v, beta, w.block, out=out, workspace=ws, debug=True, grid=grid)
    torch.cuda.synchronize()
    M = sol.n_blocks(N, w.block)
    T = (N + sol.QUERY_TILE - 1) // sol.QUERY_TILE
    kept_blocks = int(dbg["tile_kept"].sum().item())
    rho_tile = kept_blocks / (B * H * T * M)
    F_tile = sol.kept_block_flops(dbg["tile_kept"], dbg["mask"], N, d, w.block)
    # the fused kernel skips a key block per wave when none of the wave's rows keeps it: waves of
    # 16 rows at head dimension 128, of 32 rows at 64
    wave_rows = 16 if d == 128 else 32
    units = sol.union_units(dbg["mask"], N, w.block, heights=(1, wave_rows, sol.QUERY_TILE))
    F_row, F_exec = 4.0 * d * units[1], 4.0 * d * units[wave_rows]
    mask = dbg["mask"].view(torch.int32)
    row_bits = sum(int(torch.bitwise_and(torch.bitwise_right_shift(mask, s), 1).sum().item())
                   for s in range(32))
    rho_row = row_bits / (B * H * N * M)
    del dbg, mask
    log(f"beta={beta:.4f} rho_tile={rho_tile:.4f} rho_row={rho_row:.4f} F_tile={F_tile / 1e12:.2f} TF "
        f"F_exec={F_exec / 1e12:.2f} TF F_row={F_row / 1e12:.2f} TF")

    probe = mfma_probe_tflops(sol)
    log(f"matrix-core probe: {probe:.0f} TFLOP/s bf16")

    K, Wm = args.steps, args.warmup
    ev = sol.HipEvents(4 * (K + Wm))
    dense_start = [torch.cuda.Event(enable_timing=True) for _ in range(K + Wm)]
    dense_end = [torch.cuda.Event(enable_timing=True) for _ in range(K + Wm)]

    def sparse(i):
        sol.attn_fwd(q, k, v, beta, w.block, out=out, workspace=ws,
                     events=ev.handles[4 * i: 4 * i + 4], grid=grid)

    def dense(i):
        dense_start[i].record()
        sol.dense_fwd(q, k, v, out=dout)
        dense_end[i].record()

    if args.interleave:
        for i in range(Wm):
            sparse(i)
            dense(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(Wm, Wm + K):
            sparse(i)
            dense(i)
    else:
        # warm-up: dense first, so that the timed sparse passes follow sparse passes
        for i in range(Wm):
            dense(i)
        for i in range(Wm):
            sparse(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(Wm, Wm + K):
            sparse(i)
        for i in range(Wm, Wm + K):
            dense(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    idx = range(Wm, Wm + K)
    pool_ms = [ev.elapsed_ms(4 * i, 4 * i + 1) for i in idx]
    kglob_ms = [ev.elapsed_ms(4 * i + 1, 4 * i + 2) for i in idx]
    fused_ms = [ev.elapsed_ms(4 * i + 2, 4 * i + 3) for i in idx]
    sparse_ms = [ev.elapsed_ms(4 * i, 4 * i + 3) for i in idx]
    dense_ms = [dense_start[i].elapsed_time(dense_end[i]) for i in idx]
    avg = lambda xs: sum(xs) / len(xs)
    med = lambda xs: sorted(xs)[len(xs) // 2]
    t_sparse, t_dense, t_fused, t_pool = avg(sparse_ms), avg(dense_ms), avg(fused_ms), avg(pool_ms)

    dense_F = sol.dense_flops(B, H, N, d)
    pool_bytes = 2 * B * H * N * d * 2 + 2 * B * H * M * d * 4  # K,V read + Kbar,Vbar (fp32) written
    # The fused kernel's matrix-core work as executed: the exact loop's 4*d FLOPs per (row, key) of
    # each block some row of the row's wave keeps (a wave skips blocks none of its rows keeps:
    # F_exec), plus the routing sweep's products over every padded block of every row -- the
    # proxies from the three bf16 pieces of Kbar (3 x 2*d per row and block) and the pooled tokens'
    # P Vbar (2*d per row and block; skipped in the drop ablation only).
    Mp = (M + 31) // 32 * 32
    F_route = 4 * 2.0 * B * H * N * Mp * d
    F_mfma = F_exec + F_route
    achieved = F_mfma / (t_fused * 1e-3) / 1e12
    tile_rate = F_tile / (t_fused * 1e-3) / 1e12
    executed = F_exec / (t_fused * 1e-3) / 1e12
    # minimum HBM bytes of the fused kernel: Q, K, V read once, O written once
    min_bytes = 4.0 * B * H * N * d * 2
    traffic = recorded_traffic(
        [os.path.join(ROOT, "block_sparse_attention_sol_amd", "csrc", f)
         for f in FUSED_SOURCES], w.name, beta, grid is not None)
    result = {
        "metric": METRIC,
        "value": F_tile / (t_sparse * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": wall * 1e3 / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: {w.grid[0]}x{w.grid[1]}x{w.grid[2]} latent grid, positional amplitude "
                        f"{w.amp_range or w.amp}, seed 0",
            "B": B, "H": H, "N": N, "d": d, "block": w.block, "beta": round(beta, 5),
            "target_kept_block_density": None if args.row_target is not None else target,
            "target_row_density": args.row_target, "query_tile": sol.QUERY_TILE,
            "global_batch": B, "seq_len": N, "parallelism": "none (1 GPU)",
            "row_grouping": "latent grid %dx%dx%d: 2 frames x 4 rows x 16 tokens per workgroup"
                            % tuple(grid) if grid is not None and d == 128 and grid[2] % 16 == 0
                            else "contiguous 128-row tiles",
            "timing_order": "each sparse pass followed by a dense pass" if args.interleave
                            else "K sparse passes, then K dense passes",
        },
        "sparse_ms": t_sparse,
        "sparse_ms_median": med(sparse_ms),
        "dense_ms": t_dense,
        "speedup_vs_dense": t_dense / t_sparse,
        "dense_tflops": dense_F / (t_dense * 1e-3) / 1e12,
        "dense_mfma_frac": dense_F / (t_dense * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "dense_frac_of_measured_peak": dense_F / (t_dense * 1e-3) / 1e12 / probe,
        "mfma_probe_tflops": probe,
        "kernel_ms": {"pool_kv": t_pool, "row_stats": avg(kglob_ms), "fused": t_fused},
        "rho_tile": rho_tile,
        "rho_row": rho_row,
        "kept_block_tflop": F_tile / 1e12,
        "executed_block_tflop": F_exec / 1e12,
        "row_kept_tflop": F_row / 1e12,
        "fused_executed_tflops": executed,
        "fused_executed_mfma_frac": executed / PEAK_BF16_TFLOPS,
        "pool_gbs": pool_bytes / (t_pool * 1e-3) / 1e9,
        "roofline": {
            # algorithmically a dense contraction: F_mfma / min_bytes is thousands of FLOP per
            # byte, far right of the ridge (2.5 PFLOP/s / 8 TB/s = 312 FLOP/B)
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": traffic,
            "measured_peak": probe,
            "frac_of_measured_peak": achieved / probe,
            "flops": "matrix-core FLOPs as executed per launch: exact loop at the kernel's wave "
                     "granularity (F_exec) + routing sweep (three-piece proxies and pooled P Vbar "
                     "over every padded block of every row)",
            "executed_mfma_tflop": F_mfma / 1e12,
            "routing_mfma_tflop": F_route / 1e12,
            "tile_flops_rate": tile_rate,
            "tile_flops_frac": tile_rate / PEAK_BF16_TFLOPS,
            "min_hbm_bytes": min_bytes,
            "traffic_gbs": None if traffic is None else traffic / (t_fused * 1e-3) / 1e9,
            "traffic_frac_of_hbm_peak": None if traffic is None
            else traffic / (t_fused * 1e-3) / 1e9 / PEAK_HBM_GBS,
            # what the measured bytes say: if moving them at the HBM peak takes longer than the
            # executed FLOPs at the matrix peak, re-read traffic rather than the matrix cores
            # limits the kernel
            "measured_limiter": None if traffic is None else
            ("hbm (re-read traffic)" if traffic / (PEAK_HBM_GBS * 1e9) > F_mfma / (PEAK_BF16_TFLOPS * 1e12)
             else "mfma"),
            "kernel": ("sol_attn16_kernel<128,128>" if d == 128 else "sol_attn_kernel<64,64,4>")
                      + " (fused routing + pooled tokens + exact attention)",
        },
    }
    if not args.no_cpu_baseline:
        log("timing the fp64 CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, beta, F_tile)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
