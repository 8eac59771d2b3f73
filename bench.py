"""Benchmark of the AB-Attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload wan]

A step is one pass of the whole hot path over the layer's Q/K/V, which are
resident in HBM before timing starts: the plan (mean keys, IBCS k-means and
scores, SIP probabilities, draws and CSR) followed by the gathered sparse
attention. The dense flash-attention comparator is timed separately. Rank 0
prints one JSON line: `value` is the dense-equivalent flop of the layer
(4 B H N^2 d) over the step time; `roofline` rates the sparse attention
kernel (useful flop per launch over its HIP-event time, against the bf16
MFMA peak; `traffic` is the HBM bytes of one launch from the FETCH_SIZE and
WRITE_SIZE counters, valid for the attention source they were taken on);
`cpu_baseline` times the fp64 oracle on a sample of plan rows spread over
worker processes; `configs` holds the same per-layer figures for the other
workloads (tiny at 25% and 100%, small, HunyuanVideo-like) and the plan
reused over 4 drifting steps at the Wan2.1-like shape (5/10/20%).

Other modes print one JSON object instead: --schedule (the pages' 50-step
schedule on drifting inputs), --selection-study, --sampling-study,
--reuse-sweep.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-attn ms & effective TFLOP/s per layer, 75.6K tok×40 heads, ~10% keep"
PEAK_BF16_TFLOPS = 2500.0          # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0
ATTN_SOURCE = os.path.join(ROOT, "sampled_block_sparse_amd", "csrc", "attn_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sparse_attention_wan_traffic.txt")
RESULTS = os.path.join(ROOT, "results")

WORKLOADS = {
    "wan": "Wan2.1-720p-like layer: B=1 H=40 N=75600 (21x45x80) d=128 bf16, budget 10%",
    "hunyuan": "HunyuanVideo-720p-like layer: B=1 H=24 N=118800 (33x45x80) d=128 bf16, budget 8%",
    "small": "small video-shaped layer: B=1 H=8 N=8192 (8x32x32) d=128 bf16, budget 10%",
    "tiny": "tiny iid layer: B=1 H=2 N=1024 d=64 fp32, budget 25%",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan", choices=sorted(WORKLOADS))
    ap.add_argument("--budget-pct", type=int, default=None)
    ap.add_argument("--dense-iters", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=float, default=0.05,
                    help="fraction of the layer's plan rows the oracle baseline runs")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-config figures of the other workloads")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 1 GiB device copy first (counter calibration)")
    ap.add_argument("--sampling", default="poisson", choices=["poisson", "systematic"],
                    help="sampling design of the plan (default poisson)")
    ap.add_argument("--fused-plan", action="store_true",
                    help="build the timed steps' plans with the fused score + SIP kernel")
    ap.add_argument("--sampling-study", action="store_true",
                    help="design comparison instead of the benchmark line: small video-shaped "
                         "layer, budgets 5/10/20%%, 8 seeds each, Poisson against systematic "
                         "sampling: output error against dense, blocks per row, plan time")
    ap.add_argument("--schedule", action="store_true",
                    help="the pages' 50-step schedule on both video layers, Q/K/V drifting "
                         "every step: dense for the first 10 steps, then sparse with the plan "
                         "rebuilt every 4 steps; time and error against dense at every step")
    ap.add_argument("--selection-study", action="store_true",
                    help="what each selection rule retains at equal budget: exact top-K, IBCS "
                         "(C=8) and mean-query (C=1) scores with top-K or SIP, 128-token "
                         "blocks; attention mass, recall of the exact top-K and error, on the "
                         "small layer and on sampled rows of the Wan2.1-like layer")
    ap.add_argument("--reuse-sweep", action="store_true",
                    help="plan-reuse report instead of the benchmark line: small video-shaped "
                         "layer (or with --reuse-wan the Wan2.1-like one), plan built at step "
                         "0, attention at steps 0-3 on drifting Q/K/V, budgets 5/10/20%%")
    ap.add_argument("--reuse-wan", action="store_true",
                    help="with --reuse-sweep: run it on the Wan2.1-like layer")
    ap.add_argument("--out", default=None, help="also write the JSON object to this file")
    return ap.parse_args()


def emit(obj, path=None):
    line = json.dumps(obj)
    print(line, flush=True)
    if path:
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        with open(path, "w") as f:
            f.write(line + "\n")


def file_sha256(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def read_traffic():
    """HBM bytes per sparse-attention launch from the committed counter
    summary, or None when the kernel source changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            vals[key.strip()] = val.strip()
    if vals.get("kernel_source_sha256") != file_sha256(ATTN_SOURCE):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def row_stats(rowptr, N, d, B, H):
    """Useful and executed flop of one sparse-attention launch."""
    QB = (N + 127) // 128
    counts = np.diff(rowptr).reshape(B * H, QB)
    n_r = np.minimum(128, N - 128 * np.arange(QB))          # real queries per row
    useful = 4.0 * d * 4.0 * float((counts * n_r[None, :]).sum())
    active_waves = (n_r + 31) // 32
    tiles = (counts + 15) // 16
    executed = 4.0 * d * 64.0 * 32.0 * float((tiles * active_waves[None, :]).sum())
    return useful, executed, counts


# --------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a sample of plan rows, in worker processes
# forked before the GPU is touched (each worker single-threaded).
# --------------------------------------------------------------------------
_CPU = {}


def _bf16_to_f64(a16):
    return (a16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _cpu_worker_init():
    from threadpoolctl import threadpool_limits
    _CPU["limits"] = threadpool_limits(1)


def _cpu_task(task):
    """One head's sampled rows: (head setup seconds, row seconds, rows)."""
    import oracle
    b, h, rows = task
    x = _CPU
    conv = _bf16_to_f64 if x["bf16"] else (lambda a: a.astype(np.float64))
    t0 = time.perf_counter()
    Kh, Vh = conv(x["k"][b, h]), conv(x["v"][b, h])
    kb = oracle.mean_keys(Kh)
    t1 = time.perf_counter()
    N = Kh.shape[0]
    for r in rows:
        lo, hi = 128 * r, min(N, 128 * r + 128)
        Qr = conv(x["q"][b, h, lo:hi])
        s, _, _ = oracle.ibcs_row(Qr, kb)
        p = oracle.sip_probabilities(s.astype(np.float32), x["budget"])
        idx, logw, _ = oracle.sip_draw_row(p, x["seed"], b, h, r)
        oracle.ht_attention_row(Qr, Kh, Vh, idx, logw)
    return t1 - t0, time.perf_counter() - t1, len(rows)


def cpu_baseline(q, k, v, budget, seed, frac):
    """Time the oracle (k-means, scores, SIP, draws, HT attention per row;
    mean keys per head) on `frac` of the layer's rows, spread over worker
    processes (one per core of the CPU share, at most 16), and extrapolate to
    the whole layer on the same workers."""
    import multiprocessing as mp
    import torch
    B, H, N, d = (int(x) for x in q.shape)
    QB = (N + 127) // 128
    rows_total = B * H * QB
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    n_sample = max(workers, int(math.ceil(frac * rows_total)))
    rng = np.random.default_rng(0)
    pick = np.sort(rng.choice(rows_total, size=min(n_sample, rows_total), replace=False))
    tasks = {}
    for row in pick:
        bh, r = divmod(int(row), QB)
        tasks.setdefault(divmod(bh, H), []).append(r)
    task_list = [(b, h, rs) for (b, h), rs in tasks.items()]
    bf16 = q.dtype == torch.bfloat16
    view = (lambda t: t.view(torch.int16).numpy().view(np.uint16)) if bf16 else (lambda t: t.numpy())
    _CPU.update(q=view(q), k=view(k), v=view(v), bf16=bf16, budget=budget, seed=seed)
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(workers, initializer=_cpu_worker_init) as pool:
        res = pool.map(_cpu_task, task_list, chunksize=1)
    wall = time.perf_counter() - t0
    setup = [r[0] for r in res]
    row_s = sum(r[1] for r in res)
    done = sum(r[2] for r in res)
    cpu_s_layer = float(np.mean(setup)) * B * H + row_s / done * rows_total
    return dict(layer_s=cpu_s_layer / workers, rows=done, rows_total=rows_total, wall=wall,
                workers=workers, host_cpus=os.cpu_count())


# --------------------------------------------------------------------------
# GPU helpers
# --------------------------------------------------------------------------
def _timer(torch, stream):
    def timed(fn, reps=5, warm=1):
        for _ in range(warm):
            fn()
        ms = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        return float(np.median(ms))
    return timed


def _plan_ms(torch, absa, q, k, budget, seed, reps=3, **kw):
    """Wall time of absa_plan_create (it synchronises), median of reps."""
    absa.absa_plan_create(q, k, budget, seed, **kw).destroy()
    torch.cuda.synchronize()
    ms = []
    plan = None
    for _ in range(reps):
        if plan is not None:
            plan.destroy()
        t0 = time.perf_counter()
        plan = absa.absa_plan_create(q, k, budget, seed, **kw)
        ms.append((time.perf_counter() - t0) * 1e3)
    return float(np.median(ms)), plan


def _errors(torch, out, ref):
    of, rf = out.float(), ref.float()
    diff = of - rf
    return (float(torch.linalg.vector_norm(diff) / torch.linalg.vector_norm(rf)),
            float(diff.abs().max()))


def _layer_entry(torch, absa, timed, name, q, k, v, pct, reps=5, dense_reps=3):
    """Per-layer figures of one workload: plan ms, sparse and dense ms,
    TFLOP/s (dense-equivalent, executed, useful), fraction of bf16 peak,
    speed-up and error of the sparse output against dense."""
    B, H, N, d = (int(x) for x in q.shape)
    M = N // 4
    budget = synth_budget(pct, M)
    plan_ms, plan = _plan_ms(torch, absa, q, k, budget, 0x5EED0000)
    out = torch.empty_like(q)
    dense_out = torch.empty_like(q)
    sparse_ms = timed(lambda: absa.absa_sparse_attention(plan, q, k, v, out), reps=reps)
    dense_ms = timed(lambda: absa.absa_dense_attention(q, k, v, dense_out), reps=dense_reps)
    gp_rowptr = plan.export()["rowptr"]
    useful, executed, counts = row_stats(gp_rowptr, N, d, B, H)
    dense_flop = 4.0 * B * H * float(N) * N * d
    rel, mx = _errors(torch, out, dense_out)
    plan.destroy()
    return {
        "workload": WORKLOADS.get(name, name).rsplit(",", 1)[0] + f", budget {pct}%",
        "B": B, "H": H, "N": N, "d": d, "budget_blocks": budget,
        "plan_ms": round(plan_ms, 4), "sparse_attn_ms": round(sparse_ms, 4),
        "dense_ms": round(dense_ms, 4),
        "sparse_attn_effective_tflops": round(dense_flop / (sparse_ms * 1e-3) / 1e12, 2),
        "sparse_attn_executed_tflops": round(executed / (sparse_ms * 1e-3) / 1e12, 2),
        "sparse_attn_useful_tflops": round(useful / (sparse_ms * 1e-3) / 1e12, 2),
        "frac_bf16_peak_executed": round(executed / (sparse_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "dense_tflops": round(dense_flop / (dense_ms * 1e-3) / 1e12, 2),
        "speedup_vs_dense": round(dense_ms / sparse_ms, 3),
        "keep_fraction": round(float(gp_rowptr[-1]) / (B * H * ((N + 127) // 128) * M), 5),
        "rel_l2_vs_dense": round(rel, 6), "max_abs_vs_dense": round(mx, 5),
    }


def synth_budget(pct, M):
    import synth
    return synth.budget_blocks(pct, M)


def reuse_rows(torch, absa, timed, q0, k0, v0, pcts=(5, 10, 20), steps=4, on_device=True,
               sparse_reps=5, dense_reps=3):
    """[hamidun, kernel paragraph]: one plan per 4 denoising steps. The plan
    is built at step 0 and reused at steps 1..steps-1 while Q/K/V drift by
    0.05 N(0,1) per step; sparse and dense time and the error against dense
    on each step's inputs, per budget."""
    import synth
    B, H, N, d = (int(x) for x in q0.shape)
    M = N // 4
    drift = synth.drift_device if on_device else (lambda x, seed: synth.drift(x.cpu(), seed).to(x.device))
    inputs = [(q0, k0, v0)]
    for s in range(1, steps):
        inputs.append(tuple(drift(x, seed=100 * s + i) for i, x in enumerate(inputs[-1])))
    dense_out, dense_ms = [], []
    for (qs, ks, vs) in inputs:
        o = torch.empty_like(qs)
        dense_ms.append(timed(lambda: absa.absa_dense_attention(qs, ks, vs, o), reps=dense_reps))
        dense_out.append(o)
    rows = []
    for pct in pcts:
        budget = synth.budget_blocks(pct, M)
        plan_ms, plan = _plan_ms(torch, absa, q0, k0, budget, synth.sip_seed(0))
        useful, executed, _ = row_stats(plan.export()["rowptr"], N, d, B, H)
        for s, (qs, ks, vs) in enumerate(inputs):
            out = torch.empty_like(qs)
            sparse_ms = timed(lambda: absa.absa_sparse_attention(plan, qs, ks, vs, out),
                              reps=sparse_reps)
            rel, mx = _errors(torch, out, dense_out[s])
            rows.append({
                "budget_pct": pct, "budget_blocks": budget, "step": s, "plan_built_at_step": 0,
                "plan_ms": round(plan_ms, 3) if s == 0 else None,
                "sparse_attn_ms": round(sparse_ms, 4), "dense_ms": round(dense_ms[s], 4),
                "sparse_attn_executed_tflops": round(executed / (sparse_ms * 1e-3) / 1e12, 2),
                "frac_bf16_peak_executed": round(executed / (sparse_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "speedup_vs_dense": round(dense_ms[s] / sparse_ms, 3),
                "rel_l2_vs_dense": round(rel, 6), "max_abs_vs_dense": round(mx, 5),
            })
        plan.destroy()
    del inputs, dense_out
    return rows


def reuse_sweep(workload="small", out=None):
    import torch
    import sampled_block_sparse_amd as absa
    import synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = (x.to(dev) for x in synth.make_inputs(workload))
    timed = _timer(torch, torch.cuda.current_stream())
    rows = reuse_rows(torch, absa, timed, q, k, v, on_device=(workload != "small"))
    emit({"mode": "reuse_sweep", "workload": WORKLOADS[workload],
          "drift": "Q/K/V += 0.05 N(0,1) per step", "rows": rows}, out)


def sampling_study(seeds=8, out=None):
    """Poisson against fixed-size (systematic) sampling on the small
    video-shaped layer: for each budget and design, the sparse output's error
    against dense attention over several seeds (mean and spread), the spread
    of blocks per row, and the plan time; prints one JSON object."""
    import torch
    import sampled_block_sparse_amd as absa
    import synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = (x.to(dev) for x in synth.make_inputs("small"))
    B, H, N, d = (int(x) for x in q.shape)
    M = N // 4
    dense = absa.absa_dense_attention(q, k, v)
    df = dense.float()
    dn = float(torch.linalg.vector_norm(df))
    outt = torch.empty_like(q)
    rows = []
    for pct in (5, 10, 20):
        budget = synth.budget_blocks(pct, M)
        for design in ("poisson", "systematic"):
            errs, maxabs, cmin, cmax, cstd, plan_ms = [], [], [], [], [], []
            for s in range(seeds):
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                plan = absa.absa_plan_create(q, k, budget, synth.sip_seed(s), sampling=design)
                plan_ms.append((time.perf_counter() - t0) * 1e3)
                absa.absa_sparse_attention(plan, q, k, v, outt)
                torch.cuda.synchronize()
                diff = outt.float() - df
                errs.append(float(torch.linalg.vector_norm(diff)) / dn)
                maxabs.append(float(diff.abs().max()))
                c = np.diff(plan.export()["rowptr"])
                cmin.append(int(c.min()))
                cmax.append(int(c.max()))
                cstd.append(float(c.std()))
                plan.destroy()
            rows.append({
                "budget_pct": pct, "budget_blocks": budget, "sampling": design, "seeds": seeds,
                "rel_l2_vs_dense_mean": float(np.mean(errs)),
                "rel_l2_vs_dense_std": float(np.std(errs)),
                "max_abs_vs_dense_mean": float(np.mean(maxabs)),
                "blocks_per_row_min": min(cmin), "blocks_per_row_max": max(cmax),
                "blocks_per_row_std_mean": float(np.mean(cstd)),
                "plan_ms_median": float(np.median(plan_ms[1:] if seeds > 1 else plan_ms)),
            })
    emit({"mode": "sampling_study", "workload": WORKLOADS["small"], "rows": rows}, out)


# --------------------------------------------------------------------------
# Selection study: arithmetic (CPU, tested) and the GPU-driven study.
# --------------------------------------------------------------------------
def topk_plan(score, K):
    """CSR of the K best blocks of every row (ascending indices, p = 1)."""
    rows, M = score.shape
    idx = np.sort(np.argpartition(-score, K - 1, axis=1)[:, :K], axis=1).astype(np.int32)
    rowptr = np.arange(rows + 1, dtype=np.int64) * K
    return rowptr, idx.reshape(-1), np.zeros(rows * K, np.float32), np.ones(rows * K)


def block_masses(Qr, K, kv_block=4):
    """True attention mass of every KV block for one query row: the mean over
    the row's queries of the softmax probability summed over the block's keys
    (fp64). Qr [n, d], K [N, d] -> [N / kv_block], summing to 1."""
    z = Qr @ K.T / math.sqrt(Qr.shape[1])
    z = np.exp(z - z.max(axis=1, keepdims=True))
    z /= z.sum(axis=1, keepdims=True)
    return z.reshape(z.shape[0], -1, kv_block).sum(axis=2).mean(axis=0)


def retained_mass(mass, rowptr, idx):
    """Per row, the true attention mass of the blocks a plan keeps."""
    rows = np.repeat(np.arange(mass.shape[0]), np.diff(rowptr))
    kept = np.zeros(mass.shape[0])
    np.add.at(kept, rows, mass[rows, idx])
    return kept


def recall(rowptr, idx, ref_rowptr, ref_idx):
    """Per row, the fraction of the reference plan's blocks that the plan keeps."""
    out = np.zeros(len(rowptr) - 1)
    for i in range(len(out)):
        ref = ref_idx[ref_rowptr[i]:ref_rowptr[i + 1]]
        got = idx[rowptr[i]:rowptr[i + 1]]
        out[i] = np.intersect1d(ref, got).size / max(1, ref.size)
    return out


def coarse_plan(score, K, group=32):
    """K/group groups of `group` consecutive blocks per row (128-token blocks
    for group = 32), chosen by summed score; CSR with p = 1."""
    rows, M = score.shape
    Kc = max(1, K // group)
    coarse = score[:, :M // group * group].reshape(rows, -1, group).sum(axis=2)
    _, ic, _, _ = topk_plan(coarse, Kc)
    idx = (ic.reshape(-1, Kc)[:, :, None] * group + np.arange(group)).reshape(-1).astype(np.int32)
    n = Kc * group
    return (np.arange(rows + 1, dtype=np.int64) * n, idx, np.zeros(idx.size, np.float32),
            np.ones(idx.size))


def _subset_csr(gp, rows_sel):
    rp, ix, lw = gp["rowptr"], gp["idx"], gp["logw"]
    parts = [(ix[rp[r]:rp[r + 1]], lw[rp[r]:rp[r + 1]]) for r in rows_sel]
    rowptr = np.zeros(len(rows_sel) + 1, np.int64)
    rowptr[1:] = np.cumsum([p[0].size for p in parts])
    return rowptr, np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def selection_study(out=None):
    """What the plan's choices retain at equal budget. Small video-shaped
    layer (all rows; error = the GPU kernel's output on each rule's plan
    against dense) and 24 sampled rows of the Wan2.1-like layer (error = the
    fp64 oracle's HT attention of those rows against their dense rows).
    Rules: exact top-K by true mass (the bound), top-K by IBCS score (C = 8)
    and by the mean-query score (C = 1), SIP sampling on each of those two
    scores, and K/32 128-token blocks by summed IBCS score. Per rule: mean
    retained mass, recall of the exact top-K blocks, and error."""
    import torch
    import oracle
    import sampled_block_sparse_amd as absa
    import synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    result = {"mode": "selection_study", "layers": []}

    def rules(score8, score1, plan8, plan1, mass, K):
        exact = topk_plan(mass, K)
        r = {"exact top-K": exact, "C=8 top-K": topk_plan(score8, K),
             "C=1 top-K": topk_plan(score1, K), "C=8 scores + SIP": plan8,
             "C=1 scores + SIP": plan1, "128-token blocks, C=8": coarse_plan(score8, K)}
        return r, exact

    # small layer, all rows
    q, k, v = synth.make_inputs("small")
    B, H, N, d = (int(x) for x in q.shape)
    M, QB = N // 4, (N + 127) // 128
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    dense = absa.absa_dense_attention(qd, kd, vd).float()
    dn = float(torch.linalg.vector_norm(dense))
    Q64, K64 = q.double().numpy(), k.double().numpy()
    mass = np.stack([block_masses(Q64[b, h, 128 * r:128 * r + 128], K64[b, h])
                     for b in range(B) for h in range(H) for r in range(QB)])
    layer = {"workload": WORKLOADS["small"], "rows": B * H * QB, "rules": []}
    for pct in (5, 10, 20):
        K = synth.budget_blocks(pct, M)
        sc, plans = {}, {}
        for C in (8, 1):
            plan = absa.absa_plan_create(qd, kd, K, synth.sip_seed(0), n_clusters=C,
                                         keep_intermediates=True)
            sc[C] = plan.export_intermediate(absa.INTER_SCORES).reshape(-1, M).astype(np.float64)
            gp = plan.export()
            plans[C] = (gp["rowptr"], gp["idx"], gp["logw"], gp["p"])
            plan.destroy()
        rs, exact = rules(sc[8], sc[1], plans[8], plans[1], mass, K)
        for name, csr in rs.items():
            pl = absa.absa_plan_import(*csr, B, H, N, d)
            o = absa.absa_sparse_attention(pl, qd, kd, vd).float()
            torch.cuda.synchronize()
            kept = retained_mass(mass, csr[0], csr[1])
            rec = recall(csr[0], csr[1], exact[0], exact[1])
            layer["rules"].append({
                "budget_pct": pct, "budget_blocks": K, "rule": name,
                "blocks_per_row_mean": float(np.diff(csr[0]).mean()),
                "retained_mass_mean": float(kept.mean()), "retained_mass_min": float(kept.min()),
                "recall_of_exact_topk_mean": float(rec.mean()),
                "rel_l2_vs_dense": float(torch.linalg.vector_norm(o - dense)) / dn})
            pl.destroy()
    result["layers"].append(layer)
    print(f"[selection] small layer done", file=sys.stderr, flush=True)
    del qd, kd, vd, dense

    # Wan2.1-like layer, sampled rows (fp64 oracle for mass and error)
    q, k, v = synth.make_inputs("wan")
    B, H, N, d = (int(x) for x in q.shape)
    M, QB = N // 4, (N + 127) // 128
    rng = np.random.default_rng(5)
    sel = np.sort(rng.choice(B * H * QB, size=24, replace=False))
    qd, kd = q.to(dev), k.to(dev)
    heads = {}
    rowdata = []
    for row in sel:
        bh, r = divmod(int(row), QB)
        b, h = divmod(bh, H)
        if (b, h) not in heads:
            heads = {(b, h): (k[b, h].double().numpy(), v[b, h].double().numpy())}
        Kh, Vh = heads[(b, h)]
        Qr = q[b, h, 128 * r:min(N, 128 * r + 128)].double().numpy()
        rowdata.append((b, h, r, Qr, block_masses(Qr, Kh), oracle.dense_attention_rows(Qr, Kh, Vh)))
    layer = {"workload": WORKLOADS["wan"], "rows": int(sel.size), "sampled_rows": sel.tolist(),
             "rules": []}
    mass = np.stack([x[4] for x in rowdata])
    for pct in (5, 10, 20):
        K = synth.budget_blocks(pct, M)
        sc, plans = {}, {}
        for C in (8, 1):
            plan = absa.absa_plan_create(qd, kd, K, synth.sip_seed(0), n_clusters=C,
                                         keep_intermediates=True)
            sc[C] = np.stack([plan.export_intermediate(absa.INTER_SCORES, int(row) * M, M)
                              for row in sel]).astype(np.float64)
            gp = plan.export()
            rp, ix, lw = _subset_csr(gp, sel)
            plans[C] = (rp, ix, lw, np.exp(-lw.astype(np.float64)))
            plan.destroy()
        rs, exact = rules(sc[8], sc[1], plans[8], plans[1], mass, K)
        for name, csr in rs.items():
            kept = retained_mass(mass, csr[0], csr[1])
            rec = recall(csr[0], csr[1], exact[0], exact[1])
            num = den = 0.0
            for i, (b, h, r, Qr, _, dref) in enumerate(rowdata):
                Kh, Vh = k[b, h].double().numpy(), v[b, h].double().numpy()
                lo, hi = csr[0][i], csr[0][i + 1]
                o = oracle.ht_attention_row(Qr, Kh, Vh, csr[1][lo:hi], csr[2][lo:hi])
                num += float(((o - dref) ** 2).sum())
                den += float((dref ** 2).sum())
            layer["rules"].append({
                "budget_pct": pct, "budget_blocks": K, "rule": name,
                "blocks_per_row_mean": float(np.diff(csr[0]).mean()),
                "retained_mass_mean": float(kept.mean()), "retained_mass_min": float(kept.min()),
                "recall_of_exact_topk_mean": float(rec.mean()),
                "rel_l2_vs_dense": math.sqrt(num / den)})
        print(f"[selection] wan rows, {pct}% done", file=sys.stderr, flush=True)
    result["layers"].append(layer)
    emit(result, out)


def schedule_run(workloads=("wan", "hunyuan"), steps=50, dense_first=10, every=4, out_path=None):
    """The pages' denoising schedule on one attention layer [hamidun, kernel
    paragraph and "how it was measured"]: the first `dense_first` of `steps`
    steps run full attention, then each step runs the sparse kernel on a
    plan rebuilt every `every` steps. Q/K/V drift by 0.05 N(0,1) every step
    (drawn on the device), so a plan serves inputs that moved since it was
    built. Times every piece (HIP events for the kernels, wall time for the
    plan, which synchronises) and, untimed, runs dense attention at every
    sparse step for the error of that step. Prints one JSON object."""
    import torch
    import sampled_block_sparse_amd as absa
    import synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    layers = []
    for workload in workloads:
        cfg = synth.CONFIGS[workload]
        qd, kd, vd = (x.to(dev) for x in synth.make_inputs(workload))
        B, H, N, d = (int(x) for x in qd.shape)
        budget = synth.budget_blocks(cfg["budget_pct"], N // 4)
        out = torch.empty_like(qd)
        ref = torch.empty_like(qd)

        def timed(fn):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1)

        absa.absa_dense_attention(qd, kd, vd, out)            # warm-up of both paths
        absa.absa_sparse_attention(absa.absa_plan_create(qd, kd, budget, 1), qd, kd, vd, out)
        torch.cuda.synchronize()
        per_step = []
        plan = None
        plan_step = None
        for s in range(steps):
            if s:
                qd, kd, vd = (synth.drift_device(x, seed=1000 * s + i)
                              for i, x in enumerate((qd, kd, vd)))
            if s < dense_first:
                per_step.append({"step": s, "kind": "dense",
                                 "ms": timed(lambda: absa.absa_dense_attention(qd, kd, vd, out))})
                continue
            rec = {"step": s, "kind": "sparse"}
            if (s - dense_first) % every == 0:
                if plan is not None:
                    plan.destroy()
                t0 = time.perf_counter()
                plan = absa.absa_plan_create(qd, kd, budget, synth.sip_seed(s))
                torch.cuda.synchronize()
                rec["plan_ms"] = (time.perf_counter() - t0) * 1e3
                plan_step = s
            rec["plan_built_at_step"] = plan_step
            rec["ms"] = timed(lambda: absa.absa_sparse_attention(plan, qd, kd, vd, out))
            absa.absa_dense_attention(qd, kd, vd, ref)
            rel, mx = _errors(torch, out, ref)
            rec["rel_l2_vs_dense"] = round(rel, 6)
            rec["max_abs_vs_dense"] = round(mx, 5)
            per_step.append(rec)
        plan.destroy()
        dense_ms = [r["ms"] for r in per_step if r["kind"] == "dense"]
        sparse_ms = [r["ms"] for r in per_step if r["kind"] == "sparse"]
        plan_ms = [r["plan_ms"] for r in per_step if "plan_ms" in r]
        total = sum(dense_ms) + sum(sparse_ms) + sum(plan_ms)
        all_dense = steps * float(np.mean(dense_ms))
        errs = [r["rel_l2_vs_dense"] for r in per_step if r["kind"] == "sparse"]
        layers.append({
            "workload": WORKLOADS[workload], "steps": steps, "dense_first": dense_first,
            "plan_every": every, "plans": len(plan_ms),
            "drift": "Q/K/V += 0.05 N(0,1) every step",
            "dense_ms_mean": round(float(np.mean(dense_ms)), 3),
            "plan_ms_mean": round(float(np.mean(plan_ms)), 3),
            "sparse_ms_mean": round(float(np.mean(sparse_ms)), 3),
            "attention_ms_total": round(total, 1),
            "attention_ms_total_all_dense": round(all_dense, 1),
            "speedup_vs_all_dense": round(all_dense / total, 3),
            "rel_l2_vs_dense_mean": round(float(np.mean(errs)), 6),
            "rel_l2_vs_dense_max": round(float(np.max(errs)), 6),
            "per_step": [{k2: (round(v2, 4) if isinstance(v2, float) else v2)
                          for k2, v2 in r.items()} for r in per_step],
        })
        print(f"[schedule] {workload} done", file=sys.stderr, flush=True)
        del qd, kd, vd, out, ref
        torch.cuda.empty_cache()
    emit({"mode": "schedule", "layers": layers,
          "note": "all-dense total = steps x the mean measured dense step"}, out_path)


FUSED_MAX_BLOCKS = 20224     # the longest row (KV blocks) the fused plan kernel takes


def fused_plan_entry(torch, absa, q, k, budget, seed, reps=5):
    """Plan build time with the fused score pass 2 + SIP kernel against the
    two-pass build, and whether the two plans are identical."""
    two_ms, two = _plan_ms(torch, absa, q, k, budget, seed, reps=reps)
    one_ms, one = _plan_ms(torch, absa, q, k, budget, seed, reps=reps, fused=True)
    a, b = two.export(), one.export()
    same = all(np.array_equal(a[key], b[key]) for key in a)
    two.destroy()
    one.destroy()
    return {"plan_ms_two_pass": round(two_ms, 4), "plan_ms_fused": round(one_ms, 4),
            "fused_over_two_pass": round(one_ms / two_ms, 3), "bitwise_equal_plan": bool(same),
            "note": "wall time of absa_plan_create (it synchronises), median of 5"}


def other_configs(torch, absa, timed, main_inputs, main_pct):
    """Per-layer figures of the other workloads and the Wan-shape reuse."""
    import synth
    dev = torch.device("cuda:0")
    res = {}
    for name, pcts in (("tiny", (25, 100)), ("small", (10,)), ("hunyuan", (8,))):
        q, k, v = (x.to(dev) for x in synth.make_inputs(name))
        for pct in pcts:
            key = f"{name}_{pct}"
            res[key] = _layer_entry(torch, absa, timed, name, q, k, v, pct,
                                    reps=3 if name == "hunyuan" else 5,
                                    dense_reps=2 if name == "hunyuan" else 3)
            print(f"[bench] config {key} done", file=sys.stderr, flush=True)
        if name == "tiny":
            # budget 100% must equal dense attention bit for bit
            plan = absa.absa_plan_create(q, k, q.shape[2] // 4, 1)
            res["tiny_100"]["bitwise_equal_to_dense"] = bool(torch.equal(
                absa.absa_sparse_attention(plan, q, k, v), absa.absa_dense_attention(q, k, v)))
            plan.destroy()
        del q, k, v
        torch.cuda.empty_cache()
    q, k, v = main_inputs
    res["reuse_wan"] = reuse_rows(torch, absa, timed, q, k, v, sparse_reps=3, dense_reps=1)
    print("[bench] config reuse_wan done", file=sys.stderr, flush=True)
    return res


def main():
    args = parse()
    if args.schedule:
        wl = ("wan", "hunyuan") if args.workload == "wan" else (args.workload,)
        schedule_run(wl, out_path=args.out)
        return
    if args.selection_study:
        selection_study(out=args.out)
        return
    if args.reuse_sweep:
        reuse_sweep(args.workload if args.workload != "wan" or args.reuse_wan else "small",
                    out=args.out)
        return
    if args.sampling_study:
        sampling_study(out=args.out)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by head with no exchange between GPUs)", file=sys.stderr)
        sys.exit(2)
    import torch
    import sampled_block_sparse_amd as absa
    import synth

    name = args.workload
    cfg = synth.CONFIGS[name]
    q, k, v = synth.make_inputs(name)
    B, H, N, d = (int(x) for x in q.shape)
    M = N // 4
    pct = args.budget_pct if args.budget_pct is not None else cfg["budget_pct"]
    budget = synth.budget_blocks(pct, M)
    seed = synth.sip_seed(0)
    dense_flop = 4.0 * B * H * float(N) * N * d

    # the oracle baseline runs first, in processes forked before any GPU call
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 oracle on a sample of rows", file=sys.stderr, flush=True)
        cb = cpu_baseline(q, k, v, budget, seed, args.cpu_sample)
        cpu = {
            "value": round(dense_flop / cb["layer_s"] / 1e12, 6),
            "unit": "TFLOP/s",
            "cores": cb["workers"],
            "kind": "oracle",
            "sample": (f"{cb['rows']} of the layer's {cb['rows_total']} plan rows "
                       f"({100.0 * cb['rows'] / cb['rows_total']:.1f}%, random, per row: k-means, "
                       f"scores, SIP, draws, HT attention; mean keys per head) on "
                       f"{cb['workers']} single-threaded worker processes (host reports "
                       f"{cb['host_cpus']} CPUs) in {cb['wall']:.1f} s; extrapolated to the whole "
                       f"layer on the same workers: {cb['layer_s']:.1f} s per layer"),
        }

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    out = torch.empty_like(qd)
    torch.cuda.synchronize()
    print(f"[bench] workload={name} B={B} H={H} N={N} d={d} budget={budget} "
          f"steps={args.steps} warmup={args.warmup}", file=sys.stderr, flush=True)

    if args.calib_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    stream = torch.cuda.current_stream()

    def step():
        plan = absa.absa_plan_create(qd, kd, budget, seed, sampling=args.sampling,
                                     fused=args.fused_plan)
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        absa.absa_sparse_attention(plan, qd, kd, vd, out)
        ev1.record(stream)
        return plan, ev0, ev1

    for _ in range(args.warmup):
        plan, _, _ = step()
    torch.cuda.synchronize()

    attn_events = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        plan, e0, e1 = step()
        attn_events.append((e0, e1))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    attn_ms_all = [a.elapsed_time(b) for a, b in attn_events]
    attn_ms = float(np.median(attn_ms_all))
    attn_ms_mean = float(np.mean(attn_ms_all))
    plan_ms = ms_per_step - attn_ms_mean
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step, "
          f"sparse attention {attn_ms:.3f} ms", file=sys.stderr, flush=True)

    # plan statistics and flop counts of one launch
    gp = plan.export()
    useful, executed, counts = row_stats(gp["rowptr"], N, d, B, H)
    nnz = int(gp["rowptr"][-1])
    keep_fraction = nnz / float(B * H * ((N + 127) // 128) * M)

    # dense comparator (skipped with --dense-iters 0)
    dense_ms_all = []
    dense_out = torch.empty_like(qd)
    if args.dense_iters > 0:
        absa.absa_dense_attention(qd, kd, vd, dense_out)
    for _ in range(args.dense_iters):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        absa.absa_dense_attention(qd, kd, vd, dense_out)
        e1.record(stream)
        torch.cuda.synchronize()
        dense_ms_all.append(e0.elapsed_time(e1))
    dense_ms = float(np.median(dense_ms_all)) if dense_ms_all else None
    rel_l2_vs_dense = max_abs_vs_dense = None
    if dense_ms_all:
        rel_l2_vs_dense, max_abs_vs_dense = _errors(torch, out, dense_out)
    del dense_out

    achieved = useful / (attn_ms * 1e-3) / 1e12
    gathered_bytes = nnz * 2.0 * 4 * d * q.element_size()
    roofline = {
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": read_traffic(),
    }
    plan.destroy()

    configs = None
    if not args.no_configs:
        timed = _timer(torch, stream)
        configs = {f"{name}_{pct}": {
            "workload": WORKLOADS[name], "B": B, "H": H, "N": N, "d": d, "budget_blocks": budget,
            "plan_ms": round(plan_ms, 4), "sparse_attn_ms": round(attn_ms, 4),
            "dense_ms": round(dense_ms, 4) if dense_ms else None,
            "sparse_attn_effective_tflops": round(dense_flop / (attn_ms * 1e-3) / 1e12, 2),
            "sparse_attn_executed_tflops": round(executed / (attn_ms * 1e-3) / 1e12, 2),
            "sparse_attn_useful_tflops": round(achieved, 2),
            "frac_bf16_peak_executed": round(executed / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "speedup_vs_dense": round(dense_ms / attn_ms, 3) if dense_ms else None,
            "rel_l2_vs_dense": round(rel_l2_vs_dense, 6) if rel_l2_vs_dense is not None else None,
            "note": "the timed steps above"}}
        configs.update(other_configs(torch, absa, timed, (qd, kd, vd), pct))
        if M <= FUSED_MAX_BLOCKS:
            configs[f"{name}_{pct}_fused_plan"] = fused_plan_entry(torch, absa, qd, kd, budget,
                                                                    seed)
            print("[bench] config fused plan done", file=sys.stderr, flush=True)

    rec = {
        "metric": METRIC,
        "value": round(dense_flop / (ms_per_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if q.dtype == torch.bfloat16 else "f32",
        "data": "synthetic (seeded video-shaped Q/K/V generator)",
        "config": {"workload": WORKLOADS[name] if pct == cfg["budget_pct"]
                   else WORKLOADS[name].rsplit(",", 1)[0] + f", budget {pct}%",
                   "B": B, "H": H, "N": N, "d": d, "budget_blocks": budget,
                   "sampling": args.sampling,
                   "plan_kernels": "fused score pass 2 + SIP" if args.fused_plan else "two-pass",
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "sparse_attn_ms": round(attn_ms, 4),
        "sparse_attn_effective_tflops": round(dense_flop / (attn_ms * 1e-3) / 1e12, 2),
        "sparse_attn_executed_tflops": round(executed / (attn_ms * 1e-3) / 1e12, 2),
        "sparse_attn_useful_tflops": round(achieved, 2),
        "frac_bf16_peak_executed": round(executed / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "gathered_kv_GB": round(gathered_bytes / 1e9, 3),
        "plan_ms": round(plan_ms, 4),
        "amortized_ms_per_denoising_step": round(attn_ms + plan_ms / 4.0, 4),
        "dense_ms": round(dense_ms, 4) if dense_ms else None,
        "dense_tflops": round(dense_flop / (dense_ms * 1e-3) / 1e12, 2) if dense_ms else None,
        "speedup_vs_dense": round(dense_ms / attn_ms, 3) if dense_ms else None,
        "keep_fraction": round(keep_fraction, 5),
        "blocks_per_row": {"min": int(counts.min()), "max": int(counts.max()),
                           "mean": round(float(counts.mean()), 2)},
        "rel_l2_vs_dense": round(rel_l2_vs_dense, 5) if rel_l2_vs_dense is not None else None,
        "max_abs_vs_dense": round(max_abs_vs_dense, 5) if max_abs_vs_dense is not None else None,
        "value_definition": "dense-equivalent flop 4*B*H*N^2*d per step / (plan + sparse attention) time",
        "configs": configs,
    }
    emit(rec, args.out)


if __name__ == "__main__":
    main()
