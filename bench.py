"""Benchmark of the DSA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c2] [--no-cpu] [--no-long]

One step is the whole path over one batch of seeded synthetic input: indexer
scores -> top-k (index lists, mask bits, tile classes) -> sparse attention
forward -> backward (dQ, then dK/dV). Inputs are resident in HBM before the
timed region. Default workload: the 2B-model training shape (batch 12,
seq 4096, 16 heads of 192/128, indexer 64 x 128, top-k 2048, bf16).

Prints one JSON line. `value` is useful TFLOP/s of the whole step:
indexer pairs x Hi x 2 Di, plus selected pairs x H x 6 (Dqk + Dv) for
forward + backward. `indexer_topk_ms` is the selection half of the metric;
`selection` repeats it at the 32K (671B head count) and 128K workloads, where
indexer and top-k are timed alone (the attention there is forward only and not
part of the step).
Per-kernel times come from HIP events recorded on the launch stream around
each C-ABI call (each is one kernel, except dsa_topk, which is the top-k
kernel plus the small tile-class kernel).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DSA fwd+bwd useful TFLOP/s and indexer+top-k ms at S=4K/32K/128K, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def valid_counts(cfg, seg_np):
    """|valid(t)| per (b, t): causal with the diagonal, same segment."""
    B, S = cfg.B, cfg.S
    if seg_np is None:
        return np.broadcast_to(np.arange(1, S + 1, dtype=np.int64), (B, S))
    out = np.empty((B, S), np.int64)
    for b in range(B):
        row = seg_np[b]
        starts = np.r_[0, np.nonzero(np.diff(row))[0] + 1]
        start_of = np.repeat(starts, np.diff(np.r_[starts, S]))
        out[b] = np.arange(S) - start_of + 1
    return out


def work(cfg, seg_np):
    nv = valid_counts(cfg, seg_np)
    sel = np.minimum(nv, cfg.K)
    pairs, selected = int(nv.sum()), int(sel.sum())
    sb = 2 if cfg.score_dtype == "bf16" else 4
    W = (cfg.S + 63) // 64
    topk_bytes = int(nv[nv > cfg.K].sum()) * sb + cfg.B * cfg.S * cfg.K * 4 + cfg.B * cfg.S * W * 8
    return {
        "pairs": pairs, "selected": selected,
        "indexer": pairs * cfg.Hi * 2 * cfg.Di,
        "fwd": selected * cfg.H * 2 * (cfg.Dqk + cfg.Dv),
        # backward: dP = dO V^T, dV = P^T dO, dK = dS^T Q (the dK/dV kernel) and
        # dQ = dS K (the dQ kernel); recomputing S = Q K^T (both kernels) and dP
        # (the dQ kernel) is not counted
        "bwd": selected * cfg.H * 4 * (cfg.Dqk + cfg.Dv),
        "bwd_dq": selected * cfg.H * 2 * cfg.Dqk,
        "bwd_dkdv": selected * cfg.H * 2 * (cfg.Dqk + 2 * cfg.Dv),
        "topk_bytes": topk_bytes,
        # backward prologue: O and dO rows read, D and base-2 LSE written
        "bwd_prep_bytes": cfg.B * cfg.S * cfg.H * (2 * cfg.Dv * (2 if cfg.dtype == "bf16" else 4) + 8),
    }


KERNEL_SRC = {"index_scores": "indexer.hip", "topk": "topk.hip", "attn_fwd": "attn_fwd.hip",
              "attn_bwd_prep": "attn_bwd_plain.hip",
              "attn_bwd_dq": "attn_bwd.hip", "attn_bwd_dkdv": "attn_bwd.hip"}
KERNEL_SYM = {"index_scores": "index_scores_mfma_kernel", "topk": "topk_reg_kernel", "attn_fwd": "attn_fwd_mfma_kernel",
              "attn_bwd_prep": "attn_bwd_prep_kernel",
              "attn_bwd_dq": "attn_bwd_dq_kernel", "attn_bwd_dkdv": "attn_bwd_dkdv_kernel"}


def measured_traffic(call, workload_key):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, or None when it is missing or the kernel's source changed since."""
    import hashlib
    prof = os.path.join(ROOT, "profiles", f"dsa_step_{workload_key}_hbm_traffic.txt")
    src = os.path.join(ROOT, "sparse_attention_06_amd", "csrc", KERNEL_SRC[call])
    if not os.path.exists(prof) or not os.path.exists(src):
        return None
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    for line in open(prof):
        f = line.split()
        if len(f) == 5 and f[0] == "traffic_bytes" and f[1] == KERNEL_SYM[call] and f[3] == "source_sha":
            return int(f[2]) if f[4] == sha else None
    return None


def cpu_baseline(cfg, x_cpu, budget_s=15.0, max_rows=4096):
    """The float64 oracle on a bounded row sample of the same workload."""
    from oracle import dsa_oracle as ref
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    f64 = lambda t: t.float().double().numpy()  # noqa: E731
    q_idx, k_idx, w = f64(x_cpu["q_idx"]), f64(x_cpu["k_idx"]), f64(x_cpu["w"])
    q, k, v = f64(x_cpu["q"]), f64(x_cpu["k"]), f64(x_cpu["v"])
    dout = f64(x_cpu["dout"]) if cfg.backward else None
    seg = None if x_cpu["seg"] is None else x_cpu["seg"].numpy()
    rng = np.random.default_rng(1234)
    rows_all = rng.permutation(cfg.S)[:max_rows]
    flops, done = 0, 0
    t0 = time.perf_counter()
    for t in rows_all:
        rows = np.array([t])
        sc = ref.index_scores(q_idx[:1], k_idx[:1], w[:1], None if seg is None else seg[:1], rows)
        idx = ref.topk(sc, None if seg is None else seg[:1], rows, cfg.K, cfg.S)
        ref.attention_fwd(q[:1], k[:1], v[:1], idx, None if seg is None else seg[:1], cfg.softmax_scale, rows)
        if cfg.backward:
            ref.attention_bwd(q[:1], k[:1], v[:1], dout[:1], idx, None if seg is None else seg[:1],
                              cfg.softmax_scale, rows=rows)
        nv = int(np.isfinite(sc).sum())
        n = int((idx >= 0).sum())
        flops += nv * cfg.Hi * 2 * cfg.Di + n * cfg.H * (6 if cfg.backward else 2) * (cfg.Dqk + cfg.Dv)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} random query rows of batch row 0 (indexer, top-k, forward"
                      f"{', backward' if cfg.backward else ''}), {dt:.1f} s, float64 numpy",
            "seconds": dt, "rows": done}


def selection_long(key, reps=2):
    """Indexer + top-k alone at a long-sequence workload (the metric's 32K and
    128K points): one warm-up call, then `reps` timed calls of each, with HIP
    events on the launch stream. Only the selection inputs are generated."""
    import torch
    from sparse_attention_06_amd import dsa, inputs
    cfg = inputs.CONFIGS[key]
    x = inputs.make_index_inputs(cfg, device="cuda")
    sdt = torch.bfloat16 if cfg.score_dtype == "bf16" else torch.float32
    scores = torch.empty((cfg.B, cfg.S, cfg.S), dtype=sdt, device="cuda")
    idx = torch.empty((cfg.B, cfg.S, cfg.K), dtype=torch.int32, device="cuda")
    mask = torch.empty(dsa.dsa_mask_bytes(cfg.B, cfg.S), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    t_idx, t_top = [], []
    for i in range(reps + 1):
        ev[0].record(stream)
        dsa.dsa_index_scores(x["q_idx"], x["k_idx"], x["w"], x["seg"], 0, cfg.S, scores)
        ev[1].record(stream)
        dsa.dsa_topk(scores, x["seg"], cfg.B, cfg.S, cfg.K, 0, cfg.S, idx, mask)
        ev[2].record(stream)
        torch.cuda.synchronize()
        if i:
            t_idx.append(ev[0].elapsed_time(ev[1]))
            t_top.append(ev[1].elapsed_time(ev[2]))
    # the fp8 (E4M3) indexer on the same inputs, quantized on the GPU first (untimed)
    q8 = torch.empty(x["q_idx"].shape, dtype=torch.uint8, device="cuda")
    qs = torch.empty(x["q_idx"].shape[:-1], dtype=torch.float32, device="cuda")
    k8 = torch.empty(x["k_idx"].shape, dtype=torch.uint8, device="cuda")
    ks = torch.empty(x["k_idx"].shape[:-1], dtype=torch.float32, device="cuda")
    dsa.dsa_quant_fp8_rows(x["q_idx"], q8, qs)
    dsa.dsa_quant_fp8_rows(x["k_idx"], k8, ks)
    t_fp8 = []
    for i in range(reps + 1):
        ev[0].record(stream)
        dsa.dsa_index_scores_fp8(q8, qs, k8, ks, x["w"], x["seg"], 0, cfg.S, scores)
        ev[1].record(stream)
        torch.cuda.synchronize()
        if i:
            t_fp8.append(ev[0].elapsed_time(ev[1]))
    # partial RoPE (rope_dim 64) of q_idx and k_idx in place, after the timings above
    h = 32
    ang = torch.arange(cfg.S, device="cuda", dtype=torch.float64)[:, None] * \
        (10000.0 ** (-torch.arange(h, device="cuda", dtype=torch.float64) / h))[None, :]
    ct, st = torch.cos(ang).float().contiguous(), torch.sin(ang).float().contiguous()
    t_rope = []
    for i in range(reps + 1):
        ev[0].record(stream)
        dsa.dsa_indexer_rope(x["q_idx"], 64, ct, st)
        dsa.dsa_indexer_rope(x["k_idx"], 64, ct, st)
        ev[1].record(stream)
        torch.cuda.synchronize()
        if i:
            t_rope.append(ev[0].elapsed_time(ev[1]))
    # in place only the rotated dims move: bf16 read + write of 64 of every Di
    rope_bytes = 2 * (x["q_idx"].numel() + x["k_idx"].numel()) * 2 * 64 // cfg.Di
    wk = work(cfg, None if x["seg"] is None else x["seg"].cpu().numpy())
    mi, mt = float(np.mean(t_idx)), float(np.mean(t_top))
    m8 = float(np.mean(t_fp8))
    mr = float(np.mean(t_rope))
    del scores, idx, mask, x, q8, qs, k8, ks
    torch.cuda.empty_cache()
    ach_i = wk["indexer"] / (mi * 1e-3) / 1e12
    ach_8 = wk["indexer"] / (m8 * 1e-3) / 1e12
    ach_t = wk["topk_bytes"] / (mt * 1e-3) / 1e9
    return {"workload": cfg.name, "S": cfg.S, "index_scores_ms": mi, "topk_ms": mt, "indexer_topk_ms": mi + mt,
            "index_scores": {"achieved": ach_i, "unit": "TFLOP/s", "frac": ach_i / PEAK_BF16_TFLOPS,
                             "algorithmic": wk["indexer"]},
            "topk": {"achieved": ach_t, "unit": "GB/s", "frac": ach_t / PEAK_HBM_GBS,
                     "algorithmic": wk["topk_bytes"]},
            # fp8 inputs (not the metric's bf16 workload): the indexer alone and with the same top-k
            "index_scores_fp8_ms": m8, "indexer_fp8_topk_ms": m8 + mt,
            "index_scores_fp8": {"achieved": ach_8, "unit": "TFLOP/s", "frac": ach_8 / PEAK_FP8_TFLOPS,
                                 "algorithmic": wk["indexer"]},
            # input preparation before the indexer (not part of the metric): RoPE of q_idx and k_idx
            "rope_ms": mr, "rope": {"achieved": rope_bytes / (mr * 1e-3) / 1e9, "unit": "GB/s",
                                    "frac": rope_bytes / (mr * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                    "algorithmic": rope_bytes}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c2")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-long", action="store_true",
                    help="skip timing indexer + top-k at the 32K and 128K workloads")
    ap.add_argument("--long-only", action="store_true",
                    help="only time indexer + top-k at the 32K and 128K workloads (one JSON line)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_attention_06_amd import dsa, inputs
    from sparse_attention_06_amd.pipeline import DSAPath

    cfg = inputs.CONFIGS[args.config]
    dsa.lib()
    dev = "cuda"
    if args.copy_mib:
        n = args.copy_mib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {n} bytes read, {n} bytes written")
        del src, dst

    if args.long_only:
        selection = {}
        for key in ("c3", "c5"):
            log(f"indexer + top-k at {inputs.CONFIGS[key].name}")
            r = selection_long(key)
            selection[f"S{r['S']}"] = r
            log(f"  index_scores {r['index_scores_ms']:.2f} ms, topk {r['topk_ms']:.2f} ms, "
                f"fp8 index_scores {r['index_scores_fp8_ms']:.2f} ms, rope {r['rope_ms']:.3f} ms")
        print(json.dumps({"metric": "indexer + top-k ms", "selection": selection}), flush=True)
        return
    log(f"config {cfg.name}: generating inputs on the GPU")
    x = inputs.make(cfg, device=dev)
    seg_np = None if x["seg"] is None else x["seg"].cpu().numpy()
    sdt = torch.bfloat16 if cfg.score_dtype == "bf16" else torch.float32
    path = DSAPath(cfg.B, cfg.S, cfg.Hi, cfg.Di, cfg.K, cfg.H, cfg.Dqk, cfg.Dv, dtype=cfg.torch_dtype(),
                   score_dtype=sdt, backward=cfg.backward, device=dev)
    scale = cfg.softmax_scale
    seg = x["seg"]
    stream = torch.cuda.current_stream()

    calls = ["index_scores", "topk", "attn_fwd"] + (["attn_bwd_prep", "attn_bwd_dkdv", "attn_bwd_dq"]
                                                    if cfg.backward else [])

    def step(evs=None):
        def mark(i):
            if evs is not None:
                evs[i].record(stream)
        mark(0)
        dsa.dsa_index_scores(x["q_idx"], x["k_idx"], x["w"], seg, 0, cfg.S, path.scores)
        mark(1)
        dsa.dsa_topk(path.scores, seg, cfg.B, cfg.S, cfg.K, 0, cfg.S, path.idx, path.mask)
        mark(2)
        dsa.dsa_sparse_attn_fwd(x["q"], x["k"], x["v"], path.mask, scale, path.o, path.lse)
        mark(3)
        if cfg.backward:
            dsa.dsa_sparse_attn_bwd_prep(path.o, x["dout"], path.lse, cfg.Dqk, path.ws)
            mark(4)
            dsa.dsa_sparse_attn_bwd_dkdv(x["q"], x["k"], x["v"], x["dout"], path.lse, path.mask, scale,
                                         path.dk, path.dv, path.ws)
            mark(5)
            dsa.dsa_sparse_attn_bwd_dq(x["q"], x["k"], x["v"], x["dout"], path.lse, path.mask, scale,
                                       path.dq, path.ws)
            mark(6)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup {i + 1}/{args.warmup} done")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms = total_ms / args.steps
    per = {c: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps)]))
           for j, c in enumerate(calls)}
    log(f"timed {args.steps} steps: {ms:.3f} ms/step; " + ", ".join(f"{c} {v:.3f}" for c, v in per.items()))

    wk = work(cfg, seg_np)
    useful = wk["indexer"] + wk["fwd"] + (wk["bwd"] if cfg.backward else 0)
    value = useful / (ms * 1e-3) / 1e12
    kern = {
        "index_scores": ("mfma", wk["indexer"]),
        "topk": ("hbm", wk["topk_bytes"]),
        "attn_fwd": ("mfma", wk["fwd"]),
        "attn_bwd_prep": ("hbm", wk["bwd_prep_bytes"]),
        "attn_bwd_dq": ("mfma", wk["bwd_dq"]),
        "attn_bwd_dkdv": ("mfma", wk["bwd_dkdv"]),
    }
    kernels = {}
    for c in calls:
        bound, amount = kern[c]
        t = per[c] * 1e-3
        if bound == "mfma":
            ach = amount / t / 1e12
            kernels[c] = {"ms": per[c], "bound": "mfma", "achieved": ach, "unit": "TFLOP/s",
                          "frac": ach / PEAK_BF16_TFLOPS, "algorithmic": amount}
        else:
            ach = amount / t / 1e9
            kernels[c] = {"ms": per[c], "bound": "hbm", "achieved": ach, "unit": "GB/s",
                          "frac": ach / PEAK_HBM_GBS, "algorithmic": amount}
    dom = max(calls, key=lambda c: per[c])
    kd = kernels[dom]
    roofline = {"bound": kd["bound"], "achieved": kd["achieved"],
                "peak": PEAK_BF16_TFLOPS if kd["bound"] == "mfma" else PEAK_HBM_GBS, "unit": kd["unit"],
                "frac": kd["frac"], "traffic": measured_traffic(dom, args.config), "kernel": dom}

    # the metric's other sequence lengths: indexer + top-k alone at 32K and 128K
    selection = {f"S{cfg.S}": {"workload": cfg.name, "S": cfg.S, "index_scores_ms": per["index_scores"],
                               "topk_ms": per["topk"], "indexer_topk_ms": per["index_scores"] + per["topk"]}}
    if not args.no_long:
        del path
        torch.cuda.empty_cache()
        for key in ("c3", "c5"):
            log(f"indexer + top-k at {inputs.CONFIGS[key].name}")
            r = selection_long(key)
            selection[f"S{r['S']}"] = r
            log(f"  index_scores {r['index_scores_ms']:.2f} ms, topk {r['topk_ms']:.2f} ms, "
                f"fp8 index_scores {r['index_scores_fp8_ms']:.2f} ms, rope {r['rope_ms']:.3f} ms")

    cpu = None
    if not args.no_cpu:
        log("timing the float64 oracle on a row sample (cpu baseline)")
        x_cpu = {k: (None if v is None else v.cpu()) for k, v in x.items()}
        cpu = cpu_baseline(cfg, x_cpu)
        log(f"cpu baseline: {cpu['value']:.3e} TFLOP/s over {cpu['rows']} rows")

    out = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if cfg.dtype == "bf16" else "fp32", "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "S": cfg.S, "index_heads": cfg.Hi, "index_dim": cfg.Di,
                   "topk": cfg.K, "heads": cfg.H, "dqk": cfg.Dqk, "dv": cfg.Dv, "score_dtype": cfg.score_dtype,
                   "segments": cfg.segments is not None, "passes": "+".join(calls)},
        "indexer_topk_ms": per["index_scores"] + per["topk"],
        "selection": selection,
        "attention_useful_tflops": (wk["fwd"] + (wk["bwd"] if cfg.backward else 0)) /
                                   (sum(per[c] for c in calls if c.startswith("attn")) * 1e-3) / 1e12,
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
