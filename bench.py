"""Benchmark: one layer of AB-Attention's block-sparse attention on one MI355X.

A step is the whole path on one batch of synthetic video-shaped input already
resident in HBM: ab_score (IBCS k-means + block estimates), ab_sample (SIP) and
ab_attn_fwd (weighted gather attention), enqueued on one stream.

Prints one JSON line. `value` is the dense-equivalent attention throughput,
4*B*H*N^2*d / (time of one whole step), in TFLOP/s; `ms_per_step` is ms per
layer. `roofline` describes the attention kernel: its actually computed FLOPs
(4*d*sum over query rows of the kept keys) per launch divided by its average
launch time measured with HIP events on the stream it runs on, against the
dense bf16 matrix-core peak. `cpu_baseline` times the CPU oracle on a bounded
sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak (published)
PEAK_FP8_TFLOPS = 5000.0  # MI355X dense fp8 matrix-core peak (published)
METRIC = "dense-equivalent attention TFLOP/s and ms/layer at ~10% density, 1 MI355X"
# committed HBM-counter summary and kernel source of each attention variant
TRAFFIC = {
    "bf16": (os.path.join(ROOT, "profiles", "attn_fwd_wan1.3b_traffic.txt"),
             os.path.join(ROOT, "block_sparse_attention_ibcs_amd", "csrc", "attn_fwd.hip")),
    "fp8": (os.path.join(ROOT, "profiles", "attn_fp8_wan1.3b_traffic.txt"),
            os.path.join(ROOT, "block_sparse_attention_ibcs_amd", "csrc", "attn_fp8.hip")),
}


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="wan1.3b", help="wan1.3b (default), wan14b or hunyuan")
    ap.add_argument("--density", type=float, default=None)
    ap.add_argument("--k-block", type=int, default=None)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="wall time budget of the CPU oracle sample")
    ap.add_argument("--cpu-precision", default="fp32", choices=("fp32", "fp64"),
                    help="arithmetic of the timed CPU oracle: its fp32 timing mode (default) or its fp64 parity mode")
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="steps timed with the caches flushed before each (a 512 MB buffer written between steps)")
    ap.add_argument("--no-recall", action="store_true", help="skip the attention-mass recall statistic")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print a summary of a rocprofv3 --kernel-trace --stats output directory (no GPU needed)")
    ap.add_argument("--summarize-pmc", metavar="DIR", nargs="+",
                    help="print a summary of rocprofv3 --pmc output directories (no GPU needed)")
    ap.add_argument("--timed-launches", type=int, default=0,
                    help="with --summarize-trace: also average each kernel's last N launches (the timed region)")
    ap.add_argument("--fp8", action="store_true",
                    help="run the FP8 variant of the attention stage (ab_fp8_prepare + ab_attn_fwd_fp8: E4M3 "
                         "products, V-Smooth, ExpCast-FP8) instead of the bf16 kernel; not the headline line")
    ap.add_argument("--attn-order", choices=("auto", "contiguous"), default="auto",
                    help="order of the attention kernel's query blocks: auto = the kernel's own choice (head-major "
                         "when eight heads' K and V exceed the Infinity Cache, else one contiguous range per XCD); "
                         "contiguous = ab_attn_fwd_ordered with the identity order (one contiguous range per XCD "
                         "always), for comparing the two; the outputs are the same")
    ap.add_argument("--graph", action="store_true",
                    help="replay one step captured in a HIP graph instead of launching the three calls eagerly "
                         "(measured: no faster, the launches already run ahead of the GPU)")
    ap.add_argument("--intra", action="store_true",
                    help="INTRA Scatter/Gather patterns through the attention kernel on --workload; one JSON line per layer kind")
    ap.add_argument("--sweep", action="store_true",
                    help="gather-cost sweep on the 75600-token, 40-head shape: density {1, .25, .10, .05} x k_block "
                         "{16, 32, 64, 128}; one JSON line per point instead of the headline line")
    ap.add_argument("--ablation", action="store_true",
                    help="estimator comparison on --workload: relative L2 error of the layer output against dense "
                         "attention for IBCS+SIP, IBCS+top-K, pooled (C=1)+SIP and pooled+top-K over density and "
                         "k_block; one JSON line per point")
    ap.add_argument("--ablation-seeds", type=int, default=4, help="SIP seeds per ablation point")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one device copy of this many MiB before timing (reference kernel for HBM counters)")
    return ap.parse_args()


def source_digest(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(workload, variant):
    """HBM bytes per attention launch from the committed counter summary, if it was
    taken on this workload with the current kernel source; else None."""
    summary, source = TRAFFIC[variant]
    if not os.path.exists(summary):
        return None
    vals = {}
    with open(summary) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != source_digest(source) or vals.get("workload") != workload:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


MFMA_BUSY = {
    "bf16": (os.path.join(ROOT, "profiles", "attn_fwd_wan1.3b_mfma_busy.txt"),
             os.path.join(ROOT, "block_sparse_attention_ibcs_amd", "csrc", "attn_fwd.hip")),
    "fp8": (os.path.join(ROOT, "profiles", "attn_fp8_wan1.3b_mfma_busy.txt"),
            os.path.join(ROOT, "block_sparse_attention_ibcs_amd", "csrc", "attn_fp8.hip")),
}


def read_mfma_busy(workload, variant):
    """Fraction of the attention kernel's active cycles in which the matrix cores are busy
    (SQ_VALU_MFMA_BUSY_CYCLES over SIMDs x GRBM_GUI_ACTIVE per XCD), from the committed
    counter summary if it was taken on this workload with the current kernel source."""
    summary, source = MFMA_BUSY[variant]
    if not os.path.exists(summary):
        return None
    vals = {}
    with open(summary) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                vals[key.strip()] = val.strip()
    if vals.get("kernel_source_sha256_16") != source_digest(source) or vals.get("workload") != workload:
        return None
    try:
        return float(vals["mfma_busy_fraction"])
    except (KeyError, ValueError):
        return None


def attention_work(w, nqb, nkb, idx, cnt):
    """Actually computed attention work of one launch, 4*d*sum over query rows of the kept
    real keys (the ragged tail block counts its real keys only), and the realised density."""
    import torch

    tail = w.N - (nkb - 1) * w.k_block
    counts = cnt.to(torch.int64)
    last_kept = torch.zeros_like(counts)
    nz = counts > 0
    last_idx = torch.gather(idx.to(torch.int64), 3, (counts.clamp(min=1) - 1).unsqueeze(-1)).squeeze(-1)
    last_kept[nz & (last_idx == nkb - 1)] = 1
    keys = counts * w.k_block - last_kept * (w.k_block - tail)
    rows_per_block = torch.full((nqb,), w.q_block, dtype=torch.int64, device=idx.device)
    rows_per_block[-1] = w.N - (nqb - 1) * w.q_block
    flops = float((4 * w.d * (keys * rows_per_block.view(1, 1, -1)).sum()).item())
    return flops, float(counts.sum().item()) / (w.B * w.H * nqb * nkb)


SWEEP_DENSITIES = (1.0, 0.25, 0.10, 0.05)
SWEEP_K_BLOCKS = (16, 32, 64, 128)


def run_sweep(args):
    """Gather-cost sweep: the scorer once per key sub-block size, then sampler and attention
    at every density, each stage timed with HIP events on its stream over args.steps
    launches. Density 1 keeps every sub-block, so its attention time is set against the
    dense bf16 roofline of the same shape."""
    import numpy as np
    import torch

    import block_sparse_attention_ibcs_amd as ab
    import workloads

    w0 = workloads.get("wan14b")
    q, k, v = workloads.generate(w0, seed=0)
    dev = torch.device("cuda:0")
    qd, kd, vd = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (q, k, v))
    del q, k, v
    stream = torch.cuda.current_stream()
    dense = w0.dense_flops()
    dense_roof_ms = dense / (PEAK_BF16_TFLOPS * 1e12) * 1e3

    def timed(fn, reps):
        evs = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            evs.append((a, b))
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs]))

    for bk in SWEEP_K_BLOCKS:
        w = w0.with_(k_block=bk)
        desc = ab.Desc.for_tensor(qd, w.q_block, bk, w.n_clusters, w.kmeans_iters)
        nqb, nkb = desc.nqb, desc.nkb
        rows = (w.B, w.H, nqb)
        ws = ab.alloc_workspace(desc, dev)
        scores = torch.empty(rows + (nkb,), dtype=torch.float32, device=dev)
        idx = torch.empty(rows + (nkb,), dtype=torch.int32, device=dev)
        wts = torch.empty(rows + (nkb,), dtype=torch.float32, device=dev)
        cnt = torch.empty(rows, dtype=torch.int32, device=dev)
        out = torch.empty_like(qd)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        score_fn = lambda: ab.ab_score(desc, qd, kd, scores=scores, workspace=ws)  # noqa: E731
        for _ in range(args.warmup):
            score_fn()
        score_ms = timed(score_fn, args.steps)
        for rho in SWEEP_DENSITIES:
            sample_fn = lambda: ab.ab_sample(desc, scores, rho, args.seed, idx=idx, weights=wts,  # noqa: E731
                                             counts=cnt, want_mask=False)
            attn_fn = lambda: ab.ab_attn_fwd(desc, qd, kd, vd, idx, wts, cnt, out=out, lse=lse)  # noqa: E731
            sample_fn()
            attn_fn()
            torch.cuda.synchronize()
            flops, realised = attention_work(w, nqb, nkb, idx, cnt)
            for _ in range(args.warmup):
                attn_fn()
            sample_ms = timed(sample_fn, args.steps)
            attn_ms = timed(attn_fn, args.steps)
            achieved = flops / (attn_ms / 1e3) / 1e12
            layer_ms = score_ms + sample_ms + attn_ms
            print(json.dumps({
                "sweep": "gather-cost",
                "workload": f"wan14b shape: B={w.B} H={w.H} N={w.N} d={w.d} Bq={w.q_block} C={w.n_clusters}",
                "k_block": bk,
                "density": rho,
                "realised_density": realised,
                "score_ms": score_ms,
                "sample_ms": sample_ms,
                "attn_ms": attn_ms,
                "layer_ms": layer_ms,
                "attn_actual_tflops": achieved,
                "attn_mfma_frac": achieved / PEAK_BF16_TFLOPS,
                "attn_flops": flops,
                "attn_dense_equivalent_tflops": dense / (attn_ms / 1e3) / 1e12,
                "layer_dense_equivalent_tflops": dense / (layer_ms / 1e3) / 1e12,
                "dense_roofline_ms": dense_roof_ms,
                "steps": args.steps,
            }), flush=True)
        del ws, scores, idx, wts, cnt, out, lse
        torch.cuda.empty_cache()


def run_intra(args):
    """INTRA relay patterns as a second index producer for the same attention kernel:
    Scatter and Gather lists (ab_intra_lists, default neighbourhood of
    q_block*ceil(sqrt(NQB)) tokens) on the workload's inputs; list generation and
    attention timed with HIP events on their stream; one JSON line per layer kind."""
    import numpy as np
    import torch

    import block_sparse_attention_ibcs_amd as ab
    import workloads

    w = workloads.get(args.workload)
    if args.k_block:
        w = w.with_(k_block=args.k_block)
    q, k, v = workloads.generate(w, seed=0)
    dev = torch.device("cuda:0")
    qd, kd, vd = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (q, k, v))
    del q, k, v
    stream = torch.cuda.current_stream()
    desc = ab.Desc.for_tensor(qd, w.q_block, w.k_block, w.n_clusters, w.kmeans_iters)
    nqb, nkb = desc.nqb, desc.nkb
    rows = (w.B, w.H, nqb)
    idx = torch.empty(rows + (nkb,), dtype=torch.int32, device=dev)
    wts = torch.empty(rows + (nkb,), dtype=torch.float32, device=dev)
    cnt = torch.empty(rows, dtype=torch.int32, device=dev)
    out = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    dense = w.dense_flops()
    L = w.q_block * int(np.ceil(np.sqrt(nqb)))

    def timed(fn, reps):
        evs = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            evs.append((a, b))
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs]))

    order = torch.empty(w.B * w.H * nqb, dtype=torch.int32, device=dev)
    for layer, name in ((ab.AB_INTRA_SCATTER, "scatter"), (ab.AB_INTRA_GATHER, "gather")):
        list_fn = lambda: ab.ab_intra_lists(desc, layer, 0, idx=idx, weights=wts, counts=cnt,  # noqa: E731
                                            row_order=order)
        attn_fn = lambda: ab.ab_attn_fwd(desc, qd, kd, vd, idx, wts, cnt, out=out, lse=lse)  # noqa: E731
        ordered_fn = lambda: ab.ab_attn_fwd_ordered(desc, qd, kd, vd, idx, wts, cnt, order,  # noqa: E731
                                                    out=out, lse=lse)
        list_fn()
        attn_fn()
        torch.cuda.synchronize()
        flops, realised = attention_work(w, nqb, nkb, idx, cnt)
        for _ in range(args.warmup):
            attn_fn()
            ordered_fn()
        list_ms = timed(list_fn, args.steps)
        attn_ms = timed(attn_fn, args.steps)
        ordered_ms = timed(ordered_fn, args.steps)
        best_ms = min(attn_ms, ordered_ms)
        achieved = flops / (best_ms / 1e3) / 1e12
        print(json.dumps({
            "intra_layer": name,
            "workload": f"{w.name}: B={w.B} H={w.H} N={w.N} d={w.d} Bq={w.q_block} Bk={w.k_block}",
            "neighbourhood_tokens": L,
            "realised_density": realised,
            "list_ms": list_ms,
            "attn_natural_order_ms": attn_ms,
            "attn_pattern_order_ms": ordered_ms,
            "attn_ms": best_ms,
            "attn_actual_tflops": achieved,
            "attn_mfma_frac": achieved / PEAK_BF16_TFLOPS,
            "attn_flops": flops,
            "attn_dense_equivalent_tflops": dense / (best_ms / 1e3) / 1e12,
            "steps": args.steps,
        }), flush=True)


ABLATION_DENSITIES = (0.05, 0.10, 0.25)
ABLATION_K_BLOCKS = (16, 32, 64)


def run_ablation(args):
    """Estimator comparison. The dense reference is the attention kernel at density 1,
    which keeps every sub-block with weight 1 (exact dense attention). For each k_block
    and density: IBCS scores with the workload's C and pooled scores with C = 1, each
    followed by SIP with independent trials and with the systematic draw
    (args.ablation_seeds seeds each, and the average of their outputs) and by top-K
    truncation; the relative L2 error ||O - O_dense|| / ||O_dense|| over the whole
    layer output is computed in fp32 on the device."""
    import torch

    import block_sparse_attention_ibcs_amd as ab
    import workloads

    w0 = workloads.get(args.workload)
    q, k, v = workloads.generate(w0, seed=0)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w0.dtype == "bf16" else torch.float32
    qd, kd, vd = (torch.from_numpy(x).to(tdt).to(dev) for x in (q, k, v))
    del q, k, v

    def layer(desc, scores, rho, seed=None, systematic=False):
        if seed is None:
            idx, wts, cnt, _ = ab.ab_sample_topk(desc, scores, rho, want_mask=False)
        elif systematic:
            idx, wts, cnt, _ = ab.ab_sample_systematic(desc, scores, rho, seed, want_mask=False)
        else:
            idx, wts, cnt, _ = ab.ab_sample(desc, scores, rho, seed, want_mask=False)
        out, _ = ab.ab_attn_fwd(desc, qd, kd, vd, idx, wts, cnt, want_lse=False)
        kept = float(cnt.to(torch.float64).sum().item()) / (cnt.numel() * desc.nkb)
        return out.float(), kept

    d_ref = ab.Desc.for_tensor(qd, w0.q_block, w0.k_block, w0.n_clusters, w0.kmeans_iters)
    s_ref = ab.ab_score(d_ref, qd, kd)
    o_dense, _ = layer(d_ref, s_ref, 1.0, seed=0)
    ref_norm = float(torch.linalg.vector_norm(o_dense).item())
    del s_ref

    def rel(o):
        return float(torch.linalg.vector_norm(o - o_dense).item()) / ref_norm

    seeds = list(range(args.ablation_seeds))
    for bk in ABLATION_K_BLOCKS:
        scorers = {}
        for name, c in (("ibcs", w0.n_clusters), ("pooled", 1)):
            desc = ab.Desc.for_tensor(qd, w0.q_block, bk, c, w0.kmeans_iters)
            scorers[name] = (desc, ab.ab_score(desc, qd, kd))
        for rho in ABLATION_DENSITIES:
            for name, (desc, scores) in scorers.items():
                errs, kept, acc = [], [], None
                for sd in seeds:
                    o, kf = layer(desc, scores, rho, seed=sd)
                    errs.append(rel(o))
                    kept.append(kf)
                    acc = o if acc is None else acc + o
                mean_err = sum(errs) / len(errs)
                sd_err = (sum((e - mean_err) ** 2 for e in errs) / max(1, len(errs) - 1)) ** 0.5
                sys_errs, sys_acc = [], None
                for sd in seeds:
                    o, _ = layer(desc, scores, rho, seed=sd, systematic=True)
                    sys_errs.append(rel(o))
                    sys_acc = o if sys_acc is None else sys_acc + o
                o_topk, kept_topk = layer(desc, scores, rho)
                print(json.dumps({
                    "ablation": "estimator",
                    "workload": f"{args.workload}: B={w0.B} H={w0.H} N={w0.N} d={w0.d} Bq={w0.q_block} T={w0.kmeans_iters}",
                    "k_block": bk,
                    "density": rho,
                    "scorer": f"{name} (C={desc.n_clusters})",
                    "sip_rel_l2_mean": mean_err,
                    "sip_rel_l2_sd": sd_err,
                    "sip_kept": sum(kept) / len(kept),
                    "sip_seed_average_rel_l2": rel(acc / len(seeds)),
                    "systematic_rel_l2_mean": sum(sys_errs) / len(sys_errs),
                    "systematic_seed_average_rel_l2": rel(sys_acc / len(seeds)),
                    "topk_rel_l2": rel(o_topk),
                    "topk_kept": kept_topk,
                    "seeds": len(seeds),
                }), flush=True)
        del scorers
        torch.cuda.empty_cache()


def mass_recall(w, q, k, scores, idx, wts, cnt, density, n_blocks=64, seed=5):
    """Descriptive statistics of the synthetic inputs on n_blocks seeded query blocks:
    the true attention mass of a query block on key sub-block j is the mean over its
    rows of the dense softmax mass on j (float32 on the host). Reports the mass held by
    the top-ceil(rho NKB) sub-blocks ranked by the true mass, and by the IBCS scores,
    the mass on the sub-blocks the draw kept, and the draw's inverse-probability
    weighted mass (whose expectation is 1)."""
    import numpy as np

    rng = np.random.default_rng(seed)
    nqb = -(-w.N // w.q_block)
    nkb = -(-w.N // w.k_block)
    topk = min(nkb, math.ceil(density * nkb))
    pick = rng.choice(w.B * w.H * nqb, size=min(n_blocks, w.B * w.H * nqb), replace=False)
    scale = 1.0 / math.sqrt(w.d)
    stats = {"true_topk": [], "ibcs_topk": [], "kept": [], "kept_weighted": []}
    pad = nkb * w.k_block - w.N
    for t in pick.tolist():
        bh, i = divmod(t, nqb)
        b, h = divmod(bh, w.H)
        lo, hi = i * w.q_block, min(w.N, (i + 1) * w.q_block)
        logit = (q[b, h, lo:hi].astype(np.float32) @ k[b, h].astype(np.float32).T) * np.float32(scale)
        p = np.exp(logit - logit.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        if pad:
            p = np.concatenate([p, np.zeros((p.shape[0], pad), np.float32)], axis=1)
        mass = p.reshape(p.shape[0], nkb, w.k_block).sum(axis=2).mean(axis=0).astype(np.float64)
        stats["true_topk"].append(np.sort(mass)[::-1][:topk].sum())
        stats["ibcs_topk"].append(mass[np.argsort(-scores[b, h, i], kind="stable")[:topk]].sum())
        c = int(cnt[b, h, i])
        kept = idx[b, h, i, :c]
        stats["kept"].append(mass[kept].sum())
        stats["kept_weighted"].append((mass[kept] * wts[b, h, i, :c]).sum())
    out = {key: float(np.mean(val)) for key, val in stats.items()}
    out.update({"blocks": int(len(pick)), "top": int(topk)})
    return out


def cpu_baseline(w, q, k, v, density, seed, budget_s, precision="fp32"):
    """Time the oracle (IBCS + SIP + weighted attention) on query blocks for about budget_s seconds:
    a seeded spread of the blocks of head 0, then of head 1, and so on. precision: the oracle's
    fp32 timing mode (its score and attention arithmetic in float32) or its fp64 parity mode."""
    import numpy as np

    import oracle

    threads = os.cpu_count() or 1
    try:
        from threadpoolctl import threadpool_info

        info = threadpool_info()
        if info:
            threads = max(int(t.get("num_threads", 1)) for t in info)
    except Exception:
        pass
    p = oracle.Params(w.q_block, w.k_block, w.n_clusters, w.kmeans_iters, density, bf16=w.dtype == "bf16")
    order = [(0, h, int(i)) for h in range(w.B * w.H) for i in np.random.default_rng(1 + h).permutation(w.nqb)]
    t0 = time.perf_counter()
    done = []
    for (b, h, i) in order:
        oracle.run_blocks(q, k, v, p, seed, [(h // w.H, h % w.H, i)], precision=precision)
        done.append(i)
        if time.perf_counter() - t0 >= budget_s and len(done) >= 2:
            break
    dt = time.perf_counter() - t0
    heads = len({bh for (_, bh, _) in order[:len(done)]})
    rows = sum(min(w.q_block, w.N - i * w.q_block) for i in done)
    dense_flops = 4.0 * rows * w.N * w.d
    return {
        "value": dense_flops / dt / 1e12,
        "unit": "TFLOP/s (dense-equivalent)",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{len(done)} query blocks ({rows} query rows) of {heads} head(s) through IBCS k-means (fp32), "
                  f"block scores, SIP draw (integer) and weighted attention, scores and attention in "
                  f"{'float32' if precision == 'fp32' else 'float64'} numpy; {dt:.1f} s wall "
                  f"({dt / len(done) * w.H * w.nqb:.0f} s extrapolated per layer)",
        "precision": precision,
        "ms_per_layer_extrapolated": dt / len(done) * w.H * w.nqb * 1e3,
    }


def _csv_rows(path):
    import csv

    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def summarize_trace(args):
    """Kernel-time table of a rocprofv3 --kernel-trace --stats run, plus each kernel's
    average over its last --timed-launches launches (the timed region of a bench run)."""
    import glob

    stats = _csv_rows(glob.glob(os.path.join(args.summarize_trace, "*kernel_stats.csv"))[0])
    print(f"# {'kernel':<32}{'calls':>6}{'avg_us':>10}{'min_us':>10}{'max_us':>10}{'share':>9}")
    for r in stats:
        print(f"{r['Name'][:32]:<32}{int(r['Calls']):>6}{float(r['AverageNs']) / 1e3:>10.1f}"
              f"{float(r['MinNs']) / 1e3:>10.1f}{float(r['MaxNs']) / 1e3:>10.1f}{float(r['Percentage']):>8.2f}%")
    if args.timed_launches > 0:
        trace = _csv_rows(glob.glob(os.path.join(args.summarize_trace, "*kernel_trace.csv"))[0])
        by = {}
        for r in sorted(trace, key=lambda r: int(r["Start_Timestamp"])):
            by.setdefault(r["Kernel_Name"], []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        print(f"# last {args.timed_launches} launches of each kernel (timed region):")
        for name, d in by.items():
            if len(d) >= args.timed_launches:
                last = d[-args.timed_launches:]
                print(f"#   {name[:40]:<40} {sum(last) / len(last) / 1e3:10.1f} us")


def summarize_pmc(args):
    """Average per dispatch of every counter of rocprofv3 --pmc runs, per kernel; HBM
    bytes of each kernel from FETCH_SIZE / WRITE_SIZE scaled by what the same counters
    read for the device copy of known size (bench.py --copy-calibration-mib), and the
    matrix-core busy fraction SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x GRBM_GUI_ACTIVE per XCD)."""
    import glob

    per = {}
    agent = None
    for d in args.summarize_pmc:
        rows = _csv_rows(glob.glob(os.path.join(d, "*counter_collection.csv"))[0])
        for r in rows:
            key = (r["Kernel_Name"], r["Counter_Name"])
            per.setdefault(key, {}).setdefault(r["Dispatch_Id"], 0.0)
            per[key][r["Dispatch_Id"]] += float(r["Counter_Value"])
        info = glob.glob(os.path.join(d, "*agent_info.csv"))
        if info:
            for a in _csv_rows(info[0]):
                if a.get("Agent_Type") == "GPU":
                    agent = a
    avg = {key: sum(v.values()) / len(v) for key, v in per.items()}
    kernels = sorted({k for k, _ in avg})
    simds = int(agent["Simd_Count"]) if agent else 1024
    xcds = int(agent["Num_Xcc"]) if agent else 8
    for kname in kernels:
        vals = {c: v for (k, c), v in avg.items() if k == kname}
        print(f"{kname[:40]:<40} " + "  ".join(f"{c} {v:.6g}" for c, v in sorted(vals.items())))
    copy = [k for k in kernels if "copyBuffer" in k]
    mib = args.copy_calibration_mib
    fetch_scale = write_scale = None
    if copy and mib > 0:
        # the calibration copy is the largest dispatch of the copy kernel (torch issues small ones too)
        c = copy[0]
        if (c, "FETCH_SIZE") in per:
            fetch_scale = mib * 1024.0 / max(per[(c, "FETCH_SIZE")].values())
        if (c, "WRITE_SIZE") in per:
            write_scale = mib * 1024.0 / max(per[(c, "WRITE_SIZE")].values())
        print(f"# calibration: a {mib} MiB device copy; fetch scale {fetch_scale}, write scale {write_scale} "
              f"(true KiB per counted KiB)")
    for kname in kernels:
        out = []
        if fetch_scale and (kname, "FETCH_SIZE") in avg:
            out.append(f"fetch {avg[(kname, 'FETCH_SIZE')] * fetch_scale * 1024 / 1e6:.1f} MB")
        if write_scale and (kname, "WRITE_SIZE") in avg:
            out.append(f"write {avg[(kname, 'WRITE_SIZE')] * write_scale * 1024 / 1e6:.1f} MB")
        if (kname, "SQ_VALU_MFMA_BUSY_CYCLES") in avg and (kname, "GRBM_GUI_ACTIVE") in avg:
            busy = avg[(kname, "SQ_VALU_MFMA_BUSY_CYCLES")] / (simds * avg[(kname, "GRBM_GUI_ACTIVE")] / xcds)
            out.append(f"mfma_busy {busy:.4f}")
        if out:
            print(f"# {kname[:40]:<40} " + ", ".join(out))


def main():
    args = parse_args()
    if args.summarize_trace or args.summarize_pmc:
        if args.summarize_trace:
            summarize_trace(args)
        if args.summarize_pmc:
            summarize_pmc(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path is single-GPU by design "
              "(on several GPUs the heads would be split between them, each GPU running the whole path "
              "on its heads with no exchange).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import block_sparse_attention_ibcs_amd as ab
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ab.load_library()  # fails loudly if the HIP library is not built
    if args.sweep:
        run_sweep(args)
        return
    if args.intra:
        run_intra(args)
        return
    if args.ablation:
        run_ablation(args)
        return
    w = workloads.get(args.workload)
    if args.k_block:
        w = w.with_(k_block=args.k_block)
    density = w.density if args.density is None else args.density
    q, k, v = workloads.generate(w, seed=0)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    qd, kd, vd = (torch.from_numpy(x).to(tdt).to(dev) for x in (q, k, v))
    desc = ab.Desc.for_tensor(qd, w.q_block, w.k_block, w.n_clusters, w.kmeans_iters)
    nqb, nkb = desc.nqb, desc.nkb
    rows = (w.B, w.H, nqb)
    ws = ab.alloc_workspace(desc, dev)
    scores = torch.empty(rows + (nkb,), dtype=torch.float32, device=dev)
    idx = torch.empty(rows + (nkb,), dtype=torch.int32, device=dev)
    wts = torch.empty(rows + (nkb,), dtype=torch.float32, device=dev)
    cnt = torch.empty(rows, dtype=torch.int32, device=dev)
    out = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

    if args.copy_calibration_mib > 0:
        nbytes = args.copy_calibration_mib << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    stream = torch.cuda.current_stream()
    ev = {name: [] for name in ("score", "sample", "attn")}
    ident = None
    if args.attn_order == "contiguous":
        ident = torch.arange(w.B * w.H * nqb, dtype=torch.int32, device=dev)
    fp8_ops = None
    if args.fp8:
        if ident is not None:
            print("--attn-order applies to the bf16 kernel only", file=sys.stderr)
            sys.exit(2)
        if w.dtype != "bf16" or w.d != 128 or w.q_block != 128:
            print("--fp8 needs a bf16 workload with d = 128 and q_block = 128", file=sys.stderr)
            sys.exit(2)
        fp8_ops = ab.Fp8Operands(desc, dev)
        ev["fp8_prepare"] = []

    def step(record=False):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if record else None
        if record:
            e[0].record(stream)
        ab.ab_score(desc, qd, kd, scores=scores, workspace=ws)
        if record:
            e[1].record(stream)
        ab.ab_sample(desc, scores, density, args.seed, idx=idx, weights=wts, counts=cnt, want_mask=False)
        if record:
            e[2].record(stream)
        if fp8_ops is None:
            if ident is None:
                ab.ab_attn_fwd(desc, qd, kd, vd, idx, wts, cnt, out=out, lse=lse)
            else:
                ab.ab_attn_fwd_ordered(desc, qd, kd, vd, idx, wts, cnt, ident, out=out, lse=lse)
            if record:
                e[3].record(stream)
        else:
            ab.ab_fp8_prepare(desc, qd, kd, vd, ops=fp8_ops)
            if record:
                e.append(torch.cuda.Event(enable_timing=True))
                e[3].record(stream)
            ab.ab_attn_fwd_fp8(desc, fp8_ops, idx, wts, cnt, out=out, lse=lse)
            if record:
                e[4].record(stream)
        if record:
            ev["score"].append((e[0], e[1]))
            ev["sample"].append((e[1], e[2]))
            if fp8_ops is None:
                ev["attn"].append((e[2], e[3]))
            else:
                ev["fp8_prepare"].append((e[2], e[3]))
                ev["attn"].append((e[3], e[4]))

    # One step captured in a HIP graph (the same kernels on the same buffers, launched as
    # one graph): the timed loop replays it. The path issues no memsets, so the graph
    # holds kernel nodes only.
    run = step
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(3):
                step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        run = graph.replay
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3
    # per-stage durations with HIP events on the launch stream (separate pass so the headline
    # number carries no event overhead)
    for _ in range(args.steps):
        step(record=True)
    torch.cuda.synchronize()
    stage_ms = {k_: float(np.mean([a.elapsed_time(b) for a, b in v_])) for k_, v_ in ev.items()}

    # cold caches: a 512 MB buffer (twice the 256 MB Infinity Cache, far beyond the L2s)
    # written before each timed step, outside its events
    cold = None
    if args.cold_steps > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cold_ev = {name: [] for name in ev}
        for n_c in range(args.cold_steps):
            flush.fill_(n_c & 0xFF)
            saved = {name: len(v_) for name, v_ in ev.items()}
            step(record=True)
            for name in ev:
                cold_ev[name].extend(ev[name][saved[name]:])
                del ev[name][saved[name]:]
        torch.cuda.synchronize()
        cold_stage = {k_: float(np.mean([a.elapsed_time(b) for a, b in v_])) for k_, v_ in cold_ev.items()}
        cold = {"steps": args.cold_steps, "stage_ms": cold_stage, "ms_per_step": float(sum(cold_stage.values())),
                "flush": "512 MB buffer written before each step (outside the timed events)"}
        del flush

    actual_flops, realised = attention_work(w, nqb, nkb, idx, cnt)
    dense = w.dense_flops()
    K_budget = max(1, min(nkb, math.floor(density * nkb + 0.5)))

    attn_s = stage_ms["attn"] / 1e3
    achieved = actual_flops / attn_s / 1e12
    traffic = read_traffic(args.workload, "bf16" if fp8_ops is None else "fp8")
    peak = PEAK_BF16_TFLOPS if fp8_ops is None else PEAK_FP8_TFLOPS
    fp8_vs_bf16 = None
    if fp8_ops is not None:
        # accuracy of the FP8 variant: relative L2 distance of its output from the bf16
        # kernel's on the same kept lists (the bf16 path is within ~0.3% of exact)
        ref, _ = ab.ab_attn_fwd(desc, qd, kd, vd, idx, wts, cnt, want_lse=False)
        torch.cuda.synchronize()
        fp8_vs_bf16 = float(torch.linalg.vector_norm((out.float() - ref.float()).flatten()) /
                            torch.linalg.vector_norm(ref.float().flatten()))
    result = {
        "metric": METRIC,
        "value": dense / (ms_per_step / 1e3) / 1e12,
        "unit": "TFLOP/s (dense-equivalent)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16" if w.dtype == "bf16" else "f32") if fp8_ops is None else "fp8-e4m3 (attention products)",
        "data": "synthetic (seeded smooth 3D positional field + noise; no model weights)",
        "config": {
            "workload": f"{args.workload}: B={w.B} H={w.H} grid={'x'.join(map(str, w.grid))} N={w.N} d={w.d} "
                        f"Bq={w.q_block} Bk={w.k_block} C={w.n_clusters} T={w.kmeans_iters} density={density}",
            "seq_len": w.N,
            "heads": w.H,
            "density": density,
            "realised_density": realised,
            # sum of the inclusion probabilities of a row is the budget K (up to integer
            # floors below NKB 2^-24), so the expected kept fraction is K / NKB
            "expected_density": K_budget / nkb,
            "stage_ms": stage_ms,
            "cold_cache": cold,
            "hip_graph": bool(args.graph),
            "attn_order": args.attn_order,
            "attention_variant": "bf16" if fp8_ops is None else "fp8 (E4M3 QK and PV, V-Smooth, ExpCast-FP8)",
            "fp8_rel_l2_vs_bf16_path": fp8_vs_bf16,
            "attn_actual_tflops": achieved,
            "attn_dense_equivalent_tflops": dense / attn_s / 1e12,
            "layer_actual_tflops_excl_scorer": actual_flops / (ms_per_step / 1e3) / 1e12,
        },
        "roofline": {
            "kernel": "attn_fwd_bf16" if fp8_ops is None else "attn_fwd_fp8",
            "bound": "mfma",
            "achieved": achieved,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": achieved / peak,
            "traffic": traffic,
            "traffic_note": "FETCH_SIZE + WRITE_SIZE per launch scaled by a device-copy calibration: bytes between "
                            "L2 and the fabric (Infinity Cache hits included), an upper bound on HBM bytes",
            "mfma_busy": read_mfma_busy(args.workload, "bf16" if fp8_ops is None else "fp8"),
            "flops_per_launch": actual_flops,
            "launch_ms": stage_ms["attn"],
        },
        "cpu_baseline": None,
    }
    if not args.no_recall:
        result["config"]["attention_mass_recall"] = mass_recall(
            w, q, k, scores.cpu().numpy(), idx.cpu().numpy(), wts.cpu().numpy(), cnt.cpu().numpy(), density)
    if not args.no_cpu_baseline and fp8_ops is None:
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, density, args.seed, args.cpu_seconds, args.cpu_precision)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
