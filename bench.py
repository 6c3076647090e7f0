#!/usr/bin/env python3
"""Decode benchmark of the predictor-gated sparse FFN on one MI355X.

One step = one decode token (batch 1) through every layer of a model-shaped
FFN stack: for each layer, the predictor, the compaction and the sparse FFN
(one ``pi_layer`` call).  The L calls of a step are captured once into a HIP
graph that reads its inputs from a staging buffer; each step copies that
token's inputs (one vector per layer, already in HBM) into the staging buffer
and replays the graph.

Printed: one JSON line with layer-tokens/s (tokens x layers / wall time);
a roofline entry for the layer call (pi_layer: algorithmic bytes per call --
predictor weights, the active FFN rows, biases, list and vectors -- over its
event-timed average duration, against the 8 TB/s HBM peak), the same for the
gather path alone (pi_sparse_ffn) and the predictor alone (pi_predict), each
timed in its own graph over all layers; and the CPU oracle timed on a
bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload falcon40b]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

HBM_PEAK_GBPS = 8000.0
METRIC = "sparse-FFN layer tokens/s (batch 1) + achieved HBM GB/s vs peak"
ELEM_BYTES = {"f32": 4, "f16": 2}


def _row_bytes(cfg):
    if cfg.wtype == "q4_0":
        return cfg.d_model // 32 * 18
    return cfg.d_model * ELEM_BYTES[cfg.wtype]


def bytes_predict(cfg):
    """Algorithmic bytes of one pi_predict call at batch 1."""
    eb = ELEM_BYTES[cfg.pred_wtype]
    return (cfg.rank * cfg.d_model + cfg.d_ff * cfg.rank) * eb + 4 * cfg.d_ff + cfg.d_model * eb + cfg.d_ff


def bytes_compact(cfg, cnt):
    return cfg.d_ff + 4 * cnt + 4


def bytes_gather(cfg, cnt):
    """Algorithmic bytes of one pi_sparse_ffn call at batch 1: the active
    weight rows, their biases and list entries, x and y."""
    xb = 2 if cfg.wtype == "q4_0" else ELEM_BYTES[cfg.wtype]
    return cnt * cfg.n_mat * _row_bytes(cfg) + 8 * cnt + cfg.d_model * xb + 4 * cfg.d_model


def bytes_active(cfg, cnt):
    return cnt * cfg.n_mat * _row_bytes(cfg)


def bytes_layer(cfg, cnt):
    """Algorithmic bytes of one pi_layer call at batch 1: both predictor
    matrices and its bias, x, the active FFN rows with their biases, the
    active list and y."""
    eb = ELEM_BYTES[cfg.pred_wtype]
    xb = 2 if cfg.wtype == "q4_0" else ELEM_BYTES[cfg.wtype]
    return ((cfg.rank * cfg.d_model + cfg.d_ff * cfg.rank) * eb + 4 * cfg.d_ff + cfg.d_model * xb
            + bytes_active(cfg, cnt) + 8 * cnt + 4 * cfg.d_model)


def _time_graph(graph, reps, stream):
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    graph.replay()
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(reps):
        graph.replay()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / reps          # ms per replay


def cpu_baseline(cfg, layers, xs_host, budget_s=20.0, max_samples=64):
    """The oracle's layer() on host copies of a few layers and tokens."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:       # pragma: no cover - threadpoolctl missing
        threads = os.cpu_count() or 1
    done, t_total, samples = 0, 0.0, []
    for li, hl in enumerate(layers):
        for tok in range(xs_host.shape[0]):
            x = xs_host[tok, li]
            t0 = time.perf_counter()
            oracle.layer(x, hl["p1"], hl["p2"], hl["c"], cfg.tau, **hl["ffn"])
            t_total += time.perf_counter() - t0
            done += 1
            samples.append((li, tok))
            if t_total > budget_s or done >= max_samples:
                break
        if t_total > budget_s or done >= max_samples:
            break
    return {
        "value": done / t_total,
        "unit": "layer-tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"oracle layer (predict, compact, sparse FFN; float64) on {done} layer-tokens "
                  f"(layers 0-{len(layers) - 1}, tokens 0-{xs_host.shape[0] - 1}) of the same stack, "
                  f"{t_total:.1f} s on {os.cpu_count()} host cores ({threads} BLAS threads)",
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description="predictor-gated sparse FFN decode benchmark")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="falcon40b")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--reps", type=int, default=20, help="replays for the per-call timing graphs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only; the sparse FFN is not sharded across GPUs "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import activation_sparse_rank_amd as pi
    import workload

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    pi.load_library()
    cfg = workload.get_config(args.workload)
    dev = torch.device("cuda")
    L, d, f = cfg.n_layers, cfg.d_model, cfg.d_ff
    T = args.warmup + args.steps
    xdt = torch.float16 if cfg.x_dtype == "f16" else torch.float32

    n_base_layers, n_base_tok = 4, 16
    q4 = cfg.wtype == "q4_0"
    mats = ("w_up", "w_down_t", "w_gate")
    t_gen = time.perf_counter()
    layers, canon = [], []
    for li in range(L):
        lw = workload.make_layer(cfg, li, dev, args.seed)
        lw.pop("p")
        if q4:
            # the kernels read the repacked layout; the oracle reads canonical blocks
            if li < n_base_layers and not args.no_cpu_baseline:
                canon.append({k: lw[k].cpu().numpy() for k in mats if k in lw})
            for k in mats:
                if k in lw:
                    lw[k] = pi.q4_0_repack(lw[k], f, d)
        layers.append(lw)
        if (li + 1) % 10 == 0:
            print(f"[bench] generated layer {li + 1}/{L}", file=sys.stderr, flush=True)
    x_all = torch.empty((T, L, d), dtype=xdt, device=dev)
    for li in range(L):
        x_all[:, li] = workload.make_tokens(cfg, li, T, dev, args.seed)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen

    preds = [pi.Predictor(lw["p1"], lw["p2"], lw["c"]) for lw in layers]
    ffns = [pi.FFN(lw["w_up"], lw["w_down_t"], cfg.act, b_up=lw.get("b_up"), w_gate=lw.get("w_gate"),
                   b_gate=lw.get("b_gate"), d_model=d if q4 else None) for lw in layers]
    ws_bytes = pi.workspace_bytes(preds[0], ffns[0], 1)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    x_stage = torch.zeros((L, d), dtype=xdt, device=dev)
    y_all = torch.empty((L, d), dtype=torch.float32, device=dev)

    stream = torch.cuda.Stream()
    # ---------------- the decode step graph ----------------
    with torch.cuda.stream(stream):
        for li in range(L):   # eager run once before capture (also loads code objects)
            pi.layer(preds[li], ffns[li], x_stage[li:li + 1], cfg.tau, y_all[li:li + 1], ws=ws)
    torch.cuda.synchronize()
    g_step = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_step, stream=stream):
        for li in range(L):
            pi.layer(preds[li], ffns[li], x_stage[li:li + 1], cfg.tau, y_all[li:li + 1], ws=ws)
    torch.cuda.synchronize()

    def step(t):
        x_stage.copy_(x_all[t], non_blocking=True)
        g_step.replay()

    with torch.cuda.stream(stream):
        for t in range(args.warmup):
            step(t)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        start.record(stream)
        for t in range(args.warmup, T):
            step(t)
        end.record(stream)
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps
    layer_tok_s = args.steps * L / (ms_total / 1e3)

    # ---------------- per-(layer, token) counts of the timed steps ----------------
    mask = torch.empty((L, f), dtype=torch.uint8, device=dev)
    idx = torch.empty((L, f), dtype=torch.int32, device=dev)
    cnt = torch.zeros((L,), dtype=torch.int32, device=dev)
    cnt_hist = torch.empty((args.steps, L), dtype=torch.int32, device=dev)
    ws_p = torch.empty(pi.workspace_bytes(preds[0], None, 1), dtype=torch.uint8, device=dev)
    g_pc = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_pc, stream=stream):
        for li in range(L):
            pi.predict(preds[li], x_stage[li:li + 1], cfg.tau, mask[li:li + 1], ws=ws_p)
            pi.compact(mask[li:li + 1], idx[li], cnt[li:li + 1])
    with torch.cuda.stream(stream):
        for t in range(args.warmup, T):
            x_stage.copy_(x_all[t], non_blocking=True)
            g_pc.replay()
            cnt_hist[t - args.warmup].copy_(cnt, non_blocking=True)
    torch.cuda.synchronize()
    counts = cnt_hist.cpu().numpy().astype(np.int64)
    cnt_mean = float(counts.mean())

    # ---------------- per-call timing: predict, compact, sparse FFN ----------------
    # inputs of the last timed token; idx/count of every layer from g_pc
    ws_s = torch.empty(pi.workspace_bytes(None, ffns[0], 1), dtype=torch.uint8, device=dev)
    g_pred, g_comp, g_sp = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_pred, stream=stream):
        for li in range(L):
            pi.predict(preds[li], x_stage[li:li + 1], cfg.tau, mask[li:li + 1], ws=ws_p)
    with torch.cuda.graph(g_comp, stream=stream):
        for li in range(L):
            pi.compact(mask[li:li + 1], idx[li], cnt[li:li + 1])
    with torch.cuda.graph(g_sp, stream=stream):
        for li in range(L):
            pi.sparse_ffn(ffns[li], x_stage[li:li + 1], idx[li], cnt[li:li + 1], y_all[li:li + 1], ws=ws_s)
    with torch.cuda.stream(stream):
        ms_pred = _time_graph(g_pred, args.reps, stream) / L
        ms_comp = _time_graph(g_comp, args.reps, stream) / L
        ms_sp = _time_graph(g_sp, args.reps, stream) / L
    last_cnt = cnt.cpu().numpy().astype(np.int64)
    b_pred = bytes_predict(cfg)
    b_comp = float(np.mean([bytes_compact(cfg, c) for c in last_cnt]))
    b_sp = float(np.mean([bytes_gather(cfg, c) for c in last_cnt]))
    b_act = float(np.mean([bytes_active(cfg, c) for c in last_cnt]))

    def roof(kernels, b, ms):
        gbps = b / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "kernel": kernels, "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                "bytes_per_launch": int(b), "avg_launch_us": round(ms * 1e3, 3)}

    # whole-layer bytes per layer-token, averaged over the timed steps
    b_layer = float(np.mean([bytes_layer(cfg, c) for c in counts.flat]))
    ms_layer = ms_step / L
    dn = "k_down_q4" if q4 else "k_down"
    layer_roof = roof(f"pi_layer (k_pred1 + k_pred_up + {dn} + k_merge)", b_layer, ms_layer)
    parts = {
        "predict": roof("pi_predict (k_pred1 + k_pred2)", b_pred, ms_pred),
        "compact": {"kernel": "pi_compact (k_compact)", "avg_launch_us": round(ms_comp * 1e3, 3),
                    "bytes_per_launch": int(b_comp)},
        "gather": roof(f"pi_sparse_ffn (k_up + {dn} + k_merge)", b_sp, ms_sp),
    }
    parts["gather"]["active_weight_gbps"] = round(b_act / (ms_sp * 1e-3) / 1e9, 1)
    parts["gather"]["active_weight_frac"] = round(b_act / (ms_sp * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)

    out = {
        "metric": METRIC,
        "value": round(layer_tok_s, 1),
        "unit": "layer-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.wtype,
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} decode batch 1", "d_model": d, "d_ff": f, "layers": L,
                   "rank": cfg.rank, "act": cfg.act, "weights": cfg.wtype, "mean_density": cfg.rho,
                   "parallelism": "none (1 GPU)"},
        "roofline": layer_roof,
        "roofline_parts": parts,
        "count_mean": round(cnt_mean, 1),
        "count_min": int(counts.min()),
        "count_max": int(counts.max()),
        "gen_seconds": round(t_gen, 1),
    }

    if not args.no_cpu_baseline:
        import oracle  # the baseline leg is the only user of the oracle here
        host_layers = []
        for li in range(n_base_layers):
            lw = layers[li]

            def w(k):
                if k not in lw:
                    return None
                return oracle.Q4_0Matrix(canon[li][k], d) if q4 else lw[k].cpu().numpy()

            host_layers.append({
                "p1": lw["p1"].cpu().numpy(), "p2": lw["p2"].cpu().numpy(), "c": lw["c"].cpu().numpy(),
                "ffn": {"w_up": w("w_up"), "w_down_t": w("w_down_t"), "act": cfg.act,
                        "b_up": lw["b_up"].cpu().numpy() if "b_up" in lw else None,
                        "w_gate": w("w_gate"),
                        "b_gate": lw["b_gate"].cpu().numpy() if "b_gate" in lw else None},
            })
        xs = x_all[args.warmup:args.warmup + n_base_tok, :n_base_layers].cpu().numpy()
        out["cpu_baseline"] = cpu_baseline(cfg, host_layers, xs)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
