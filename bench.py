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
import glob
import hashlib
import json
import os
import re
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


def bytes_predict(cfg, n_tok=1):
    """Algorithmic bytes of one pi_predict call: both predictor matrices and
    its bias, x, and the masks."""
    eb = ELEM_BYTES[cfg.pred_wtype]
    return (cfg.rank * cfg.d_model + cfg.d_ff * cfg.rank) * eb + 4 * cfg.d_ff + n_tok * (cfg.d_model * eb + cfg.d_ff)


def bytes_compact(cfg, cnt, n_tok=1):
    return n_tok * cfg.d_ff + 4 * cnt + 4


def bytes_active(cfg, cnt, down_rows=None, up_rows=None):
    """Bytes of the FFN weight rows a call needs: the gate rows of the cnt
    listed neurons (ReGLU), their up rows -- every listed row, or up_rows
    when given (the fused ReGLU kernel leaves out the up rows of neurons
    whose gate fires for no token, and counts the rows it reads) -- and the
    down rows that are read: every listed row, or down_rows when given (the
    down projection leaves out rows whose h is zero for every token, and
    counts the rows it reads)."""
    down = cnt if down_rows is None else down_rows
    up = cnt if up_rows is None else up_rows
    gate = cnt if cfg.n_mat == 3 else 0
    return (gate + up + down) * _row_bytes(cfg)


def bytes_gather(cfg, cnt, n_tok=1, down_rows=None, up_rows=None):
    """Algorithmic bytes of one pi_sparse_ffn call: the weight rows it needs
    (each read once for all tokens), the biases and list entries of the
    listed neurons, x and y."""
    xb = 2 if cfg.wtype == "q4_0" else ELEM_BYTES[cfg.wtype]
    return bytes_active(cfg, cnt, down_rows, up_rows) + 8 * cnt + n_tok * (cfg.d_model * xb + 4 * cfg.d_model)


def bytes_layer(cfg, cnt, n_tok=1, down_rows=None, up_rows=None):
    """Algorithmic bytes of one pi_layer call: both predictor matrices and
    its bias, x, the FFN rows it needs (once for all tokens), the biases and
    list entries of the listed neurons, and y."""
    eb = ELEM_BYTES[cfg.pred_wtype]
    xb = 2 if cfg.wtype == "q4_0" else ELEM_BYTES[cfg.wtype]
    return ((cfg.rank * cfg.d_model + cfg.d_ff * cfg.rank) * eb + 4 * cfg.d_ff
            + bytes_active(cfg, cnt, down_rows, up_rows) + 8 * cnt + n_tok * (cfg.d_model * xb + 4 * cfg.d_model))


def flops_ffn(cfg, cnt, n_tok):
    """Multiply-adds x 2 of the sparse FFN over cnt listed neurons."""
    return 2.0 * cnt * cfg.n_mat * cfg.d_model * n_tok


ROOT = os.path.dirname(os.path.abspath(__file__))


def kernel_source_sha256(names=None):
    """sha256 over include/pi.h and the kernel sources (all of csrc/, or the
    csrc/ files in names), in name order."""
    files = [os.path.join(ROOT, "include", "pi.h")]
    d = os.path.join(ROOT, "activation_sparse_rank_amd", "csrc")
    files += [os.path.join(d, f) for f in sorted(os.listdir(d))
              if f.endswith((".hip", ".h")) and (names is None or f in names)]
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode())
        h.update(b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


# Sources every kernel's behaviour depends on besides the file that defines
# it: the host launch code (grids, chunking) and the shared device headers.
KERNEL_COMMON_SOURCES = ["abi.hip", "pi_internal.h", "predict_device.h"]


def kernel_defining_file(name):
    """The csrc .hip file that defines the __global__ kernel `name`, or None."""
    d = os.path.join(ROOT, "activation_sparse_rank_amd", "csrc")
    pat = re.compile(r"__global__[^;{]*?\b" + re.escape(name) + r"\s*\(", re.S)
    for f in sorted(os.listdir(d)):
        if f.endswith(".hip"):
            with open(os.path.join(d, f)) as fh:
                if pat.search(fh.read()):
                    return f
    return None


def kernel_sources(name):
    """The csrc files kernel `name` is built from (defining file + common sources)."""
    f = kernel_defining_file(name)
    return None if f is None else sorted(set([f] + KERNEL_COMMON_SOURCES))


def load_traffic(workload):
    """HBM bytes per dispatch of each kernel, from the committed rocprofv3 PMC
    summary of this workload (profiles/*_traffic.md).  Each kernel's entry
    names the sources it was built from and their hash when the counters were
    taken; a kernel whose sources have changed since is left out (its traffic
    is then unknown), so one changed file never passes stale counts along.
    None when there is no summary for the workload."""
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.md"))):
        with open(path) as fh:
            m = re.search(r"```json\n(.*?)\n```", fh.read(), re.S)
        if not m:
            continue
        data = json.loads(m.group(1))
        if data.get("workload") != workload:
            continue
        fs, ws = data["fetch_scale"], data["write_scale"]
        out = {}
        for k, v in data["kernels"].items():
            files = v.get("source_files")
            if files and v.get("source_sha256") == kernel_source_sha256(files):
                out[k] = (v["fetch_kib"] * fs + v["write_kib"] * ws) * 1024.0
        return out
    return None


def _time_graph(graph, reps, stream):
    """ms per replay of graph over reps replays, after one untimed replay."""
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


def _oracle_rate(cfg, layers, xs_host, budget_s):
    """layer-tokens/s of the oracle's layer() over every (layer, step) of the
    sample, in order, stopping early once budget_s seconds are spent."""
    import oracle
    # xs_host: [steps][layers][batch][d]; one oracle call takes one step's batch of one layer
    done, calls, t_total = 0, 0, 0.0
    for li, hl in enumerate(layers):
        for tok in range(xs_host.shape[0]):
            x = xs_host[tok, li]
            t0 = time.perf_counter()
            oracle.layer(x, hl["p1"], hl["p2"], hl["c"], cfg.tau, **hl["ffn"])
            t_total += time.perf_counter() - t0
            done += x.shape[0]
            calls += 1
            if t_total > budget_s:
                break
        if t_total > budget_s:
            break
    return done / t_total, done, calls, t_total


def cpu_baseline(cfg, layers, xs_host, budget_s=15.0):
    """The oracle's layer() (float64 numpy) on host copies of the first layers
    and steps of the same stack: once with the BLAS pool on every core it may
    use, once limited to one thread."""
    from threadpoolctl import threadpool_info, threadpool_limits

    blas = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    affinity = len(os.sched_getaffinity(0))
    v_all, done, calls, t_all = _oracle_rate(cfg, layers, xs_host, budget_s)
    with threadpool_limits(limits=1):
        v_one, done1, _, t_one = _oracle_rate(cfg, layers, xs_host, budget_s)
    return {
        "value": round(v_all, 3),
        "unit": "layer-tokens/s",
        "cores": blas,
        "kind": "oracle",
        "value_1_thread": round(v_one, 3),
        "cpu_count": os.cpu_count(),
        "affinity_cpus": affinity,
        "blas_threads": blas,
        "sample": f"oracle layer (predict, compact, sparse FFN; float64) on layers 0-{len(layers) - 1} x steps "
                  f"0-{xs_host.shape[0] - 1} (batch {xs_host.shape[2]}) of the same stack: {done} layer-tokens in "
                  f"{calls} calls, {t_all:.1f} s with {blas} BLAS threads; {done1} layer-tokens in {t_one:.1f} s "
                  f"with 1 thread; {os.cpu_count()} host cores, {affinity} in this process's affinity mask",
    }


def _tile(cfg):
    """Tokens per pass of the list path (fp16 / fp32: 8; Q4_0: x tile <= 32 KB)."""
    if cfg.wtype != "q4_0":
        return 8
    t = 8
    while t > 1 and t * cfg.d_model * 2 > 32768:
        t //= 2
    return t


def measure_stream(pi, dev, stream, nbytes=8 << 30, reps=10):
    """GB/s of pi_stream_read over an nbytes buffer (event-timed on stream)."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    out = torch.empty(pi._lib.PI_STREAM_BLOCKS, dtype=torch.int32, device=dev)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        pi.stream_read(buf, out)
        start.record(stream)
        for _ in range(reps):
            pi.stream_read(buf, out)
        end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    del buf
    return round(nbytes / (ms * 1e-3) / 1e9, 1)


def place_by_hotness(pi, cfg, lw, layer, seed, n_cal, dev, order="hot"):
    """Offline placement of one layer's neurons: run the layer's predictor on
    n_cal calibration tokens (a token stream of their own, never timed),
    count each neuron's predicted firings, and permute every per-neuron array
    into the order pi_hot_order gives ("hot": hot neurons dealt evenly over
    the fused kernel's segments) or pi_rank_order gives ("rank": neurons by
    firing count, the always-firing ones contiguous in the first rows);
    canonical Q4_0 blocks are permuted before the repack."""
    import workload

    xc = workload.make_tokens(cfg, layer, n_cal, dev, seed, stream=2)
    mask = torch.empty((n_cal, cfg.d_ff), dtype=torch.uint8, device=dev)
    pi.predict(pi.Predictor(lw["p1"], lw["p2"], lw["c"]), xc, cfg.tau, mask)
    counts = torch.zeros(cfg.d_ff, dtype=torch.int32, device=dev)
    pi.count_active(mask, counts)
    return pi.place_layer(lw, pi.hot_order(counts) if order == "hot" else pi.rank_order(counts))


def matrix_rows(cfg, lw, key):
    """(tensor view, row bytes) pieces of one weight matrix whose rows a
    gather reads: the matrix itself, or for repacked Q4_0 its code rows and
    its scale rows."""
    f, d = cfg.d_ff, cfg.d_model
    w = lw[key]
    if cfg.wtype != "q4_0":
        return [(w, d * ELEM_BYTES[cfg.wtype])]
    nb = d // 32
    flat = w.reshape(-1)
    codes = flat[:f * nb * 16].view(f, nb * 16)
    scales = flat[f * nb * 16:].view(f, nb * 2)
    return [(codes, nb * 16)] + ([(scales, nb * 2)] if (nb * 2) % 16 == 0 else [])


def _pred_kernels(cfg, n_tok):
    """Kernels of one pi_predict call (labels only)."""
    if cfg.pred_wtype == "f16" and cfg.d_model % 128 == 0 and cfg.rank % 128 == 0 and n_tok > 2:
        return "k_mp1 + k_tsplit + k_mp2"
    return "k_pred1 + k_pred2"


def _ffn_kernels(cfg, n_tok):
    """Kernels of one pi_sparse_ffn call (labels only)."""
    q4 = cfg.wtype == "q4_0"
    mfma_from = 3 if cfg.wtype == "f16" else _tile(cfg) + 1
    if n_tok >= mfma_from and cfg.wtype in ("f16", "q4_0") and cfg.d_model % 128 == 0:
        wide = min(n_tok, 64) > 32
        down_wide = "k_mdown_w4" if cfg.wtype == "f16" else "k_mdown_wide"
        return f"k_xstep + {'k_mup_wide + k_mfin + ' + down_wide if wide else 'k_mup + k_mdown'} + k_merge"
    return f"k_up + {'k_down_q4' if q4 else 'k_down'} + k_merge"


def _kernels(cfg, n_tok):
    """Kernels of one pi_layer call (labels only)."""
    pred = _pred_kernels(cfg, n_tok)
    if n_tok <= _tile(cfg) and pred == "k_pred1 + k_pred2" and _ffn_kernels(cfg, n_tok).startswith("k_up"):
        return f"k_pred1 + k_pred_up + {'k_down_q4' if cfg.wtype == 'q4_0' else 'k_down'} + k_merge"
    ffn = _ffn_kernels(cfg, n_tok)
    if pred.startswith("k_mp1"):
        # the matrix-core predictor also lists the union, and its first
        # product leaves the step-major copy of x that an fp16 FFN over one
        # token tile reuses
        if cfg.wtype == "f16" and n_tok <= 64 and ffn.startswith("k_xstep + "):
            ffn = ffn[len("k_xstep + "):]
        return f"{pred} (+ list) + {ffn}"
    return f"{pred} + {_compact_kernel(cfg)} + {ffn}"


def _compact_kernel(cfg):
    """pi_compact's kernel: one workgroup per tile for 16-byte aligned mask
    rows (the benchmark's masks are torch allocations, so aligned), else one."""
    return "k_compact_tiles" if cfg.d_ff % 16 == 0 else "k_compact"


def main(argv=None):
    ap = argparse.ArgumentParser(description="predictor-gated sparse FFN decode benchmark")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="falcon40b")
    ap.add_argument("--batch", type=int, default=1, help="tokens per decode step (their masks are OR-ed)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--reps", type=int, default=20, help="replays for the per-call timing graphs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prompt", action="store_true", help="skip the multi-token prompt measurement")
    ap.add_argument("--no-hot-order", action="store_true",
                    help="keep the generated neuron order (same as --order none)")
    ap.add_argument("--order", choices=("hot", "rank", "none"), default="hot",
                    help="neuron placement from the calibration profile: hot neurons dealt over the fused kernel's "
                         "segments (hot), neurons by firing rank (rank), or the generated order (none)")
    ap.add_argument("--calib", type=int, default=256, help="calibration tokens per layer for the hotness profile")
    ap.add_argument("--repeats", type=int, default=5, help="timed runs of the step loop (median and minimum reported)")
    args = ap.parse_args(argv)

    order = "none" if args.no_hot_order else args.order
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: runs on one GPU only; the sparse FFN is not sharded across GPUs "
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
    L, d, f, B = cfg.n_layers, cfg.d_model, cfg.d_ff, args.batch
    T = args.warmup + args.steps
    xdt = torch.float16 if cfg.x_dtype == "f16" else torch.float32
    n_prompt = cfg.prompt if (B == 1 and cfg.prompt > 0 and not args.no_prompt) else 0

    n_base_layers, n_base_tok = 2, 32   # about 10 s of oracle work per timing
    q4 = cfg.wtype == "q4_0"
    mats = ("w_up", "w_down_t", "w_gate")
    t_gen = time.perf_counter()
    layers, canon = [], []
    for li in range(L):
        lw = workload.make_layer(cfg, li, dev, args.seed)
        lw.pop("p")
        if order != "none":
            lw = place_by_hotness(pi, cfg, lw, li, args.seed, args.calib, dev, order)
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
    # decode inputs: T steps x L layers x B tokens, already in HBM
    x_all = torch.empty((T, L, B, d), dtype=xdt, device=dev)
    for li in range(L):
        x_all[:, li] = workload.make_tokens(cfg, li, T * B, dev, args.seed).view(T, B, d)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen

    preds = [pi.Predictor(lw["p1"], lw["p2"], lw["c"]) for lw in layers]
    ffns = [pi.FFN(lw["w_up"], lw["w_down_t"], cfg.act, b_up=lw.get("b_up"), w_gate=lw.get("w_gate"),
                   b_gate=lw.get("b_gate"), d_model=d if q4 else None) for lw in layers]
    ws = pi.alloc_workspace(preds[0], ffns[0], B, dev)        # zero-filled: fault flags clear
    x_stage = torch.zeros((L, B, d), dtype=xdt, device=dev)
    y_all = torch.empty((L, B, d), dtype=torch.float32, device=dev)

    stream = torch.cuda.Stream()
    # ---------------- the decode step graph ----------------
    with torch.cuda.stream(stream):
        for li in range(L):   # eager run once before capture (also loads code objects)
            pi.layer(preds[li], ffns[li], x_stage[li], cfg.tau, y_all[li], ws=ws)
    torch.cuda.synchronize()
    g_step = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_step, stream=stream):
        for li in range(L):
            pi.layer(preds[li], ffns[li], x_stage[li], cfg.tau, y_all[li], ws=ws)
    torch.cuda.synchronize()

    def step(t):
        x_stage.copy_(x_all[t], non_blocking=True)
        g_step.replay()

    with torch.cuda.stream(stream):
        for t in range(args.warmup):
            step(t)
    torch.cuda.synchronize()
    # the timed steps, repeated: each repeat replays the same K steps
    rows_before = pi.read_down_rows(ws, stream)
    up_before = pi.read_up_rows(ws, stream)
    rep_ms = []
    for r in range(max(1, args.repeats)):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            start.record(stream)
            for t in range(args.warmup, T):
                step(t)
            end.record(stream)
        torch.cuda.synchronize()
        rep_ms.append(start.elapsed_time(end))
        print(f"[bench] repeat {r + 1}: {args.steps} steps, {rep_ms[-1] / args.steps:.4f} ms/step", file=sys.stderr,
              flush=True)
    ms_total = float(np.median(rep_ms))
    ms_step = ms_total / args.steps
    layer_tok_s = args.steps * L * B / (ms_total / 1e3)
    flags_step = pi.read_flags(ws, stream)
    # down-projection rows the timed layer calls read (the workspace header's count)
    down_mean = (pi.read_down_rows(ws, stream) - rows_before) / (len(rep_ms) * args.steps * L)
    up_mean = (pi.read_up_rows(ws, stream) - up_before) / (len(rep_ms) * args.steps * L)
    if flags_step:
        print(f"[bench] fault flags raised during the timed steps: {flags_step:#x}", file=sys.stderr, flush=True)

    # ---------------- per-(layer, step) list lengths of the timed steps ----------------
    mask = torch.empty((L, B, f), dtype=torch.uint8, device=dev)
    idx = torch.empty((L, f), dtype=torch.int32, device=dev)
    cnt = torch.zeros((L,), dtype=torch.int32, device=dev)
    cnt_hist = torch.empty((args.steps, L), dtype=torch.int32, device=dev)
    ws_p = torch.empty(pi.workspace_bytes(preds[0], None, B), dtype=torch.uint8, device=dev)
    g_pc = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_pc, stream=stream):
        for li in range(L):
            pi.predict(preds[li], x_stage[li], cfg.tau, mask[li], ws=ws_p)
            pi.compact(mask[li], idx[li], cnt[li:li + 1])
    with torch.cuda.stream(stream):
        for t in range(args.warmup, T):
            x_stage.copy_(x_all[t], non_blocking=True)
            g_pc.replay()
            cnt_hist[t - args.warmup].copy_(cnt, non_blocking=True)
    torch.cuda.synchronize()
    counts = cnt_hist.cpu().numpy().astype(np.int64)
    cnt_mean = float(counts.mean())

    # ---------------- per-call timing: predict, compact, sparse FFN ----------------
    # inputs of the last timed step; idx/count of every layer from g_pc
    ws_s = torch.zeros(pi.workspace_bytes(None, ffns[0], B), dtype=torch.uint8, device=dev)   # header clear
    g_pred, g_comp, g_sp = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_pred, stream=stream):
        for li in range(L):
            pi.predict(preds[li], x_stage[li], cfg.tau, mask[li], ws=ws_p)
    with torch.cuda.graph(g_comp, stream=stream):
        for li in range(L):
            pi.compact(mask[li], idx[li], cnt[li:li + 1])
    with torch.cuda.graph(g_sp, stream=stream):
        for li in range(L):
            pi.sparse_ffn(ffns[li], x_stage[li], idx[li], cnt[li:li + 1], y_all[li], ws=ws_s)
    # the gather ceiling: the same active rows of every weight matrix read
    # with no arithmetic (pi_gather_read), over the same lists
    g_gr = torch.cuda.CUDAGraph()
    gr_out = torch.empty(pi._lib.PI_STREAM_BLOCKS, dtype=torch.int32, device=dev)
    mat_keys = [k for k in ("w_up", "w_gate", "w_down_t") if k in layers[0]]
    with torch.cuda.graph(g_gr, stream=stream):
        for li in range(L):
            for k in mat_keys:
                for view, rb in matrix_rows(cfg, layers[li], k):
                    pi.gather_read(view, idx[li], cnt[li:li + 1], row_bytes=rb, max_count=f, out=gr_out)
    sp_rows0, sp_up0 = pi.read_down_rows(ws_s, stream), pi.read_up_rows(ws_s, stream)
    # the dense-stream floor of the predictor: p1 and p2 of every layer read
    # with no arithmetic (pi_stream_read), each its own launch as in k_pred1 / k_pred2
    g_r1, g_r2 = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_r1, stream=stream):
        for li in range(L):
            pi.stream_read(layers[li]["p1"], gr_out)
    with torch.cuda.graph(g_r2, stream=stream):
        for li in range(L):
            pi.stream_read(layers[li]["p2"], gr_out)
    with torch.cuda.stream(stream):
        ms_r1 = _time_graph(g_r1, args.reps, stream) / L
        ms_r2 = _time_graph(g_r2, args.reps, stream) / L
    with torch.cuda.stream(stream):
        ms_pred = _time_graph(g_pred, args.reps, stream) / L
        ms_comp = _time_graph(g_comp, args.reps, stream) / L
        ms_sp = _time_graph(g_sp, args.reps, stream) / L
        ms_gr = _time_graph(g_gr, args.reps, stream) / L
    sp_down = (pi.read_down_rows(ws_s, stream) - sp_rows0) / ((args.reps + 1) * L)
    sp_up = (pi.read_up_rows(ws_s, stream) - sp_up0) / ((args.reps + 1) * L)
    last_cnt = cnt.cpu().numpy().astype(np.int64)
    last_mean = float(last_cnt.mean())
    b_pred = bytes_predict(cfg, B)
    b_comp = float(np.mean([bytes_compact(cfg, c, B) for c in last_cnt]))
    b_sp = bytes_gather(cfg, last_mean, B, sp_down, sp_up)
    b_act = bytes_active(cfg, last_mean, sp_down, sp_up)
    b_listed = bytes_active(cfg, last_mean)          # every listed row of every matrix

    traffic_table = load_traffic(f"{cfg.name} decode batch {B}")

    def traffic_of(kernels, table=traffic_table):
        # measured HBM bytes per call of the kernel set named in the label
        names = re.findall(r"k_[a-z0-9_]+", kernels)
        if table is None or not names or any(k not in table for k in names):
            return None
        return int(sum(table[k] for k in names))

    def roof(kernels, b, ms, table=traffic_table):
        gbps = b / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "kernel": kernels, "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic_of(kernels, table),
                "bytes_per_launch": int(b), "avg_launch_us": round(ms * 1e3, 3)}

    # achievable HBM read bandwidth: a plain streaming read (pi_stream_read)
    # of an 8 GiB buffer, the reference the path's streams are compared with
    stream_gbps = measure_stream(pi, dev, stream)

    # whole-layer bytes per layer call, averaged over the timed steps (bytes
    # are linear in the list length and the up and down rows read)
    b_layer = bytes_layer(cfg, cnt_mean, B, down_mean, up_mean)
    ms_layer = ms_step / L
    kern = _kernels(cfg, B)
    layer_roof = roof(f"pi_layer ({kern})", b_layer, ms_layer)
    parts = {
        "predict": roof(f"pi_predict ({_pred_kernels(cfg, B)})", b_pred, ms_pred),
        "compact": {"kernel": f"pi_compact ({_compact_kernel(cfg)})", "avg_launch_us": round(ms_comp * 1e3, 3),
                    "bytes_per_launch": int(b_comp), "traffic": traffic_of(_compact_kernel(cfg))},
        "gather": roof(f"pi_sparse_ffn ({_ffn_kernels(cfg, B)})", b_sp, ms_sp),
    }
    gather_read_gbps = round(b_listed / (ms_gr * 1e-3) / 1e9, 1)
    for r in (layer_roof, parts["predict"], parts["gather"]):
        r["stream_read_gbps"] = stream_gbps
        r["frac_of_stream_read"] = round(r["achieved"] / stream_gbps, 4)
        r["gather_read_gbps"] = gather_read_gbps
    parts["gather"]["active_weight_gbps"] = round(b_act / (ms_sp * 1e-3) / 1e9, 1)
    parts["gather"]["active_weight_frac"] = round(b_act / (ms_sp * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
    parts["gather"]["frac_of_gather_read"] = round(parts["gather"]["active_weight_gbps"] / gather_read_gbps, 4)
    parts["gather_read"] = {"what": "pi_gather_read of every listed row of every weight matrix, no arithmetic",
                            "avg_us_per_layer": round(ms_gr * 1e3, 3), "bytes_per_layer": int(b_listed),
                            "gbps": gather_read_gbps}
    b_p1 = layers[0]["p1"].numel() * layers[0]["p1"].element_size()
    b_p2 = layers[0]["p2"].numel() * layers[0]["p2"].element_size()
    parts["predictor_read"] = {"what": "pi_stream_read of p1, and separately of p2, of every layer, no arithmetic",
                               "p1_us_per_layer": round(ms_r1 * 1e3, 3), "p1_bytes": b_p1,
                               "p1_gbps": round(b_p1 / (ms_r1 * 1e-3) / 1e9, 1),
                               "p2_us_per_layer": round(ms_r2 * 1e3, 3), "p2_bytes": b_p2,
                               "p2_gbps": round(b_p2 / (ms_r2 * 1e-3) / 1e9, 1)}

    out = {
        "metric": METRIC if B == 1 else METRIC.replace("(batch 1)", f"(batch {B})"),
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
        "config": {"workload": f"{cfg.name} decode batch {B}", "d_model": d, "d_ff": f, "layers": L,
                   "rank": cfg.rank, "act": cfg.act, "weights": cfg.wtype, "batch": B,
                   "mean_density": cfg.rho, "parallelism": "none (1 GPU)",
                   "neuron_order": {"none": "as generated",
                                    "hot": f"by hotness, dealt over segments ({args.calib} calibration tokens "
                                           f"per layer)",
                                    "rank": f"by firing rank ({args.calib} calibration tokens per layer)"}[order]},
        "repeats": {"n": len(rep_ms), "value": "median",
                    "ms_per_step_median": round(ms_step, 4),
                    "ms_per_step_min": round(min(rep_ms) / args.steps, 4),
                    "ms_per_step_max": round(max(rep_ms) / args.steps, 4),
                    "value_at_min": round(args.steps * L * B / (min(rep_ms) / 1e3), 1)},
        "fault_flags": flags_step,
        "roofline": layer_roof,
        "roofline_parts": parts,
        "count_mean": round(cnt_mean, 1),
        "down_rows_mean": round(down_mean, 1),
        "up_rows_mean": round(up_mean, 1),
        "count_min": int(counts.min()),
        "count_max": int(counts.max()),
        "gen_seconds": round(t_gen, 1),
    }

    # ---------------- multi-token prompt: per-token masks OR-ed, matrix-core path ----------------
    if n_prompt:
        n = n_prompt
        x_pr = torch.empty((L, n, d), dtype=xdt, device=dev)
        for li in range(L):
            x_pr[li] = workload.make_tokens(cfg, li, n, dev, args.seed, stream=1)
        y_pr = torch.empty((L, n, d), dtype=torch.float32, device=dev)
        ws_m = torch.zeros(pi.workspace_bytes(preds[0], ffns[0], n), dtype=torch.uint8, device=dev)
        mask_m = torch.empty((L, n, f), dtype=torch.uint8, device=dev)
        idx_m = torch.empty((L, f), dtype=torch.int32, device=dev)
        cnt_m = torch.zeros((L,), dtype=torch.int32, device=dev)
        ws_mp = torch.empty(pi.workspace_bytes(preds[0], None, n), dtype=torch.uint8, device=dev)
        ws_ms = torch.empty(pi.workspace_bytes(None, ffns[0], n), dtype=torch.uint8, device=dev)
        with torch.cuda.stream(stream):
            for li in range(L):
                pi.predict(preds[li], x_pr[li], cfg.tau, mask_m[li], ws=ws_mp)
                pi.compact(mask_m[li], idx_m[li], cnt_m[li:li + 1])
                pi.layer(preds[li], ffns[li], x_pr[li], cfg.tau, y_pr[li], ws=ws_m)
        torch.cuda.synchronize()
        g_ml, g_mp, g_ms = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_ml, stream=stream):
            for li in range(L):
                pi.layer(preds[li], ffns[li], x_pr[li], cfg.tau, y_pr[li], ws=ws_m)
        with torch.cuda.graph(g_mp, stream=stream):
            for li in range(L):
                pi.predict(preds[li], x_pr[li], cfg.tau, mask_m[li], ws=ws_mp)
        with torch.cuda.graph(g_ms, stream=stream):
            for li in range(L):
                pi.sparse_ffn(ffns[li], x_pr[li], idx_m[li], cnt_m[li:li + 1], y_pr[li], ws=ws_ms)
        reps = max(2, args.reps // 4)
        ml_rows0, ml_up0 = pi.read_down_rows(ws_m, stream), pi.read_up_rows(ws_m, stream)
        with torch.cuda.stream(stream):
            ms_ml = _time_graph(g_ml, reps, stream) / L
            ms_mp = _time_graph(g_mp, reps, stream) / L
            ms_ms = _time_graph(g_ms, reps, stream) / L
        ml_down = (pi.read_down_rows(ws_m, stream) - ml_rows0) / ((reps + 1) * L)
        ml_up = (pi.read_up_rows(ws_m, stream) - ml_up0) / ((reps + 1) * L)
        # the union's rows of every weight matrix read with no arithmetic
        g_mgr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_mgr, stream=stream):
            for li in range(L):
                for k in mat_keys:
                    for view, rb in matrix_rows(cfg, layers[li], k):
                        pi.gather_read(view, idx_m[li], cnt_m[li:li + 1], row_bytes=rb, max_count=f, out=gr_out)
        with torch.cuda.stream(stream):
            ms_mgr = _time_graph(g_mgr, reps, stream) / L
        uc = cnt_m.cpu().numpy().astype(np.int64)
        uc_mean = float(uc.mean())
        b_ml = bytes_layer(cfg, uc_mean, n, ml_down, ml_up)
        b_ms = bytes_gather(cfg, uc_mean, n)
        fl = float(np.mean([flops_ffn(cfg, c, n) for c in uc]))
        tflops = fl / (ms_ms * 1e-3) / 1e12
        mk = _kernels(cfg, n)
        traffic_pr = load_traffic(f"{cfg.name} prompt {n}")
        out["multi_token"] = {
            "what": f"one prompt of {n} tokens per layer, per-token masks OR-ed into one list",
            "n_tok": n,
            "union_count_mean": round(uc_mean, 1),
            "down_rows_mean": round(ml_down, 1),
            "up_rows_mean": round(ml_up, 1),
            "layer_tokens_per_s": round(n / (ms_ml * 1e-3), 1),
            "layer": roof(f"pi_layer ({mk})", b_ml, ms_ml, traffic_pr),
            "predict": roof(f"pi_predict ({_pred_kernels(cfg, n)})", bytes_predict(cfg, n), ms_mp, traffic_pr),
            "gather": roof(f"pi_sparse_ffn ({_ffn_kernels(cfg, n)})", b_ms, ms_ms, traffic_pr),
            "gather_mfma": {"bound": "mfma", "achieved": round(tflops, 1), "peak": 2500.0, "unit": "TFLOP/s",
                            "frac": round(tflops / 2500.0, 4), "flops_per_launch": fl},
            "gather_read": {"what": "pi_gather_read of the union's rows of every weight matrix, no arithmetic",
                            "avg_us_per_layer": round(ms_mgr * 1e3, 3),
                            "bytes_per_layer": int(np.mean([bytes_active(cfg, c) for c in uc])),
                            "gbps": round(float(np.mean([bytes_active(cfg, c) for c in uc])) / (ms_mgr * 1e-3) / 1e9,
                                          1)},
        }
        print(f"[bench] prompt {n}: layer {ms_ml * 1e3:.1f} us, gather {ms_ms * 1e3:.1f} us", file=sys.stderr,
              flush=True)

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
