"""The benchmark's algorithmic byte counts (the roofline numerators), written
out by hand for the model shapes: per layer call at batch 1, the predictor
(p1 [r][d] and p2 [d_ff][r] in fp16, c fp32), the active rows of the FFN
matrices (one row per listed neuron per matrix: 2 bytes per weight for fp16,
18 bytes per 32 weights for Q4_0), a bias and a list entry per listed neuron,
x in and y (fp32) out.  CPU only."""

import bench
import workload


def _by_hand(d, d_ff, r, n_mat, row_bytes, cnt, x_bytes=2):
    pred = (r * d + d_ff * r) * 2 + 4 * d_ff
    active = cnt * n_mat * row_bytes
    return pred + active + 8 * cnt + d * x_bytes + 4 * d


def test_falcon_fp16_layer_bytes():
    cfg = workload.get_config("falcon40b")
    cnt = 3277
    assert bench.bytes_layer(cfg, cnt) == _by_hand(8192, 32768, 1024, 2, 8192 * 2, cnt)
    # about 191.5 MB at the mean list length: 84.0 MB of predictor, 107.4 MB of rows
    assert abs(bench.bytes_layer(cfg, cnt) / 1e6 - 191.5) < 0.2
    assert bench.bytes_active(cfg, cnt) == 3277 * 2 * 16384


def test_llama_reglu_and_q4_layer_bytes():
    cfg = workload.get_config("llama70b")
    assert bench.bytes_layer(cfg, 2867) == _by_hand(8192, 28672, 1024, 3, 8192 * 2, 2867)
    q = workload.get_config("falcon40b_q4")
    assert bench.bytes_active(q, 3277) == 3277 * 2 * (8192 // 32 * 18)
    assert bench.bytes_layer(q, 3277) == _by_hand(8192, 32768, 1024, 2, 4608, 3277)


def test_gather_and_predict_bytes():
    cfg = workload.get_config("falcon40b")
    assert bench.bytes_gather(cfg, 100) == 100 * 2 * 16384 + 800 + 8192 * 2 + 8192 * 4
    assert bench.bytes_predict(cfg) == (1024 * 8192 + 32768 * 1024) * 2 + 4 * 32768 + 8192 * 2 + 32768


def test_down_rows_read_replace_listed_down_rows():
    # The down projection leaves out rows whose h is zero for every token and
    # counts the rows it reads; the bytes then take that count for the down
    # matrix only (the up and gate rows of every listed neuron are still read).
    cfg = workload.get_config("falcon40b")
    rb = 8192 * 2
    assert bench.bytes_active(cfg, 3277, 1456) == (3277 + 1456) * rb
    assert bench.bytes_layer(cfg, 3277, 1, 1456) == bench.bytes_layer(cfg, 3277) - (3277 - 1456) * rb
    assert bench.bytes_gather(cfg, 3277, 1, 3277) == bench.bytes_gather(cfg, 3277)
    ll = workload.get_config("llama70b")
    assert bench.bytes_active(ll, 2867, 1000) == (2 * 2867 + 1000) * rb


def test_up_rows_read_replace_listed_up_rows():
    # The fused ReGLU kernel reads a listed neuron's up row only when its gate
    # fires for some token and counts the up rows it reads; the gate rows of
    # every listed neuron are still read.
    ll = workload.get_config("llama70b")
    rb = 8192 * 2
    assert bench.bytes_active(ll, 2867, 1000, 1200) == (2867 + 1200 + 1000) * rb
    assert bench.bytes_active(ll, 2867, None, 2867) == bench.bytes_active(ll, 2867)
    assert bench.bytes_layer(ll, 2867, 1, 1000, 1200) == bench.bytes_layer(ll, 2867, 1, 1000) - (2867 - 1200) * rb
    assert bench.bytes_gather(ll, 2867, 1, None, 0) == bench.bytes_gather(ll, 2867) - 2867 * rb
    fc = workload.get_config("falcon40b")     # ReLU: no gate matrix
    assert bench.bytes_active(fc, 3277, 1456, 3000) == (3000 + 1456) * rb


def test_kernel_defining_file():
    # the traffic summaries hash each kernel's own sources: the file that
    # defines it is found by its __global__ declaration
    assert bench.kernel_defining_file("k_mp2") == "k_mfma.hip"
    assert bench.kernel_defining_file("k_down") == "k_gather.hip"
    assert bench.kernel_defining_file("k_down_q4") == "k_gather.hip"
    assert bench.kernel_defining_file("k_pred1") == "k_predict.hip"
    assert bench.kernel_defining_file("k_compact_tiles") == "k_compact.hip"
    assert bench.kernel_defining_file("k_no_such_kernel") is None
    assert bench.kernel_sources("k_merge") == sorted({"k_gather.hip", *bench.KERNEL_COMMON_SOURCES})


def test_traffic_counts_go_stale_per_kernel(tmp_path, monkeypatch):
    # A tree with two kernels in two files: after one file changes, only the
    # kernel it defines loses its counts.
    import json
    csrc = tmp_path / "activation_sparse_rank_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "include").mkdir()
    (tmp_path / "include" / "pi.h").write_text("// header\n")
    (csrc / "a.hip").write_text("__global__ void k_one(int* p) { *p = 1; }\n")
    (csrc / "b.hip").write_text("__global__ __launch_bounds__(64) void k_two(int* p) { *p = 2; }\n")
    for f in bench.KERNEL_COMMON_SOURCES:
        (csrc / f).write_text("// common\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    kern = {}
    for k in ("k_one", "k_two"):
        src = bench.kernel_sources(k)
        kern[k] = {"fetch_kib": 1.0, "write_kib": 1.0, "dispatches": 1, "source_files": src,
                   "source_sha256": bench.kernel_source_sha256(src)}
    data = {"workload": "w", "fetch_scale": 2.0, "write_scale": 1.0, "kernels": kern}
    (tmp_path / "profiles" / "w_traffic.md").write_text("```json\n" + json.dumps(data) + "\n```\n")
    assert set(bench.load_traffic("w")) == {"k_one", "k_two"}
    assert bench.load_traffic("w")["k_one"] == 3.0 * 1024
    (csrc / "b.hip").write_text("__global__ __launch_bounds__(64) void k_two(int* p) { *p = 3; }\n")
    assert set(bench.load_traffic("w")) == {"k_one"}
    (csrc / "abi.hip").write_text("// changed\n")        # a common source: every kernel
    assert bench.load_traffic("w") == {}
    assert bench.load_traffic("other") is None


def test_committed_traffic_summaries_have_per_kernel_sources():
    import glob, json, os, re
    for path in glob.glob(os.path.join(bench.ROOT, "profiles", "*_traffic.md")):
        data = json.loads(re.search(r"```json\n(.*?)\n```", open(path).read(), re.S).group(1))
        assert data["kernels"], path
        for k, v in data["kernels"].items():
            assert v["source_files"] == bench.kernel_sources(k), (path, k)
