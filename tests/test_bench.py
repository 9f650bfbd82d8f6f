"""Host-side checks of bench.py's bookkeeping (no GPU)."""
import dataclasses
import os
import subprocess
import sys

import numpy as np

import bench
from draft_token_verification_10_amd import workloads as W


def test_algorithmic_bytes_workload2():
    s = W.SPECS[2]
    # the figures the benchmark is quoted on
    assert bench.algorithmic_bytes(s, "stochastic") == 1_116_367_872
    assert bench.algorithmic_bytes(s, "greedy") == 591_023_104


def test_ragged_bytes_reduce_to_dense():
    s = W.SPECS[2]
    kb = np.full(s.B, s.k)
    cu_bytes = 4 * (s.B + 1)
    assert bench.algorithmic_bytes(s, "ragged", kb) == \
        bench.algorithmic_bytes(s, "stochastic") + cu_bytes
    # greedy: the same minus best_cand, plus cu
    assert bench.algorithmic_bytes(s, "ragged", kb, greedy=True) == \
        bench.algorithmic_bytes(s, "greedy") - 4 * s.B + cu_bytes


def test_sample_bytes():
    s = W.SPECS[2]
    assert bench.algorithmic_bytes(s, "sample") == s.B * s.V * 2 + 8 * s.B
    assert bench.algorithmic_bytes(s, "sample", greedy=True) == s.B * s.V * 2 + 4 * s.B


def test_copies_defeat_last_level_cache():
    assert bench.n_copies(1_116_367_872, None) == 1
    assert bench.n_copies(147_750_912, None) * 147_750_912 >= bench.COLD_BYTES
    assert bench.n_copies(10, None) == bench.MAX_COPIES
    assert bench.n_copies(10, 3) == 3


def test_ragged_batch_packing():
    b = W.make(1, seqs=range(5))
    r = W.ragged(b)
    assert r.cu[0] == 0 and np.all(np.diff(r.cu) == r.kb) and np.all((r.kb >= 1) & (r.kb <= 4))
    for i in range(5):
        k, d0 = int(r.kb[i]), int(r.cu[i])
        assert np.array_equal(r.target[d0 + i:d0 + i + k + 1], b.target[i, :k + 1])
        assert np.array_equal(r.draft[d0:d0 + k], b.draft[i, :k])
        assert np.array_equal(r.draft_tokens[d0:d0 + k], b.draft_tokens[i, :k])


def test_several_gpus_refused():
    p = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True,
                       text=True, cwd=bench.ROOT, timeout=120)
    assert p.returncode == 2 and "one GPU" in p.stderr


def test_tree_workload_shape():
    par = W.tree_parents()
    assert len(par) == sum(W.TREE_LEVELS) == 64
    assert par[0] == -1 and all(0 <= par[j] < j for j in range(1, 64))
    depth = [0] * 64
    for j in range(1, 64):
        depth[j] = depth[par[j]] + 1
    assert [depth.count(d) for d in range(len(W.TREE_LEVELS))] == list(W.TREE_LEVELS)
    tb = W.tree_batch(B=2, V=300)
    assert tb.target.shape == (2, 64, 300) and tb.node_tokens[:, 0].tolist() == [-1, -1]
    assert bench.tree_bytes(32, 64, 128256, 2) == 32 * 64 * 128256 * 2 + 16 * 32 * 64 + 4 * 32


def test_commit_bytes():
    assert bench.commit_bytes([0, 2], 3) == 4 * 2 + 4 * 6 + 4 * 2 + 4 * 4 + 4 * 2 + 4 * 2


def test_kernel_names_follow_layouts():
    s2, s1 = W.SPECS[2], W.SPECS[1]
    assert bench.kernel_name(s2, "stochastic") == "k_stochastic_seq_exit (full read)"
    # 512-thread groups: position order from 384 sequences on rows of at
    # least 160000 bytes (B=512, V=129280 bf16), else pair 0 streamed last
    assert bench.kernel_name(W.SPECS[3], "stochastic") == "k_stochastic_seq_exit (full read)"
    s3 = W.SPECS[3]
    assert bench.kernel_name(dataclasses.replace(s3, B=383), "stochastic") == "k_stochastic_seq"
    assert bench.kernel_name(dataclasses.replace(s3, B=513), "stochastic") == "k_stochastic_seq"
    assert bench.kernel_name(dataclasses.replace(s3, V=79999), "stochastic") == "k_stochastic_seq"
    assert bench.kernel_name(dataclasses.replace(s3, V=80000), "stochastic").startswith("k_stochastic_seq_exit")
    assert bench.kernel_name(dataclasses.replace(s3, V=40000, dtype=W.F32), "stochastic").startswith(
        "k_stochastic_seq_exit")
    # without diagnostics: the capped early exit for k >= 6 (B=256, k=8), the
    # plain one below (B=512, k=3)
    assert bench.kernel_name(s2, "stochastic", diagnostics=False).startswith(
        "k_stochastic_seq_exit (capped) + k_exit_stats")
    assert bench.kernel_name(W.SPECS[3], "stochastic", diagnostics=False) == "k_stochastic_seq_exit"
    assert bench.kernel_name(s2, "greedy") == "k_greedy_seq"
    assert bench.kernel_name(s2, "ragged", uniform=False) == "k_row_stats"
    assert bench.kernel_name(s2, "ragged", uniform=True) == "k_stochastic_seq_exit (full read)"
    assert bench.kernel_name(s2, "sample") == "k_sample_seq"
    assert bench.kernel_name(s1, "sample") == "k_row_stats"
    assert bench.sample_one_pass(512, 98304, 2) and not bench.sample_one_pass(512, 128256, 2)
    assert bench.sample_one_pass(257, 32000, 2) and not bench.sample_one_pass(300, 65536, 2)
    assert bench.kernel_name(s1, "sample", greedy=True) == "k_row_stats"
    assert bench.kernel_name(s2, "sample", greedy=True) == "k_greedy_seq"
    assert bench.kernel_name(s1, "stochastic") == "k_row_stats"


def test_cpu_baseline_reports_threads_and_single_thread():
    """The oracle timing leg: the threaded figure, a one-thread pass beside
    it, and the oracle's thread count restored afterwards."""
    import numpy as np
    from oracle import svo
    rng = np.random.default_rng(3)
    rows = rng.standard_normal((4, 1000)).astype(np.float32)
    u = np.full(4, 0.5, np.float32)
    before = svo.num_threads()
    nbytes = rows.nbytes + 8 * 4
    out = bench.cpu_baseline(lambda: svo.sample(rows, u, B=4, V=1000), 4, "a tiny batch",
                             nbytes, 1e6, min_reps=3, target_s=0.05)
    assert svo.num_threads() == before
    assert out["kind"] == "oracle" and out["cores"] == before and out["value"] > 0
    assert out["threads"] == before and out["logical_cpus"] == os.cpu_count()
    assert out["cpu_model"] and out["physical_cores"] >= 1
    # the oracle's rate on the same bytes, and the GPU's lead over it
    med = 4 / out["value"]
    assert abs(out["GBps"] - nbytes / med / 1e9) <= 1e-3 + 1e-3 * out["GBps"]
    assert abs(out["gpu_speedup"] - 1e6 / out["value"]) <= 0.05 + 1e-3 * out["gpu_speedup"]
    st = out["single_thread"]
    assert st["cores"] == 1 and st["value"] > 0 and st["unit"] == "seqs/s"
    assert st["GBps"] > 0 and st["gpu_speedup"] > 0


def test_fetched_rate():
    r = bench.fetched_rate(8e9, 1000.0)  # 8 GB in one second
    assert r == {"fetched_GBps": 8.0, "fetched_frac": 0.001}
    assert bench.fetched_rate(None, 1.0) == {"fetched_GBps": None, "fetched_frac": None}


def test_record_traffic(tmp_path, monkeypatch):
    """Counter CSVs -> bytes per call: the copy calibration's factor, then a
    two-kernel call summed over its kernels (median over dispatches), tagged
    with the kernel source hash so a later source change voids it."""
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))

    def csv_file(name, rows):
        p = tmp_path / name
        p.write_text("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n" +
                     "".join(f"{i},{k},C,{v}\n" for i, (k, v) in enumerate(rows)))
        return str(p)

    gib_kib = (1 << 30) / 1024
    fc = csv_file("fc.csv", [("__amd_rocclr_copyBuffer", gib_kib / 2)] * 3)
    wc = csv_file("wc.csv", [("__amd_rocclr_copyBuffer", gib_kib)] * 3)
    cal = bench.record_traffic("_calibration", fc, wc, ["__amd_rocclr_copyBuffer"], "cal")
    assert cal["fetch_scale"] == 2.0 and cal["write_scale"] == 1.0
    rows_f = [("void sv::k_a<1>(sv::Params)", 100.0), ("void sv::k_a_exit<1>(sv::Params)", 7.0),
              ("void sv::k_b<1>(sv::Params)", 10.0), ("void sv::k_a<1>(sv::Params)", 102.0),
              ("void sv::k_a<1>(sv::Params)", 1000.0), ("void sv::k_b<1>(sv::Params)", 12.0)]
    rows_w = [(k, v / 10) for k, v in rows_f]
    e = bench.record_traffic("x/y", csv_file("f.csv", rows_f), csv_file("w.csv", rows_w),
                             ["sv::k_a<", "sv::k_b<"], "src")
    # medians: k_a 102 (k_a_exit not matched), k_b 11
    assert e["fetch_bytes_per_launch"] == int((102 + 11) * 1024 * 2)
    assert e["write_bytes_per_launch"] == int(round((10.2 + 1.1) * 1024))
    assert e["bytes_per_launch"] == e["fetch_bytes_per_launch"] + e["write_bytes_per_launch"]
    assert bench.traffic_for("x/y") == e["bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_hash", lambda: "other")
    assert bench.traffic_for("x/y") is None
