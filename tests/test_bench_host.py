"""Host-side logic of bench.py that needs no GPU: the clock summary drops the
samples read before the firmware's clock table first refreshed."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _sampler(samples):
    c = bench.ClockSampler.__new__(bench.ClockSampler)
    c._thread = None
    c.handle = None
    c.error = None
    c.samples = samples
    return c


def test_clock_summary_drops_samples_before_the_first_refresh():
    s = _sampler([(150.0, 2000.0, 0.00), (150.0, 2000.0, 0.01), (1700.0, 1900.0, 0.02),
                  (1800.0, 2000.0, 0.03), (1600.0, 2000.0, 0.04)]).stop()
    assert s["samples"] == 3
    assert s["gfx_mhz_median"] == 1700.0
    assert s["gfx_mhz_min"] == 1600.0 and s["gfx_mhz_max"] == 1800.0
    assert s["mem_mhz_median"] == 2000.0
    assert abs(s["window_s"] - 0.04) < 1e-9


def test_clock_summary_reports_a_table_that_never_refreshed():
    s = _sampler([(150.0, 2000.0, 0.0), (150.0, 2000.0, 0.01)]).stop()
    assert "gfx_mhz_median" not in s and "note" in s


def test_clock_summary_without_samples_gives_the_reason():
    c = _sampler([])
    c.error = "AmdSmiLibraryException: driver not loaded"
    s = c.stop()
    assert s["samples"] == 0 and "driver" in s["error"]


def _write_counter_csv(path, rows):
    import csv
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for name, counter, value in rows:
            wr.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def _summarize(tmp_path, monkeypatch, class_split):
    import argparse
    import json
    import types
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "_plan",
                        lambda args: types.SimpleNamespace(path=2, class_split=class_split))
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    cfetch, cwrite = tmp_path / "cf.csv", tmp_path / "cw.csv"
    # the copy of 1 MiB reads 512 KiB and writes 1024 KiB as counted: scales 2 and 1
    _write_counter_csv(cfetch, [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 512.0)])
    _write_counter_csv(cwrite, [("__amd_rocclr_copyBuffer", "WRITE_SIZE", 1024.0)])
    _write_counter_csv(fetch, [("ua_attn_kernel<...>", "FETCH_SIZE", 10.0),
                               ("ua_decode16_kernel<...>", "FETCH_SIZE", 100.0),
                               ("ua_decode16_kernel<...>", "FETCH_SIZE", 102.0),
                               ("ua_reduce_kernel<...>", "FETCH_SIZE", 5.0)])
    _write_counter_csv(write, [("ua_attn_kernel<...>", "WRITE_SIZE", 8.0),
                               ("ua_decode16_kernel<...>", "WRITE_SIZE", 3.0),
                               ("ua_reduce_kernel<...>", "WRITE_SIZE", 1.0)])
    args = argparse.Namespace(workload="variant_mix", summarize_traffic=[
        str(fetch), str(write), str(cfetch), str(cwrite), str(1 << 20)])
    bench.summarize_traffic(args)
    return json.load(open(tmp_path / "profiles" / "variant_mix_hbm_traffic.json"))


def test_traffic_of_one_launch_is_its_dominant_attention_kernel(tmp_path, monkeypatch):
    t = _summarize(tmp_path, monkeypatch, class_split=0)
    assert t["fetch_scale"] == 2.0 and t["write_scale"] == 1.0
    assert t["attention_kernel"] == "ua_decode16_kernel"
    # decode16: (100 + 102) / 2 KiB read x 2, 3 KiB written
    assert t["bytes_per_launch"] == 101 * 1024 * 2 + 3 * 1024


def test_traffic_of_a_class_split_sums_its_timed_span(tmp_path, monkeypatch):
    t = _summarize(tmp_path, monkeypatch, class_split=1)
    assert t["attention_kernel"] == "ua_attn_kernel+ua_decode16_kernel+ua_reduce_kernel"
    read = (10 + 101 + 5) * 1024 * 2
    written = (8 + 3 + 1) * 1024
    assert t["bytes_per_launch"] == read + written


def test_select_repacks_queries_and_keeps_the_pool():
    from varlen_attention_serving_amd import workloads as W
    w = W.random_small(11, num_seqs=5)
    s = w.select([3, 0])
    assert list(s.q_lens) == [w.q_lens[3], w.q_lens[0]]
    assert list(s.seq_lens) == [w.seq_lens[3], w.seq_lens[0]]
    assert list(s.cu_seqlens_q) == [0, w.q_lens[3], w.q_lens[3] + w.q_lens[0]]
    lo3, hi3 = w.cu_seqlens_q[3], w.cu_seqlens_q[4]
    assert (s.q[:hi3 - lo3] == w.q[lo3:hi3]).all()
    assert (s.q[hi3 - lo3:] == w.q[:w.q_lens[0]]).all()
    assert (s.block_table[0] == w.block_table[3]).all()
    assert s.k_cache is w.k_cache and s.v_cache is w.v_cache


def test_parts_split_a_mixed_batch_and_switch_features_off():
    from varlen_attention_serving_amd import workloads as W
    w = W.named("chunked_prefill_mix")
    parts = dict(bench.part_batches(w))
    assert list(parts) == ["all", "decode_seqs", "wide_seqs", "no_softcap", "no_window"]
    assert parts["decode_seqs"].num_seqs + parts["wide_seqs"].num_seqs == w.num_seqs
    assert parts["decode_seqs"].total_q + parts["wide_seqs"].total_q == w.total_q
    # bytes split between the two classes: the second batch adds one cu_seqlens_q entry
    total = bench.algorithmic_work(w)["bytes"]
    assert (bench.algorithmic_work(parts["decode_seqs"])["bytes"]
            + bench.algorithmic_work(parts["wide_seqs"])["bytes"]) == total + 4
    assert parts["no_softcap"].softcap == 0.0 and parts["no_window"].window == 0
    assert dict(bench.part_batches(W.named("long_prefill"))).keys() == {"all"}
