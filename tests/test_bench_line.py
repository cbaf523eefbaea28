"""bench.py's last stdout line stays compact (the driver keeps only the tail
of stdout) and carries the fields the measurement contract names.  Built
from synthetic numbers on the CPU; no GPU involved."""
import json

import bench


def _head():
    per = {k: {"launches": n, "us_per_launch": us, "bytes_per_launch": b, "gbs": b / us / 1e3}
           for k, n, us, b in [("qkv", 32, 8.2, 26779648), ("o", 32, 5.5, 17825792),
                               ("gate_up", 32, 23.1, 124911616), ("down", 32, 13.4, 62390272),
                               ("lm_head", 1, 90.0, 558726144)]}
    return {"steps": 50, "graph": True, "launches_per_step": 129, "bytes_per_step": 7984714752,
            "ms_per_step": 1.6832, "gpu_ms_per_step": 1.6811, "gbs_wall": 4743.7, "gbs_gpu": 4749.6,
            "kernel_ms_per_step": 1.6123, "gbs_kernel": 4952.4, "tok_s_wall": 594.1, "tok_s_kernel": 620.2,
            "per_matrix": per, "pct_peak_wall": 59.3, "pct_peak_kernel": 61.9}


def test_final_line_is_compact_and_complete():
    ceiling = {"value": 6784.2, "best": 6811.0, "unit": "GB/s", "bytes": 4 << 30, "frac_of_peak": 0.848,
               "launches": 7, "statistic": "median", "kernel": "stream_read_kernel (qmv_stream_read)"}
    cpu = {"value": 1.288, "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": "one batch-1 Q8_0 8B token: a layer's 7 matrices timed once x32 + lm_head, "
                     "7984714752 B in 6.20 s, 1 thread",
           "host_cpus": 16, "cpu_model": "AMD EPYC 9575F 64-Core Processor", "tok_s_equiv": 0.1613}
    # more sweeps, with longer names, than a default run produces
    summary = {f"llama8b_q4_1_fused_grouped_chain_b{i}": [12345, 123456] for i in range(40)}
    line = bench.final_line(_head(), ceiling, cpu, summary, 50, 3)
    text = json.dumps(line)
    assert len(text) < 4096, len(text)
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline", "read_ceiling", "cpu_baseline"):
        assert k in line, k
    assert line["config"]["workload"]
    roof = line["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in roof, k
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert line["cpu_baseline"]["kind"] == "oracle" and line["cpu_baseline"]["cores"] == 1
    assert "\n" not in text
