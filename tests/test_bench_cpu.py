"""bench.py's host logic, no GPU: the single-GPU exit, the choice of the M=1
decode figures, and the workload constants the roofline divides by."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one MI355X" in r.stderr and "--gpus 1" in r.stderr
    assert r.stdout == ""                       # no JSON line for an unsupported request


def test_workload_flop_and_bytes():
    """2MNK and packed bytes of the step's shapes, against the figures worked out
    for these shapes beforehand (4.5 bits per packed element: codes + E4M3 scales)."""
    assert bench.FLOP["gate_up"] == 1_460_288_880_640
    assert bench.FLOP["down"] == 730_144_440_320
    assert bench.FLOP["gdn"] == 691_221_299_200
    assert bench.FLOP["decode"] == 178_257_920
    assert bench.DECODE_W_BYTES == 50_135_040
    # A codes+scales, W codes+scales, bf16 output
    assert bench.ALGO_BYTES["gdn"] == 10_485_760 + 1_310_720 + 42_188_800 + 5_273_600 + 135_004_160
    assert bench.ALGO_BYTES["gate_up"] == 10_485_760 + 1_310_720 + 89_128_960 + 11_141_120 + 142_606_336
    assert bench.ALGO_BYTES["down"] == 35_651_584 + 4_456_448 + 44_564_480 + 5_570_560 + 41_943_040
    assert bench.REC_FLOP_PER_HEAD_TOKEN == 114_688


def test_decode_headline_prefers_the_graph_replays():
    dur = {"decode_all": 0.0201}                            # ms, from events around the decode part
    sweep = {"stream_read_us": 8.4,
             "M1": {"gemm_us": 12.0, "quantize_plus_gemm_us": 14.5, "gemm_over_stream_read": 12.0 / 8.4}}
    d = bench.decode_summary(dur, sweep)
    assert d["gemm_us"] == 12.0 and d["quantize_plus_gemm_us"] == 14.5
    assert abs(d["weight_GBps"] - 50_135_040 / 12.0 / 1e3) < 0.1
    assert d["in_step_events"] == {"quantize_plus_gemm_us": 20.1}
    assert d["stream_read_us"] == 8.4 and abs(d["gemm_over_stream_read"] - 12.0 / 8.4) < 1e-12
    d0 = bench.decode_summary(dur, None)
    assert d0["gemm_us"] is None and d0["quantize_plus_gemm_us"] == 20.1 and d0["sweep"] is None


def test_config_switch_choices_and_single_gpu_rule():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "nope"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2 and "invalid choice" in r.stderr and r.stdout == ""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "linear", "--gpus", "2"],
                       cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 2 and "--gpus 1" in r.stderr and r.stdout == ""
    assert bench.CONFIGS[0] == "step"          # the default keeps the one-line bench contract
