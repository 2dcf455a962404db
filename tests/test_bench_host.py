"""Host-side checks of bench.py: the one-GPU contract, the roofline each
workload is reported against, that a traffic figure is only reported
for the kernel and source it was measured on, and that clock figures come
only from metrics refreshed while a leg ran."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""


def test_config_rooflines():
    mlp = dict(us=35.0, tflops=368.0, gbps=3000.0, kernel="k", flops=2.0 * 128 * 12288 * 4096,
               alg_bytes=2.0 * (128 * 4096 + 12288 * 4096 + 128 * 12288))
    r = bench.config_roofline("mlp_up_128x12288x4096", mlp)
    assert r["bound"] == "hbm" and r["peak"] == bench.PEAK_HBM_GBPS and r["frac"] == round(3000.0 / 8000.0, 4)
    pre = dict(us=280.0, tflops=1470.0, gbps=800.0, kernel="k", flops=2.0 * 4096 * 4096 * 12288,
               alg_bytes=2.0 * (2 * 4096 * 12288 + 4096 * 4096))
    r = bench.config_roofline("prefill_down_4096x4096x12288", pre)
    assert r["bound"] == "mfma" and r["peak"] == bench.PEAK_BF16_TFLOPS
    r = bench.config_roofline("tiny_256", dict(us=4.0, kernel="k", flops=1.0, alg_bytes=1.0))
    assert r["bound"] == "latency" and r["peak"] is None


def test_traffic_only_for_its_kernel_and_source():
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as f:
        rec = json.load(f)
    for workload, e in rec["workloads"].items():
        got = bench.measured_traffic(workload, e["kernel"])
        current = e["source_digest"] == bench.source_digest(e["source"])
        assert (got == e["bytes_per_launch"]) if current else got is None
        assert bench.measured_traffic(workload, e["kernel"] + "_other") is None
    assert bench.measured_traffic("no_such_workload", "tile_256x256x64_s2_w4x2_p5") is None


def test_clock_sampler_keeps_only_refreshes_made_while_the_leg_ran():
    # (engine MHz, memory MHz, activity %, socket W, firmware timestamp): the
    # first reading's table predates the leg, so only later refreshes count.
    cs = bench.ClockSampler.__new__(bench.ClockSampler)
    cs._thread = None
    cs.samples = [(2400.0, 2000, 0, 300, 10), (2400.0, 2000, 0, 300, 10), (1800.0, 2000, 100, 1390, 11),
                  (1800.0, 2000, 100, 1390, 11), (1790.0, 2000, 100, 1395, 12)]
    r = cs.stop()
    assert r["metric_refreshes"] == 2 and r["samples"] == 3
    assert r["sclk_mhz_median"] == 1800.0 and r["sclk_mhz_min"] == 1790.0
    assert r["socket_power_w_median"] == 1390.0
    cs.samples = [(2400.0, 2000, 0, 300, 10)] * 3
    r = cs.stop()
    assert r["metric_refreshes"] == 0 and r["sclk_mhz_median"] is None
