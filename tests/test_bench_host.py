"""Host logic of bench.py that needs no GPU: the sysfs clock/power sampler."""
import os
import time

import bench


def fake_sysfs(tmp_path, current_mhz, watts):
    dev = tmp_path / "card0" / "device"
    (dev / "hwmon" / "hwmon3").mkdir(parents=True)
    (dev / "pp_dpm_sclk").write_text(f"0: 500Mhz\n1: {current_mhz}Mhz *\n2: 2400Mhz\n")
    (dev / "hwmon" / "hwmon3" / "power1_input").write_text(str(int(watts * 1e6)))
    (dev / "hwmon" / "hwmon3" / "power1_cap").write_text(str(1400 * 10 ** 6))
    return str(dev)


def test_sampler_reads_current_level_and_power(tmp_path, monkeypatch):
    dev = fake_sysfs(tmp_path, 2158, 1398.5)
    monkeypatch.setattr(bench, "_gpu_sysfs_dir", lambda: dev)
    s = bench.ClockSampler(period_s=0.005).start()
    time.sleep(0.05)
    s.stop()
    c = s.summary()
    assert c["sclk_mhz"] == 2158 and c["power_w"] == 1398.5 and c["power_cap_w"] == 1400.0
    assert c["samples"] >= 2
    assert s.summary(time.perf_counter() + 1) is None  # no samples after the run


def test_sampler_without_sysfs_records_nothing(monkeypatch):
    monkeypatch.setattr(bench, "_gpu_sysfs_dir", lambda: None)
    s = bench.ClockSampler().start()
    s.stop()
    assert s.summary() is None


def test_clock_context_scales_the_spec_peak():
    t = {"launch_ms_mean": 0.25, "clock": {"sclk_mhz": 1200, "power_w": 1000.0,
                                          "power_cap_w": 1400.0, "samples": 5}}
    fl = 2.5e11  # 1000 TFLOP/s at 0.25 ms
    c = bench.clock_context(fl, t, 2516.6)
    assert c["peak_at_sclk_tflops"] == round(2516.6 / 2, 1)
    assert abs(c["frac_at_sclk"] - 1000 / (2516.6 / 2)) < 1e-4
    assert bench.clock_context(fl, {"launch_ms_mean": 0.25, "clock": None}, 2516.6) is None
