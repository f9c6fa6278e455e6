"""Host-side checks of bench.py (no GPU needed): the one-GPU refusal and the
rule that a traffic figure from a committed counter summary is reported only
while the kernel sources it was taken on are unchanged."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    rec = json.loads(res.stdout.strip().splitlines()[-1])
    assert rec["n_gpus"] == 2 and "one GPU" in rec["error"]


def test_source_digest_follows_the_sources(tmp_path):
    b = _bench()
    d1 = b.kernel_sources_digest(["bwd.hip", "sla_device.h"])
    assert d1 == b.kernel_sources_digest(["bwd.hip", "sla_device.h"])
    assert d1 != b.kernel_sources_digest(["attn_fwd.hip", "sla_device.h"])
    assert d1 != b.kernel_sources_digest(["bwd.hip"])


def test_traffic_only_for_the_profiled_sources(tmp_path, monkeypatch):
    b = _bench()
    (tmp_path / "profiles").mkdir()
    rec = {"kernel": "k", "source_digest": "abc123", "hbm_bytes_per_launch": 12345}
    (tmp_path / "profiles" / "traffic_k_wl.json").write_text(json.dumps(rec))
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    assert b.traffic_from_profile("k", "wl", "abc123") == 12345
    assert b.traffic_from_profile("k", "wl", "stale") is None          # kernel changed since
    assert b.traffic_from_profile("other", "wl", "abc123") is None     # never profiled


def test_step_stats_nearest_rank():
    b = _bench()
    st = b.step_stats([5.0, 1.0, 3.0, 2.0, 4.0, None])
    assert st == {"median": 3.0, "min": 1.0, "p90": 5.0, "mean": 3.0, "n": 5}
    assert b.step_stats([None]) is None
    assert b.step_stats(list(map(float, range(1, 21))))["p90"] == 18.0


def test_trace_summary_drops_warmup_launches(tmp_path):
    """Every kernel runs the same number of times per step: the first
    warmup / (warmup + steps) of each kernel's launches (by start time) are
    dropped, whatever order the trace lists them in."""
    b = _bench()
    rows = ['"Kind","Kernel_Name","Start_Timestamp","End_Timestamp"']
    # kernel a: once per step, warm-up launch 100 us, timed 10, 20 us
    for t0, dur in ((0, 100_000), (1_000_000, 10_000), (2_000_000, 20_000)):
        rows.append(f'"KERNEL_DISPATCH","a",{t0},{t0 + dur}')
    # kernel b: twice per step, listed out of order
    for t0, dur in ((2_500_000, 3_000), (500, 90_000), (1_500_000, 1_000), (600, 80_000),
                    (1_600_000, 2_000), (2_600_000, 4_000)):
        rows.append(f'"KERNEL_DISPATCH","b",{t0},{t0 + dur}')
    path = tmp_path / "trace.csv"
    path.write_text("\n".join(rows) + "\n")
    out = b.trace_summary(str(path), warmup=1, steps=2)
    line_a = next(ln for ln in out.splitlines() if "`a`" in ln)
    line_b = next(ln for ln in out.splitlines() if "`b`" in ln)
    # a: timed 10 and 20 us -> nearest-rank median 10, min 10, p90 20, mean 15
    assert "| 3 | 2 | 10.0 | 10.0 | 20.0 | 15.0 |" in line_a
    # b: the two warm-up launches (90 and 80 us) dropped; timed 1, 2, 3, 4 us
    assert "| 6 | 4 | 2.0 | 1.0 | 4.0 | 2.5 |" in line_b
    assert "(2 steps, 1 warm-up steps dropped)" in out


def test_counter_summary_scales_by_the_copy_probe(tmp_path, monkeypatch):
    """Counter values are divided by what the same counter reads for the
    closing 256 MiB copy; engine cycles are per XCD over the duration."""
    b = _bench()
    hdr = '"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"'

    def write(name, rows):
        p = tmp_path / name
        p.write_text("\n".join([hdr] + [",".join(map(str, r)) for r in rows]) + "\n")
        return str(p)

    k = '"void sla::bwd_kv_kernel<128>(int)"'
    fetch = write("f.csv", [(1, k, '"FETCH_SIZE"', 1000.0, 0, 1_000_000),
                            (2, k, '"FETCH_SIZE"', 3000.0, 0, 1_000_000),
                            (3, '"__amd_rocclr_copyBuffer"', '"FETCH_SIZE"', 131072.0, 0, 100)])
    wr = write("w.csv", [(1, k, '"WRITE_SIZE"', 500.0, 0, 1_000_000),
                         (2, k, '"WRITE_SIZE"', 500.0, 0, 1_000_000),
                         (3, '"__amd_rocclr_copyBuffer"', '"WRITE_SIZE"', 262144.0, 0, 100)])
    # 8 XCDs x 2.0e6 cycles in 1 ms -> 2000 MHz
    gr = write("g.csv", [(1, k, '"GRBM_COUNT"', 16e6, 0, 1_000_000),
                         (1, k, '"GRBM_GUI_ACTIVE"', 16e6, 0, 1_000_000),
                         (2, k, '"GRBM_COUNT"', 16e6, 0, 1_000_000),
                         (2, k, '"GRBM_GUI_ACTIVE"', 16e6, 0, 1_000_000)])
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    monkeypatch.setattr(b, "kernel_sources_digest", lambda names: "d1")
    out = b.counter_summary(fetch, wr, gr, "wl")
    rec = json.loads((tmp_path / "profiles" / "traffic_bwd_kv_wl.json").read_text())
    assert rec["fetch_factor"] == 0.5 and rec["write_factor"] == 1.0
    # mean fetch 2000 KiB / 0.5 + write 500 KiB / 1.0
    assert rec["hbm_bytes_per_launch"] == (4000 + 500) * 1024
    assert rec["clock_mhz_under_counters"] == 2000.0 and rec["source_digest"] == "d1"
    assert "| `sla::bwd_kv_kernel<128>` | 2 |" in out


def test_sustained_clock_skips_the_first_refresh(monkeypatch):
    """The metrics table refreshes about once a second; the first refresh
    after the start also covers idle time, so only later windows count."""
    import sys
    import types

    b = _bench()
    # refresh counter moves on every third read; clocks per window
    state = {"reads": 0}
    windows = [[100, 100], [2000, 2200], [2100, 2300], [2150, 2250]]

    def metrics(_h):
        state["reads"] += 1
        w = min(state["reads"] // 3, len(windows) - 1)
        return {"system_clock_counter": w, "current_gfxclks": windows[w] + [0xFFFF],
                "current_socket_power": 1000 + w}

    fake = types.SimpleNamespace(
        amdsmi_init=lambda: None, amdsmi_shut_down=lambda: None,
        amdsmi_get_processor_handles=lambda: ["gpu0"],
        amdsmi_get_gpu_metrics_info=metrics)
    monkeypatch.setitem(sys.modules, "amdsmi", fake)
    steps = []
    rec = b.sustained_clock(lambda: steps.append(1), max_s=5.0, sync=lambda: None)
    # windows 2 and 3 (the first refresh, window 1, is skipped; 0xFFFF entries ignored)
    assert rec["windows"] == 2
    assert rec["gfx_mhz"] == round(((2100 + 2300) / 2 + (2150 + 2250) / 2) / 2, 1)
    assert rec["gfx_mhz_per_xcd"] == [2150.0, 2250.0] and rec["socket_power_w"] == 1003
    assert steps   # the step ran while the clock was read


def test_sustained_clock_without_amdsmi(monkeypatch):
    import sys

    b = _bench()
    monkeypatch.setitem(sys.modules, "amdsmi", None)   # import fails
    rec = b.sustained_clock(lambda: None, sync=lambda: None)
    assert rec["gfx_mhz"] is None and "error" in rec


def test_sq_summary_normalisation(tmp_path):
    """MFMA busy is per SIMD over the kernel's cycles (SQ_BUSY_CYCLES per
    engine); instruction counts are per critical pair."""
    b = _bench()
    hdr = '"Kernel_Name","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"'
    k = '"void sla::bwd_kv_kernel<128>(int)"'
    a = tmp_path / "a.csv"
    # 2 engines busy 2000 cycles each over 1 us -> 2000 MHz; 4 SIMDs, MFMA busy 2000 of 8000
    a.write_text("\n".join([hdr, f'{k},"SQ_BUSY_CYCLES",4000,0,1000',
                            f'{k},"SQ_VALU_MFMA_BUSY_CYCLES",2000,0,1000',
                            f'{k},"SQ_WAVE_CYCLES",1000,0,1000',
                            f'{k},"SQ_WAIT_INST_ANY",250,0,1000']) + "\n")
    bb = tmp_path / "b.csv"
    bb.write_text("\n".join([hdr] + [f'{k},"SQ_INSTS_{c}",{v},0,1000' for c, v in
                                     (("MFMA", 40), ("VALU", 80), ("LDS", 20), ("VMEM", 4), ("SALU", 8))]) + "\n")
    out = b.sq_summary(str(a), str(bb), pairs=4, simds=4, engines=2)
    row = next(ln for ln in out.splitlines() if "bwd_kv_kernel" in ln)
    assert "| 1.0 | 2000 | 25.0 | 25.0 | 10 / 20 / 5 / 1 / 2 |" in row
