"""Host-side logic of bench.py, without a GPU: the one-GPU rule, the pair
counts and flop credits the throughput is built on, and the summaries made
from rocprofv3 counter files (fed with small synthetic files here)."""

import csv
import os
import subprocess
import sys

import pytest

import bench
import synthetic_inputs as si

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("N,causal,window", [(1, False, None), (7, False, None), (7, True, None),
                                             (64, True, None), (65, True, 1), (65, True, 16),
                                             (16, True, 16), (10, True, 64)])
def test_pair_counts_match_brute_force(N, causal, window):
    w = si.Workload("t", 1, 1, 1, N, 64, causal, False, 0, "", window, "bf16", "bhsd", None, 0.0)
    brute = sum(1 for i in range(N) for j in range(N)
                if (not causal or j <= i) and (window is None or i - j < window))
    assert w.pairs() == brute


def test_decode_pair_counts_match_brute_force():
    for causal, window in ((True, None), (False, None), (True, 5)):
        w = si.Workload("t", 1, 1, 1, 40, 64, causal, False, 0, "", window, "bf16", "bhsd", 3, 0.0)
        rows = range(37, 40)
        brute = sum(1 for i in rows for j in range(40)
                    if (not causal or j <= i) and (window is None or i - j < window))
        assert w.pairs() == brute


def test_flop_credits_split_the_backward_products():
    w = si.WORKLOADS["c5_bwd_d128"]
    c = bench.kernel_flop_credit(w)
    per_pair = w.pairs() * w.B * w.Hq * w.d
    # forward: S and PV (2 products x 2 flops); backward: 5 products x 2 flops
    assert c["fwd"] == 4 * per_pair
    assert c["bwd_dkdv"] + c["bwd_dq"] == 10 * per_pair


def _write_counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "pmc_counter_collection.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value",
                                           "Start_Timestamp", "End_Timestamp"])
        wr.writeheader()
        for kname, cname, val, t0, t1 in rows:
            wr.writerow(dict(Kernel_Name=kname, Counter_Name=cname, Counter_Value=val,
                             Start_Timestamp=t0, End_Timestamp=t1))


def test_traffic_summary_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "traffic_file", lambda k, wl: str(tmp_path / f"traffic_{k}_{wl}.txt"))
    cal = "void at::native::vectorized_elementwise_kernel<neg_kernel>"
    dk = "void attn::bwd_dkdv_kernel<0, 128, 1, false>(attn::BwdParams)"
    mib = 4
    # the copy reads and writes 4 MiB; FETCH_SIZE reports half of it, WRITE_SIZE all
    _write_counters(tmp_path / "f", [(cal, "FETCH_SIZE", mib * 512.0, 0, 1),
                                     (dk, "FETCH_SIZE", 1000.0, 0, 1), (dk, "FETCH_SIZE", 1200.0, 0, 1)])
    _write_counters(tmp_path / "w", [(cal, "WRITE_SIZE", mib * 1024.0, 0, 1),
                                     (dk, "WRITE_SIZE", 300.0, 0, 1)])
    bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path), "c5_bwd_d128", mib)
    got = bench.read_traffic("bwd_dkdv_kernel", "c5_bwd_d128")
    # (1100 KiB * 2 + 300 KiB) per dispatch
    assert got == pytest.approx((1100.0 * 2 + 300.0) * 1024.0)
    # a summary measured on other source is not reported
    path = tmp_path / "traffic_bwd_dkdv_kernel_c5_bwd_d128.txt"
    text = path.read_text().replace(bench.source_hash("bwd_dkdv_kernel"), "0000000000000000")
    path.write_text(text)
    assert bench.read_traffic("bwd_dkdv_kernel", "c5_bwd_d128") is None


def test_busy_summary(tmp_path):
    dk = "void attn::bwd_dkdv_kernel<0, 128, 1, false>(attn::BwdParams)"
    # 2 ms at 2 GHz = 4e6 cycles per XCD; matrix cores busy half of them on every SIMD
    _write_counters(tmp_path / "g", [(dk, "GRBM_GUI_ACTIVE", 4e6 * bench.XCDS, 0, 2_000_000)])
    _write_counters(tmp_path / "m", [(dk, "SQ_VALU_MFMA_BUSY_CYCLES", 2e6 * bench.SIMDS, 0, 2_000_000)])
    out = tmp_path / "busy.txt"
    bench.summarize_busy(str(tmp_path / "g"), str(tmp_path / "m"), str(out), "c5_bwd_d128")
    line = [x for x in out.read_text().splitlines() if x.startswith("void attn::bwd_dkdv")][0]
    cols = [c.strip() for c in line.split("|")]
    assert cols[3].startswith("2.000")      # clock, GHz
    assert float(cols[6]) == pytest.approx(0.5)  # busy share


def test_wave_summary_shares_add_up(tmp_path):
    fw = "void attn::fwd_kernel<0, 128, 1, 8, false>(attn::FwdParams)"
    vals = dict(SQ_WAVE_CYCLES=1000, SQ_ACTIVE_INST_ANY=400, SQ_WAIT_INST_ANY=350, SQ_WAIT_ANY=250,
                SQ_ACTIVE_INST_VALU=200, SQ_ACTIVE_INST_LDS=50, SQ_WAIT_INST_LDS=10,
                SQ_VALU_MFMA_COEXEC_CYCLES=30)
    _write_counters(tmp_path / "s", [(fw, k, v, 0, 1) for k, v in vals.items()])
    out = tmp_path / "waves.txt"
    bench.summarize_waves(str(tmp_path / "s"), str(out), "c5_bwd_d128")
    line = [x for x in out.read_text().splitlines() if x.startswith("void attn::fwd")][0]
    cols = [float(c) for c in line.split("|")[1:]]
    assert cols[:4] == pytest.approx([0.4, 0.35, 0.25, 1.0])
    assert cols[4:] == pytest.approx([0.2, 0.05])


def test_counter_summary_lists_every_counter(tmp_path):
    dk = "void attn::bwd_dkdv_kernel<0, 128, 1, false>(attn::BwdParams)"
    other = "void at::native::vectorized_elementwise_kernel<neg_kernel>"
    _write_counters(tmp_path / "c", [(dk, "SQ_INSTS_VALU", 10, 0, 1), (dk, "SQ_INSTS_VALU", 30, 0, 1),
                                     (dk, "SQ_LDS_BANK_CONFLICT", 0, 0, 1), (other, "SQ_INSTS_VALU", 5, 0, 1)])
    out = tmp_path / "c.txt"
    bench.summarize_counters(str(tmp_path / "c"), str(out), "c5_bwd_d128")
    text = out.read_text()
    assert "--pmc SQ_INSTS_VALU SQ_LDS_BANK_CONFLICT " in text
    rows = [x for x in text.splitlines() if x.startswith("void ")]
    assert rows == ["void attn::bwd_dkdv_kernel<0, 128, 1, false> | 20 | 0"]


def test_traffic_summary_finds_the_wide_dkdv_kernel(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "traffic_file", lambda k, wl: str(tmp_path / f"traffic_{k}_{wl}.txt"))
    cal = "void at::native::vectorized_elementwise_kernel<neg_kernel>"
    dk = "void attn::bwd_dkdv_wide_kernel<0, 1>(attn::BwdParams)"
    _write_counters(tmp_path / "f", [(cal, "FETCH_SIZE", 2048.0, 0, 1), (dk, "FETCH_SIZE", 500.0, 0, 1)])
    _write_counters(tmp_path / "w", [(cal, "WRITE_SIZE", 4096.0, 0, 1), (dk, "WRITE_SIZE", 100.0, 0, 1)])
    bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path), "c5_bwd_d128", 4)
    assert bench.read_traffic("bwd_dkdv_kernel", "c5_bwd_d128") == pytest.approx((500.0 * 2 + 100.0) * 1024.0)


@pytest.mark.parametrize("kernel,symbol", [
    ("fwd_kernel", "void attn::fwd_m16_kernel<0, 128, 1, 4>(attn::FwdParams)"),
    ("fwd_kernel", "void attn::fwd_split_kernel<0, 64, 0, 8>(attn::FwdParams)"),
    ("bwd_dq_kernel", "void attn::bwd_dq_m16_kernel<0, 1>(attn::BwdParams)"),
])
def test_traffic_summary_finds_the_16x16x32_and_split_kernels(tmp_path, monkeypatch, kernel, symbol):
    # the forward and dQ pass run other kernels than their 32x32x16 step loops
    # on some plans; the traffic summary must count them under the pass's name
    monkeypatch.setattr(bench, "traffic_file", lambda k, wl: str(tmp_path / f"traffic_{k}_{wl}.txt"))
    cal = "void at::native::vectorized_elementwise_kernel<neg_kernel>"
    _write_counters(tmp_path / "f", [(cal, "FETCH_SIZE", 2048.0, 0, 1), (symbol, "FETCH_SIZE", 300.0, 0, 1)])
    _write_counters(tmp_path / "w", [(cal, "WRITE_SIZE", 4096.0, 0, 1), (symbol, "WRITE_SIZE", 50.0, 0, 1)])
    bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path), "c5_bwd_d128", 4)
    assert bench.read_traffic(kernel, "c5_bwd_d128") == pytest.approx((300.0 * 2 + 50.0) * 1024.0)
