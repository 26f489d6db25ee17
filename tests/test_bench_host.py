"""CPU checks of bench.py's host-side logic (no GPU): the one-GPU guard, the
timing spread, the rocminfo device record, the counter-summary gate and the
all-cores oracle worker."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus 2" in r.stderr and "one GPU" in r.stderr
    assert r.stdout == ""


def test_spread_percentiles_and_units():
    s = bench.spread([i * 1e-3 for i in range(1, 11)])       # 1..10 us, given in ms
    assert s["min"] == pytest.approx(1.0)
    assert s["avg"] == pytest.approx(5.5)
    assert s["median"] == pytest.approx(5.5)
    assert s["p10"] == pytest.approx(1.9)
    assert s["p90"] == pytest.approx(9.1)
    one = bench.spread([0.25])
    assert one["p10"] == one["p90"] == one["median"] == pytest.approx(250.0)


ROCMINFO = """*******
Agent 1
*******
  Name:                    Some CPU
  Marketing Name:          Some CPU
  Device Type:             CPU
  Compute Unit:            128
*******
Agent 2
*******
  Name:                    gfx950
  Uuid:                    GPU-0000
  Marketing Name:          
  Vendor Name:             AMD
  Device Type:             GPU
  Max Clock Freq. (MHz):   2400
  Compute Unit:            256
"""


def test_device_record_reads_the_first_gpu_agent(monkeypatch):
    class R:
        stdout = ROCMINFO
    monkeypatch.setattr(subprocess, "run", lambda *a, **k: R)
    rec = bench.device_record()
    assert rec == {"marketing_name": "", "isa": "gfx950", "compute_units": "256",
                   "max_clock_mhz": "2400"}


def test_device_record_reports_a_missing_tool(monkeypatch):
    def boom(*a, **k):
        raise FileNotFoundError("rocminfo")
    monkeypatch.setattr(subprocess, "run", boom)
    assert "error" in bench.device_record()


def test_traffic_figure_is_dropped_once_the_kernel_source_changes(tmp_path, monkeypatch):
    src = tmp_path / "kernels.hip"
    src.write_text("// kernel source\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    rec = {"kernels_hip_sha256_16": bench.kernel_source_hash(), "hbm_bytes_per_launch": 123.0}
    summary = tmp_path / "traffic.md"
    summary.write_text("# traffic\n\n```json\n" + json.dumps(rec) + "\n```\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(summary))
    assert bench.read_traffic() == 123.0
    src.write_text("// kernel source, edited\n")
    assert bench.read_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.md"))
    assert bench.read_traffic() is None


def test_cpu_worker_reports_its_rate():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--cpu-worker",
                        "8", "0", "4096", "2048", "0.05"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    rec = json.loads(r.stdout.strip().splitlines()[-1])
    assert rec["elements"] >= 2 * 2048 and rec["elements"] % 2048 == 0
    assert rec["seconds"] > 0


def test_trace_gaps_reads_spans_and_gaps(tmp_path, capsys):
    """Two units per step, one warm-up step: spans, kernel sums and gaps from a
    synthetic rocprofv3 kernel trace (other kernels ignored)."""
    hdr = '"Kind","Kernel_Name","Start_Timestamp","End_Timestamp"\n'
    rows = []
    t = 1000
    for step in range(3):
        for u in range(2):
            rows.append(f'"KERNEL_DISPATCH","void k_step_vec<x>(StepArgs)",{t},{t + 4000}\n')
            t += 4000 + (500 if u == 0 else 0)        # a 0.5 us gap inside each step
        rows.append(f'"KERNEL_DISPATCH","torch_fill",{t},{t + 100}\n')
        t += 1000
    path = tmp_path / "trace.csv"
    path.write_text(hdr + "".join(rows))
    bench.trace_gaps(str(path), 2, 2, 1)
    out = capsys.readouterr().out
    assert "| 1 | 0.009 | 0.008 | 5.88% | 0.5 | 0.5 |" in out
    assert "span 0.009 ms, kernels 0.008 ms" in out
    with pytest.raises(SystemExit):
        bench.trace_gaps(str(path), 2, 5, 1)


def _counter_csv(path, dispatches):
    """A rocprofv3 counter_collection.csv holding `dispatches` = [(kernel, {counter: value})]."""
    lines = ['"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"\n']
    for i, (kernel, counters) in enumerate(dispatches):
        for c, v in counters.items():
            # two instances per counter, summed by the reader
            lines.append(f'"{i + 1}","{kernel}","{c}","{v / 2}"\n')
            lines.append(f'"{i + 1}","{kernel}","{c}","{v / 2}"\n')
    path.mkdir()
    (path / "run_counter_collection.csv").write_text("".join(lines))


def test_traffic_summary_from_raw_request_counts(tmp_path, capsys):
    """Bytes from 128-byte read and 64-byte write requests; the two 1 GiB copies of known
    size gate the result, and a copy whose counts do not match its size stops it."""
    U, S = 202383360, 25297920
    fused = "void (anonymous namespace)::k_step_one<8, true, 0, false>((anonymous namespace)::StepArgs)"
    gather = "void (anonymous namespace)::k_segcopy<1>((anonymous namespace)::SegArgs)"
    lcopy = "void (anonymous namespace)::k_segcopy<0>((anonymous namespace)::SegArgs)"
    rcopy = "__amd_rocclr_copyBuffer"
    gib = 1 << 30

    def rd(nbytes):
        return {"TCC_EA0_RDREQ_sum": nbytes / 128, "TCC_EA0_RDREQ_32B_sum": 0.0,
                "TCC_BUBBLE_sum": 0.0, "TCC_EA0_RDREQ_DRAM_sum": nbytes / 128}

    def wr(nbytes):
        return {"TCC_EA0_WRREQ_sum": nbytes / 64, "TCC_EA0_WRREQ_64B_sum": nbytes / 64,
                "TCC_EA0_WRREQ_DRAM_sum": nbytes / 64}

    seq = [(fused, 28 * S, 14 * S), (gather, 2 * U, 2 * U), (gather, 2 * S, 2 * S),
           (fused, 28 * S + 128, 14 * S), (lcopy, gib, gib), (rcopy, gib, gib)]
    _counter_csv(tmp_path / "rd", [(k, rd(r)) for k, r, _ in seq])
    _counter_csv(tmp_path / "wr", [(k, wr(w)) for k, _, w in seq])
    bench.pmc_summary(str(tmp_path / "rd"), str(tmp_path / "wr"))
    rec = json.loads(capsys.readouterr().out.split("```json")[1].split("```")[0])
    assert rec["hbm_bytes_per_launch"] == pytest.approx(42 * S + 64)
    assert rec["traffic_over_algorithmic"] == pytest.approx(1 + 64 / (42 * S))
    assert rec["gather"]["dispatches"] == 1          # the init-size copy is left out
    assert rec["gather"]["traffic_over_algorithmic"] == pytest.approx(1.0)
    bad = [(k, r if k != rcopy else gib // 2, w) for k, r, w in seq]
    _counter_csv(tmp_path / "rd2", [(k, rd(r)) for k, r, _ in bad])
    _counter_csv(tmp_path / "wr2", [(k, wr(w)) for k, _, w in bad])
    with pytest.raises(SystemExit):
        bench.pmc_summary(str(tmp_path / "rd2"), str(tmp_path / "wr2"))


def test_fused_kernel_name_matching():
    """The profile readers find the fused kernel by its demangled name: the one-tile
    kernel of the staged step, or the general vector kernel, for the given row count."""
    r8 = bench.fused_kernel_re(8)
    assert r8.search("void (anonymous namespace)::k_step_one<8, true, 0, false>((anonymous namespace)::StepArgs)")
    assert r8.search("void (anonymous namespace)::k_step_vec<((anonymous namespace)::Op)2, 8, true, 0, false>(x)")
    assert not r8.search("void (anonymous namespace)::k_step_one<8, false, 0, false>(x)")      # no emission
    assert not r8.search("void (anonymous namespace)::k_step_one<16, true, 8, false>(x)")      # hybrid 2 x 8
    assert not r8.search("void (anonymous namespace)::k_step_vec<((anonymous namespace)::Op)0, 8, false, 0, false>(x)")
    assert bench.fused_kernel_re(16).search("k_step_one<16, true, 0, false>")
