"""CPU tests of the benchmark's profile summariser: splitting a kernel trace's
attention launches by bench phase, including an alone leg measured again."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _write_trace(path, durations_us, kernel="attn_kernel<4, 4>"):
    t = 1_000_000
    rows = ["Kernel_Name,Start_Timestamp,End_Timestamp"]
    for d in durations_us:
        rows.append(f"\"{kernel}\",{t},{t + int(d * 1000)}")
        t += int(d * 1000) + 5000
    # a kernel of another kind between them changes nothing
    rows.append(f"score_kernel,{t},{t + 1000}")
    open(path, "w").write("\n".join(rows) + "\n")


def _write_log(path, phases, extra_lines=(), avg_launch_us=100.0):
    lines = ["[bench] attention launches: " + json.dumps(phases)]
    lines += list(extra_lines)
    lines.append(json.dumps({"roofline": {"avg_launch_us": avg_launch_us}}))
    open(path, "w").write("\n".join(lines) + "\n")


def test_phases_split_in_launch_order(tmp_path):
    phases = {"warmup": 2, "timed": 3, "extra": 1, "alone": 4}
    durs = [50, 50] + [100, 110, 120] + [70] + [40, 40, 40, 40]
    _write_trace(tmp_path / "t.csv", durs)
    _write_log(tmp_path / "b.log", phases, avg_launch_us=110.0)
    out = "\n".join(bench._attention_phases(str(tmp_path / "t.csv"), str(tmp_path / "b.log")))
    assert "not split" not in out
    assert "timed       3 launches  mean    110.00 us" in out
    assert "alone       4 launches  mean     40.00 us" in out
    assert "trace mean / events = 1.000" in out


def test_alone_leg_measured_again_is_counted(tmp_path):
    # the alone leg took three attempts of 4 launches after 2 untimed ones
    phases = {"warmup": 1, "timed": 2, "extra": 0, "alone": 2 + 4}
    durs = [50] + [100, 100] + [40] * (2 + 3 * 4)
    _write_trace(tmp_path / "t.csv", durs)
    retry = "[bench] alone launches: the host fell behind the GPU (enqueue 1.00 ms, fills 0.50 ms); measuring again"
    made = "[bench] attention alone launches made: 14"
    _write_log(tmp_path / "b.log", phases, extra_lines=[retry, retry, made])
    out = "\n".join(bench._attention_phases(str(tmp_path / "t.csv"), str(tmp_path / "b.log")))
    assert "not split" not in out
    assert "alone      14 launches" in out


def test_count_mismatch_is_reported_not_split(tmp_path):
    phases = {"warmup": 1, "timed": 2, "extra": 0, "alone": 3}
    _write_trace(tmp_path / "t.csv", [10] * 7)
    _write_log(tmp_path / "b.log", phases)
    out = bench._attention_phases(str(tmp_path / "t.csv"), str(tmp_path / "b.log"))
    assert any("launch count 7 differs from the bench's 6: not split" in x for x in out)
