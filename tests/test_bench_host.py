"""Host-side checks of bench.py (no GPU): the one-GPU contract and the summaries it writes
from profiler databases."""
import os
import sqlite3
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_counter_summary_groups_workloads(tmp_path, monkeypatch):
    """A synthetic counter database in rocprofv3's schema (the columns the summary reads):
    two workloads, each opened by the bench's marker kernel, with upload copies between;
    warm-up dispatches left out, per-wave ratios."""
    sys.path.insert(0, ROOT)
    import bench
    db = sqlite3.connect(tmp_path / "run_results.db")
    db.execute("create table counters_collection (dispatch_id int, kernel_name text, "
               "counter_name text, value real)")
    att = "void pa::(anonymous namespace)::paged_attn_balanced_kernel<X>(pa::AttnArgs)"
    mrg = "void pa::(anonymous namespace)::balanced_merge_kernel<128>(pa::AttnArgs, int)"
    marker = ("void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<short>,"
              " std::array<char*, 1ul> >(int, at::native::FillFunctor<short>, std::array<char*, 1ul>)")
    rows, did = [], 0

    def dispatch(name, waves, insts):
        nonlocal did
        did += 1
        rows.append((did, name, "SQ_WAVES", waves))
        rows.append((did, name, "SQ_INSTS_VALU", insts))
    dispatch(marker, 1, 1)
    dispatch("__amd_rocclr_copyBuffer", 1, 1)
    for i in range(4):                       # 2 warm-up + 2 timed, first workload
        dispatch(att, 100, 1000 if i < 2 else 2000)
        dispatch(mrg, 10, 7)
    dispatch(marker, 1, 1)
    dispatch("__amd_rocclr_copyBuffer", 1, 1)
    for i in range(5):                       # 3 warm-up + 2 timed, second workload
        dispatch(att, 50, 10 if i < 3 else 500)
    db.executemany("insert into counters_collection values (?, ?, ?, ?)", rows)
    db.commit()
    db.close()
    out_dir = tmp_path / "profiles"
    out_dir.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "test")

    class A:
        steps, warmup, event_steps, no_cpu, path, layout = 2, 2, 2, True, "step", "interleaved"
        calibrate = False
    bench.counter_summary(A(), str(tmp_path), "unit")
    text = (out_dir / "unit.md").read_text()
    lines = [l for l in text.splitlines() if l.startswith(("| llama", "| tiny"))]
    assert len(lines) == 3
    first, merge, second = (l.split("|") for l in lines)
    assert first[1].strip() == bench.ORDER[0] and first[3].strip() == "2"
    assert "balanced_merge_kernel" in merge[2]
    assert second[1].strip() == bench.ORDER[1] and second[3].strip() == "2"
    # VALU per wave: 2000 / 100 and 500 / 50 (warm-ups excluded)
    assert first[-4].strip() == "20" and second[-4].strip() == "10"
