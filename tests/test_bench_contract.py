"""bench.py's parts that need no GPU: the one-GPU guard, and the committed counter figures it
reports (HBM traffic, matrix-core busy fraction), which it must drop once any source of the
kernel kind they were measured on has changed."""
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode != 0
    assert "one GPU" in res.stderr


@pytest.fixture()
def tree_copy(tmp_path, monkeypatch):
    """A copy of the kernel sources and profiles that bench's lookups read."""
    csrc = tmp_path / "paged_kv_attention_05_amd" / "csrc"
    shutil.copytree(os.path.join(ROOT, "paged_kv_attention_05_amd", "csrc"), csrc)
    shutil.copytree(os.path.join(ROOT, "profiles"), tmp_path / "profiles")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path


@pytest.mark.parametrize("kind", sorted(bench.KERNEL_SOURCES))
def test_a_figure_goes_stale_when_any_source_of_its_kind_changes(tree_copy, kind):
    sha0 = bench.kernel_sha(kind)
    for name in bench.KERNEL_SOURCES[kind] + bench.COMMON_SOURCES:
        path = tree_copy / "paged_kv_attention_05_amd" / "csrc" / name
        text = path.read_bytes()
        path.write_bytes(text + b"\n// edited\n")
        assert bench.kernel_sha(kind) != sha0, name
        path.write_bytes(text)
    assert bench.kernel_sha(kind) == sha0


def test_stale_figures_are_not_reported(tree_copy):
    data = {"w": {"prefill": {"kernel_sha": bench.kernel_sha("prefill"), "mfma_busy": 0.5,
                              "hbm_bytes_per_launch": 123.0}}}
    for f in ("mfma.json", "traffic.json"):
        (tree_copy / "profiles" / f).write_text(json.dumps(data))
    assert bench.measured_mfma_busy("prefill", "w") == 0.5
    assert bench.measured_traffic("prefill", "w") == 123.0
    assert bench.measured_mfma_busy("prefill", "other") is None
    (tree_copy / "paged_kv_attention_05_amd" / "csrc" / "v16_stage.hip").write_text("// changed\n")
    assert bench.measured_mfma_busy("prefill", "w") is None
    assert bench.measured_traffic("prefill", "w") is None


def test_committed_counter_figures_cite_their_summaries():
    for f in ("mfma.json", "traffic.json"):
        path = os.path.join(ROOT, "profiles", f)
        if not os.path.exists(path):
            continue
        for workload, kinds in json.load(open(path)).items():
            for kind, entry in kinds.items():
                assert kind in bench.KERNEL_SOURCES, (f, workload, kind)
                assert os.path.exists(os.path.join(ROOT, entry["source"])), (f, workload, entry["source"])
                if f == "mfma.json":
                    assert 0.0 < entry["mfma_busy"] <= 1.0
