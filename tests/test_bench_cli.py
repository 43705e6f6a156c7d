"""Host logic of bench.py that runs without a GPU: the one-GPU contract and
the lookup of the committed HBM byte counters (used only when they were taken
on the kernel source in the tree)."""
import hashlib
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_counters_are_used_only_for_the_source_they_were_taken_on(tmp_path):
    bench = load_bench()
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel source\n")
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    counters = tmp_path / "counters.json"
    bench.KERNEL_SRC = str(src)
    bench.COUNTERS = str(counters)
    assert bench.measured_traffic() is None                      # no counters
    counters.write_text(json.dumps({"kernel_source_sha256": sha, "hbm_bytes_per_launch": 1234.0}))
    assert bench.measured_traffic() == 1234
    src.write_text("// kernel source, changed\n")
    assert bench.measured_traffic() is None                      # taken on another source
    counters.write_text("not json")
    assert bench.measured_traffic() is None


def test_stack_groups_hold_the_stack_matrices():
    # the grouped layout the benchmark draws the stack in: every matrix is a
    # contiguous slice of its group with the values torch_stack_matrix gives
    torch = __import__("pytest").importorskip("torch")
    sys.path.insert(0, ROOT)
    from post_weight_quantization_row_amd import synth
    groups, members = synth.torch_stack_grouped("cpu", n_layers=1)
    assert [(t, tuple(x.shape), r) for t, x, _, r in groups] == [
        ("q4_0", (4 * 4096, 4096), 4096), ("q5_1", (2 * 11008, 4096), 11008), ("q5_1", (4096, 11008), 4096)]
    views = synth.torch_stack_views(groups, members, n_layers=1)
    for which in (0, 3, 5, 6):   # first and last member of each group
        t, x, q = views[which]
        t2, x2, q2 = synth.torch_stack_matrix(0, which, "cpu")
        assert t == t2 and x.is_contiguous() and torch.equal(x, x2) and torch.equal(q, q2)
