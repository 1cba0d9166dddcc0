"""Host-side parts of the benchmark's contract (no GPU): the single-GPU refusal and the
fingerprint that ties the stored HBM-traffic figure to the kernel code."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def _load_bench():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_traffic_fingerprint_follows_code_not_comments(tmp_path):
    """The stored HBM-traffic figure is tied to the kernel sources' code: a comment edit
    keeps the fingerprint, a code edit changes it (and the figure is then not reported)."""
    import shutil
    bench = _load_bench()
    src = os.path.join(ROOT, "long_context_block_qsa_amd", "csrc")
    dst = tmp_path / "long_context_block_qsa_amd" / "csrc"
    shutil.copytree(src, dst)
    bench.ROOT = str(tmp_path)
    base = bench.sources_sha256()
    f = dst / "qsa_kernels.hip"
    text = f.read_text()
    f.write_text(text.replace("namespace qsa {", "namespace qsa {  // a comment\n/* and another */", 1))
    assert bench.sources_sha256() == base
    other = dst / "qsa_backward.hip"   # another translation unit: not the scoring kernel's
    other.write_text(other.read_text() + "\nnamespace qsa { constexpr int UNUSED_X = 1; }\n")
    assert bench.sources_sha256() == base
    f.write_text(text.replace("constexpr int SCORE_BATCH = 8;", "constexpr int SCORE_BATCH = 4;", 1))
    assert bench.sources_sha256() != base
    bench.TRAFFIC = {"score": {"bytes": 1, "sources_sha256": base}}
    assert bench.traffic_of("score") is None
