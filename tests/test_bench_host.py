"""Host logic of bench.py (CPU): the one-GPU contract, the source digest that
keeps counter profiles honest, and the committed profiles' format."""
import glob
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""


SRC = """// a kernel
__global__ void k(float* x) {   // trailing comment
    x[0] = 1.0f;

}
"""


def test_source_digest_ignores_comments_and_blank_lines():
    d = bench.source_digest([SRC])
    assert d == bench.source_digest([SRC.replace("// a kernel", "// reworded")])
    assert d == bench.source_digest([SRC.replace("\n\n", "\n\n\n\n")])
    assert d == bench.source_digest([SRC.replace("// trailing comment", "")])
    assert d != bench.source_digest([SRC.replace("1.0f", "2.0f")])
    assert d != bench.source_digest([SRC, "int y;"])


def write_profile(dirpath, name, digest, hbm=1.5e8):
    with open(os.path.join(dirpath, f"{name}_pmc.txt"), "w") as f:
        f.write(f"# test profile\nhbm_bytes_per_launch: {hbm:e}\nsource_sha256: {digest}\n")


def test_kernel_traffic_only_while_the_sources_match(tmp_path, monkeypatch):
    src_dir = tmp_path / "src"
    src_dir.mkdir()
    (src_dir / "k.hip").write_text(SRC)
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "PROFILES", str(prof))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    write_profile(prof, "kern", bench.source_digest([SRC]))
    assert bench.kernel_traffic("kern", ["src/k.hip"]) == pytest.approx(1.5e8)
    # a comment edit keeps the counters; a code edit retires them
    (src_dir / "k.hip").write_text(SRC.replace("// a kernel", "// the kernel"))
    assert bench.kernel_traffic("kern", ["src/k.hip"]) == pytest.approx(1.5e8)
    (src_dir / "k.hip").write_text(SRC.replace("1.0f", "3.0f"))
    assert bench.kernel_traffic("kern", ["src/k.hip"]) is None
    # no profile, or one without its digest: no traffic figure
    assert bench.kernel_traffic("missing", ["src/k.hip"]) is None
    (prof / "nodigest_pmc.txt").write_text("hbm_bytes_per_launch: 1e8\n")
    assert bench.kernel_traffic("nodigest", ["src/k.hip"]) is None


def test_committed_counter_profiles_carry_command_digest_and_bytes():
    files = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_pmc.txt")))
    assert files
    for f in files:
        text = open(f).read()
        assert re.search(r"rocprofv3 --pmc FETCH_SIZE", text), f
        assert re.search(r"rocprofv3 --pmc WRITE_SIZE", text), f
        assert re.search(r"^source_sha256:\s*[0-9a-f]{64}$", text, re.M), f
    # every profile the benchmark line reads exists and states its bytes
    for name in bench.TRAFFIC_PROFILE.values():
        path = os.path.join(ROOT, "profiles", f"{name}_pmc.txt")
        assert os.path.exists(path), name
        m = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)$", open(path).read(), re.M)
        assert m and float(m.group(1)) > 0, name
