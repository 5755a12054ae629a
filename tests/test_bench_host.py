"""Host-side parts of bench.py that need no GPU: the refusal of more than one
GPU (the contract: N above 1 exits with a message saying so), and the
HBM-traffic table, whose figures count only while the kernel source they were
measured on is unchanged."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                       env={**os.environ, **env}, capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""          # no JSON line


def test_traffic_table_uses_only_current_sources(tmp_path):
    src = "remask_commit.hip"
    sha = hashlib.sha256(open(os.path.join(ROOT, "block_diffusion_amd", "csrc", src), "rb").read()).hexdigest()
    f = tmp_path / "traffic_x.md"
    f.write_text(
        "text\n"
        f"<!-- traffic dbd_remask_commit rows=512 bytes=123456 src={src} sha256={sha} -->\n"
        f"<!-- traffic dbd_remask_commit rows=128 bytes=999 src={src} sha256={'0' * 64} -->\n"
        "<!-- traffic dbd_nothing rows=512 bytes=5 src=no_such_file.hip sha256=" + "a" * 64 + " -->\n")
    t = bench.traffic_table("x", path=str(f))
    assert t[("dbd_remask_commit", 512)] == 123456       # source unchanged: the figure counts
    assert t[("dbd_remask_commit", 128)] is None         # recorded on another source: null
    assert t[("dbd_nothing", 512)] is None               # source missing: null
    assert bench.traffic_table("x", path=str(tmp_path / "missing.md")) == {}


def test_committed_traffic_markers_parse():
    t = bench.traffic_table("sdar4b_b4_bs128")
    assert ("dbd_lmhead_conf", 512) in t and ("dbd_attn_paged", 512) in t
    for k, v in t.items():
        assert v is None or v > 0, k
