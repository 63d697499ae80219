"""Host-side checks of bench.py that need no GPU: it refuses more than one
GPU before touching the device, and the counter figures it reads from the
committed rocprofv3 summaries are reported only for the kernel source they
were taken on."""
import hashlib
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    for argv, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv, capture_output=True,
                           text=True, env=dict(os.environ, **env), timeout=120)
        assert r.returncode == 2, (argv, env, r.returncode)
        assert "one GPU" in r.stderr
        assert r.stdout == ""  # no JSON line


def _summary(tmp_path, source_bytes, workload="cfg2", value="12345"):
    src = tmp_path / "kernel.hip"
    src.write_bytes(source_bytes)
    digest = hashlib.sha256(source_bytes).hexdigest()
    summary = tmp_path / "summary.md"
    summary.write_text(f"# counters\n\n- workload: `{workload}`\n- source_sha256: `{digest}`\n"
                       f"- hbm_bytes_per_launch: `{value}`\n")
    return str(summary), str(src)


def test_summary_figure_follows_the_source_hash(tmp_path):
    summary, src = _summary(tmp_path, b"kernel v1")
    assert bench._summary_figure(summary, src, "cfg2", "hbm_bytes_per_launch") == 12345.0
    # another workload, a missing field, a changed source, a missing file
    assert bench._summary_figure(summary, src, "cfg3", "hbm_bytes_per_launch") is None
    assert bench._summary_figure(summary, src, "cfg2", "fetch_factor") is None
    open(src, "wb").write(b"kernel v2")
    assert bench._summary_figure(summary, src, "cfg2", "hbm_bytes_per_launch") is None
    assert bench._summary_figure(str(tmp_path / "absent.md"), src, "cfg2", "hbm_bytes_per_launch") is None


def test_committed_summaries_name_a_workload_and_a_source():
    """The two counter summaries bench.py reads carry the fields it parses."""
    import re
    for path, field in ((bench.TRAFFIC_SUMMARY, "hbm_bytes_per_launch"),
                        (bench.BIN_TRAFFIC_SUMMARY, "hbm_bytes_per_call")):
        fields = dict(re.findall(r"^- (\w+): `([^`]*)`", open(path).read(), flags=re.M))
        assert fields.get("workload") == "cfg2", path
        assert re.fullmatch(r"[0-9a-f]{64}", fields.get("source_sha256", "")), path
        assert float(fields[field]) > 0, path
