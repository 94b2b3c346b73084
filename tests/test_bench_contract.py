"""CPU checks of bench.py's command-line contract and of the committed
counter summaries it reads (no GPU needed)."""

import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_distributed_launch_is_refused():
    r = _run([], {"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_no_gpu_exits_with_a_message():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: the bench would run")
    r = _run(["--steps", "1", "--warmup", "0", "--no-cpu-baseline"])
    assert r.returncode == 2
    assert "needs a GPU" in r.stderr


def _fields(path):
    out = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(" ") and not line.startswith("#"):
                k, v = line.split(":", 1)
                out[k.strip()] = v.strip()
    return out


@pytest.mark.parametrize("name", ["attn_decode_llama8b_bf16_bs16_counters.txt",
                                  "attn_decode_long_context_bf16_counters.txt"])
def test_counter_summaries_are_consistent(name):
    """HBM bytes per launch are the two counters scaled by their calibration
    factors, and the algorithmic bytes match the workload's definition."""
    f = _fields(os.path.join(ROOT, "profiles", name))
    fetch = float(f["fetch_size_kib_per_launch"]) * 1024 * float(f["fetch_factor"])
    write = float(f["write_size_kib_per_launch"]) * 1024 * float(f["write_factor"])
    hbm = int(f["hbm_bytes_per_launch"])
    assert abs(hbm - (fetch + write)) <= 1024
    alg = int(f["algorithmic_kv_bytes_per_launch"])
    assert abs(float(f["traffic_over_algorithmic"]) - hbm / alg) < 1e-3
    assert hbm >= alg   # every valid K/V byte is read at least once
    assert re.fullmatch(r"[0-9a-f]{16}", f["kernel_source"])


def test_traffic_is_reported_only_for_the_current_sources(tmp_path, monkeypatch):
    """A counter summary taken on another version of the kernel sources is
    not reported (traffic null)."""
    src = os.path.join(ROOT, "profiles", "attn_decode_llama8b_bf16_bs16_counters.txt")
    with open(src) as fh:
        text = fh.read()
    digest = bench.source_digest()
    cur = re.search(r"^kernel_source: (\S+)$", text, re.M).group(1)
    stale = text.replace(f"kernel_source: {cur}", "kernel_source: 0000000000000000")
    fresh = text.replace(f"kernel_source: {cur}", f"kernel_source: {digest}")
    for body, want_none in ((stale, True), (fresh, False)):
        (tmp_path / "attn_decode_llama8b_bf16_bs16_counters.txt").write_text(body)
        monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
        got = bench.traffic_for("llama8b_bf16_bs16")
        assert (got is None) == want_none
        if not want_none:
            assert got == int(_fields(src)["hbm_bytes_per_launch"])
