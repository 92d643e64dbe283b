"""Host logic of bench.py, no GPU: the algorithmic byte and flop counts against their
formulas written out, the reading of the committed counter summaries (and its refusal when
the kernel sources have changed), and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth import get_config  # noqa: E402


def test_single_token_costs():
    """One token on the OPT-6.7B shape: stage 1 reads P1, the token and writes q; the
    middle kernel reads P2, the predictor and activation biases, q, the token and the
    listed rows; the down kernel reads the listed rows and writes y once."""
    c = get_config("C2_10")
    d, n, r, U = c.d, c.n, c.rank, 1638
    cost = bench.kernel_cost(c, 1, U)
    assert set(cost) == {"stage1", "mid", "down"}
    assert cost["stage1"][0] == r * d * 2 + 4 * d + 4 * r
    assert cost["mid"][0] == n * r * 2 + 8 * n + 4 * r + 4 * d + U * (d * 2 + 12)
    assert cost["down"][0] == U * (d * 2 + 16) + 4 * d
    # the weight rows dominate: more than 97% of the middle kernel's bytes are P2 and rows
    assert (n * r * 2 + U * d * 2) / cost["mid"][0] > 0.97


def test_batch_tile_costs_and_flops():
    """Sixteen tokens on the gated Llama-7B shape: the up tile kernel reads gate and up
    rows, the down tile kernel one row each; flops are the products as defined, 2 per
    multiply-add, every token against every union row."""
    c = get_config("C4")
    d, U, B = c.d, 6200, 16
    cost = bench.kernel_cost(c, B, U)
    assert set(cost) == {"stage1", "up_tiles", "down_tiles"}
    up_bytes, up_fl = cost["up_tiles"]
    dn_bytes, dn_fl = cost["down_tiles"]
    assert up_bytes == U * (2 * d * 2 + 16 + 4 * B) + 4 * B * d
    assert dn_bytes == U * (d * 2 + 4 + 4 * B) + 4 * B * d
    assert up_fl == 2.0 * 2 * d * U * B
    assert dn_fl == 2.0 * d * U * B


def test_measured_traffic_follows_the_sources(monkeypatch, tmp_path):
    """A counter summary is read only while the kernel sources hash to the value recorded
    in it; a missing summary gives None."""
    (tmp_path / "profiles").mkdir()
    summary = tmp_path / "profiles" / "k_demo_work_b1_pmc.md"
    summary.write_text("# demo\n\n- kernel source sha256: `%s`\n- fetch KiB per dispatch: 1.0\n"
                       "- write KiB per dispatch: 2.0\n- traffic bytes per dispatch: 12345\n"
                       % ("a" * 64), encoding="utf-8")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: "a" * 64)
    assert bench.measured_traffic("k_demo", "work_b1") == 12345.0
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: "b" * 64)
    assert bench.measured_traffic("k_demo", "work_b1") is None
    assert bench.measured_traffic("no_such_kernel", "no_such_workload") is None


def test_committed_summaries_are_complete():
    """Every summary under profiles/ gives the command that made it and the kernel source
    hash it was taken on; the counter summaries also give the fields bench.py reads."""
    prof = os.path.join(ROOT, "profiles")
    names = [f for f in os.listdir(prof) if f.endswith(".md")]
    assert any(f.endswith("_pmc.md") for f in names) and any(f.endswith("_stats.md") for f in names)
    for f in names:
        text = open(os.path.join(prof, f), encoding="utf-8").read()
        assert "rocprofv3 " in text and " -- python3 -u bench.py" in text, f
        assert "- kernel source sha256: `" in text, f
        if f.endswith("_pmc.md"):
            assert "--pmc FETCH_SIZE" in text and "--pmc WRITE_SIZE" in text, f
            for field in ("fetch KiB per dispatch", "write KiB per dispatch",
                          "traffic bytes per dispatch"):
                assert f"- {field}: " in text, (f, field)
        else:
            assert "--kernel-trace --stats" in text, f


@pytest.mark.parametrize("gpus", ["2", "8"])
def test_one_gpu_guard(gpus):
    """bench.py measures one GPU: asked for more, it exits with status 2 and says so,
    before touching any device."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", gpus],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
