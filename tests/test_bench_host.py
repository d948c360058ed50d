"""CPU checks of bench.py's host logic: the one-GPU guard and the algorithmic
work per launch that the roofline fractions are computed from (the block's
per-token FLOP and byte counts, evaluated at the workloads' sizes)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from runtime_routed_transformer_amd.workloads import CONFIG_BY_NAME  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_grouped_gemm_flops_per_depth():
    # mid workload: T = 16,384 tokens, d = 1,024, f = 4,096 (SwiGLU)
    f = bench.gemm_flops(CONFIG_BY_NAME["mid_bf16"])
    assert f["gemm_qkv"] == 2 * 16384 * 3072 * 1024
    assert f["gemm_o"] == 2 * 16384 * 1024 * 1024
    assert f["gemm_gate_up"] == 2 * 16384 * 8192 * 1024
    assert f["gemm_down"] == 2 * 16384 * 1024 * 4096
    # per forward: 2 (4 d^2 + 3 d f) per token and depth, 4,398 GFLOP at 8 depths
    per_fwd = sum(f.values()) * 8
    assert per_fwd == 2 * (4 * 1024 ** 2 + 3 * 1024 * 4096) * 16384 * 8
    assert round(per_fwd / 1e9, 1) == 4398.0
    # GELU (two matrices): the up projection has f rows, not 2 f
    g = bench.gemm_flops(CONFIG_BY_NAME["tiny_fp32"])
    assert g["gemm_gate_up"] == 2 * 64 * 256 * 64


def test_bandwidth_kernel_bytes():
    b = bench.hbm_bytes(CONFIG_BY_NAME["mid_bf16"])
    T, d = 16384, 1024
    assert b["pool"] == 4 * T * d                       # 67.1 MB: read s once
    assert b["norm_attn"] == (4 + 2) * T * d            # read s, write bf16 u
    assert b["win_attn"] == 2 * 4 * T * d               # q, k, v in, o out (bf16)
    assert b["gemm_down (scatter epilogue)"] == 8 * T * d


def test_decode_bytes_per_launch():
    cfg = CONFIG_BY_NAME["mid_bf16"]
    w = bench.decode_weight_bytes(cfg)
    d, f = 1024, 4096
    assert w == {"gemm_qkv": 3 * d * d * 2, "gemm_o": d * d * 2, "gemm_gate_up": 2 * f * d * 2,
                 "gemm_down": f * d * 2}
    # one expert's whole block in bf16: 2 (4 d^2 + 3 d f) bytes = 33.6 MB
    assert sum(w.values()) == 2 * (4 * d * d + 3 * d * f)
    # three distinct experts at a depth read three experts' gate/up rows,
    # plus the 4 documents' input (bf16) and hidden (bf16) rows
    assert bench.decode_launch_bytes(cfg, "gemm_gate_up", 3) == 3 * w["gemm_gate_up"] + 4 * (d * 2 + f * 2)


def test_stored_traffic_is_ignored_once_sources_change(tmp_path, monkeypatch):
    # a profile whose digest does not match the current sources gives None
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "gemm_qkv_mid_bf16_traffic.md").write_text(
        'x\n```json\n{"bytes_per_launch": 1.0, "sources_sha256": "0"}\n```\n')
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "runtime_routed_transformer_amd" / "csrc").mkdir(parents=True)
    for name in ("gemm.hip", "lol_internal.h"):
        (tmp_path / "runtime_routed_transformer_amd" / "csrc" / name).write_text("src")
    assert bench.stored_traffic("gemm_qkv", "mid_bf16") is None
    digest = bench.kernel_sources_digest("gemm_qkv")
    (prof / "gemm_qkv_mid_bf16_traffic.md").write_text(
        'x\n```json\n{"bytes_per_launch": 123.0, "sources_sha256": "%s"}\n```\n' % digest)
    assert bench.stored_traffic("gemm_qkv", "mid_bf16") == pytest.approx(123.0)


def test_stored_skewed_bias_equals_a_fresh_calibration():
    """The benchmark reads the skewed workloads' balancing bias from a
    fixture written by oracle/write_bias_fixture.py (so its GPU legs never
    run the oracle); the fixture must still be what the calibration gives
    for the current config, bit for bit."""
    import numpy as np
    from oracle import write_bias_fixture as wbf
    from runtime_routed_transformer_amd.workloads import generate, load_skewed_bias
    cfgs = wbf.fixture_configs()
    assert cfgs, "no skewed workload"
    for cfg in cfgs:
        inp = generate(cfg)
        load_skewed_bias(inp)
        np.testing.assert_array_equal(inp.expert_bias.view(np.uint32),
                                      wbf.calibrated(cfg).view(np.uint32), err_msg=cfg.name)


def test_bench_gpu_legs_do_not_import_the_oracle():
    """Only the cpu_baseline code of bench.py may import oracle/: every
    import of it sits inside a baseline block."""
    import ast
    src = open(os.path.join(ROOT, "bench.py")).read()
    tree = ast.parse(src)
    for node in ast.walk(tree):
        if isinstance(node, (ast.Import, ast.ImportFrom)):
            names = [a.name for a in node.names] if isinstance(node, ast.Import) else [node.module or ""]
            if any(n == "oracle" or n.startswith("oracle.") for n in names):
                line = src.splitlines()[node.lineno - 1]
                ctx = "\n".join(src.splitlines()[max(0, node.lineno - 12):node.lineno])
                assert "cpu_baseline" in ctx or "no_cpu_baseline" in ctx, line
