"""Host-side checks of the measurement script and of the product/oracle split
(no GPU needed)."""
import ast
import importlib.util
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mixture_experts_layer_09_amd")


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_record_digest_and_lookup():
    b = _bench_module()
    d = b.kernel_sources_digest()
    assert re.fullmatch(r"[0-9a-f]{16}", d)
    assert d == b.kernel_sources_digest()                      # stable
    assert b.traffic_record("no_such_workload") is None
    rec = b.traffic_record("cfg2_M64")
    # either the committed counters still describe these sources, or null
    assert rec is None or rec > 0


def test_workload_names_resolve():
    b = _bench_module()
    cfg, M = b.workload("cfg2_M64")
    assert (cfg.H, cfg.E_routed, cfg.top_k, cfg.I, M) == (2048, 128, 8, 768, 64)
    cfg, M = b.workload("cfg5_M8192")
    assert (cfg.H, cfg.E_routed, cfg.quant, M) == (6144, 20, "w4a8", 8192)


def _imported_modules(path):
    tree = ast.parse(open(path).read())
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            for a in node.names:
                yield a.name
        elif isinstance(node, ast.ImportFrom):
            yield node.module or ""


@pytest.mark.parametrize("name", sorted(f for f in os.listdir(PKG) if f.endswith(".py")))
def test_product_package_does_not_use_the_oracle(name):
    """The oracle is test infrastructure: nothing in the package imports it."""
    mods = list(_imported_modules(os.path.join(PKG, name)))
    assert not any(m == "oracle" or m.startswith("oracle.") for m in mods), mods
    assert "oracle" not in open(os.path.join(PKG, name)).read()


def test_native_sources_do_not_reference_the_oracle():
    for root, _, files in os.walk(os.path.join(PKG, "csrc")):
        for f in files:
            txt = open(os.path.join(root, f)).read()
            assert "oracle" not in txt.lower(), f


def test_weight_bytes_count_every_format_and_scale():
    """Algorithmic bytes per expert: elements at the format's width plus its
    scales (one fp32 per 128x128 block, one bf16 per row per 128 K, one E8M0
    byte per row per 32 K)."""
    import dataclasses
    b = _bench_module()
    cfg, _ = b.workload("cfg2_M64")                  # N1 = 1536, H = 2048, I = 768
    n13, n2 = 1536 * 2048, 2048 * 768
    want = {"bf16": (2 * n13, 2 * n2),
            "fp8_tensor": (n13 + 4, n2 + 4),
            "fp8_block": (n13 + 12 * 16 * 4, n2 + 16 * 6 * 4),
            "w4a8": (n13 // 2 + 1536 * 16 * 2, n2 // 2 + 2048 * 6 * 2),
            "mxfp8": (n13 + n13 // 32, n2 + n2 // 32),
            "mxfp4": (n13 // 2 + n13 // 32, n2 // 2 + n2 // 32)}
    for q, (w13, w2) in want.items():
        assert b.weight_bytes_per_expert(dataclasses.replace(cfg, quant=q)) == (w13, w2), q


def test_overridden_workloads_have_no_traffic_record():
    b = _bench_module()
    assert b.traffic_record("cfg2_M64_gelu_tanh") is None
    assert b.traffic_record("cfg2_M64_mxfp4") is None
