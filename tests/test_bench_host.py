"""Host logic of bench.py (no GPU): the one-GPU guard, the algorithmic byte and
flop counts behind the roofline fraction, the kernel names it reports, and the
gating of the counter-based HBM traffic."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from block_diffusion_decoding_attn_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_lm_head_bytes_and_flops_qwen7b_bs4():
    cfg = synth.get_config("qwen2.5-7b_bs4")
    M, H, V = 32, 3584, 152064
    byts, flops = bench.lm_head_bytes_flops(cfg, fused=True)
    # weights and rows read once; per row token, confidence, commit flag, token and masked updates; per sequence
    # the commit count
    assert byts == V * H * 2 + M * H * 2 + M * (4 + 4 + 1 + 4 + 1) + 4 * 4
    assert byts == 1090224128 + 464
    assert flops == 2.0 * M * H * V
    byts_u, _ = bench.lm_head_bytes_flops(cfg, fused=False)
    assert byts_u == V * H * 2 + M * H * 2 + M * V * 4


def test_roofline_bound_by_arithmetic_intensity():
    ridge = bench.BF16_MFMA_PEAK_TFLOPS * 1e12 / (bench.HBM_PEAK_GBS * 1e9)
    for name, bound in [("qwen2.5-7b_bs4", "hbm"), ("qwen2.5-1.5b_bs1", "hbm"), ("llada-8b_dualcache", "hbm"),
                        ("qwen2.5-7b_long_bs16", "mfma")]:
        byts, flops = bench.lm_head_bytes_flops(synth.get_config(name), fused=True)
        assert (flops / byts > ridge) == (bound == "mfma"), name


@pytest.mark.parametrize("name,lm,fin", [
    ("qwen2.5-7b_bs4", "lm_head_skinny_bf16_one", "select_finalize_row_kernel"),
    ("qwen2.5-1.5b_bs1", "lm_head_skinny_bf16_one", "select_finalize_row_kernel"),
    ("llada-8b_dualcache", "lm_head_skinny_bf16_one", "select_finalize_row_kernel"),
    ("qwen2.5-7b_long_bs16", "lm_head_tiled_bf16", "select_finalize_seq_kernel"),
    ("tiny_fp32", "lm_head_skinny_f32", "select_finalize_row_kernel"),
])
def test_reported_kernel_names(name, lm, fin):
    cfg = synth.get_config(name)
    assert bench.lm_head_kernel_name(cfg) == lm
    assert bench.finalize_kernel_name(cfg) == fin


def _pmc_fields(path):
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    return kv


def test_default_workload_has_a_counter_summary():
    assert os.path.exists(bench.pmc_profile(synth.get_config(2).name))


@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_counter_traffic_only_for_its_workload_and_source(name):
    path = bench.pmc_profile(name)
    if not os.path.exists(path):
        assert bench.pmc_traffic(name) is None
        return
    kv = _pmc_fields(path)
    assert kv["workload"] == name
    cfg = synth.get_config(name)
    assert kv["kernel"] == bench.lm_head_kernel_name(cfg)
    sha = hashlib.sha256(open(bench.LM_HEAD_SRC, "rb").read()).hexdigest()
    got = bench.pmc_traffic(name)
    if kv["source_sha256"] != sha:
        assert got is None          # taken on other sources: not reported
        return
    fetch = float(kv["fetch_kib_per_dispatch"]) * 1024 * float(kv["copy_fetch_scale"])
    write = float(kv["write_kib_per_dispatch"]) * 1024 * float(kv["copy_write_scale"])
    assert got == pytest.approx(fetch + write)
    byts, _ = bench.lm_head_bytes_flops(cfg, fused=True)
    if cfg.rows <= 64:
        # skinny: the weights leave HBM once, within 1% of the algorithmic bytes of the call
        assert abs(got - byts) / byts < 0.01
    else:
        # tiled: at least the algorithmic bytes (row tiles of a weight tile share one XCD's L2)
        assert got >= 0.99 * byts
