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
    sha = bench.source_sha256("lm_head")
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


def test_attention_counter_summary_long_context():
    """The long-context attention summary: K/V leave HBM once; the rest of the
    counted traffic is the split partials (written by the attention, read
    back by the merge) and Q / O."""
    name = "qwen2.5-7b_long_bs16"
    path = bench.pmc_profile(name, "attn")
    assert os.path.exists(path)
    kv = _pmc_fields(path)
    assert kv["workload"] == name
    assert kv["kernel"] == "block_attn_bf16_kernel + block_attn_bf16_merge_kernel"
    if kv["source_sha256"] != bench.source_sha256("attn"):
        assert bench.pmc_traffic(name, "attn") is None  # taken on other sources: not reported
        pytest.skip("attention counter summary taken on another source")
    cfg = synth.get_config(name)
    lk = cfg.prompt_len + cfg.block
    pairs = cfg.batch * cfg.n_kv_heads
    rows = cfg.n_q_heads // cfg.n_kv_heads * cfg.sub_block  # query rows per KV head
    live_waves = (rows + 31) // 32
    nsplit = 4                                           # 256 workgroups over 64 KV heads
    partials = nsplit * pairs * live_waves * (cfg.head_dim // 4 + 2) * 64 * 4  # O / l as bf16, m, l
    q = cfg.batch * cfg.sub_block * cfg.n_q_heads * cfg.head_dim * 2
    kvb = 2 * pairs * lk * cfg.head_dim * 2
    assert bench.attn_bytes(cfg, lk) == kvb + 2 * q
    fetch = float(kv["fetch_bytes_per_dispatch"])
    write = float(kv["write_bytes_per_dispatch"])
    assert abs(fetch - (kvb + q + partials)) / kvb < 0.02
    assert abs(write - (partials + q)) / (partials + q) < 0.02


def _sqlite(path, tables):
    import sqlite3
    con = sqlite3.connect(path)
    for name, cols, rows in tables:
        con.execute(f"create table {name}({', '.join(cols)})")
        con.executemany(f"insert into {name} values ({', '.join('?' * len(cols))})", rows)
    con.commit()
    con.close()


def test_summarize_trace_and_counters(tmp_path, capsys):
    tr = str(tmp_path / "t.db")
    _sqlite(tr, [("kernels", ["name", "duration"], [("k_a", 3000), ("k_a", 5000), ("k_b", 1000)])])
    bench.summarize_trace(tr)
    out = capsys.readouterr().out.splitlines()
    assert out[2] == "| `k_a` | 2 | 4.00 | 3.00 | 5.00 | 88.9% |"
    assert out[3] == "| `k_b` | 1 | 1.00 | 1.00 | 1.00 | 11.1% |"
    pc = str(tmp_path / "c.db")
    _sqlite(pc, [("counters_collection", ["kernel_name", "counter_name", "dispatch_id", "value"],
                  [("k_a", "X", 1, 2.0), ("k_a", "X", 1, 3.0), ("k_a", "X", 2, 7.0), ("k_a", "Y", 1, 1.0),
                   ("k_a", "Y", 2, 3.0)]),
                 ("kernels", ["name", "duration"], [("k_a", 2000), ("k_a", 4000)])])
    bench.summarize_counters(pc)
    out = capsys.readouterr().out.splitlines()
    # dispatch 1: X = 2 + 3 (records summed), dispatch 2: X = 7 -> mean 6; Y mean 2
    assert out[2] == "| `k_a` | 2 | 3.00 | 6 | 2 |"


def test_summarize_pmc_scales_by_the_copy(tmp_path, capsys):
    rows_f = [("void fdl::block_attn_bf16_kernel<128, 8>(fdl::AttnArgs)", "FETCH_SIZE", d, v)
              for d, v in [(1, 100.0), (1, 50.0), (2, 150.0)]]
    rows_f += [("void fdl::block_attn_bf16_merge_kernel<128, 8, 16, 4, 4>(fdl::AttnArgs)", "FETCH_SIZE", 3, 20.0)]
    rows_w = [("void fdl::block_attn_bf16_kernel<128, 8>(fdl::AttnArgs)", "WRITE_SIZE", 1, 10.0),
              ("void fdl::block_attn_bf16_merge_kernel<128, 8, 16, 4, 4>(fdl::AttnArgs)", "WRITE_SIZE", 2, 5.0)]
    cols = ["kernel_name", "counter_name", "dispatch_id", "value"]
    dbs = []
    for nm, rows in [("f", rows_f), ("w", rows_w), ("cf", [("copy", "FETCH_SIZE", 1, 512.0)]),
                     ("cw", [("copy", "WRITE_SIZE", 1, 1024.0)])]:
        p = str(tmp_path / f"{nm}.db")
        _sqlite(p, [("counters_collection", cols, rows)])
        dbs.append(p)

    class A:
        summarize_pmc = dbs
        pmc_kernel = "attn"
        workload = "qwen2.5-7b_long_bs16"
        pmc_copy_mib = 1
    bench.summarize_pmc(A)
    kv = dict(line.split(": ", 1) for line in capsys.readouterr().out.splitlines())
    # kernel 150 KiB per dispatch + merge 20 KiB, a 1 MiB copy read as 512 KiB -> scale 2
    assert float(kv["fetch_kib_per_dispatch"]) == 170.0
    assert float(kv["copy_fetch_scale"]) == 2.0
    assert int(kv["fetch_bytes_per_dispatch"]) == 170 * 1024 * 2
    assert int(kv["write_bytes_per_dispatch"]) == 15 * 1024


def test_cpu_baseline_sample_and_cores():
    """The oracle leg on the CPU: per-stage seconds, the threads it ran on
    within the affinity mask, blocks taken from their own cache states."""
    from block_diffusion_decoding_attn_amd.runner import StepRunner
    cfg = synth.get_config("qwen2.5-1.5b_bs1")
    run = StepRunner(cfg, device="cpu", keep_host=True)
    r = bench.cpu_baseline(run, 3.0)
    assert r["kind"] == "oracle" and r["unit"] == "steps/s" and r["value"] > 0
    assert 1 <= r["cores"] <= r["affinity_cores"] == bench.host_cores()
    assert set(r["stage_seconds_per_step"]) == {"attention", "lm_head", "select", "append"}
    assert "blocks 0," in r["sample"] and "of 8" in r["sample"]
    assert 0.0 <= r["exceed_tau_fraction"] <= 1.0


def test_prefill_shape_and_pairs():
    """The multi-block bench line: prompt prefill under the block-causal mask,
    the whole cache bidirectionally for DualCache; visible pairs counted by
    brute force over the mask on small sizes."""
    from block_diffusion_decoding_attn_amd import synth
    assert bench.prefill_shape(synth.get_config("qwen2.5-7b_bs4")) == (1024, True)
    llada = synth.get_config("llada-8b_dualcache")
    assert bench.prefill_shape(llada) == (llada.cap, False)
    for n, blk in [(1, 32), (31, 32), (64, 32), (100, 16), (257, 32)]:
        brute = sum(1 for p in range(n) for j in range(n) if j // blk <= p // blk)
        assert bench.prefill_pairs(n, blk, True) == brute
        assert bench.prefill_pairs(n, blk, False) == n * n
