"""Benchmark: cached block-diffusion denoising steps on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
    python bench.py --decode-loop [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch: block attention over
the prefix cache + block, LM head, confidence select (with the commit-state
update) and, after the last sub-block of a block, the KV append.  The default
workload is the Qwen2.5-7B-shaped one (batch 4, 28/4 heads, d 128, prompt
1024, answer 512, block 32, sub-block 8, vocab 152064, tau 0.9); its 64-step
schedule is replayed until K steps have been timed.  Inputs are resident in
HBM before timing starts.  Prints one JSON line.

With --decode-loop a timed unit is instead one whole generation of the batch
through fdl_decode (the device-side decode loop with its stand-in model):
every block, sub-block and step until all positions are committed or EOS
stops the sequences; K generations are timed after W warmup generations, and
the line reports steps/s and committed tokens/s of those generations.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "denoise-steps/s and committed tokens/s, Qwen2.5-7B shapes; % of HBM/MFMA roof"
HBM_PEAK_GBS = 8000.0
# The dominant call is bracketed by HIP events on every EV_EVERY-th timed step
# (on its launch stream, inside the timed region).  Bracketing every step cost
# ~5 us of GPU time per step (2.8% of the 7B/bs4 step) for the same average.
EV_EVERY = 8
BF16_MFMA_PEAK_TFLOPS = 2500.0
def pmc_profile(workload):
    """Path of the committed FETCH_SIZE / WRITE_SIZE summary of a workload's LM head."""
    return os.path.join(ROOT, "profiles", f"lm_head_{workload}_pmc.txt")
LM_HEAD_SRC = os.path.join(ROOT, "block_diffusion_decoding_attn_amd", "csrc", "lm_head.hip")


def lm_head_bytes_flops(cfg, fused: bool):
    """Algorithmic bytes and flops of one LM-head (+ select) call.

    Unfused fdl_lm_head: W and X read once, the f32 logits written once.
    Fused fdl_lm_head_select: W and X read once, the select's per-row outputs
    (token, confidence, commit flag, the in-place token/masked updates) and
    per-sequence counts written; the logits never exist."""
    esz = 4 if cfg.dtype == "f32" else 2
    M = cfg.rows
    byts = cfg.vocab * cfg.hidden * esz + M * cfg.hidden * esz
    byts += M * (4 + 4 + 1 + 4 + 1) + cfg.batch * 4 if fused else M * cfg.vocab * 4
    flops = 2.0 * M * cfg.hidden * cfg.vocab
    return byts, flops


def lm_head_kernel_name(cfg):
    """The LM-head kernel the library launches for this workload's rows."""
    if cfg.dtype == "f32":
        return "lm_head_skinny_f32"
    if cfg.rows <= 32:
        return "lm_head_skinny_bf16_one"
    return "lm_head_skinny_bf16" if cfg.rows <= 64 else "lm_head_tiled_bf16"


def finalize_kernel_name(cfg):
    """The select finalize kernel the library launches after the fused LM head."""
    r, rows = cfg.rows // cfg.batch, cfg.rows
    if r > 64:
        return "select_finalize_kernel"
    return "select_finalize_row_kernel" if rows <= 256 else "select_finalize_seq_kernel"


def pmc_traffic(workload, per_launch_units=1):
    """HBM bytes per launch from the committed rocprofv3 counter summary, scaled
    by the copy-kernel calibration; None when missing, taken on another
    workload, or the kernel source changed since."""
    path = pmc_profile(workload)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    try:
        sha = hashlib.sha256(open(LM_HEAD_SRC, "rb").read()).hexdigest()
        if kv.get("source_sha256") != sha or kv.get("workload") != workload:
            return None
        fetch = float(kv["fetch_kib_per_dispatch"]) * 1024 * float(kv["copy_fetch_scale"])
        write = float(kv["write_kib_per_dispatch"]) * 1024 * float(kv["copy_write_scale"])
        return (fetch + write) * per_launch_units
    except (KeyError, ValueError):
        return None


def cpu_baseline(run, budget_s: float):
    """The oracle, as it stands, on the same workload's first steps (bounded)."""
    import numpy as np
    from oracle import fdl_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    cfg = run.cfg
    kc = run.kc_host.float().numpy().copy()
    vc = run.vc_host.float().numpy().copy()
    length = np.full(cfg.batch, cfg.prompt_len)
    t0 = time.perf_counter()
    n = 0
    commits = 0
    for i in run.step_ids:
        inp = run.host_inputs[i]
        kb, vb = run.kb_host[inp.block_idx]
        O.block_attention(inp.q, kc, vc, kb, vb, length, mode=cfg.attn_mode, total_len=cfg.cap)
        logits = O.lm_head(inp.x, run.w_host)
        res = O.conf_select(logits.reshape(cfg.batch, cfg.sub_block, cfg.vocab), inp.masked.numpy(),
                            inp.tau.numpy())
        commits += int(res["n_commit"].sum())
        if inp.append_after:
            kc, _ = O.kv_append(kc, kb.float().numpy(), length)
            vc, length = O.kv_append(vc, vb.float().numpy(), length)
        n += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} steps of the {cfg.name} schedule (fp64 numpy oracle: attention, LM head, "
                      f"select, append), {dt:.1f} s; {commits / dt:.3f} committed tokens/s"}


def attn_bytes(cfg, lk: int) -> int:
    """Algorithmic bytes of one attention call: Q and O once, every visible
    K/V row of every KV head once."""
    esz = 4 if cfg.dtype == "f32" else 2
    qo = 2 * cfg.batch * cfg.sub_block * cfg.n_q_heads * cfg.head_dim * esz
    return qo + 2 * cfg.batch * cfg.n_kv_heads * lk * cfg.head_dim * esz


def bench_decode_loop(args, cfg):
    import numpy as np
    import torch
    from block_diffusion_decoding_attn_amd.runner import DecodeRunner

    run = DecodeRunner(cfg, select=args.select, k=args.k, boost=args.boost, trace=True)
    for _ in range(max(args.warmup, 1)):
        run.run()
    torch.cuda.synchronize()
    res = run.results()
    steps = res["steps"]
    # committed positions: every position of the blocks a sequence generated
    committed = int(sum((res["eos_block"][b] + 1 if res["eos_block"][b] >= 0 else res["blocks_run"]) * cfg.block
                        for b in range(cfg.batch)))
    # algorithmic HBM bytes of the steps that ran: LM head + attention
    lm_b, _ = lm_head_bytes_flops(cfg, True)
    att_b = 0
    for t in res["trace"]:
        lp = cfg.prompt_len + t["block"] * cfg.block
        lk = cfg.cap if cfg.attn_mode == "dual_cache" else lp + cfg.block
        att_b += attn_bytes(cfg, lk)
    byts = steps * lm_b + att_b
    graph = run.capture(trace=False) if args.graph else None
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    host = []
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        h = time.perf_counter()
        if graph is not None:
            graph.replay()
        else:
            run.run(trace=False)
        host.append(time.perf_counter() - h)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    if int(run.counters[0]) != steps:
        raise RuntimeError("the timed generations ran a different number of steps")
    achieved = byts / (ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": steps / (ms * 1e-3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms / steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if cfg.dtype == "f32" else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} decode loop", "batch": cfg.batch, "prompt_len": cfg.prompt_len,
                   "gen_len": cfg.gen_len, "block": cfg.block, "sub_block": cfg.sub_block, "hidden": cfg.hidden,
                   "vocab": cfg.vocab, "attn_mode": cfg.attn_mode, "select": args.select, "tau": list(cfg.tau),
                   "gain": run.inp.gain, "timed_unit": "one generation (fdl_decode call)",
                   "launch": "hip graph replay" if args.graph else "eager enqueue",
                   "parallelism": "single-gpu"},
        "committed_tokens_per_s": committed / (ms * 1e-3),
        "ms_per_generation": ms,
        "steps_per_generation": steps,
        "step_slots_enqueued": run.slots,
        "blocks_run": res["blocks_run"],
        "eos_block": [int(x) for x in res["eos_block"]],
        "host_enqueue_ms": 1e3 * float(np.median(host)),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "whole loop: LM head + attention algorithmic bytes of the steps run / loop time",
                     "algorithmic_bytes": byts},
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1280)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default="qwen2.5-7b_bs4")
    ap.add_argument("--select", default="threshold", choices=["threshold", "topk", "factor"])
    ap.add_argument("--k", type=int, default=4)
    ap.add_argument("--boost", default="calibrated", choices=["calibrated", "literal"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unfused", action="store_true",
                    help="fdl_lm_head + fdl_conf_select (logits materialized) instead of fdl_lm_head_select")
    ap.add_argument("--decode-loop", action="store_true",
                    help="time whole generations through fdl_decode instead of single steps")
    ap.add_argument("--graph", action="store_true",
                    help="with --decode-loop: capture the generation in a HIP graph and time its replays")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the batch dimension would shard across GPUs with no exchange)", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_diffusion_decoding_attn_amd import fdl, synth
    from block_diffusion_decoding_attn_amd.runner import StepRunner

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fdl.lib()
    cfg = synth.get_config(args.workload)
    if args.decode_loop:
        bench_decode_loop(args, cfg)
        return
    t_setup = time.perf_counter()
    run = StepRunner(cfg, select=args.select, k=args.k, boost=args.boost, keep_host=not args.no_cpu_baseline,
                     fused=not args.unfused)
    print(f"# setup {time.perf_counter() - t_setup:.1f} s", file=sys.stderr, flush=True)
    nsched = len(run.step_ids)

    # commits per schedule step (deterministic: the same inputs every pass)
    run.reset()
    commits = []
    for i in run.step_ids:
        run.step(i)
        commits.append(int(run.n_commit.sum()))
    torch.cuda.synchronize()

    def do_steps(n, start, ev=None):
        pos = start
        for j in range(n):
            if pos == 0:
                run.reset()
            i = run.step_ids[pos]
            inp = run.inputs[i]
            if run.dual and inp.sub_idx == 0:
                run.refresh_block(inp.block_idx)
            run.attention(i)
            timed = ev is not None and j % EV_EVERY == 0
            if timed:
                ev[j // EV_EVERY][0].record()
            if run.fused:
                run.lm_head_select(i)
            else:
                run.lm_head(i)
            if timed:
                ev[j // EV_EVERY][1].record()
            if not run.fused:
                run.select(i)
            if inp.append_after and not run.dual:
                run.append(i)
            pos = (pos + 1) % nsched
        return pos

    pos = do_steps(args.warmup, 0)
    torch.cuda.synchronize()
    n_ev = (args.steps + EV_EVERY - 1) // EV_EVERY
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_ev)]
    start_pos = pos
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    do_steps(args.steps, start_pos, ev)
    t_end.record()
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end)
    ms_per_step = ms / args.steps
    committed = sum(commits[(start_pos + j) % nsched] for j in range(args.steps))
    lm_ms = sum(a.elapsed_time(b) for a, b in ev) / n_ev

    byts, flops = lm_head_bytes_flops(cfg, run.fused)
    ai = flops / byts
    if ai > BF16_MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        roof = {"bound": "mfma", "achieved": flops / (lm_ms * 1e-3) / 1e12, "peak": BF16_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": byts / (lm_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = pmc_traffic(cfg.name) if run.fused else None
    kname = lm_head_kernel_name(cfg)
    roof["kernel"] = (f"fdl_lm_head_select ({kname} with the select epilogue + {finalize_kernel_name(cfg)})"
                      if run.fused else f"fdl_lm_head ({kname})")
    roof["kernel_us"] = lm_ms * 1e3
    roof["kernel_calls_timed"] = n_ev
    roof["algorithmic_bytes"] = byts

    out = {
        "metric": METRIC,
        "value": 1e3 / ms_per_step,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if cfg.dtype == "f32" else "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "prompt_len": cfg.prompt_len, "gen_len": cfg.gen_len,
                   "block": cfg.block, "sub_block": cfg.sub_block, "n_q_heads": cfg.n_q_heads,
                   "n_kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim, "hidden": cfg.hidden, "vocab": cfg.vocab,
                   "attn_mode": cfg.attn_mode, "select": args.select, "tau": list(cfg.tau), "boost": args.boost,
                   "lm_head_select": "unfused" if args.unfused else "fused", "parallelism": "single-gpu"},
        "committed_tokens_per_s": committed / (ms * 1e-3),
        "commits_per_step": committed / args.steps,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(run, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
