"""Benchmark: cached block-diffusion denoising steps on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
    python bench.py --decode-loop [--steps K] [--warmup W] [--workload NAME]
    python bench.py --prefill [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch: block attention over
the prefix cache + block, LM head, confidence select (with the commit-state
update) and, after the last sub-block of a block, the KV append.  The default
workload is the Qwen2.5-7B-shaped one (batch 4, 28/4 heads, d 128, prompt
1024, answer 512, block 32, sub-block 8, vocab 152064, tau 0.9); its 64-step
schedule is replayed until K steps have been timed.  Inputs are resident in
HBM before timing starts.  Prints one JSON line.

Two kernels carry a roofline entry: the LM head + select call (`roofline`,
the step's dominant launch) and the block attention (`roofline_attention`);
each is bracketed by HIP events on every EV_EVERY-th timed step, on the stream
it is launched on.

    python bench.py --calibrate-counters [MiB]

runs only a plain device copy of a known size, for rocprofv3 --pmc runs that
calibrate the FETCH_SIZE / WRITE_SIZE counters (what they report for a copy
that moves exactly that many bytes each way).

With --decode-loop a timed unit is instead one whole generation of the batch
through fdl_decode (the device-side decode loop with its stand-in model):
every block, sub-block and step until all positions are committed or EOS
stops the sequences; K generations are timed after W warmup generations, and
the line reports steps/s and committed tokens/s of those generations.

With --prefill a timed unit is one fdl_prefill_attn call on the workload's
multi-block attention: the prompt prefill under the block-causal mask (the v1
refresh of the whole cache, every key visible, for the DualCache workload);
the line reports positions/s and the call's MFMA roofline fraction.
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
CSRC = os.path.join(ROOT, "block_diffusion_decoding_attn_amd", "csrc")
LM_HEAD_SRC = os.path.join(CSRC, "lm_head.hip")
ATTN_SRC = os.path.join(CSRC, "attn.hip")
# the sources a kernel's counter summary was taken on (the hash covers them all)
KERNEL_SOURCES = {"lm_head": [LM_HEAD_SRC], "attn": [ATTN_SRC, os.path.join(CSRC, "kv_tiles.h")]}


def source_sha256(kernel):
    h = hashlib.sha256()
    for path in KERNEL_SOURCES[kernel]:
        h.update(open(path, "rb").read())
    return h.hexdigest()


def pmc_profile(workload, kernel="lm_head"):
    """Path of the committed FETCH_SIZE / WRITE_SIZE summary of a workload's
    LM head ("lm_head") or block attention ("attn")."""
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.txt")


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


def pmc_traffic(workload, kernel="lm_head", per_launch_units=1):
    """HBM bytes per launch from the committed rocprofv3 counter summary, scaled
    by the copy-kernel calibration; None when missing, taken on another
    workload, or the kernel source changed since.  For the attention the
    summary's figure covers the attention kernel and its split merge."""
    path = pmc_profile(workload, kernel)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    try:
        if kv.get("source_sha256") != source_sha256(kernel) or kv.get("workload") != workload:
            return None
        fetch = float(kv["fetch_kib_per_dispatch"]) * 1024 * float(kv["copy_fetch_scale"])
        write = float(kv["write_kib_per_dispatch"]) * 1024 * float(kv["copy_write_scale"])
        return (fetch + write) * per_launch_units
    except (KeyError, ValueError):
        return None


def host_cores():
    """Cores this process may run on (its CPU affinity mask)."""
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        return 1


def _oracle_steps(run, steps, kc, vc, length, stage):
    """Run the oracle over `steps` (schedule indices, in order) from the cache
    state (kc, vc, length); add each stage's seconds to `stage`.  Returns
    (kc, vc, length, commits, rows above tau, candidate rows)."""
    import numpy as np
    from oracle import fdl_oracle as O
    cfg = run.cfg
    commits = above = cands = 0
    for i in steps:
        inp = run.host_inputs[i]
        kb, vb = run.kb_host[inp.block_idx]
        t = time.perf_counter()
        O.block_attention(inp.q, kc, vc, kb, vb, length, mode=cfg.attn_mode, total_len=cfg.cap)
        t1 = time.perf_counter()
        logits = O.lm_head(inp.x, run.w_host)
        t2 = time.perf_counter()
        masked = inp.masked.numpy()
        tau = inp.tau.numpy()
        res = O.conf_select(logits.reshape(cfg.batch, cfg.sub_block, cfg.vocab), masked, tau)
        t3 = time.perf_counter()
        commits += int(res["n_commit"].sum())
        above += int(((res["conf"] > tau[:, None]) & (masked > 0)).sum())
        cands += int((masked > 0).sum())
        if inp.append_after and cfg.attn_mode != "dual_cache":
            kc, _ = O.kv_append(kc, kb.float().numpy(), length)
            vc, length = O.kv_append(vc, vb.float().numpy(), length)
        t4 = time.perf_counter()
        for key, dt in (("attention", t1 - t), ("lm_head", t2 - t1), ("select", t3 - t2), ("append", t4 - t3)):
            stage[key] += dt
    return kc, vc, length, commits, above, cands


def cpu_baseline(run, budget_s: float):
    """The oracle, as it stands, on a bounded sample of the same workload.

    The sample is the steps of four blocks of the schedule -- the first, the
    last and two spread between them -- each from the cache state it has in
    the schedule (the blocks in between are appended by the oracle, untimed),
    each stage timed on its own (the eq 15 decomposition of the Fast-dLLM
    review, section 7: attention, LM head, select, append); the first block's
    steps are then re-run on one thread.  Steps stop early once `budget_s`
    seconds have gone by."""
    import numpy as np
    from oracle import fdl_oracle as O
    from block_diffusion_decoding_attn_amd import synth
    cfg = run.cfg
    cores = host_cores()
    threads = blas_threads()
    dual = cfg.attn_mode == "dual_cache"
    kc = run.kc_host.float().numpy().copy()
    vc = run.vc_host.float().numpy().copy()
    length = np.full(cfg.batch, cfg.prompt_len)
    blocks = sorted({run.host_inputs[i].block_idx for i in run.step_ids})
    picks = sorted({blocks[0], blocks[len(blocks) // 3], blocks[2 * len(blocks) // 3], blocks[-1]})
    stage = dict(attention=0.0, lm_head=0.0, select=0.0, append=0.0)
    n = commits = above = cands = 0
    t0 = time.perf_counter()
    cur = blocks[0]  # the cache holds every block before `cur`
    for blk in picks:
        if time.perf_counter() - t0 > budget_s:
            break
        if dual:
            length = np.full(cfg.batch, cfg.prompt_len + blk * cfg.block)
        else:
            for b in range(cur, blk):  # untimed: the blocks the sample skips
                kb, vb = run.kb_host[b] if b in run.kb_host else synth.block_kv(cfg, b, run.seed)
                kc, _ = O.kv_append(kc, kb.float().numpy(), length)
                vc, length = O.kv_append(vc, vb.float().numpy(), length)
        for i in [i for i in run.step_ids if run.host_inputs[i].block_idx == blk]:
            kc, vc, length, c, a, m = _oracle_steps(run, [i], kc, vc, length, stage)
            n, commits, above, cands = n + 1, commits + c, above + a, cands + m
            if time.perf_counter() - t0 > budget_s:
                break
        cur = blk + 1
    first = [i for i in run.step_ids if run.host_inputs[i].block_idx == blocks[0]]
    busy = sum(stage.values())
    # one thread, the first block's steps again (bounded by a third of the budget)
    one = None
    try:
        from threadpoolctl import threadpool_limits
        kc1 = run.kc_host.float().numpy().copy()
        vc1 = run.vc_host.float().numpy().copy()
        len1 = np.full(cfg.batch, cfg.prompt_len)
        st1 = dict(attention=0.0, lm_head=0.0, select=0.0, append=0.0)
        n1 = 0
        t1 = time.perf_counter()
        with threadpool_limits(limits=1):
            for i in first:
                kc1, vc1, len1, _, _, _ = _oracle_steps(run, [i], kc1, vc1, len1, st1)
                n1 += 1
                if time.perf_counter() - t1 > budget_s / 3:
                    break
        one = {"value": n1 / sum(st1.values()), "steps": n1}
    except Exception:  # noqa: BLE001
        one = None
    sample = (f"{n} steps of the {cfg.name} schedule (blocks {', '.join(map(str, picks))} of {len(blocks)}, each "
              f"from its own cache state: fp64 numpy oracle of attention, LM head, select, append), {busy:.1f} s; "
              f"{commits / busy:.3f} committed tokens/s")
    # cores: the threads the oracle ran on -- its BLAS pool (the LM head's
    # product; the rest of the oracle is single-threaded numpy), within the
    # process's CPU affinity, which is reported beside it
    return {"value": n / busy, "unit": "steps/s", "cores": min(threads, cores), "kind": "oracle", "sample": sample,
            "affinity_cores": cores, "blas_threads": threads,
            "stage_seconds_per_step": {k: v / max(n, 1) for k, v in stage.items()},
            "committed_tokens_per_s": commits / busy,
            "exceed_tau_fraction": above / max(cands, 1),
            "one_thread": one}


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


def prefill_shape(cfg):
    """The multi-block attention a workload runs: the v1 refresh of the whole
    cache (every key visible) for DualCache, else the prompt prefill under the
    block-causal mask.  Returns (n_q = n_keys, causal)."""
    if cfg.attn_mode == "dual_cache":
        return cfg.cap, False
    return cfg.prompt_len, True


def prefill_pairs(n: int, block: int, causal: bool) -> int:
    """Visible (query, key) pairs of one head: block-causal position p sees the
    keys below the end of its block."""
    if not causal:
        return n * n
    return sum(min(n, (p // block + 1) * block) for p in range(n))


def bench_prefill(args, cfg):
    import torch
    from block_diffusion_decoding_attn_amd import fdl, synth

    if cfg.dtype != "bf16":
        print("bench.py --prefill: the multi-block attention is bf16 only", file=sys.stderr)
        sys.exit(2)
    n, causal = prefill_shape(cfg)
    d = fdl.make_dims(cfg)
    dev = torch.device("cuda")
    q = synth.normal((cfg.batch, n, cfg.n_q_heads, cfg.head_dim), 0, cfg.cfg_id, 40, n, dtype=cfg.torch_dtype).to(dev)
    k, v = synth.kv_cache(cfg)
    k, v = k.to(dev), v.to(dev)
    out = torch.empty_like(q)
    for _ in range(max(args.warmup, 1)):
        fdl.fdl_prefill_attn(d, 0, n, causal, q, k, v, out)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        fdl.fdl_prefill_attn(d, 0, n, causal, q, k, v, out)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    flops = 4.0 * cfg.head_dim * prefill_pairs(n, cfg.block, causal) * cfg.n_q_heads * cfg.batch
    byts = 2 * (2 * cfg.batch * n * cfg.n_q_heads * cfg.head_dim + 2 * cfg.batch * cfg.n_kv_heads * n * cfg.head_dim)
    tflops = flops / (ms * 1e-3) / 1e12
    out_line = {
        "metric": "multi-block attention positions/s (prompt prefill or v1 refresh)",
        "value": cfg.batch * n / (ms * 1e-3),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} {'v1 refresh' if not causal else 'prompt prefill'}",
                   "batch": cfg.batch, "positions": n, "n_q_heads": cfg.n_q_heads, "n_kv_heads": cfg.n_kv_heads,
                   "head_dim": cfg.head_dim, "block": cfg.block, "mask": "block-causal" if causal else "bidirectional",
                   "timed_unit": "one fdl_prefill_attn call", "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / BF16_MFMA_PEAK_TFLOPS, "traffic": None,
                     "kernel": "prefill_attn_bf16_kernel (one launch per call)",
                     "algorithmic_flops": flops, "algorithmic_bytes": byts,
                     "arithmetic_intensity": flops / byts},
    }
    print(json.dumps(out_line), flush=True)


def calibrate_counters(mib: int, reps: int = 4):
    """A plain device copy that moves exactly `mib` MiB each way, `reps` times:
    under rocprofv3 --pmc FETCH_SIZE (or WRITE_SIZE) it gives the factor
    between what the counter reports and the bytes actually moved."""
    import torch
    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {mib} MiB x {reps}", flush=True)


def exceed_tau(run, cfg, other_boost: str, n_steps: int = 8):
    """Fraction of candidate rows whose confidence clears their tau, for the
    run's own boost generator (its whole schedule, from the commit-counting
    pass) and for the other one (the first n_steps steps, through
    fdl_lm_head_select on separate buffers)."""
    import torch
    from block_diffusion_decoding_attn_amd import fdl, synth
    dev = run.dev
    B, S = cfg.batch, cfg.sub_block
    above = cands = 0
    for i in run.step_ids[:n_steps]:
        x, _, _ = synth.hidden_rows(cfg, run.w_host, i, run.seed, other_boost)
        masked = synth.masked_rows(cfg, i, run.seed).to(dev)
        m0 = masked.clone()
        tau = synth.taus(cfg, i, run.seed).to(dev)
        conf = torch.empty((B, S), dtype=torch.float32, device=dev)
        outs = [torch.empty((B, S), dtype=torch.int32, device=dev), conf,
                torch.empty((B, S), dtype=torch.uint8, device=dev), torch.empty((B,), dtype=torch.int32, device=dev)]
        fdl.fdl_lm_head_select(run.dims, S, x.to(dev), run.w, None, masked, tau, fdl.FDL_SELECT_THRESHOLD, 0, 1.0,
                               *outs, None, None, run.ws_sel)
        torch.cuda.synchronize()
        sel = m0.bool()
        above += int(((conf > tau[:, None]) & sel).sum())
        cands += int(sel.sum())
    return above / max(cands, 1), n_steps


def _pmc_per_kernel(db, counter):
    """{kernel name: (dispatches, mean per-dispatch value)} of one rocprofv3
    --pmc results database (values summed over a dispatch's records)."""
    import sqlite3
    con = sqlite3.connect(db)
    rows = con.execute("select kernel_name, dispatch_id, sum(value) from counters_collection "
                       "where counter_name = ? group by dispatch_id", (counter,)).fetchall()
    out = {}
    for name, _, v in rows:
        n, tot = out.get(name, (0, 0.0))
        out[name] = (n + 1, tot + v)
    return {k: (n, tot / n) for k, (n, tot) in out.items()}


def summarize_pmc(args):
    """Write the FETCH_SIZE / WRITE_SIZE summary that pmc_traffic() reads, from
    four rocprofv3 --pmc databases: the workload's FETCH_SIZE and WRITE_SIZE
    runs and the same two counters over the calibration copy."""
    fetch_db, write_db, cal_fetch_db, cal_write_db = args.summarize_pmc
    kernel = args.pmc_kernel
    names = ["block_attn_bf16_kernel", "block_attn_bf16_merge_kernel"] if kernel == "attn" else [
        lm_head_kernel_name(__import__("block_diffusion_decoding_attn_amd.synth", fromlist=["x"]).get_config(
            args.workload))]

    def pick(db, counter):
        got = _pmc_per_kernel(db, counter)
        n, tot = 0, 0.0
        for nm in names:
            hits = [(k, v) for k, v in got.items() if nm + "<" in k or nm + "(" in k]
            if hits:
                k, (cnt, val) = max(hits, key=lambda kv: kv[1][0])
                n = max(n, cnt)
                tot += val
        return n, tot

    nf, fetch = pick(fetch_db, "FETCH_SIZE")
    nw, write = pick(write_db, "WRITE_SIZE")
    cal_f = max(_pmc_per_kernel(cal_fetch_db, "FETCH_SIZE").items(), key=lambda kv: kv[1][1])[1][1]
    cal_w = max(_pmc_per_kernel(cal_write_db, "WRITE_SIZE").items(), key=lambda kv: kv[1][1])[1][1]
    mib = args.pmc_copy_mib
    sf, sw = mib * 1024 / cal_f, mib * 1024 / cal_w
    sha = source_sha256(kernel)
    lines = [f"kernel: {' + '.join(names)}", f"workload: {args.workload}",
             f"source: {' + '.join(os.path.relpath(p, ROOT) for p in KERNEL_SOURCES[kernel])}",
             f"source_sha256: {sha}",
             f"dispatches_fetch: {nf}", f"dispatches_write: {nw}",
             f"fetch_kib_per_dispatch: {fetch:.1f}", f"write_kib_per_dispatch: {write:.1f}",
             f"copy_fetch_kib_per_dispatch: {cal_f:.1f}", f"copy_write_kib_per_dispatch: {cal_w:.1f}",
             f"copy_fetch_scale: {sf:.4f}", f"copy_write_scale: {sw:.4f}",
             f"fetch_bytes_per_dispatch: {fetch * 1024 * sf:.0f}",
             f"write_bytes_per_dispatch: {write * 1024 * sw:.0f}"]
    print("\n".join(lines))


def summarize_trace(db):
    """Print per-kernel duration statistics (markdown) of a rocprofv3
    --kernel-trace results database (no GPU needed)."""
    import sqlite3
    con = sqlite3.connect(db)
    rows = con.execute("select name, count(*), avg(duration), min(duration), max(duration), sum(duration) "
                       "from kernels group by name order by sum(duration) desc").fetchall()
    total = sum(r[5] for r in rows) or 1
    print("| kernel | calls | avg us | min us | max us | share |")
    print("|---|---|---|---|---|---|")
    for name, n, avg, lo, hi, tot in rows[:12]:
        print(f"| `{name[:80]}` | {n} | {avg / 1e3:.2f} | {lo / 1e3:.2f} | {hi / 1e3:.2f} | {100.0 * tot / total:.1f}% |")


def summarize_counters(db):
    """Print, per kernel and counter, the mean per-dispatch value (records of a
    dispatch summed) and the mean duration of a rocprofv3 --pmc database."""
    import sqlite3
    con = sqlite3.connect(db)
    rows = con.execute("select kernel_name, counter_name, dispatch_id, sum(value) from counters_collection "
                       "group by kernel_name, counter_name, dispatch_id").fetchall()
    acc = {}
    for name, ctr, _, v in rows:
        n, tot = acc.get((name, ctr), (0, 0.0))
        acc[(name, ctr)] = (n + 1, tot + v)
    kernels = sorted({k for k, _ in acc}, key=lambda k: -max(n for (kk, _), (n, _) in acc.items() if kk == k))
    ctrs = sorted({c for _, c in acc})
    dur = {}
    try:
        for name, avg in con.execute("select name, avg(duration) from kernels group by name"):
            dur[name] = avg / 1e3
    except sqlite3.Error:
        pass
    print("| kernel | dispatches | us | " + " | ".join(ctrs) + " |")
    print("|---|---|---|" + "---|" * len(ctrs))
    for k in kernels[:12]:
        n = max(acc[(k, c)][0] for c in ctrs if (k, c) in acc)
        vals = [f"{acc[(k, c)][1] / acc[(k, c)][0]:.6g}" if (k, c) in acc else "" for c in ctrs]
        us = f"{dur[k]:.2f}" if k in dur else ""
        print(f"| `{k[:80]}` | {n} | {us} | " + " | ".join(vals) + " |")


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
    ap.add_argument("--prefill", action="store_true",
                    help="time fdl_prefill_attn on the workload's prompt prefill (v1 refresh for DualCache)")
    ap.add_argument("--graph", action="store_true",
                    help="with --decode-loop: capture the generation in a HIP graph and time its replays")
    ap.add_argument("--calibrate-counters", type=int, nargs="?", const=1024, default=None, metavar="MIB",
                    help="only run a plain device copy of MIB MiB, 4 times (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_DB", "WRITE_DB", "COPY_FETCH_DB", "COPY_WRITE_DB"),
                    help="print the counter-traffic summary of --pmc-kernel on --workload from four rocprofv3 "
                         "--pmc databases (no GPU needed)")
    ap.add_argument("--summarize-trace", metavar="TRACE_DB",
                    help="print per-kernel durations from a rocprofv3 --kernel-trace database (no GPU needed)")
    ap.add_argument("--summarize-counters", metavar="PMC_DB",
                    help="print per-kernel mean counter values from a rocprofv3 --pmc database (no GPU needed)")
    ap.add_argument("--pmc-kernel", default="attn", choices=["attn", "lm_head"])
    ap.add_argument("--pmc-copy-mib", type=int, default=1024)
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.calibrate_counters is not None:
        calibrate_counters(args.calibrate_counters)
        return
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
    if args.prefill:
        bench_prefill(args, cfg)
        return
    t_setup = time.perf_counter()
    run = StepRunner(cfg, select=args.select, k=args.k, boost=args.boost, keep_host=not args.no_cpu_baseline,
                     fused=not args.unfused)
    print(f"# setup {time.perf_counter() - t_setup:.1f} s", file=sys.stderr, flush=True)
    nsched = len(run.step_ids)

    # commits per schedule step (deterministic: the same inputs every pass),
    # and the rows whose confidence clears tau
    run.reset()
    commits = []
    above = cands = 0
    for i in run.step_ids:
        m0 = run.inputs[i].masked.clone().bool()
        run.step(i)
        commits.append(int(run.n_commit.sum()))
        above += int(((run.conf > run.inputs[i].tau[:, None]) & m0).sum())
        cands += int(m0.sum())
    torch.cuda.synchronize()

    # HIP events on the launch stream (torch's current stream, which the
    # binding passes to every call): the LM head + select call on steps
    # j % EV_EVERY == 0, the attention (kernel + split merge) on steps
    # j % EV_EVERY == EV_EVERY // 2
    def do_steps(n, start, ev=None, ev_attn=None):
        pos = start
        for j in range(n):
            if pos == 0:
                run.reset()
            i = run.step_ids[pos]
            inp = run.inputs[i]
            if run.dual and inp.sub_idx == 0:
                run.refresh_block(inp.block_idx)
            t_attn = ev_attn is not None and j % EV_EVERY == EV_EVERY // 2
            if t_attn:
                ev_attn[j // EV_EVERY][0].record()
            run.attention(i)
            if t_attn:
                ev_attn[j // EV_EVERY][1].record()
                ev_attn[j // EV_EVERY][2] = i
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
    ev_attn = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True), None]
               for _ in range(n_ev)]
    start_pos = pos
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    do_steps(args.steps, start_pos, ev, ev_attn)
    t_end.record()
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end)
    ms_per_step = ms / args.steps
    committed = sum(commits[(start_pos + j) % nsched] for j in range(args.steps))
    lm_ms = sum(a.elapsed_time(b) for a, b in ev) / n_ev
    ev_attn = [e for e in ev_attn if e[2] is not None]
    attn_ms = sum(a.elapsed_time(b) for a, b, _ in ev_attn) / len(ev_attn)
    attn_b = 0
    for _, _, i in ev_attn:
        lp = cfg.prompt_len + run.inputs[i].block_idx * cfg.block
        attn_b += attn_bytes(cfg, cfg.cap if run.dual else lp + cfg.block)
    attn_b /= len(ev_attn)

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

    # the attention: HBM-bound at every workload (arithmetic intensity 31-212
    # flop/B, below the bf16 ridge of 312)
    a_ach = attn_b / (attn_ms * 1e-3) / 1e9
    roof_attn = {"bound": "hbm", "achieved": a_ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": a_ach / HBM_PEAK_GBS, "traffic": pmc_traffic(cfg.name, "attn"),
                 "kernel": "fdl_block_attn (block_attn kernel + split merge)", "kernel_us": attn_ms * 1e3,
                 "kernel_calls_timed": len(ev_attn), "algorithmic_bytes": attn_b}
    other = "literal" if args.boost == "calibrated" else "calibrated"
    ex_other, n_other = exceed_tau(run, cfg, other)

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
        "roofline_attention": roof_attn,
        "exceed_tau_fraction": {args.boost: above / max(cands, 1), other: ex_other,
                                "note": f"candidate rows with confidence > tau: {args.boost} over the whole "
                                        f"schedule, {other} over its first {n_other} steps"},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(run, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
