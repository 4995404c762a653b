"""Workload-level parity: whole denoising steps of every workload, run through
the C ABI in the launch configuration the benchmark times, against the oracle.
Full sizes; the oracle evaluates sampled sequences / KV groups / vocab
columns, each one in full."""
import numpy as np
import pytest
import torch

from block_diffusion_decoding_attn_amd import synth
from block_diffusion_decoding_attn_amd.runner import StepRunner
from oracle import fdl_oracle as O
from parity import compare_select, normwise, rowwise

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _oracle_logits(x, w, chunk=16384):
    """Oracle logits of rows x over the whole vocabulary, evaluated per vocab slice."""
    parts = [O.lm_head(x, w[v0:v0 + chunk]) for v0 in range(0, w.shape[0], chunk)]
    return np.concatenate(parts, axis=1)


def _host_cache_at_block(cfg, b, seed=0):
    """Cache contents before block b: prompt K/V, then the K/V of blocks 0..b-1."""
    kc, vc = synth.kv_cache(cfg, seed, fill=cfg.prompt_len)
    for bb in range(b):
        kb, vb = synth.block_kv(cfg, bb, seed)
        lo = cfg.prompt_len + bb * cfg.block
        kc[:, :, lo:lo + cfg.block] = kb
        vc[:, :, lo:lo + cfg.block] = vb
    return kc, vc


def _check_step(run: StepRunner, i: int, seqs, groups, vocab_sample=2048, select="threshold", k=4, factor=1.0):
    cfg = run.cfg
    inp = run.host_inputs[i]
    b = inp.block_idx
    dual = cfg.attn_mode == synth.DUAL_CACHE
    if dual:
        kc, vc = run.refresh[b][2]
    else:
        kc, vc = _host_cache_at_block(cfg, b, run.seed)
        run.k_cache.copy_(kc)
        run.v_cache.copy_(vc)
        run.len.fill_(cfg.prompt_len + b * cfg.block)
    run.step(i)
    torch.cuda.synchronize()
    tol = TOL[cfg.dtype]
    G = cfg.n_q_heads // cfg.n_kv_heads
    kb, vb = run.kb_host[b]
    out = run.out.float().cpu().numpy()
    lse = run.lse.cpu().numpy()
    lp = cfg.prompt_len + b * cfg.block
    # attention: sampled (sequence, KV group) pairs, every row of the group
    for s in seqs:
        for g in groups:
            hs = slice(g * G, (g + 1) * G)
            ref_o, ref_l = O.block_attention(inp.q[s:s + 1, :, hs], kc[s:s + 1, g:g + 1], vc[s:s + 1, g:g + 1],
                                             kb[s:s + 1, g:g + 1], vb[s:s + 1, g:g + 1], [lp],
                                             mode=cfg.attn_mode, total_len=cfg.cap)
            e = normwise(out[s:s + 1, :, hs], ref_o)
            rw = rowwise(out[s:s + 1, :, hs], ref_o)
            assert e <= tol, ("attn", s, g, e)
            assert rw["max"] <= tol, ("attn per row", s, g, rw)
            assert np.abs(lse[s:s + 1, hs] - ref_l).max() <= 1e-3 * np.abs(ref_l).max()
    # LM head: sampled vocab columns of every row
    logits = run.logits.cpu().numpy()
    rng = np.random.default_rng(i)
    cols = rng.choice(cfg.vocab, size=min(vocab_sample, cfg.vocab), replace=False)
    ref_cols = O.lm_head(inp.x, run.w_host[torch.as_tensor(cols)])
    e = normwise(logits[:, cols], ref_cols)
    assert e <= (1e-5 if cfg.dtype == "f32" else 1e-4), ("lm_head", e)
    # select: sampled sequences, from the oracle's own full logits rows
    S = cfg.sub_block
    rows = np.concatenate([np.arange(s * S, (s + 1) * S) for s in seqs])
    ref_logits = _oracle_logits(inp.x[torch.as_tensor(rows)], run.w_host)
    masked0 = inp.masked.numpy()[seqs]
    tau = inp.tau.numpy()[seqs]
    mode = {"threshold": O.SELECT_THRESHOLD, "topk": O.SELECT_TOPK, "factor": O.SELECT_FACTOR}[select]
    ref = O.conf_select(ref_logits.reshape(len(seqs), S, cfg.vocab), masked0, tau, mode, k, factor)
    got = dict(token=run.token.cpu().numpy()[seqs], conf=run.conf.cpu().numpy()[seqs],
               commit=run.commit.cpu().numpy()[seqs], n_commit=run.n_commit.cpu().numpy()[seqs])
    st = compare_select(ref, got, masked0, tau, mode, k, factor, eps=1e-3)
    np.testing.assert_allclose(got["conf"], ref["conf"], rtol=2e-3, atol=1e-6)
    # commit-state update: committed rows left the masked set and carry their token
    new_mask = run.masked_all[run.step_ids.index(i)].cpu().numpy()[seqs]
    np.testing.assert_array_equal(new_mask, masked0 * (1 - got["commit"]))
    toks = run.tokens.cpu().numpy()[seqs]
    com = got["commit"].astype(bool)
    assert (toks[com] == got["token"][com]).all()
    # append after the block's last sub-block: the block's K/V now sit in the cache
    if inp.append_after and not dual:
        lo = lp
        bits = torch.int16 if cfg.dtype == "bf16" else torch.int32
        assert torch.equal(run.k_cache[:, :, lo:lo + cfg.block].cpu().view(bits), kb.view(bits))
        assert torch.equal(run.v_cache[:, :, lo:lo + cfg.block].cpu().view(bits), vb.view(bits))
        assert run.len.cpu().tolist() == [lo + cfg.block] * cfg.batch
    return st


def test_tiny_fp32_step_exact_sizes():
    _need_gpu()
    cfg = synth.get_config("tiny_fp32")
    run = StepRunner(cfg, keep_host=True, write_logits=True)
    st = _check_step(run, 0, seqs=[0], groups=[0, 1], vocab_sample=512)
    assert st["seq_checked"] == 1
    # whole attention output and logits at this size
    inp = run.host_inputs[0]
    kc, vc = _host_cache_at_block(cfg, 0)
    kb, vb = run.kb_host[0]
    ref_o, _ = O.block_attention(inp.q, kc, vc, kb, vb, [cfg.prompt_len])
    # the step appended block 0; attention ran before that, so compare against the pre-append cache
    assert normwise(run.out.cpu().numpy(), ref_o) <= 1e-5


@pytest.mark.parametrize("name,steps,seqs,groups,select,fused,boost", [
    ("qwen2.5-1.5b_bs1", [0, 3, 31], [0], [0, 1], "threshold", True, "calibrated"),
    ("qwen2.5-7b_bs4", [0, 63], [0, 3], [0, 3], "threshold", True, "calibrated"),
    ("qwen2.5-7b_bs4", [2, 3], [1, 2], [1, 2], "threshold", False, "calibrated"),
    ("qwen2.5-7b_bs4", [5], [1, 2], [1], "topk", True, "calibrated"),
    ("llada-8b_dualcache", [0, 31], [0], [0, 17, 31], "threshold", True, "calibrated"),
    ("qwen2.5-7b_long_bs16", [0], [0, 9], [0, 2], "threshold", True, "calibrated"),
    ("qwen2.5-7b_long_bs16", [0], [3, 12], [3], "threshold", False, "calibrated"),
    ("qwen2.5-7b_long_bs16", [0], [4], [1], "factor", True, "calibrated"),
    # the boost exactly as the workloads state it, U(0,12): at V ~ 126k-152k
    # no position clears tau = 0.9, so every sequence commits by the fallback
    ("qwen2.5-1.5b_bs1", [0, 5, 31], [0], [1], "threshold", True, "literal"),
    ("qwen2.5-7b_bs4", [0, 1], [0, 1, 2, 3], [2], "threshold", True, "literal"),
    ("llada-8b_dualcache", [0, 7], [0], [5], "threshold", True, "literal"),
])
def test_workload_step_parity(name, steps, seqs, groups, select, fused, boost):
    _need_gpu()
    cfg = synth.get_config(name)
    run = StepRunner(cfg, steps=steps, keep_host=True, select=select, k=4, factor=1.0, fused=fused,
                     write_logits=True, boost=boost)
    total = dict(seq_checked=0, seq_excluded=0, token_checked=0, token_excluded=0, commit_excluded_rows=0)
    exceed = 0
    for i in steps:
        st = _check_step(run, i, seqs, groups, select=select, k=4, factor=1.0)
        for key in total:
            total[key] += st[key]
        conf = run.conf.cpu().numpy()[seqs]
        exceed += int((conf > run.host_inputs[i].tau.numpy()[seqs][:, None]).sum())
        if boost == "literal":
            # every checked sequence commits exactly one position (the fallback)
            assert (run.n_commit.cpu().numpy()[seqs] == 1).all()
    print(name, select, "fused" if fused else "unfused", boost, total, "rows above tau", exceed, flush=True)
    assert total["seq_checked"] >= 1
    assert total["token_checked"] >= 1


@pytest.mark.parametrize("name,causal", [("llada-8b_dualcache", False), ("qwen2.5-7b_bs4", True)])
def test_prefill_full_size_sampled(name, causal):
    """Full-size multi-block attention: the v1 refresh over all P + L positions
    (bidirectional) and the 7B prompt prefill (block-causal); the oracle
    evaluates sampled heads and position windows in full."""
    _need_gpu()
    from block_diffusion_decoding_attn_amd import fdl
    cfg = synth.get_config(name)
    d = fdl.make_dims(cfg)
    dev = torch.device("cuda")
    n = cfg.cap if not causal else cfg.prompt_len
    k, v = synth.kv_cache(cfg)
    q = synth.normal((cfg.batch, n, cfg.n_q_heads, cfg.head_dim), 0, cfg.cfg_id, 31, dtype=cfg.torch_dtype)
    out = torch.empty_like(q, device=dev)
    fdl.fdl_prefill_attn(d, 0, n, causal, q.to(dev), k.to(dev), v.to(dev), out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    G = cfg.n_q_heads // cfg.n_kv_heads
    for b, h, p0 in [(0, 0, 0), (cfg.batch - 1, cfg.n_q_heads - 1, n - 16), (0, cfg.n_q_heads // 2, n // 2 + 3)]:
        g = h // G
        ref, _ = O.prefill_attention(q[b:b + 1, p0:p0 + 16, h:h + 1], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1],
                                     p0, n, cfg.block, causal)
        assert normwise(got[b:b + 1, p0:p0 + 16, h:h + 1], ref) <= 2e-2, (b, h, p0)
