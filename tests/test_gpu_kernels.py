"""Kernel-by-kernel parity of the HIP path (through the C ABI) against the
CPU oracle on identical seeded inputs: sizes that span several tiles with a
ragged tail, plus the degenerate cases."""
import dataclasses

import numpy as np
import pytest
import torch

from block_diffusion_decoding_attn_amd import fdl, synth
from oracle import fdl_oracle as O
from parity import compare_select, normwise, rowwise

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda")


def _cfg(**kw):
    base = dict(name="case", cfg_id=50, dtype="bf16", batch=2, n_q_heads=14, n_kv_heads=2, head_dim=128,
                prompt_len=100, gen_len=96, block=32, sub_block=8, hidden=512, vocab=1000,
                attn_mode=synth.BLOCK_CAUSAL)
    base.update(kw)
    return synth.Config(**base)


def _attn_case(cfg, block_idx, sub_idx=0, prefix=None, seed=0, oracle=True):
    dev = _dev()
    d = fdl.make_dims(cfg)
    q = synth.queries(cfg, 7 + block_idx, seed)
    kc, vc = synth.kv_cache(cfg, seed)
    kb, vb = synth.block_kv(cfg, block_idx, seed)
    out = torch.empty_like(q, device=dev)
    lse = torch.empty((cfg.batch, cfg.n_q_heads, cfg.sub_block), dtype=torch.float32, device=dev)
    ws = torch.zeros((max(fdl.fdl_block_attn_workspace_size(d), 16),), dtype=torch.uint8, device=dev)
    pl = None if prefix is None else torch.tensor(prefix, dtype=torch.int32, device=dev)
    fdl.fdl_block_attn(d, block_idx, sub_idx, q.to(dev), kc.to(dev), vc.to(dev), pl, kb.to(dev), vb.to(dev),
                       out, lse, ws)
    torch.cuda.synchronize()
    if not oracle:
        return out.float().cpu().numpy(), lse.cpu().numpy(), None, None
    lp = prefix if prefix is not None else [cfg.prompt_len + block_idx * cfg.block] * cfg.batch
    ref_o, ref_l = O.block_attention(q, kc, vc, kb, vb, lp, mode=cfg.attn_mode, total_len=cfg.cap)
    return out.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l


@pytest.mark.parametrize("kw,block_idx,prefix", [
    (dict(), 0, None),                                                   # 132 keys: 3 tiles, ragged
    (dict(), 2, None),                                                   # 196 keys
    (dict(), 1, [0, 131]),                                               # per-sequence prefix, empty prefix
    (dict(n_q_heads=2, n_kv_heads=2, sub_block=32), 0, None),             # MHA, 32 rows
    (dict(n_q_heads=12, n_kv_heads=2, sub_block=8, prompt_len=512, gen_len=256), 7, None),   # 1.5B shapes
    (dict(n_q_heads=28, n_kv_heads=4, sub_block=32, prompt_len=300, gen_len=64), 1, None),   # 224 rows / group
    (dict(head_dim=64), 1, None),
    (dict(attn_mode=synth.DUAL_CACHE, n_q_heads=4, n_kv_heads=4, sub_block=32), 1, None),    # v1 DualCache
    (dict(dtype="f32", n_q_heads=4, n_kv_heads=2, head_dim=64, sub_block=32, prompt_len=96, gen_len=32), 0, None),
    (dict(dtype="f32", n_q_heads=4, n_kv_heads=2, head_dim=64, sub_block=32, prompt_len=70, gen_len=64), 1, [3, 102]),
    (dict(prompt_len=0, gen_len=32, sub_block=32, n_q_heads=2, n_kv_heads=1), 0, None),      # only the block
    (dict(batch=3, prompt_len=2000, gen_len=64), 1, [2000, 5, 2032]),   # many splits, some empty
    # more than 128 rows per KV head: the eight-wave kernel (a padding-only wave when 224 rows)
    (dict(n_q_heads=8, n_kv_heads=1, sub_block=32, prompt_len=0, gen_len=32), 0, None),      # 256 rows, one tile
    (dict(n_q_heads=28, n_kv_heads=4, sub_block=32, prompt_len=64, gen_len=64), 0, None),    # two tiles, one split
    (dict(n_q_heads=16, n_kv_heads=2, sub_block=32, prompt_len=200, gen_len=96), 2, [0, 203]),
    (dict(n_q_heads=20, n_kv_heads=4, sub_block=32, batch=1, prompt_len=1000, gen_len=64), 1, None),  # 160 rows
    (dict(n_q_heads=28, n_kv_heads=4, sub_block=32, batch=8, prompt_len=1440, gen_len=96), 2, None),  # 3-tile splits
    (dict(attn_mode=synth.DUAL_CACHE, n_q_heads=8, n_kv_heads=1, sub_block=32), 1, None),    # DualCache, 256 rows
    # at most 64 rows per KV head, several splits with empty ones, DualCache, d 64
    (dict(n_q_heads=4, n_kv_heads=4, sub_block=32, batch=3, prompt_len=700, gen_len=64), 1, [700, 3, 731]),
    (dict(attn_mode=synth.DUAL_CACHE, n_q_heads=8, n_kv_heads=4, sub_block=32), 1, None),    # DualCache, 64 rows
    (dict(head_dim=64, n_q_heads=2, n_kv_heads=2, sub_block=16), 2, None),                   # d 64, 16 rows
    (dict(n_q_heads=1, n_kv_heads=1, sub_block=8, prompt_len=190, gen_len=64), 0, None),     # 8 rows, 4 tiles
    # 65-128 rows per KV head: the four-wave kernel (all rows live, a padding wave, d 64,
    # DualCache, many splits with the one-wave-per-four-values merge)
    (dict(n_q_heads=4, n_kv_heads=1, sub_block=32), 1, None),                                # 128 rows
    (dict(n_q_heads=6, n_kv_heads=2, sub_block=32), 2, [0, 163]),                            # 96 rows
    (dict(n_q_heads=9, n_kv_heads=1, head_dim=64), 1, None),                                 # 72 rows, d 64
    (dict(attn_mode=synth.DUAL_CACHE, n_q_heads=8, n_kv_heads=2, sub_block=32), 1, None),    # DualCache, 128 rows
    (dict(n_q_heads=6, n_kv_heads=2, sub_block=32, batch=3, prompt_len=700, gen_len=64), 1, [700, 3, 731]),
])
def test_block_attn_parity(kw, block_idx, prefix):
    cfg = _cfg(**kw)
    got_o, got_l, ref_o, ref_l = _attn_case(cfg, block_idx, prefix=prefix)
    tol = TOL[cfg.dtype]
    e_o = normwise(got_o, ref_o)
    rw = rowwise(got_o, ref_o)
    e_l = np.abs(got_l - ref_l).max() / np.abs(ref_l).max()
    print(f"attn {kw} block {block_idx}: tensor {e_o:.2e} per-row {rw}", flush=True)
    assert e_o <= tol, e_o
    assert rw["max"] <= tol, rw
    assert e_l <= (1e-5 if cfg.dtype == "f32" else 1e-3), e_l


def test_block_attn_all_sub_blocks_same_keys():
    """Every sub-block of a block sees the same keys: sub_idx only selects rows."""
    cfg = _cfg()
    a = _attn_case(cfg, 1, sub_idx=0)[0]
    b = _attn_case(cfg, 1, sub_idx=3)[0]
    np.testing.assert_array_equal(a, b)


def test_block_attn_deterministic():
    cfg = _cfg(batch=3, prompt_len=2000, gen_len=64)
    a = _attn_case(cfg, 1)[0]
    b = _attn_case(cfg, 1)[0]
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("kw", [dict(), dict(n_q_heads=8, n_kv_heads=1, sub_block=32),
                                dict(dtype="f32", n_q_heads=4, n_kv_heads=2, head_dim=64, sub_block=32)])
def test_block_attn_prefix_out_of_contract(kw):
    """Per-sequence prefix lengths outside 0 <= Lp <= P + L - D are clamped to
    that range (the header's contract): the result equals the clamped call's,
    bit for bit, and the oracle's at the clamped lengths."""
    cfg = _cfg(**kw)
    hi = cfg.cap - cfg.block
    got_o, got_l, _, _ = _attn_case(cfg, 1, prefix=[-7, 10 ** 6], oracle=False)
    cl_o, cl_l, ref_o, _ = _attn_case(cfg, 1, prefix=[0, hi])
    np.testing.assert_array_equal(got_o, cl_o)
    np.testing.assert_array_equal(got_l, cl_l)
    assert rowwise(got_o, ref_o)["max"] <= TOL[cfg.dtype]


@pytest.mark.parametrize("M,H,V,dtype", [
    (1, 512, 1000, "bf16"), (7, 512, 1003, "bf16"), (16, 256, 4096, "bf16"), (32, 3584, 2048, "bf16"),
    (33, 512, 1000, "bf16"), (64, 1024, 1000, "bf16"), (100, 512, 1000, "bf16"), (300, 512, 1003, "bf16"),
    (32, 256, 512, "f32"), (5, 260, 77, "f32"), (64, 256, 512, "f32"),
    (16, 256, 100003, "bf16"), (32, 128, 152064, "bf16"),     # 79 / 119 vocabulary rows per workgroup
])
def test_lm_head_parity(M, H, V, dtype):
    dev = _dev()
    cfg = _cfg(hidden=H, vocab=V, dtype=dtype)
    d = fdl.make_dims(cfg)
    w = synth.weights(cfg)
    x = synth.normal((M, H), 0, cfg.cfg_id, synth.T_X, M, dtype=cfg.torch_dtype)
    out = torch.empty((M, V), dtype=torch.float32, device=dev)
    fdl.fdl_lm_head(d, x.to(dev), w.to(dev), out)
    torch.cuda.synchronize()
    ref = O.lm_head(x, w)
    e = normwise(out.cpu().numpy(), ref)
    assert e <= (1e-5 if dtype == "f32" else 1e-4), e


def _select_case(B, R, V, masked, tau, mode=O.SELECT_THRESHOLD, k=0, factor=1.0, logits=None, step=0,
                 inout=False):
    dev = _dev()
    cfg = _cfg(batch=B, vocab=V, sub_block=R, block=R, gen_len=R)
    d = fdl.make_dims(cfg)
    lg = synth.logits_direct(B * R, V, step) if logits is None else logits
    m = torch.as_tensor(masked, dtype=torch.uint8).reshape(B, R)
    t = torch.as_tensor(tau, dtype=torch.float32).reshape(B)
    outs = dict(token=torch.empty((B, R), dtype=torch.int32, device=dev),
                conf=torch.empty((B, R), dtype=torch.float32, device=dev),
                commit=torch.empty((B, R), dtype=torch.uint8, device=dev),
                n_commit=torch.empty((B,), dtype=torch.int32, device=dev))
    ws = torch.empty((fdl.fdl_conf_select_workspace_size(d, R),), dtype=torch.uint8, device=dev)
    mdev = m.to(dev)
    toks = torch.full((B, R), -1, dtype=torch.int32, device=dev) if inout else None
    gmode = {O.SELECT_THRESHOLD: 0, O.SELECT_TOPK: 1, O.SELECT_FACTOR: 2}[mode]
    fdl.fdl_conf_select(d, R, lg.to(dev), mdev, t.to(dev), gmode, k, factor, outs["token"], outs["conf"],
                        outs["commit"], outs["n_commit"], toks, mdev if inout else None, ws)
    torch.cuda.synchronize()
    got = {k_: v.cpu().numpy() for k_, v in outs.items()}
    ref = O.conf_select(lg.reshape(B, R, V), m.numpy(), t.numpy(), mode, k, factor)
    extra = (toks.cpu().numpy(), mdev.cpu().numpy()) if inout else None
    return got, ref, m.numpy(), t.numpy(), extra


# finalize variants: up to 256 rows one wave per row; more rows one workgroup per
# sequence (8, 16, 32 or 64 row slots: R = 8, 16, 32, 40); R > 64 the 256-thread per-row kernel
@pytest.mark.parametrize("B,R,V", [(1, 32, 512), (4, 8, 152064), (3, 8, 1003), (2, 256, 4096), (16, 32, 2048),
                                   (1, 1, 2), (5, 3, 100000), (9, 8, 5000), (3, 24, 3001),
                                   (40, 8, 3000), (20, 16, 2000), (9, 40, 777),
                                   (300, 1, 2000), (32, 8, 1500)])   # one row per sequence; exactly 256 rows
@pytest.mark.parametrize("mode", [O.SELECT_THRESHOLD, O.SELECT_TOPK, O.SELECT_FACTOR])
def test_conf_select_parity(B, R, V, mode):
    rng = np.random.default_rng(B * 1000 + R + V)
    masked = (rng.random((B, R)) < 0.7).astype(np.uint8)
    masked[0, 0] = 1
    tau = rng.choice([0.5, 0.7, 0.9, 0.95], B)
    got, ref, m, t, _ = _select_case(B, R, V, masked, tau, mode, k=4, factor=1.5, step=B + R)
    # identical fp32 inputs on both sides: argmax ties resolve identically, so no token exclusions
    np.testing.assert_array_equal(got["token"], ref["token"])
    np.testing.assert_allclose(got["conf"], ref["conf"], rtol=1e-5, atol=0)
    st = compare_select(ref, got, m, t, mode, 4, 1.5, eps=1e-5)
    assert st["seq_checked"] >= 1


def test_conf_select_eq4_worked_example_on_gpu():
    lg = torch.log(torch.tensor([[0.66, 0.34], [0.66, 0.34]], dtype=torch.float32))
    got, ref, *_ = _select_case(1, 2, 2, [[1, 1]], [0.9], logits=lg)
    assert got["token"].tolist() == [[0, 0]]
    assert got["commit"].tolist() == [[1, 0]]          # tie between rows: the lower row
    assert got["n_commit"].tolist() == [1]
    np.testing.assert_allclose(got["conf"], 0.66, rtol=1e-6)


def test_conf_select_ties_and_empty():
    # all-equal rows: argmax 0, conf 1/V; nothing masked in sequence 1 -> no commit
    V = 3000
    lg = torch.zeros((4, V))
    lg[1, 17] = 3.0
    lg[1, 2000] = 3.0                                  # equal maxima: the lower id
    got, ref, m, t, _ = _select_case(2, 2, V, [[1, 1], [0, 0]], [0.9, 0.9], logits=lg)
    assert got["token"].tolist() == [[0, 17], [0, 0]]
    np.testing.assert_allclose(got["conf"][0, 0], 1.0 / V, rtol=1e-6)
    assert got["n_commit"].tolist() == [1, 0]
    assert got["commit"].tolist() == [[0, 1], [0, 0]]


@pytest.mark.parametrize("B,R,V", [(3, 8, 5000), (40, 8, 3000), (2, 96, 1000)])   # the three finalize forms
def test_conf_select_threshold_extremes_and_large_k(B, R, V):
    """tau = 0 commits every candidate (every confidence is at least 1/V);
    tau = 1 commits none by threshold, so exactly the most confident candidate
    of each sequence that has one (the fallback); top-k with k above the
    candidate count commits every candidate."""
    rng = np.random.default_rng(B + R + V)
    masked = (rng.random((B, R)) < 0.6).astype(np.uint8)
    masked[0, :] = 0                                   # a sequence without candidates
    masked[1, 0] = 1
    n_cand = masked.sum(axis=1)
    for tau, mode, k in [(0.0, O.SELECT_THRESHOLD, 0), (1.0, O.SELECT_THRESHOLD, 0), (0.9, O.SELECT_TOPK, R + 3)]:
        got, ref, m, t, _ = _select_case(B, R, V, masked, np.full(B, tau), mode, k=k, step=7)
        np.testing.assert_array_equal(got["token"], ref["token"])
        st = compare_select(ref, got, m, t, mode, k, 1.0, eps=1e-5)
        assert st["seq_checked"] >= 1
        want = np.minimum(n_cand, 1) if tau == 1.0 else n_cand
        assert got["n_commit"].tolist() == want.tolist(), (tau, mode)
        assert (got["commit"].astype(bool) <= masked.astype(bool)).all()


def test_conf_select_inplace_update():
    B, R, V = 3, 8, 5000
    masked = np.ones((B, R), np.uint8)
    masked[1, :4] = 0
    got, ref, m, t, (toks, mnew) = _select_case(B, R, V, masked, [0.9] * B, inout=True, step=3)
    com = got["commit"].astype(bool)
    assert (toks[com] == got["token"][com]).all()
    assert (toks[~com] == -1).all()
    np.testing.assert_array_equal(mnew, masked * (1 - got["commit"]))


def _append_case(cfg, lens, n_new, seed=0):
    dev = _dev()
    d = fdl.make_dims(cfg)
    kc, vc = synth.kv_cache(cfg, seed)
    kn = synth.normal((cfg.batch, cfg.n_kv_heads, n_new, cfg.head_dim), seed, cfg.cfg_id, 40, dtype=cfg.torch_dtype)
    vn = synth.normal((cfg.batch, cfg.n_kv_heads, n_new, cfg.head_dim), seed, cfg.cfg_id, 41, dtype=cfg.torch_dtype)
    ln = torch.tensor(lens, dtype=torch.int32)
    kcd, vcd, lnd = kc.to(dev), vc.to(dev), ln.to(dev)
    fdl.fdl_kv_append(d, kcd, vcd, kn.to(dev), vn.to(dev), lnd)
    torch.cuda.synchronize()
    return kc, vc, kn, vn, ln, kcd.cpu(), vcd.cpu(), lnd.cpu()


@pytest.mark.parametrize("kw,lens,n_new", [
    (dict(), [100, 164], 32),
    (dict(dtype="f32", head_dim=64), [0, 5], 7),
    (dict(), [196 - 32, 196 - 31], 32),            # second sequence would overflow: untouched
    (dict(), [0, 0], 196),                         # refresh: rewrite every position
    (dict(), [-1, 10], 8),                         # negative length: untouched
])
def test_kv_append_bitwise(kw, lens, n_new):
    cfg = _cfg(**kw)
    kc, vc, kn, vn, ln, kg, vg, lg = _append_case(cfg, lens, n_new)
    ref_k, ref_l = kc.clone(), ln.clone()
    ref_v = vc.clone()
    for b in range(cfg.batch):
        lo = int(ln[b])
        if lo < 0 or lo + n_new > cfg.cap:
            continue
        ref_k[b, :, lo:lo + n_new] = kn[b]
        ref_v[b, :, lo:lo + n_new] = vn[b]
        ref_l[b] = lo + n_new
    assert torch.equal(kg.view(torch.int16 if cfg.dtype == "bf16" else torch.int32),
                       ref_k.view(torch.int16 if cfg.dtype == "bf16" else torch.int32))
    assert torch.equal(vg.view(torch.int16 if cfg.dtype == "bf16" else torch.int32),
                       ref_v.view(torch.int16 if cfg.dtype == "bf16" else torch.int32))
    assert lg.tolist() == ref_l.tolist()
    # and the oracle's append agrees where it applies
    ok = [b for b in range(cfg.batch) if 0 <= int(ln[b]) and int(ln[b]) + n_new <= cfg.cap]
    if len(ok) == cfg.batch:
        ok_k, ok_l = O.kv_append(kc.float().numpy(), kn.float().numpy(), ln.numpy())
        np.testing.assert_array_equal(kg.float().numpy(), ok_k)
        assert lg.tolist() == ok_l.tolist()


@pytest.mark.parametrize("kw,pos,n_new,with_len", [
    (dict(), 0, 128, True),                                                  # refresh: every position from 0
    (dict(), 64, 32, True),                                                  # one block at a position
    (dict(dtype="bf16", n_kv_heads=4, head_dim=128, prompt_len=100, gen_len=64, batch=3), 131, 33, False),
    (dict(dtype="bf16", n_kv_heads=1, head_dim=64, prompt_len=0, gen_len=32, batch=2), 0, 32, True),
])
def test_kv_write_bitwise(kw, pos, n_new, with_len):
    cfg = dataclasses.replace(synth.get_config("tiny_fp32"), **kw)
    dev = _dev()
    d = fdl.make_dims(cfg)
    kc, vc = synth.kv_cache(cfg, 0)
    kn = synth.normal((cfg.batch, cfg.n_kv_heads, n_new, cfg.head_dim), 0, cfg.cfg_id, 42, dtype=cfg.torch_dtype)
    vn = synth.normal((cfg.batch, cfg.n_kv_heads, n_new, cfg.head_dim), 0, cfg.cfg_id, 43, dtype=cfg.torch_dtype)
    lnd = torch.full((cfg.batch,), -7, dtype=torch.int32, device=dev)
    kcd, vcd = kc.to(dev), vc.to(dev)
    fdl.fdl_kv_write(d, kcd, vcd, kn.to(dev), vn.to(dev), pos, lnd if with_len else None)
    torch.cuda.synchronize()
    bits = torch.int16 if cfg.torch_dtype == torch.bfloat16 else torch.int32
    for got, cache, new in ((kcd, kc, kn), (vcd, vc, vn)):
        ref, ref_len = O.kv_write(cache.view(bits).numpy(), new.view(bits).numpy(), pos)
        np.testing.assert_array_equal(got.cpu().view(bits).numpy(), ref)
    assert lnd.cpu().tolist() == (ref_len.tolist() if with_len else [-7] * cfg.batch)


@pytest.mark.parametrize("B,R,H,V,dtype,mode", [
    (4, 8, 512, 1000, "bf16", O.SELECT_THRESHOLD),      # V not a multiple of the 128-row tile
    (1, 8, 256, 4096, "bf16", O.SELECT_TOPK),
    (2, 32, 512, 2003, "bf16", O.SELECT_FACTOR),        # M = 64
    (5, 32, 256, 1000, "bf16", O.SELECT_THRESHOLD),     # M = 160: tiled kernel
    (1, 32, 256, 512, "f32", O.SELECT_THRESHOLD),
    (2, 8, 260, 77, "f32", O.SELECT_TOPK),
    # large vocabularies, up to 32 rows: all workgroups resident, 64-128 rows each
    (2, 8, 256, 100003, "bf16", O.SELECT_THRESHOLD),    # 79 rows per workgroup, ragged last
    (4, 8, 128, 152064, "bf16", O.SELECT_TOPK),         # the Qwen2.5 vocabulary: 119 rows each
    (1, 32, 192, 126464, "bf16", O.SELECT_FACTOR),      # the LLaDA vocabulary: 99 rows each
])
def test_lm_head_select_parity(B, R, H, V, dtype, mode):
    """Fused LM head + select against the oracle (logits in fp64, select on
    them) and against the unfused GPU path on the same inputs."""
    dev = _dev()
    cfg = _cfg(batch=B, sub_block=R, block=R, gen_len=R, hidden=H, vocab=V, dtype=dtype)
    d = fdl.make_dims(cfg)
    w = synth.weights(cfg)
    x, _, _ = synth.hidden_rows(cfg, w, 3)
    rng = np.random.default_rng(B * R + V)
    masked = torch.as_tensor((rng.random((B, R)) < 0.8).astype(np.uint8))
    masked[0, 0] = 1
    tau = torch.as_tensor(rng.choice([0.5, 0.7, 0.9], B).astype(np.float32))
    gmode = {O.SELECT_THRESHOLD: 0, O.SELECT_TOPK: 1, O.SELECT_FACTOR: 2}[mode]

    def outs():
        return dict(token=torch.empty((B, R), dtype=torch.int32, device=dev),
                    conf=torch.empty((B, R), dtype=torch.float32, device=dev),
                    commit=torch.empty((B, R), dtype=torch.uint8, device=dev),
                    n_commit=torch.empty((B,), dtype=torch.int32, device=dev))
    xd, wd, md, td = x.to(dev), w.to(dev), masked.to(dev), tau.to(dev)
    fused, unfused = outs(), outs()
    lg_f = torch.empty((B * R, V), dtype=torch.float32, device=dev)
    lg_u = torch.empty((B * R, V), dtype=torch.float32, device=dev)
    ws = torch.empty((fdl.fdl_lm_head_select_workspace_size(d, R),), dtype=torch.uint8, device=dev)
    fdl.fdl_lm_head_select(d, R, xd, wd, lg_f, md, td, gmode, 3, 1.5, fused["token"], fused["conf"],
                           fused["commit"], fused["n_commit"], None, None, ws)
    fused2 = outs()
    fdl.fdl_lm_head_select(d, R, xd, wd, None, md, td, gmode, 3, 1.5, fused2["token"], fused2["conf"],
                           fused2["commit"], fused2["n_commit"], None, None, ws)
    fdl.fdl_lm_head(d, xd, wd, lg_u)
    ws2 = torch.empty((fdl.fdl_conf_select_workspace_size(d, R),), dtype=torch.uint8, device=dev)
    fdl.fdl_conf_select(d, R, lg_u, md, td, gmode, 3, 1.5, unfused["token"], unfused["conf"], unfused["commit"],
                        unfused["n_commit"], None, None, ws2)
    torch.cuda.synchronize()
    # logits written by the fused call are the LM head's, bit for bit
    assert torch.equal(lg_f, lg_u)
    got = {k_: v.cpu().numpy() for k_, v in fused.items()}
    got2 = {k_: v.cpu().numpy() for k_, v in fused2.items()}
    for k_ in got:
        np.testing.assert_array_equal(got[k_], got2[k_])       # writing logits or not changes nothing
    gu = {k_: v.cpu().numpy() for k_, v in unfused.items()}
    np.testing.assert_array_equal(got["token"], gu["token"])   # same fp32 logits: same argmax
    np.testing.assert_allclose(got["conf"], gu["conf"], rtol=1e-5)
    ref_logits = O.lm_head(x, w)
    assert normwise(lg_f.cpu().numpy(), ref_logits) <= (1e-5 if dtype == "f32" else 1e-4)
    ref = O.conf_select(ref_logits.reshape(B, R, V), masked.numpy(), tau.numpy(), mode, 3, 1.5)
    st = compare_select(ref, got, masked.numpy(), tau.numpy(), mode, 3, 1.5, eps=1e-3)
    assert st["seq_checked"] + st["seq_excluded"] == B


@pytest.mark.parametrize("kw,q_start,n_q,n_keys,causal", [
    (dict(), 0, 196, 196, True),                    # prompt prefill of a whole ragged sequence
    (dict(), 64, 70, 160, True),                    # a window of positions, keys past the window
    (dict(n_q_heads=4, n_kv_heads=4), 0, 196, 196, False),   # v1 refresh: all keys visible
    (dict(head_dim=64, block=16, sub_block=16), 5, 40, 100, True),
    (dict(n_q_heads=28, n_kv_heads=4), 100, 33, 140, True),
    (dict(), 0, 20, 20, True),                      # fewer keys than one tile
    (dict(n_q_heads=2, n_kv_heads=1), 0, 64, 64, False),     # exactly one full tile, GQA
    (dict(), 0, 1, 1, True),                        # one query, one key
    (dict(), 37, 1, 196, False),                    # one query over every key
    (dict(), 150, 8, 100, True),                    # queries past the last key: each sees all of them
])
def test_prefill_attn_parity(kw, q_start, n_q, n_keys, causal):
    dev = _dev()
    cfg = _cfg(**kw)
    d = fdl.make_dims(cfg)
    q = synth.normal((cfg.batch, n_q, cfg.n_q_heads, cfg.head_dim), 0, cfg.cfg_id, 30, n_q, dtype=cfg.torch_dtype)
    k, v = synth.kv_cache(cfg)
    out = torch.empty_like(q, device=dev)
    lse = torch.empty((cfg.batch, cfg.n_q_heads, n_q), dtype=torch.float32, device=dev)
    fdl.fdl_prefill_attn(d, q_start, n_keys, causal, q.to(dev), k.to(dev), v.to(dev), out, lse)
    torch.cuda.synchronize()
    ref_o, ref_l = O.prefill_attention(q, k, v, q_start, n_keys, cfg.block, causal)
    got = out.float().cpu().numpy()
    rw = rowwise(got, ref_o)
    print(f"prefill {kw} q {q_start}+{n_q} keys {n_keys} causal {causal}: per-row {rw}", flush=True)
    assert normwise(got, ref_o) <= 2e-2
    assert rw["max"] <= 2e-2, rw
    assert np.abs(lse.cpu().numpy() - ref_l).max() <= 1e-3 * np.abs(ref_l).max()
