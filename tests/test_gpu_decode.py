"""Decode loop (fdl_decode) against the oracle's loop, step by step.

Both sides start from the same seeded inputs and run independently.  Every
step the device records is compared with the oracle's step of the same index:
block and sub-block, argmax and confidence of every active row, the commit
set (through the block's masked flags) and the block's tokens after the step,
under the parity rules of the single-step tests (decisions within 1e-3 of a
boundary in the oracle's own values are excluded and counted).  If the two
runs ever take different decisions, the differing rows must all be excluded
ones -- the runs have then legitimately forked and the comparison stops there;
otherwise the whole run must agree, including the final tokens, the cache, the
per-sequence step counts and the EOS blocks."""
import dataclasses

import numpy as np
import pytest
import torch

from block_diffusion_decoding_attn_amd import synth
from block_diffusion_decoding_attn_amd.runner import DecodeRunner
from oracle import fdl_decode_oracle as DO
from oracle import fdl_oracle as O
from parity import compare_select, normwise

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}
SELECT = {"threshold": O.SELECT_THRESHOLD, "topk": O.SELECT_TOPK, "factor": O.SELECT_FACTOR}


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _dims(cfg):
    return dict(batch=cfg.batch, prompt_len=cfg.prompt_len, gen_len=cfg.gen_len, block=cfg.block,
                sub_block=cfg.sub_block, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
                head_dim=cfg.head_dim,
                attn_mode=O.DUAL_CACHE if cfg.attn_mode == synth.DUAL_CACHE else O.BLOCK_CAUSAL)


def _oracle(run: DecodeRunner):
    inp = run.inp
    return DO.decode(_dims(run.cfg), run.w_host, inp.prompt.numpy(), inp.boost_tok.numpy(), inp.boost_val.numpy(),
                     inp.tau.numpy(), SELECT[run.select], run.k, run.factor, inp.mask_id, inp.eos_id, inp.gain,
                     run.max_blocks)


def _compare(run: DecodeRunner, got: dict, ref: dict):
    cfg = run.cfg
    S, D = cfg.sub_block, cfg.block
    tol = TOL[cfg.dtype]
    tau = run.inp.tau.numpy()
    gt, rt = got["trace"], ref["trace"]
    assert got["steps"] == len(gt)
    forked = None
    excluded = 0
    prev = None
    for s in range(min(len(gt), len(rt))):
        g, r = gt[s], rt[s]
        assert (g["block"], g["sub"]) == (r["block"], r["sub"]), s
        if prev is None or prev[0] != r["block"]:
            # block start: every position of a sequence still generating is masked
            stopped = (ref["eos_block"] >= 0) & (ref["eos_block"] < r["block"])
            m_before = np.repeat(~stopped[:, None], D, axis=1)
        else:
            m_before = prev[1]
        sl = slice(r["sub"] * S, r["sub"] * S + S)
        cand = m_before[:, sl]
        g_commit = cand & ~g["masked"][:, sl]
        stats = compare_select(dict(conf=r["conf"], p2=r["p2"], token=r["token"], commit=r["commit"],
                                    n_commit=r["commit"].sum(1)),
                               dict(token=g["token"], conf=g["conf"], commit=g_commit, n_commit=g_commit.sum(1)),
                               cand, tau, SELECT[run.select], run.k, run.factor)
        assert normwise(g["conf"], r["conf"]) <= tol, (s, normwise(g["conf"], r["conf"]))
        excluded += stats["token_excluded"] + stats["seq_excluded"] + stats["commit_excluded_rows"]
        same = (np.array_equal(g["masked"], r["masked"]) and np.array_equal(g["tokens"], r["tokens"]))
        if not same:
            assert stats["token_excluded"] + stats["seq_excluded"] + stats["commit_excluded_rows"] > 0, s
            forked = s
            break
        prev = (r["block"], r["masked"])
    if forked is not None:
        print(f"runs forked at step {forked} on an excluded decision (steps compared: {forked + 1})")
        return dict(forked=forked, excluded=excluded)
    assert len(gt) == len(rt)
    np.testing.assert_array_equal(got["tokens"], ref["tokens"])
    assert not got["masked"].any() and not ref["masked"].any()
    np.testing.assert_array_equal(got["eos_block"], ref["eos_block"])
    np.testing.assert_array_equal(got["seq_steps"], ref["seq_steps"])
    np.testing.assert_array_equal(got["length"], ref["length"])
    assert got["blocks_run"] == ref["blocks_run"]
    n = int(ref["length"].min())
    ktol = 1e-6 if cfg.dtype == "f32" else 2.0 ** -8
    assert normwise(got["k_cache"][:, :, :n], ref["k_cache"][:, :, :n]) <= ktol
    assert normwise(got["v_cache"][:, :, :n], ref["v_cache"][:, :, :n]) <= ktol
    return dict(forked=None, excluded=excluded)


def _tiny(**over):
    base = dict(batch=3, gen_len=128, sub_block=8)
    base.update(over)
    return dataclasses.replace(synth.get_config("tiny_fp32"), **base)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decode_tiny_fp32_threshold(seed):
    _need_gpu()
    print(f"decode tiny fp32 threshold seed {seed}", flush=True)
    run = DecodeRunner(_tiny(), seed=seed)
    run.run()
    torch.cuda.synchronize()
    got = run.results()
    ref = _oracle(run)
    res = _compare(run, got, ref)
    assert res["forked"] is None or res["forked"] >= 10
    assert got["steps"] > run.cfg.gen_len // run.cfg.sub_block   # parallel decoding took several steps


@pytest.mark.parametrize("select,k,factor", [("topk", 3, 1.0), ("factor", 0, 1.0)])
def test_decode_tiny_fp32_other_rules(select, k, factor):
    _need_gpu()
    print(f"decode tiny fp32 {select}", flush=True)
    run = DecodeRunner(_tiny(), seed=3, select=select, k=k, factor=factor)
    run.run()
    torch.cuda.synchronize()
    _compare(run, run.results(), _oracle(run))


def test_decode_tiny_fp32_dual_cache():
    _need_gpu()
    print("decode tiny fp32 dual cache", flush=True)
    cfg = _tiny(attn_mode=synth.DUAL_CACHE, batch=2)
    run = DecodeRunner(cfg, seed=4)
    run.run()
    torch.cuda.synchronize()
    _compare(run, run.results(), _oracle(run))


def test_decode_eos_and_padding():
    """Sequence 0 produces EOS in block 0 and sequence 2 in block 2; both get
    padding blocks afterwards while sequence 1 runs to the end."""
    _need_gpu()
    print("decode tiny fp32 eos", flush=True)
    cfg = _tiny()
    inp = synth.decode_inputs(cfg, seed=5, eos=False)
    for b, p in ((0, 3), (2, 70)):
        inp.boost_tok[b, p] = inp.eos_id
        inp.boost_val[b, p] = 60.0
    run = DecodeRunner(cfg, seed=5, inputs=inp)
    run.run()
    torch.cuda.synchronize()
    got = run.results()
    ref = _oracle(run)
    res = _compare(run, got, ref)
    assert res["forked"] is None
    assert list(got["eos_block"]) == [0, -1, 2]
    P, D = cfg.prompt_len, cfg.block
    assert (got["tokens"][0, P + D:] == inp.mask_id).all()
    assert (got["tokens"][2, P + 3 * D:] == inp.mask_id).all()


def test_decode_all_stop_early():
    _need_gpu()
    cfg = _tiny()
    inp = synth.decode_inputs(cfg, seed=6, eos=False)
    for b in range(cfg.batch):
        inp.boost_tok[b, b + 1] = inp.eos_id
        inp.boost_val[b, b + 1] = 60.0
    run = DecodeRunner(cfg, seed=6, inputs=inp)
    run.run()
    torch.cuda.synchronize()
    got = run.results()
    assert got["blocks_run"] == 1
    assert {t["block"] for t in got["trace"]} == {0}
    _compare(run, got, _oracle(run))


def test_decode_rerun_is_identical():
    """The loop reinitializes all of its state: a second run gives the same result."""
    _need_gpu()
    run = DecodeRunner(_tiny(), seed=7)
    run.run()
    first = run.results()
    run.run()
    second = run.results()
    for key in ("tokens", "seq_steps", "eos_block", "length"):
        np.testing.assert_array_equal(first[key], second[key])
    assert first["steps"] == second["steps"]


@pytest.mark.parametrize("select", ["threshold", "factor"])
def test_decode_many_rows_bf16(select):
    """bf16, 9 sequences x 32 rows per step: inside the loop the LM head takes
    its tiled path (more than 64 rows, a partial second row tile) and the
    select its one-workgroup-per-sequence finalize (more than 256 rows)."""
    _need_gpu()
    print(f"decode many rows bf16 {select}", flush=True)
    cfg = _tiny(dtype="bf16", batch=9, gen_len=64, sub_block=32)
    assert cfg.rows == 288
    run = DecodeRunner(cfg, seed=3, select=select, k=4, factor=1.0)
    run.run()
    torch.cuda.synchronize()
    res = _compare(run, run.results(), _oracle(run))
    assert res["forked"] is None or res["forked"] >= 10


@pytest.mark.parametrize("name,max_blocks", [("qwen2.5-1.5b_bs1", 2), ("qwen2.5-7b_bs4", 1),
                                             ("llada-8b_dualcache", 1)])
def test_decode_workload_shapes_bf16(name, max_blocks):
    """Full-size bf16 shapes, the first blocks of the generation."""
    _need_gpu()
    print(f"decode {name} max_blocks {max_blocks}", flush=True)
    cfg = synth.get_config(name)
    run = DecodeRunner(cfg, seed=0, max_blocks=max_blocks)
    run.run()
    torch.cuda.synchronize()
    got = run.results()
    ref = _oracle(run)
    res = _compare(run, got, ref)
    print(f"steps {got['steps']} excluded {res['excluded']} forked {res['forked']}", flush=True)
    # a fork is only allowed at an excluded decision, and not before ten steps
    # have been compared
    assert res["forked"] is None or res["forked"] >= 10, res


def test_decode_graph_replay():
    """The whole generation captured in a HIP graph: every replay, with eager
    work of another run and synchronizations in between, equals the eager run."""
    _need_gpu()
    print("decode graph replay", flush=True)
    cfg = _tiny()
    run = DecodeRunner(cfg, seed=8)
    other = DecodeRunner(cfg, seed=9)
    run.run()
    torch.cuda.synchronize()
    eager = run.results()
    graph = run.capture()
    torch.cuda.synchronize()
    for rep in range(3):
        other.run()                       # eager work between replays
        torch.cuda.synchronize()
        run.tokens.zero_()
        run.masked.fill_(1)
        run.counters.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = run.results()
        for key in ("tokens", "masked", "seq_steps", "eos_block", "length", "k_cache", "v_cache"):
            np.testing.assert_array_equal(got[key], eager[key], err_msg=f"replay {rep}: {key}")
        assert (got["steps"], got["blocks_run"]) == (eager["steps"], eager["blocks_run"])
        for a, b in zip(got["trace"], eager["trace"]):
            np.testing.assert_array_equal(a["tokens"], b["tokens"])
            np.testing.assert_array_equal(a["conf"], b["conf"])
