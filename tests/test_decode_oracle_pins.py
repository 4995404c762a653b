"""Pins for the decode-loop oracle (oracle/fdl_decode_oracle.py): every step
it records must equal a full recomputation of the stand-in model over the
whole token sequence (no cache), its bookkeeping must follow the commit rule
and the block/EOS rules, and its special cases must reduce to closed forms.
CPU only."""
import math

import numpy as np
import pytest

from oracle import fdl_decode_oracle as D
from oracle import fdl_oracle as O

# a small stand-in model: hidden = n_q_heads * head_dim; the prompt fills whole
# blocks, as in every workload, so that block boundaries of the M_BC mask over
# absolute positions coincide with the generated blocks
DIMS = dict(batch=3, prompt_len=16, gen_len=48, block=16, sub_block=4, n_q_heads=4, n_kv_heads=2, head_dim=8)
H, V = 32, 64
MASK_ID, EOS_ID = V - 1, V - 2


def _w(seed=0):
    r = np.random.default_rng(1000 + seed)
    return r.standard_normal((V, H)) / math.sqrt(H)


def _inputs(seed=0, dims=DIMS, eos_at=None, boost_hi=12.0):
    r = np.random.default_rng(2000 + seed)
    B, P, L = dims["batch"], dims["prompt_len"], dims["gen_len"]
    prompt = r.integers(0, V - 2, (B, P))
    tok = r.integers(0, V - 2, (B, L))
    val = r.uniform(0.0, boost_hi, (B, L))
    if eos_at is not None:
        for b, p in enumerate(eos_at):
            if p is not None:
                tok[b, p] = EOS_ID
                val[b, p] = 60.0        # certain: committed at the first step that sees it
    return prompt, tok, val


def _run(seed=0, tau=0.9, mode=O.SELECT_THRESHOLD, k=0, factor=1.0, gain=2.0, dims=DIMS, eos_at=None,
         max_blocks=0):
    w = _w(seed)
    prompt, tok, val = _inputs(seed, dims, eos_at)
    taus = np.full(dims["batch"], tau)
    res = D.decode(dims, w, prompt, tok, val, taus, mode, k, factor, MASK_ID, EOS_ID, gain, max_blocks)
    return w, prompt, tok, val, taus, res


# ----------------------------------------------------------------------------
# D-1  every recorded step == full recomputation over the token sequence
# ----------------------------------------------------------------------------

def _dense_step(w, dims, seq, rows_abs, tok, val, gain, causal):
    """Recompute one step from scratch: embed every position of the sequence,
    attend with the block-causal mask M_BC (or no mask: v1) over the whole
    sequence, build the hidden rows, project, take argmax and confidence."""
    Hq, Hkv, d, blk = dims["n_q_heads"], dims["n_kv_heads"], dims["head_dim"], dims["block"]
    n = seq.shape[0]
    e = math.sqrt(H) * w[seq]                               # [n][H]
    q_all = e.reshape(n, Hq, d)
    k_all = e[:, : Hkv * d].reshape(n, Hkv, d)
    v_all = e[:, H - Hkv * d:].reshape(n, Hkv, d)[:, :, ::-1]
    G = Hq // Hkv
    out = np.zeros((len(rows_abs), Hq, d))
    for h in range(Hq):
        g = h // G
        mask = np.array([[(not causal) or O.block_of(j, blk) <= O.block_of(p, blk) for j in range(n)]
                         for p in rows_abs])
        out[:, h] = O.dense_masked_attention(q_all[rows_abs, h], k_all[:, g], v_all[:, g], mask)
    toks, confs = [], []
    for i, p in enumerate(rows_abs):
        wt = w[tok[i]]
        x = gain * out[i].reshape(-1) + val[i] * wt / (wt @ wt)
        logits = w @ x
        t, c, _ = O.row_confidence(logits)
        toks.append(t)
        confs.append(c)
    return np.array(toks), np.array(confs)


def _replay(w, dims, tok, val, res, gain, causal=True):
    B, P, Dk, S = dims["batch"], dims["prompt_len"], dims["block"], dims["sub_block"]
    final = res["tokens"]
    prev_blk, prev = -1, None
    for st in res["trace"]:
        blk, sub = st["block"], st["sub"]
        base = P + blk * Dk
        pre = np.full((B, Dk), MASK_ID) if blk != prev_blk else prev
        for b in range(B):
            seq = final[b].copy()
            seq[base:base + Dk] = pre[b]
            seq[base + Dk:] = MASK_ID
            r0 = blk * Dk + sub * S
            rows_abs = np.arange(P + r0, P + r0 + S)
            t, c = _dense_step(w, dims, seq, rows_abs, tok[b, r0:r0 + S], val[b, r0:r0 + S], gain, causal)
            np.testing.assert_array_equal(st["token"][b], t)
            np.testing.assert_allclose(st["conf"][b], c, rtol=1e-10, atol=0)
        prev_blk, prev = blk, st["tokens"]


@pytest.mark.parametrize("seed,tau", [(0, 0.9), (1, 0.5)])
def test_d1_steps_equal_full_recomputation(seed, tau):
    w, _, tok, val, _, res = _run(seed, tau)
    assert len(res["trace"]) > 10
    _replay(w, DIMS, tok, val, res, 2.0)


def test_d1_dual_cache_steps_equal_full_bidirectional_recomputation():
    dims = dict(DIMS, attn_mode=O.DUAL_CACHE, batch=2)
    w, _, tok, val, _, res = _run(3, 0.9, dims=dims, max_blocks=2)
    _replay(w, dims, tok, val, res, 2.0, causal=False)


# ----------------------------------------------------------------------------
# D-2  bookkeeping of every step follows the commit rule
# ----------------------------------------------------------------------------

def test_d2_step_bookkeeping():
    w, _, _, _, taus, res = _run(4, 0.9)
    Dk, S = DIMS["block"], DIMS["sub_block"]
    prev_blk, pm, pt = -1, None, None
    for st in res["trace"]:
        blk, sub = st["block"], st["sub"]
        if blk != prev_blk:
            pm = np.ones((DIMS["batch"], Dk), dtype=bool)
            pt = np.full((DIMS["batch"], Dk), MASK_ID)
        sl = slice(sub * S, sub * S + S)
        cand = pm[:, sl]
        for b in range(DIMS["batch"]):
            c = st["commit"][b]
            assert not (c & ~cand[b]).any(), "committed a row that was not masked"
            assert st["live"][b] == cand[b].any()
            if cand[b].any():
                above = cand[b] & (st["conf"][b] > taus[b])
                if above.any():
                    np.testing.assert_array_equal(c, above)
                else:                         # fallback: exactly the most confident candidate
                    assert c.sum() == 1
                    best = max(np.flatnonzero(cand[b]), key=lambda r: (st["conf"][b][r], -r))
                    assert c[best]
            else:
                assert not c.any()
        exp_m = pm.copy()
        exp_m[:, sl] &= ~st["commit"]
        np.testing.assert_array_equal(st["masked"], exp_m)
        exp_t = pt.copy()
        exp_t[:, sl] = np.where(st["commit"], st["token"], pt[:, sl])
        np.testing.assert_array_equal(st["tokens"], exp_t)
        prev_blk, pm, pt = blk, st["masked"], st["tokens"]
    assert not res["masked"].any()


# ----------------------------------------------------------------------------
# D-3 / D-4 / D-7  step counts in the special cases
# ----------------------------------------------------------------------------

def _steps_per_sub(res):
    out = {}
    for st in res["trace"]:
        out[(st["block"], st["sub"])] = out.get((st["block"], st["sub"]), 0) + 1
    return out


def test_d3_tau_one_commits_one_row_per_step():
    """tau = 1 disables parallel decoding ([v2] Level 2): no confidence exceeds
    1, so every step commits the single most confident masked row."""
    _, _, _, _, _, res = _run(5, 1.0)
    for st in res["trace"]:
        np.testing.assert_array_equal(st["commit"].sum(1), st["live"].astype(int))
    assert set(_steps_per_sub(res).values()) == {DIMS["sub_block"]}


def test_d4_tau_zero_commits_whole_sub_block():
    _, _, _, _, _, res = _run(6, 0.0)
    n_sub = DIMS["gen_len"] // DIMS["sub_block"]
    assert len(res["trace"]) == n_sub
    assert all(st["commit"].all() for st in res["trace"])


def test_d7_topk_step_count():
    k = 3
    _, _, _, _, _, res = _run(7, mode=O.SELECT_TOPK, k=k)
    assert set(_steps_per_sub(res).values()) == {math.ceil(DIMS["sub_block"] / k)}
    for st in res["trace"]:
        assert set(st["commit"].sum(1)) <= {0, k, DIMS["sub_block"] % k}


# ----------------------------------------------------------------------------
# D-5  EOS stops a sequence; the batch runs until every sequence stops
# ----------------------------------------------------------------------------

def test_d5_eos_stops_sequence_and_pads_the_rest():
    _, _, _, _, _, res = _run(8, eos_at=[5, None, 20])     # blocks 0 and 1
    assert list(res["eos_block"]) == [0, -1, 1]
    assert res["blocks_run"] == DIMS["gen_len"] // DIMS["block"]
    P, Dk = DIMS["prompt_len"], DIMS["block"]
    for st in res["trace"]:
        if st["block"] >= 1:
            assert not st["live"][0] and not st["commit"][0].any()
        if st["block"] >= 2:
            assert not st["live"][2]
    assert (res["tokens"][0, P + Dk:] == MASK_ID).all()
    assert (res["tokens"][2, P + 2 * Dk:] == MASK_ID).all()
    assert res["tokens"][0, P + 5] == EOS_ID


def test_d5_all_sequences_stop():
    _, _, _, _, _, res = _run(9, eos_at=[1, 2, 3])
    assert res["blocks_run"] == 1
    assert {st["block"] for st in res["trace"]} == {0}
    assert list(res["eos_block"]) == [0, 0, 0]


def test_d5_max_blocks():
    _, _, _, _, _, res = _run(10, max_blocks=2)
    assert res["blocks_run"] == 2
    assert list(res["length"]) == [DIMS["prompt_len"] + 2 * DIMS["block"]] * DIMS["batch"]


# ----------------------------------------------------------------------------
# D-6  the block-level cache is exact ([v2] Level 3)
# ----------------------------------------------------------------------------

def test_d6_cache_equals_embedding_of_final_tokens():
    w, _, _, _, _, res = _run(11)
    Hkv, d = DIMS["n_kv_heads"], DIMS["head_dim"]
    assert list(res["length"]) == [DIMS["prompt_len"] + DIMS["gen_len"]] * DIMS["batch"]
    for b in range(DIMS["batch"]):
        for p in range(int(res["length"][b])):
            e = math.sqrt(H) * w[res["tokens"][b, p]]
            np.testing.assert_array_equal(res["k_cache"][b, :, p], e[: Hkv * d].reshape(Hkv, d))
            np.testing.assert_array_equal(res["v_cache"][b, :, p], e[H - Hkv * d:].reshape(Hkv, d)[:, ::-1])


# ----------------------------------------------------------------------------
# D-8  the stand-in model's closed forms
# ----------------------------------------------------------------------------

def test_d8_stand_in_model_closed_forms():
    w = _w(12)
    Hq, Hkv, d = DIMS["n_q_heads"], DIMS["n_kv_heads"], DIMS["head_dim"]
    q, k, v = D.sm_embed(w, 7, Hq, Hkv, d)
    e = math.sqrt(H) * w[7]
    np.testing.assert_array_equal(q.reshape(-1), e)
    np.testing.assert_array_equal(k[1], e[d:2 * d])
    np.testing.assert_array_equal(v[0], e[H - 2 * d:H - d][::-1])
    np.testing.assert_array_equal(v[1, 0], e[H - 1])
    o = np.random.default_rng(3).standard_normal((Hq, d))
    x0 = D.sm_hidden(o, w, 9, 5.5, 0.0)
    assert abs(w[9] @ x0 - 5.5) < 1e-12                  # the boost raises logit 9 by exactly beta
    x1 = D.sm_hidden(o, w, 9, 5.5, 2.0)
    np.testing.assert_allclose(x1 - x0, 2.0 * o.reshape(-1), rtol=0, atol=1e-14)
