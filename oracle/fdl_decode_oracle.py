"""CPU fp64 oracle of the block-diffusion decode loop (generation of whole
blocks, step after step, until every position is committed or EOS appears).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module.  It shares no code with
the HIP library and must never serve as a fallback for it.

The loop follows "Fast-dLLM v2: Efficient Block-Diffusion LLM" (technical
breakdown), Inference Pipeline:
  Level 1  blocks are generated left to right; each starts fully masked, is
           refined until no position is masked, then its K/V enter the
           block-level cache; generation stops once a completed block holds
           EOS, or after a maximum number of blocks.
  Level 2  inside a block, every step predicts all masked positions and
           commits by the confidence rule; the block is decoded sub-block by
           sub-block ("Sub-block size as a decoding granularity knob").
  Level 3  the block-level cache is exact: cached K/V equal those a full
           recomputation would give.
  "Batch decoding with length padding": all sequences of a batch advance
           together; a sequence that has produced EOS keeps running through
           the same operations, its remaining blocks being padding.
and, for the v1 DualCache variant, "Fast-dLLM: Reusing Bidirectional State
...", section 3 and Algorithm 1 (the cache is refreshed once per block and the
active block also attends to the cached suffix).

Synthetic model.  The pages' transformer is replaced by a stand-in whose
every input to the step is a function of the current tokens, so that the
loop's control flow depends on what it commits:
  * token embedding  e(t) = sqrt(H) * W[t]  (tied to the LM-head weight
    W[V][H]; H = Hq * d);
  * query of head h  = e(t)[h d : (h+1) d];
    key of KV head g = e(t)[g d : (g+1) d];
    value of KV head g = e(t)[H - (Hkv-g) d : H - (Hkv-g-1) d] in reverse
    order (so that no head's output lines up with its own value slice, which
    would make the stand-in copy attended tokens with certainty);
    (K/V depend on the token only, so cached K/V of a fixed token are exact);
  * hidden row of an active position p = gain * (attention output of p,
    heads concatenated) + beta_p * W[t_p] / |W[t_p]|^2, which raises the
    logit of the drawn token t_p by exactly beta_p (the peaking boost of the
    single-step workloads);
  * row i of the active sub-block predicts its own position (the one-position
    shift of the v2 pages is a property of the trained model's rows, which
    this stand-in does not have).
Reading of the pages used here (each listed in the design notes):
  * a sequence that has produced EOS gets padding blocks: their positions are
    MASK tokens that are never candidates, so they commit nothing and never
    hold the batch back;
  * every step of a sub-block runs while any sequence of the batch still has
    a masked position in it; a sequence without one commits nothing.
"""
from __future__ import annotations

import math
from typing import Dict, List

import numpy as np

from . import fdl_oracle as O


# ----------------------------------------------------------------------------
# The synthetic model
# ----------------------------------------------------------------------------

def sm_embed(w64: np.ndarray, token: int, n_q_heads: int, n_kv_heads: int, head_dim: int):
    """(q [Hq][d], k [Hkv][d], v [Hkv][d]) of one token under the stand-in model."""
    H = w64.shape[1]
    e = math.sqrt(H) * w64[token]
    q = e.reshape(n_q_heads, head_dim)
    k = e[: n_kv_heads * head_dim].reshape(n_kv_heads, head_dim)
    v = e[H - n_kv_heads * head_dim:].reshape(n_kv_heads, head_dim)[:, ::-1]
    return q, k, v


def sm_hidden(o_heads: np.ndarray, w64: np.ndarray, boost_tok: int, boost_val: float, gain: float):
    """Hidden row fed to the LM head: gain * o (heads concatenated) plus the
    boost vector beta * W[t] / |W[t]|^2 (W[t] . that vector = beta)."""
    wt = w64[boost_tok]
    return gain * o_heads.reshape(-1) + boost_val * wt / float(wt @ wt)


def embed_kv(w64, tokens_row, positions, n_q_heads, n_kv_heads, head_dim):
    """K/V [Hkv][n][d] of the given positions of one sequence."""
    ks, vs = [], []
    for p in positions:
        _, k, v = sm_embed(w64, int(tokens_row[p]), n_q_heads, n_kv_heads, head_dim)
        ks.append(k)
        vs.append(v)
    return np.stack(ks, axis=1), np.stack(vs, axis=1)


# ----------------------------------------------------------------------------
# Bookkeeping of the loop (separate functions so that each can be checked)
# ----------------------------------------------------------------------------

def block_start(prompt_len: int, block_size: int, blk: int) -> int:
    """Absolute position of the first token of generated block blk."""
    return prompt_len + blk * block_size


def sub_rows(block_size: int, sub_size: int, blk: int, sub: int) -> range:
    """Generated-position indices (0-based after the prompt) of a sub-block."""
    r0 = blk * block_size + sub * sub_size
    return range(r0, r0 + sub_size)


def holds_eos(block_tokens: np.ndarray, eos_id: int) -> bool:
    return bool(np.any(np.asarray(block_tokens) == eos_id))


# ----------------------------------------------------------------------------
# The loop
# ----------------------------------------------------------------------------

def decode(dims: Dict, w, prompt, boost_tok, boost_val, tau, mode: str = O.SELECT_THRESHOLD, k: int = 0,
           factor: float = 1.0, mask_id: int = 0, eos_id: int = 0, gain: float = 1.0,
           max_blocks: int = 0) -> Dict:
    """Run the decode loop.  dims: batch, prompt_len, gen_len, block,
    sub_block, n_q_heads, n_kv_heads, head_dim, attn_mode (O.BLOCK_CAUSAL or
    O.DUAL_CACHE).  w [V][H]; prompt [B][P]; boost_tok, boost_val [B][L];
    tau [B].

    Returns tokens [B][P+L], masked [B][L], k/v cache [B][Hkv][P+L][d],
    length [B], seq_steps [B] (steps in which the sequence had a masked row),
    eos_block [B] (-1: none), blocks_run, and the per-step trace: a list of
    dicts with block, sub, conf/token/p2 [B][S] of the active rows, commit
    [B][S], and the block's tokens/masked [B][D] after the step."""
    B, P, L = dims["batch"], dims["prompt_len"], dims["gen_len"]
    D, S = dims["block"], dims["sub_block"]
    Hq, Hkv, d = dims["n_q_heads"], dims["n_kv_heads"], dims["head_dim"]
    mode_attn = dims.get("attn_mode", O.BLOCK_CAUSAL)
    dual = mode_attn == O.DUAL_CACHE
    w64 = O._f64(w)
    V, H = w64.shape
    if H != Hq * d:
        raise ValueError("the stand-in model needs hidden = n_q_heads * head_dim")
    cap = P + L
    n_blocks = max_blocks if max_blocks > 0 else L // D
    prompt = np.asarray(prompt)
    boost_tok = np.asarray(boost_tok)
    boost_val = np.asarray(boost_val, dtype=np.float64)
    tau = np.asarray(tau, dtype=np.float64).reshape(-1)

    tokens = np.full((B, cap), mask_id, dtype=np.int64)
    tokens[:, :P] = prompt
    masked = np.zeros((B, L), dtype=bool)
    kc = np.zeros((B, Hkv, cap, d))
    vc = np.zeros((B, Hkv, cap, d))
    length = np.zeros(B, dtype=np.int64)
    # the prompt is the initial prefix (Level 1): its K/V fill the cache
    if P > 0 and not dual:
        for b in range(B):
            kn, vn = embed_kv(w64, tokens[b], range(P), Hq, Hkv, d)
            kc[b, :, :P], vc[b, :, :P] = kn, vn
        length[:] = P
    done = np.zeros(B, dtype=bool)
    eos_block = np.full(B, -1, dtype=np.int64)
    seq_steps = np.zeros(B, dtype=np.int64)
    trace: List[Dict] = []
    blocks_run = 0

    for blk in range(n_blocks):
        if done.all():
            break
        blocks_run += 1
        base = block_start(P, D, blk)
        for b in range(B):
            tokens[b, base:base + D] = mask_id
            masked[b, blk * D:(blk + 1) * D] = not done[b]
        if dual:
            # [v1] Algorithm 1: refresh, i.e. recompute the K/V of every position
            for b in range(B):
                kn, vn = embed_kv(w64, tokens[b], range(cap), Hq, Hkv, d)
                kc[b], vc[b] = kn, vn
            length[:] = cap
        for sub in range(D // S):
            rows = sub_rows(D, S, blk, sub)
            while masked[:, rows.start:rows.stop].any():
                live = masked[:, rows.start:rows.stop].any(axis=1)
                seq_steps += live
                q = np.zeros((B, S, Hq, d))
                kb = np.zeros((B, Hkv, D, d))
                vb = np.zeros((B, Hkv, D, d))
                for b in range(B):
                    for i, r in enumerate(rows):
                        q[b, i] = sm_embed(w64, int(tokens[b, P + r]), Hq, Hkv, d)[0]
                    kb[b], vb[b] = embed_kv(w64, tokens[b], range(base, base + D), Hq, Hkv, d)
                lp = np.full(B, base)
                out, _ = O.block_attention(q, kc, vc, kb, vb, lp, mode_attn, cap)
                x = np.zeros((B * S, H))
                for b in range(B):
                    for i, r in enumerate(rows):
                        x[b * S + i] = sm_hidden(out[b, i], w64, int(boost_tok[b, r]), boost_val[b, r], gain)
                logits = O.lm_head(x, w64).reshape(B, S, V)
                res = O.conf_select(logits, masked[:, rows.start:rows.stop], tau, mode, k, factor)
                t_new, m_new = O.commit_update(tokens[:, P + rows.start:P + rows.stop],
                                               masked[:, rows.start:rows.stop], res["token"], res["commit"])
                tokens[:, P + rows.start:P + rows.stop] = t_new
                masked[:, rows.start:rows.stop] = m_new
                trace.append(dict(block=blk, sub=sub, conf=res["conf"], token=res["token"], p2=res["p2"],
                                  commit=res["commit"], live=live,
                                  tokens=tokens[:, base:base + D].copy(),
                                  masked=masked[:, blk * D:(blk + 1) * D].copy()))
        if not dual:
            # Level 3: the completed block's K/V enter the block-level cache
            kn = np.zeros((B, Hkv, D, d))
            vn = np.zeros((B, Hkv, D, d))
            for b in range(B):
                kn[b], vn[b] = embed_kv(w64, tokens[b], range(base, base + D), Hq, Hkv, d)
            kc, length2 = O.kv_append(kc, kn, length)
            vc, _ = O.kv_append(vc, vn, length)
            length = length2
        for b in range(B):
            if not done[b] and holds_eos(tokens[b, base:base + D], eos_id):
                done[b] = True
                eos_block[b] = blk
    return dict(tokens=tokens, masked=masked, k_cache=kc, v_cache=vc, length=length, seq_steps=seq_steps,
                eos_block=eos_block, blocks_run=blocks_run, trace=trace)
