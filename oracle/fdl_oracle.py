"""CPU fp64 oracle for one cached block-diffusion denoising step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module.  It shares no code with
the HIP library and must never serve as a fallback for it.

Each function is the plain definition of one step of the method, in float64,
with no blocking, fusion or reordering beyond what that definition states.
Inputs are numpy arrays (any float dtype; they are upcast exactly to float64).

Pages followed (cited by title and section):
  [v2]  "Fast-dLLM v2: Efficient Block-Diffusion LLM" (technical breakdown):
        "Attention Mask Design", "Inference-time attention mask (Figure 7b)",
        "Inference Pipeline" Levels 1-3, "Batch decoding with length padding",
        "Sub-block size as a decoding granularity knob".
  [v1]  "Fast-dLLM: Reusing Bidirectional State and Spending Confidence on
        Parallel Tokens": eq 3 (attention), section 3 "PrefixCache and
        DualCache" with Algorithm 1, section 4 Algorithm 2 (threshold
        selection with guaranteed progress), section 6 eq 13 / Algorithm 3
        (factor selection).
  [rq]  "Diffusion language models: review questions": commit every position
        above the threshold, else the single most confident one; fixed
        count per step.

Every function here is pinned by the CPU test suite (tests/test_oracle_pins.py)
against brute force, closed forms, the pages' worked example or invariants.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np

BLOCK_CAUSAL = "block_causal"
DUAL_CACHE = "dual_cache"

SELECT_THRESHOLD = "threshold"
SELECT_TOPK = "topk"
SELECT_FACTOR = "factor"


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):          # a torch tensor: upcast exactly via float64
        a = a.detach().cpu().double().numpy()
    return np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------
# Attention  ([v1] eq 3; [v2] "Inference-time attention mask (Figure 7b)")
# ----------------------------------------------------------------------------

def score_scale(head_dim: int) -> float:
    """[v1] eq 3: scores are QK^T divided by sqrt(d)."""
    return 1.0 / math.sqrt(head_dim)


def kv_head_of(h: int, n_q_heads: int, n_kv_heads: int) -> int:
    """Grouped-query mapping: query heads are split into n_kv_heads contiguous
    groups of G = Hq/Hkv heads, group g reading KV head g.  (The pages do not
    mention GQA; the contiguous grouping is the convention of the Qwen2.5
    models whose shapes the workloads use.)"""
    return h // (n_q_heads // n_kv_heads)


def visible_keys(prefix_len: int, block: int, mode: str, total_len: int):
    """Logical key list for every query row of the active block, as
    (position, source) pairs, source 'cache' or 'block'.

    [v2] Figure 7b: the active block attends bidirectionally to all of its own
    D positions and to every cached prefix position; nothing after the block
    is visible.  [v1] section 3 DualCache: the active block additionally sees
    the cached suffix (all remaining masked positions after it), whose K/V sit
    in the cache at their own positions."""
    keys = [(j, "cache") for j in range(prefix_len)]
    keys += [(prefix_len + j, "block") for j in range(block)]
    if mode == DUAL_CACHE:
        keys += [(j, "cache") for j in range(prefix_len + block, total_len)]
    elif mode != BLOCK_CAUSAL:
        raise ValueError(mode)
    return keys


def softmax_weights(scores: np.ndarray):
    """Softmax of one row of scores with its log-sum-exp (natural log)."""
    m = scores.max()
    e = np.exp(scores - m)
    s = e.sum()
    return e / s, m + math.log(s)


def block_attention(q, k_cache, v_cache, k_blk, v_blk, prefix_len: Sequence[int],
                    mode: str = BLOCK_CAUSAL, total_len: Optional[int] = None):
    """Attention of the active block's query rows over prefix cache + block (+ suffix).

    q        [B][S][Hq][d]   query rows of the active (sub-)block
    k_cache  [B][Hkv][cap][d], v_cache likewise (positions by absolute index)
    k_blk    [B][Hkv][D][d], v_blk likewise  (fresh K/V of the active block)
    prefix_len[B]            cached prefix length Lp per sequence
    total_len                P + L (only used by the DualCache mode)

    Returns (out [B][S][Hq][d], lse [B][Hq][S]) in float64.
    o = sum_j softmax_j(q.k_j / sqrt(d)) v_j over the visible keys ([v1] eq 3).
    """
    q, kc, vc, kb, vb = map(_f64, (q, k_cache, v_cache, k_blk, v_blk))
    B, S, Hq, d = q.shape
    Hkv, D = kb.shape[1], kb.shape[2]
    if total_len is None:
        total_len = kc.shape[2]
    out = np.zeros((B, S, Hq, d))
    lse = np.zeros((B, Hq, S))
    scale = score_scale(d)
    for b in range(B):
        lp = int(prefix_len[b])
        keys = visible_keys(lp, D, mode, total_len)
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            K = np.stack([kc[b, g, j] if src == "cache" else kb[b, g, j - lp] for j, src in keys])
            V = np.stack([vc[b, g, j] if src == "cache" else vb[b, g, j - lp] for j, src in keys])
            for i in range(S):
                w, l = softmax_weights(K @ q[b, i, h] * scale)
                out[b, i, h] = w @ V
                lse[b, h, i] = l
    return out, lse


# ----------------------------------------------------------------------------
# Training-time mask (for brute-force pins) ([v2] "Attention Mask Design")
# ----------------------------------------------------------------------------

def block_of(i: int, block: int) -> int:
    return i // block


def mask_full(L: int, block: int) -> np.ndarray:
    """M_full in {0,1}^{2L x 2L} = [[M_BD, M_OBC], [0, M_BC]] over the
    concatenation [x_t ; x_0] of the noised and clean sequences.
    M_BD: same block.  M_OBC: key block strictly before the query's block.
    M_BC: key block at or before the query's block.  Bottom-left: zero."""
    M = np.zeros((2 * L, 2 * L), dtype=bool)
    for i in range(L):
        for j in range(L):
            bi, bj = block_of(i, block), block_of(j, block)
            M[i, j] = bi == bj                 # M_BD
            M[i, L + j] = bj < bi              # M_OBC
            M[L + i, L + j] = bj <= bi         # M_BC
    return M


def dense_masked_attention(q, k, v, mask):
    """Dense attention of rows q[n][d] over keys k[m][d] with a boolean mask[n][m]:
    blocked scores are set to -inf before the softmax ([v2] "Attention Mask Design")."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    s = (q @ k.T) * score_scale(q.shape[1])
    s = np.where(mask, s, -np.inf)
    out = np.zeros((q.shape[0], v.shape[1]))
    for i in range(q.shape[0]):
        w, _ = softmax_weights(s[i])
        out[i] = w @ v
    return out


def bc_visible(p: int, j: int, block: int) -> bool:
    """M_BC ([v2] "Attention Mask Design"): key j is visible to position p when
    j's block is the same as or earlier than p's block."""
    return block_of(j, block) <= block_of(p, block)


def prefill_attention(q, k, v, q_start: int, n_keys: int, block: int, causal: bool = True):
    """Attention of query positions q_start .. q_start+n_q-1 over key positions
    0 .. n_keys-1 of one K/V sequence.

    q [B][n_q][Hq][d]; k, v [B][Hkv][>= n_keys][d].  causal: the block-causal
    M_BC pattern ([v2] "Attention Mask Design": a position sees its own block
    and every earlier block), as in the prompt prefill; otherwise every key is
    visible, as in the [v1] Algorithm 1 refresh.  Returns (out [B][n_q][Hq][d],
    lse [B][Hq][n_q])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, nq, Hq, d = q.shape
    Hkv = k.shape[1]
    out = np.zeros((B, nq, Hq, d))
    lse = np.zeros((B, Hq, nq))
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            for i in range(nq):
                p = q_start + i
                keys = [j for j in range(n_keys) if (bc_visible(p, j, block) or not causal)]
                sc = k[b, g, keys] @ q[b, i, h] * score_scale(d)
                w, l = softmax_weights(sc)
                out[b, i, h] = w @ v[b, g, keys]
                lse[b, h, i] = l
    return out, lse


# ----------------------------------------------------------------------------
# LM head  ([v2] Inference Pipeline Level 2: distributions over the vocabulary)
# ----------------------------------------------------------------------------

def lm_head(x, w):
    """logits[M][V] = X[M][H] . W[V][H]^T in float64.

    Token shift ([v2] Step 5): the row that predicts block position i is the
    hidden state at i-1; that is the caller's choice of rows, not arithmetic."""
    return _f64(x) @ _f64(w).T


# ----------------------------------------------------------------------------
# Confidence select  ([v1] Algorithm 2; [v2] Level 2; [rq])
# ----------------------------------------------------------------------------

def row_confidence(logits_row: np.ndarray):
    """Greedy prediction and its confidence for one row of logits.

    token = argmax (lowest id on equal logits), conf = softmax probability of
    that token = 1 / sum_v exp(l_v - l_max), p2 = the runner-up probability
    (equal to conf when the maximum is shared)."""
    l = _f64(logits_row)
    tok = int(np.argmax(l))                     # numpy returns the first maximum
    m = l[tok]
    z = np.exp(l - m).sum()
    top2 = np.partition(l, -2)[-2] if l.size > 1 else -np.inf
    return tok, 1.0 / z, math.exp(top2 - m) / z


def above_threshold(c: float, tau: float) -> bool:
    """Strict comparison: a position is finalized when its confidence exceeds
    tau ([v2] Level 2; [rq]).  ([v1] Algorithm 2 prints >=; that page itself
    warns against silently replacing a strict premise by >=.)"""
    return c > tau


def _order_by_conf(cands, conf):
    """Candidates by decreasing confidence, lower row first on equal confidence."""
    return sorted(cands, key=lambda r: (-conf[r], r))


def select_rows(conf: np.ndarray, masked: np.ndarray, tau: float, mode: str = SELECT_THRESHOLD,
                k: int = 0, factor: float = 1.0) -> np.ndarray:
    """Commit mask for one sequence's rows.

    THRESHOLD ([v1] Algorithm 2): S = {masked r : conf_r > tau}; if S is empty
      and some row is masked, S = {the masked row of maximum conf} (lowest row
      on ties).
    TOPK ([rq] fixed count per step): the min(k, #masked) most confident
      masked rows (lower row first on ties).
    FACTOR ([v1] eq 13 / Algorithm 3): with masked rows sorted by decreasing
      confidence c_(1) >= ... >= c_(m), commit the first n for the largest n
      with (n+1)(1 - c_(n)) < f; if no n qualifies, the first row alone."""
    R = conf.shape[0]
    commit = np.zeros(R, dtype=bool)
    cands = [r for r in range(R) if masked[r]]
    if not cands:
        return commit
    if mode == SELECT_THRESHOLD:
        for r in cands:
            if above_threshold(conf[r], tau):
                commit[r] = True
        if not commit.any():
            commit[_order_by_conf(cands, conf)[0]] = True
    elif mode == SELECT_TOPK:
        for r in _order_by_conf(cands, conf)[:k]:
            commit[r] = True
    elif mode == SELECT_FACTOR:
        order = _order_by_conf(cands, conf)
        best = 0
        for n in range(1, len(order) + 1):
            if (n + 1) * (1.0 - conf[order[n - 1]]) < factor:
                best = n
        for r in order[: max(best, 1)]:
            commit[r] = True
    else:
        raise ValueError(mode)
    return commit


def conf_select(logits, masked, tau, mode: str = SELECT_THRESHOLD, k: int = 0,
                factor: float = 1.0) -> Dict[str, np.ndarray]:
    """Confidence select over logits[B][R][V] with masked[B][R] and tau[B].

    Returns token, conf, p2 [B][R], commit [B][R] (bool), n_commit [B]."""
    lg = _f64(logits)
    B, R, _ = lg.shape
    masked = np.asarray(masked).astype(bool)
    tau = np.asarray(tau, dtype=np.float64).reshape(-1)
    token = np.zeros((B, R), dtype=np.int64)
    conf = np.zeros((B, R))
    p2 = np.zeros((B, R))
    commit = np.zeros((B, R), dtype=bool)
    for b in range(B):
        for r in range(R):
            token[b, r], conf[b, r], p2[b, r] = row_confidence(lg[b, r])
        commit[b] = select_rows(conf[b], masked[b], tau[b], mode, k, factor)
    return dict(token=token, conf=conf, p2=p2, commit=commit, n_commit=commit.sum(1))


def commit_update(tokens, masked, token, commit):
    """Apply a commit set: finalized rows take their predicted token and leave
    the masked set ([v2] Level 2; [v1] Algorithm 2, last step)."""
    tokens = np.array(tokens, copy=True)
    masked = np.array(masked, copy=True)
    tokens[commit] = token[commit]
    masked[commit] = 0
    return tokens, masked


# ----------------------------------------------------------------------------
# KV append  ([v2] Level 3 block-level cache; [v1] Algorithm 1 refresh)
# ----------------------------------------------------------------------------

def kv_write(cache, new, pos):
    """[v1] Algorithm 1 refresh: write new[B][Hkv][n][d] into every sequence's
    cache at positions pos .. pos+n-1; the lengths become pos + n.  Returns
    copies."""
    cache = np.array(cache, copy=True)
    n = new.shape[2]
    if pos < 0 or pos + n > cache.shape[2]:
        raise ValueError("write outside the cache")
    cache[:, :, pos:pos + n] = new
    return cache, np.full(cache.shape[0], pos + n, dtype=np.int64)


def kv_append(cache, new, length):
    """Write new[B][Hkv][n][d] into cache[B][Hkv][cap][d] at positions
    length[b] .. length[b]+n-1 and advance length[b] by n.  Returns copies."""
    cache = np.array(cache, copy=True)
    length = np.array(length, copy=True)
    n = new.shape[2]
    for b in range(cache.shape[0]):
        lo = int(length[b])
        if lo + n > cache.shape[2]:
            raise ValueError("append past capacity")
        cache[b, :, lo:lo + n] = new[b]
        length[b] = lo + n
    return cache, length
