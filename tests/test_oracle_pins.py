"""Pins for the CPU oracle: each check ties it to something other than itself
(brute force from the mask definitions, closed forms, the pages' worked
numbers, invariants).  CPU only."""
import json
import math
import os

import numpy as np
import pytest

from oracle import fdl_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------
# C-1  mask semantics: cached block step == rows of the dense masked attention
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("n_blocks_prompt,block_idx,D", [(4, 0, 16), (4, 3, 16), (2, 5, 8), (3, 1, 4)])
def test_c1_cached_step_equals_training_mask_rows(n_blocks_prompt, block_idx, D):
    """Training mask M_full over [x_t ; x_0] (built from the M_BD / M_OBC /
    M_BC definitions): the rows of the noised active block attend to their own
    noised block and to the clean earlier blocks.  With the clean earlier
    blocks' K/V as the cache and the noised block's K/V as the block buffer,
    the cached step must give the same rows."""
    r = rng(1)
    Ltot = (n_blocks_prompt + block_idx + 3) * D      # whole sequence incl. later blocks
    d = 8
    lp = (n_blocks_prompt + block_idx) * D             # prefix = prompt + decoded blocks
    # clean and noised K/V/Q for every position
    kc, vc = r.standard_normal((Ltot, d)), r.standard_normal((Ltot, d))
    kn, vn, qn = r.standard_normal((Ltot, d)), r.standard_normal((Ltot, d)), r.standard_normal((Ltot, d))
    M = O.mask_full(Ltot, D)
    rows = np.arange(lp, lp + D)                       # noised rows of the active block
    K = np.concatenate([kn, kc])                       # keys: [x_t ; x_0]
    V = np.concatenate([vn, vc])
    dense = O.dense_masked_attention(qn[rows], K, V, M[rows])
    out, _ = O.block_attention(qn[rows][None, :, None, :], kc[None, None], vc[None, None],
                               kn[rows][None, None], vn[rows][None, None], [lp])
    np.testing.assert_allclose(out[0, :, 0], dense, rtol=0, atol=1e-12)


def test_c1_block_causal_equals_bc_mask_over_sequence():
    """Inference view ([v2] Figure 7b): with one K/V per position, the active
    block's rows equal the M_BC-masked (block-causal) dense attention over the
    whole sequence, later blocks included and masked out."""
    r = rng(2)
    D, d, lp = 16, 8, 64
    Ltot = lp + 3 * D
    q, k, v = (r.standard_normal((Ltot, d)) for _ in range(3))
    M = O.mask_full(Ltot, D)[Ltot:, Ltot:]             # M_BC quadrant
    rows = np.arange(lp, lp + D)
    dense = O.dense_masked_attention(q[rows], k, v, M[rows])
    out, _ = O.block_attention(q[rows][None, :, None], k[None, None], v[None, None],
                               k[rows][None, None], v[rows][None, None], [lp])
    np.testing.assert_allclose(out[0, :, 0], dense, rtol=0, atol=1e-12)


def test_c1_dual_cache_equals_full_bidirectional():
    """[v1] section 3 DualCache: prefix cache + fresh block + cached suffix is a
    full bidirectional attention over all P+L positions in which the block's
    positions use the fresh K/V."""
    r = rng(3)
    D, d, P, L, b = 8, 8, 24, 32, 2
    T = P + L
    kc, vc = r.standard_normal((T, d)), r.standard_normal((T, d))
    kb, vb, q = r.standard_normal((D, d)), r.standard_normal((D, d)), r.standard_normal((D, d))
    lp = P + b * D
    K, V = kc.copy(), vc.copy()
    K[lp:lp + D], V[lp:lp + D] = kb, vb
    dense = O.dense_masked_attention(q, K, V, np.ones((D, T), dtype=bool))
    out, _ = O.block_attention(q[None, :, None], kc[None, None], vc[None, None], kb[None, None],
                               vb[None, None], [lp], mode=O.DUAL_CACHE, total_len=T)
    np.testing.assert_allclose(out[0, :, 0], dense, rtol=0, atol=1e-12)


def test_c1_mask_full_quadrants_small():
    """M_full for L = 4, D = 2, written out by hand from the three definitions."""
    BD = [[1, 1, 0, 0], [1, 1, 0, 0], [0, 0, 1, 1], [0, 0, 1, 1]]
    OBC = [[0, 0, 0, 0], [0, 0, 0, 0], [1, 1, 0, 0], [1, 1, 0, 0]]
    BC = [[1, 1, 0, 0], [1, 1, 0, 0], [1, 1, 1, 1], [1, 1, 1, 1]]
    Z = [[0] * 4] * 4
    want = np.block([[np.array(BD), np.array(OBC)], [np.array(Z), np.array(BC)]]).astype(bool)
    np.testing.assert_array_equal(O.mask_full(4, 2), want)


# ----------------------------------------------------------------------------
# C-2  exact block cache: cached decoding == full recomputation (2-layer toy)
# ----------------------------------------------------------------------------

def _toy_model(r, V, H, n_layers):
    E = r.standard_normal((V, H))
    Ws = [tuple(r.standard_normal((H, H)) / math.sqrt(H) for _ in range(3)) for _ in range(n_layers)]
    return E, Ws


def _full_forward(tokens, E, Ws, mask):
    """Dense forward of a residual toy transformer (attention only)."""
    h = E[tokens]
    per_layer_kv = []
    for Wq, Wk, Wv in Ws:
        q, k, v = h @ Wq, h @ Wk, h @ Wv
        per_layer_kv.append((k, v))
        h = h + O.dense_masked_attention(q, k, v, mask)
    return h, per_layer_kv


def test_c2_block_cache_is_exact():
    """[v2] Level 3: block-level KV cache is exact.  Decoding block by block
    with the cached step + append gives exactly the full block-causal forward
    over the final sequence, at every layer."""
    r = rng(4)
    Vv, H, D, P, nb = 50, 16, 8, 16, 3
    E, Ws = _toy_model(r, Vv, H, 2)
    tokens = r.integers(0, Vv, P + nb * D)
    T = len(tokens)
    M_bc = O.mask_full(T, D)[T:, T:]
    h_full, _ = _full_forward(tokens, E, Ws, M_bc)
    # prefill the prompt's cache with its own dense forward (prompt only)
    Mp = O.mask_full(P, D)[P:, P:]
    _, kv_prompt = _full_forward(tokens[:P], E, Ws, Mp)
    caches = []
    for k, v in kv_prompt:
        kc, vc = np.zeros((1, 1, T, H)), np.zeros((1, 1, T, H))
        kc[0, 0, :P], vc[0, 0, :P] = k, v
        caches.append([kc, vc, np.array([P])])
    for b in range(nb):
        lo = P + b * D
        h = E[tokens[lo:lo + D]]
        for li, (Wq, Wk, Wv) in enumerate(Ws):
            kc, vc, ln = caches[li]
            q, k, v = h @ Wq, h @ Wk, h @ Wv
            out, _ = O.block_attention(q[None, :, None], kc, vc, k[None, None], v[None, None], ln)
            # block finished: append its K/V
            kc2, ln2 = O.kv_append(kc, k[None, None], ln)
            vc2, _ = O.kv_append(vc, v[None, None], ln)
            caches[li] = [kc2, vc2, ln2]
            h = h + out[0, :, 0]
        np.testing.assert_allclose(h, h_full[lo:lo + D], rtol=0, atol=1e-11)


def test_c2_negative_control_dualcache_is_approximate():
    """[v1] section 3: under bidirectional attention the cache is only an
    approximation: a 2-layer toy whose DualCache was filled before the block's
    tokens were revealed differs from the full recomputation afterwards."""
    r = rng(5)
    Vv, H, D, P, L = 50, 16, 8, 16, 24
    E, Ws = _toy_model(r, Vv, H, 2)
    MASK = 0
    final = r.integers(1, Vv, P + L)
    T = P + L
    full_bidir = np.ones((T, T), dtype=bool)
    h_full, _ = _full_forward(final, E, Ws, full_bidir)
    # refresh at the first block boundary: answer still all masked
    start = final.copy()
    start[P:] = MASK
    _, kv_ref = _full_forward(start, E, Ws, full_bidir)
    h = E[final[P:P + D]]
    for li, (Wq, Wk, Wv) in enumerate(Ws):
        k_ref, v_ref = kv_ref[li]
        q, k, v = h @ Wq, h @ Wk, h @ Wv
        out, _ = O.block_attention(q[None, :, None], k_ref[None, None], v_ref[None, None], k[None, None],
                                   v[None, None], [P], mode=O.DUAL_CACHE, total_len=T)
        h = h + out[0, :, 0]
    assert np.abs(h - h_full[P:P + D]).max() > 1e-3


# ----------------------------------------------------------------------------
# C-3 / C-4  softmax rows and closed forms
# ----------------------------------------------------------------------------

def _attn(q, kc, vc, kb, vb, lp, **kw):
    return O.block_attention(q, kc, vc, kb, vb, lp, **kw)


def test_c3_weights_sum_to_one_and_lse_counts_keys():
    """V = 1 everywhere gives o = 1 (weights sum to one); q = 0 gives equal
    scores, so lse = ln(number of visible keys) = ln(Lp + D) (block-causal)
    and ln(P + L) (DualCache)."""
    r = rng(6)
    B, S, Hq, Hkv, d, cap, D = 2, 4, 4, 2, 8, 40, 8
    kc = r.standard_normal((B, Hkv, cap, d))
    kb = r.standard_normal((B, Hkv, D, d))
    ones_c, ones_b = np.ones((B, Hkv, cap, d)), np.ones((B, Hkv, D, d))
    q = r.standard_normal((B, S, Hq, d))
    out, _ = _attn(q, kc, ones_c, kb, ones_b, [16, 24])
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-14)
    _, lse = _attn(np.zeros_like(q), kc, kc, kb, kb, [16, 24])
    np.testing.assert_allclose(lse[0], math.log(16 + D), atol=1e-14)
    np.testing.assert_allclose(lse[1], math.log(24 + D), atol=1e-14)
    _, lse = _attn(np.zeros_like(q), kc, kc, kb, kb, [16, 24], mode=O.DUAL_CACHE, total_len=cap)
    np.testing.assert_allclose(lse, math.log(cap), atol=1e-14)


def test_c4_identical_keys_give_mean_of_values():
    r = rng(7)
    B, S, Hq, Hkv, d, cap, D, lp = 1, 3, 2, 1, 4, 20, 4, 12
    kvec = r.standard_normal(d)
    kc = np.tile(kvec, (B, Hkv, cap, 1))
    kb = np.tile(kvec, (B, Hkv, D, 1))
    vc, vb = r.standard_normal((B, Hkv, cap, d)), r.standard_normal((B, Hkv, D, d))
    out, _ = _attn(r.standard_normal((B, S, Hq, d)), kc, vc, kb, vb, [lp])
    want = np.concatenate([vc[0, 0, :lp], vb[0, 0]]).mean(0)
    np.testing.assert_allclose(out[0, :, 0], np.tile(want, (S, 1)), atol=1e-14)


def test_c4_single_key_and_dominant_key():
    r = rng(8)
    d = 4
    v = r.standard_normal((1, 1, 1, d))
    k = r.standard_normal((1, 1, 1, d))
    out, _ = _attn(r.standard_normal((1, 2, 1, d)), np.zeros((1, 1, 0, d)), np.zeros((1, 1, 0, d)), k, v, [0])
    np.testing.assert_allclose(out[0, :, 0], np.tile(v[0, 0, 0], (2, 1)), atol=1e-15)
    # one key aligned with q at a huge score: its value wins
    kc = r.standard_normal((1, 1, 10, d)) * 0.01
    vc = r.standard_normal((1, 1, 10, d))
    q = np.zeros((1, 1, 1, d)); q[..., 0] = 200.0
    kc[0, 0, 3] = [10.0, 0, 0, 0]
    out, _ = _attn(q, kc, vc, kc[:, :, :2] * 0, vc[:, :, :2], [10])
    np.testing.assert_allclose(out[0, 0, 0], vc[0, 0, 3], atol=1e-12)


def test_c4_two_key_closed_form_fixes_scale():
    """Two keys, d = 4, q = (2,0,0,0), k1 = (1,0,0,0), k2 = 0: scores are
    q.k/sqrt(4) = 1 and 0, so o = (e v1 + v2)/(e + 1) ([v1] eq 3)."""
    q = np.array([2.0, 0, 0, 0]).reshape(1, 1, 1, 4)
    kc = np.array([[1.0, 0, 0, 0]]).reshape(1, 1, 1, 4)
    kb = np.zeros((1, 1, 1, 4))
    v1, v2 = np.array([1.0, 2, 3, 4]), np.array([-1.0, 0, 5, 1])
    out, lse = _attn(q, kc, v1.reshape(1, 1, 1, 4), kb, v2.reshape(1, 1, 1, 4), [1])
    e = math.e
    np.testing.assert_allclose(out[0, 0, 0], (e * v1 + v2) / (e + 1), atol=1e-15)
    assert abs(lse[0, 0, 0] - math.log(e + 1)) < 1e-15


def test_c4_gqa_equals_mha_with_repeated_kv():
    r = rng(9)
    B, S, Hq, Hkv, d, cap, D = 2, 4, 6, 2, 8, 24, 4
    q = r.standard_normal((B, S, Hq, d))
    kc, vc = r.standard_normal((B, Hkv, cap, d)), r.standard_normal((B, Hkv, cap, d))
    kb, vb = r.standard_normal((B, Hkv, D, d)), r.standard_normal((B, Hkv, D, d))
    G = Hq // Hkv
    rep = lambda t: np.repeat(t, G, axis=1)          # head h <- kv head h // G
    a, _ = _attn(q, kc, vc, kb, vb, [8, 20])
    b, _ = _attn(q, rep(kc), rep(vc), rep(kb), rep(vb), [8, 20])
    np.testing.assert_allclose(a, b, atol=1e-14)
    # a different KV head per group really matters
    kc2 = kc.copy(); kc2[:, 1] += 1.0
    c, _ = _attn(q, kc2, vc, kb, vb, [8, 20])
    assert np.abs(c[:, :, :G] - a[:, :, :G]).max() < 1e-14
    assert np.abs(c[:, :, G:] - a[:, :, G:]).max() > 1e-6


def test_c4_brute_force_tiny_loops():
    """Pure-Python loop evaluation of eq 3 on a tiny case."""
    r = rng(10)
    d, lp, D = 3, 2, 2
    q = r.standard_normal((1, 1, 1, d))
    kc, vc = r.standard_normal((1, 1, 5, d)), r.standard_normal((1, 1, 5, d))
    kb, vb = r.standard_normal((1, 1, D, d)), r.standard_normal((1, 1, D, d))
    keys = [kc[0, 0, 0], kc[0, 0, 1], kb[0, 0, 0], kb[0, 0, 1]]
    vals = [vc[0, 0, 0], vc[0, 0, 1], vb[0, 0, 0], vb[0, 0, 1]]
    s = [sum(q[0, 0, 0, t] * k[t] for t in range(d)) / math.sqrt(d) for k in keys]
    z = sum(math.exp(x) for x in s)
    want = [sum(math.exp(s[j]) * vals[j][t] for j in range(4)) / z for t in range(d)]
    out, _ = _attn(q, kc, vc, kb, vb, [lp])
    np.testing.assert_allclose(out[0, 0, 0], want, atol=1e-14)


# ----------------------------------------------------------------------------
# C-5 / C-6  commit rule and confidence
# ----------------------------------------------------------------------------

def test_c6_eq4_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "eq4_marginals.json")))
    j = g["joint"]
    p0 = [j["00"] + j["01"], j["00"] + j["10"]]        # marginal of token 0 at each position
    logits = np.log(np.array([[[p0[0], 1 - p0[0]], [p0[1], 1 - p0[1]]]]))
    res = O.conf_select(logits, np.ones((1, 2)), [g["tau"]])
    e = g["expected"]
    assert res["token"][0].tolist() == e["token"]
    np.testing.assert_allclose(res["conf"][0], e["conf"], atol=1e-12)
    assert res["commit"][0].tolist() == e["commit"]
    assert int(res["n_commit"][0]) == e["n_commit"]


def test_c6_closed_form_confidence():
    """One logit a, V-1 zeros: c = e^a / (e^a + V - 1); p2 = 1/(e^a + V - 1)."""
    for V, a in [(2, 0.3), (512, 7.0), (151936, 14.5), (1000, -2.0)]:
        row = np.zeros(V); row[V // 3] = a
        tok, c, p2 = O.row_confidence(row)
        if a > 0:
            assert tok == V // 3
            assert abs(c - math.exp(a) / (math.exp(a) + V - 1)) < 1e-15
            assert abs(p2 - 1 / (math.exp(a) + V - 1)) < 1e-15
        else:
            assert tok == 0                           # lowest of the equal maxima
            assert abs(c - 1 / (math.exp(a) + V - 1)) < 1e-15
            assert c == p2


def test_c6_argmax_tie_lowest_id():
    row = np.array([0.0, 3.0, 1.0, 3.0, 3.0])
    tok, c, p2 = O.row_confidence(row)
    assert tok == 1 and c == p2


def test_c5_commit_rule_properties():
    r = rng(11)
    for trial in range(300):
        R = int(r.integers(1, 33))
        conf = r.random(R) ** 0.3
        masked = r.random(R) < 0.7
        tau = float(r.choice([0.5, 0.7, 0.9, 0.95]))
        c = O.select_rows(conf, masked, tau)
        if not masked.any():
            assert not c.any()
            continue
        assert c.sum() >= 1
        assert not (c & ~masked).any()
        above = masked & (conf > tau)
        if above.any():
            np.testing.assert_array_equal(c, above)
        else:
            best = max(np.flatnonzero(masked), key=lambda i: (conf[i], -i))
            assert c.sum() == 1 and c[best]
        k = int(r.integers(1, 6))
        t = O.select_rows(conf, masked, tau, O.SELECT_TOPK, k=k)
        assert t.sum() == min(k, masked.sum())
        if t.any() and (masked & ~t).any():
            assert conf[t].min() >= conf[masked & ~t].max()


def test_c5_threshold_is_strict_at_equality():
    conf = np.array([0.5, 0.5, 0.25])
    c = O.select_rows(conf, np.ones(3, bool), 0.5)
    assert c.tolist() == [True, False, False]          # none exceeds 0.5: fallback, lowest row


def test_c5_factor_rule_page_values():
    g = json.load(open(os.path.join(GOLDEN, "factor_rule.json")))
    conf = np.full(g["block"], g["conf_all"])
    m = np.ones(g["block"], bool)
    f = O.select_rows(conf, m, g["tau"], O.SELECT_FACTOR, factor=g["factor"])
    t = O.select_rows(conf, m, g["tau"])
    assert f.sum() == g["expected"]["factor_n_commit"]
    assert t.sum() == g["expected"]["threshold_n_commit"]


def test_c5_factor_rule_strict_boundary_and_fallback():
    """(n+1)(1-c_(n)) < f with f = 1 is c_(n) > n/(n+1): exactly at the
    boundary the size is not admitted; with no admissible size the most
    confident row alone is committed."""
    conf = np.array([0.5, 0.9, 0.25])   # sorted: 0.9 (row 1), 0.5 (row 0), 0.25
    c = O.select_rows(conf, np.ones(3, bool), 0.9, O.SELECT_FACTOR, factor=1.0)
    assert c.tolist() == [False, True, False]         # n=1: 2*0.1 < 1; n=2: 3*0.5 = 1.5
    conf = np.array([0.5, 0.5])
    c = O.select_rows(conf, np.ones(2, bool), 0.9, O.SELECT_FACTOR, factor=1.0)
    assert c.tolist() == [True, False]                # 2*(1-0.5) = 1 is not < 1: fallback
    conf = np.array([0.75, 0.5])
    c = O.select_rows(conf, np.ones(2, bool), 0.9, O.SELECT_FACTOR, factor=1.5)
    assert c.tolist() == [True, False]                # n=2: 3*(1-0.5) = 1.5 is not < 1.5
    conf = np.array([0.8, 0.95, 0.7, 0.1])
    c = O.select_rows(conf, np.ones(4, bool), 0.9, O.SELECT_FACTOR, factor=2.0)
    assert c.tolist() == [True, True, True, False]    # 4*0.3 = 1.2 < 2; 5*0.9 = 4.5


def test_commit_update_applies_only_committed():
    tokens = np.array([[5, 6, 7]])
    masked = np.array([[1, 1, 0]], dtype=np.uint8)
    t, m = O.commit_update(tokens, masked, np.array([[9, 8, 7]]), np.array([[False, True, False]]))
    assert t.tolist() == [[5, 8, 7]] and m.tolist() == [[1, 0, 0]]


# ----------------------------------------------------------------------------
# C-7  LM head, C-8 append
# ----------------------------------------------------------------------------

def test_c7_lm_head_exact_on_integers():
    r = rng(12)
    M, H, V = 5, 7, 11
    x = r.integers(-4, 5, (M, H))
    w = r.integers(-4, 5, (V, H))
    got = O.lm_head(x, w)
    for i in range(M):
        for v in range(V):
            assert got[i, v] == sum(int(x[i, k]) * int(w[v, k]) for k in range(H))


def test_c8_append_reproduces_concatenation():
    r = rng(13)
    B, Hkv, cap, d, D = 2, 3, 20, 4, 4
    cache = np.zeros((B, Hkv, cap, d))
    ln = np.array([0, 4])
    parts = [[], []]
    pre = r.standard_normal((B, Hkv, 4, d))
    cache[1, :, :4] = pre[1]
    parts[1].append(pre[1])
    for _ in range(3):
        new = r.standard_normal((B, Hkv, D, d))
        cache, ln = O.kv_append(cache, new, ln)
        parts[0].append(new[0]); parts[1].append(new[1])
    assert ln.tolist() == [12, 16]
    for b in range(B):
        cat = np.concatenate(parts[b], axis=1)
        np.testing.assert_array_equal(cache[b, :, :cat.shape[1]], cat)
        assert not cache[b, :, cat.shape[1]:].any()
    with pytest.raises(ValueError):
        O.kv_append(cache, r.standard_normal((B, Hkv, 8, d)), ln)


def test_kv_write_refresh_and_append_agree():
    """[v1] Algorithm 1 refresh: writing all P + L positions from 0 leaves
    exactly the new K/V and lengths P + L; a write at the common length of
    every sequence is the append of the same block."""
    r = rng(33)
    B, Hkv, cap, d = 3, 2, 24, 4
    cache = r.standard_normal((B, Hkv, cap, d))
    full = r.standard_normal((B, Hkv, cap, d))
    c2, ln = O.kv_write(cache, full, 0)
    np.testing.assert_array_equal(c2, full)
    assert ln.tolist() == [cap] * B
    blk = r.standard_normal((B, Hkv, 8, d))
    cw, lw = O.kv_write(cache, blk, 8)
    ca, la = O.kv_append(cache, blk, np.full(B, 8))
    np.testing.assert_array_equal(cw, ca)
    assert lw.tolist() == la.tolist() == [16] * B
    np.testing.assert_array_equal(cw[:, :, :8], cache[:, :, :8])
    np.testing.assert_array_equal(cw[:, :, 16:], cache[:, :, 16:])
    with pytest.raises(ValueError):
        O.kv_write(cache, blk, cap - 7)
    with pytest.raises(ValueError):
        O.kv_write(cache, blk, -1)


# ----------------------------------------------------------------------------
# prefill / refresh attention (multi-block queries)
# ----------------------------------------------------------------------------

def test_prefill_rows_equal_cached_block_steps():
    """Block-causal prefill of a sequence: the rows of each block equal the
    cached step of that block (prefix = everything before it, block = itself)."""
    r = rng(20)
    B, Hq, Hkv, d, D, T = 2, 4, 2, 8, 8, 40
    q = r.standard_normal((B, T, Hq, d))
    k, v = r.standard_normal((B, Hkv, T, d)), r.standard_normal((B, Hkv, T, d))
    out, lse = O.prefill_attention(q, k, v, 0, T, D, causal=True)
    for blk in range(T // D):
        lp = blk * D
        o2, l2 = O.block_attention(q[:, lp:lp + D], k, v, k[:, :, lp:lp + D], v[:, :, lp:lp + D], [lp] * B)
        np.testing.assert_allclose(out[:, lp:lp + D], o2, atol=1e-12)
        np.testing.assert_allclose(lse[:, :, lp:lp + D], l2, atol=1e-12)


def test_prefill_key_counts_and_bidirectional():
    """q = 0 gives equal scores, so lse = ln(number of visible keys): the
    block end for the causal rule (capped at n_keys), all n_keys otherwise;
    the bidirectional form equals the DualCache step with the block fresh."""
    r = rng(21)
    B, Hq, Hkv, d, D, nk = 1, 2, 1, 4, 8, 30
    q0 = np.zeros((B, 12, Hq, d))
    k, v = r.standard_normal((B, Hkv, 32, d)), r.standard_normal((B, Hkv, 32, d))
    _, lse = O.prefill_attention(q0, k, v, 10, nk, D, causal=True)
    for i in range(12):
        p = 10 + i
        assert abs(lse[0, 0, i] - math.log(min(nk, (p // D + 1) * D))) < 1e-14
    _, lse = O.prefill_attention(q0, k, v, 10, nk, D, causal=False)
    np.testing.assert_allclose(lse, math.log(nk), atol=1e-14)
    q = r.standard_normal((B, D, Hq, d))
    out, _ = O.prefill_attention(q, k, v, 16, 32, D, causal=False)
    o2, _ = O.block_attention(q, k, v, k[:, :, 16:24], v[:, :, 16:24], [16], mode=O.DUAL_CACHE, total_len=32)
    np.testing.assert_allclose(out, o2, atol=1e-12)
