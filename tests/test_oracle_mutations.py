"""Each plausible mistake planted in the oracle (on the CPU, via monkeypatch)
must make at least one pin fail: those of test_oracle_pins for the step
functions, those of test_decode_oracle_pins for the decode loop."""
import math

import numpy as np
import pytest

import test_decode_oracle_pins as DP
import test_oracle_pins as P
from oracle import fdl_decode_oracle as D
from oracle import fdl_oracle as O


def _pins(module):
    out = []
    for name, fn in sorted(vars(module).items()):
        if not name.startswith("test_") or not callable(fn):
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if params:
            for args in params[0].args[1]:
                out.append((f"{name}{args}", fn, args))
        else:
            out.append((name, fn, ()))
    return out


def _failures(module=P):
    bad = []
    for name, fn, args in _pins(module):
        try:
            fn(*args)
        except Exception:          # noqa: BLE001 - any failure counts
            bad.append(name)
    return bad


def test_pins_all_pass_unmutated():
    assert _failures(P) == []
    assert _failures(DP) == []


def _m_scale(d):
    return 1.0 / d


def _m_gqa(h, hq, hkv):
    return h % hkv


def _m_ge(c, tau):
    return c >= tau


def _m_order_high(cands, conf):
    return sorted(cands, key=lambda r: (-conf[r], -r))


_orig_visible = O.visible_keys


def _m_drop_last_key(lp, D, mode, total):
    return _orig_visible(lp, D, mode, total)[:-1]


def _m_no_block(lp, D, mode, total):
    return [k for k in _orig_visible(lp, D, mode, total) if k[1] != "block"]


def _m_no_suffix(lp, D, mode, total):
    return _orig_visible(lp, D, O.BLOCK_CAUSAL, total)


def _m_prefix_off_by_one(lp, D, mode, total):
    keys = _orig_visible(lp, D, mode, total)
    return [(j - 1, s) if s == "cache" and j > 0 else (j, s) for j, s in keys]


def _m_unnormalized(scores):
    m = scores.max()
    e = np.exp(scores - m)
    return e, m + math.log(e.sum())


def _m_last_argmax(row):
    l = np.asarray(row, dtype=np.float64)
    tok = len(l) - 1 - int(np.argmax(l[::-1]))
    m = l[tok]
    z = np.exp(l - m).sum()
    top2 = np.partition(l, -2)[-2]
    return tok, 1.0 / z, math.exp(top2 - m) / z


def _m_conf_logit(row):
    l = np.asarray(row, dtype=np.float64)
    tok = int(np.argmax(l))
    z = np.exp(l - l[tok]).sum()
    top2 = np.partition(l, -2)[-2]
    return tok, 1.0 / (z - 1.0 + 1e-300) if z > 1 else 1.0, math.exp(top2 - l[tok]) / z


_orig_append = O.kv_append


def _m_append_shift(cache, new, length):
    cache, length2 = _orig_append(cache, new, np.asarray(length))
    cache = np.roll(cache, 1, axis=2)
    return cache, length2


_orig_write = O.kv_write


def _m_write_keeps_length(cache, new, pos):
    c, ln = _orig_write(cache, new, pos)
    return c, ln - new.shape[2]


def _m_write_one_late(cache, new, pos):
    c, ln = _orig_write(cache, new, pos)
    return np.roll(c, 1, axis=2), ln


def _m_lm_head_transposed(x, w):
    return O._f64(x) @ O._f64(w)


_orig_select = O.select_rows


def _m_factor_le(conf, masked, tau, mode=O.SELECT_THRESHOLD, k=0, factor=1.0):
    if mode != O.SELECT_FACTOR:
        return _orig_select(conf, masked, tau, mode, k, factor)
    return _orig_select(conf, masked, tau, mode, k, factor + 1e-12)


def _m_no_fallback(conf, masked, tau, mode=O.SELECT_THRESHOLD, k=0, factor=1.0):
    if mode != O.SELECT_THRESHOLD:
        return _orig_select(conf, masked, tau, mode, k, factor)
    return np.asarray(masked, bool) & (np.asarray(conf) > tau)


def _m_bc_strict(p, j, block):
    return O.block_of(j, block) < O.block_of(p, block)


def _m_bc_token_causal(p, j, block):
    return j <= p


_orig_embed_kv = D.embed_kv


def _m_embed_kv_prev_token(w64, tokens_row, positions, hq, hkv, d):
    return _orig_embed_kv(w64, tokens_row, [max(p - 1, 0) for p in positions], hq, hkv, d)


def _m_sub_rows_no_block(block_size, sub_size, blk, sub):
    return range(sub * sub_size, sub * sub_size + sub_size)


def _m_never_eos(block_tokens, eos_id):
    return False


def _m_block_start_late(prompt_len, block_size, blk):
    return prompt_len + blk * block_size + 1


_orig_sm_embed = D.sm_embed


def _m_value_not_reversed(w64, token, hq, hkv, d):
    q, k, v = _orig_sm_embed(w64, token, hq, hkv, d)
    return q, k, v[:, ::-1]


def _m_hidden_no_attention(o_heads, w64, boost_tok, boost_val, gain):
    wt = w64[boost_tok]
    return boost_val * wt / float(wt @ wt) + 0.0 * o_heads.reshape(-1)


DECODE_MUTATIONS = [
    ("decode: K/V embedded from the previous position's token", "embed_kv", _m_embed_kv_prev_token),
    ("decode: sub-block rows without the block offset", "sub_rows", _m_sub_rows_no_block),
    ("decode: EOS never stops a sequence", "holds_eos", _m_never_eos),
    ("decode: block starts one position late", "block_start", _m_block_start_late),
    ("decode: value slice not reversed", "sm_embed", _m_value_not_reversed),
    ("decode: hidden row without the attention output", "sm_hidden", _m_hidden_no_attention),
]


MUTATIONS = [
    ("prefill: strictly earlier blocks only", "bc_visible", _m_bc_strict),
    ("prefill: token-causal instead of block-causal", "bc_visible", _m_bc_token_causal),
    ("score scale 1/d instead of 1/sqrt(d)", "score_scale", _m_scale),
    ("GQA head h % Hkv instead of h // G", "kv_head_of", _m_gqa),
    (">= tau instead of > tau", "above_threshold", _m_ge),
    ("ties to the higher row", "_order_by_conf", _m_order_high),
    ("last block key dropped", "visible_keys", _m_drop_last_key),
    ("block keys omitted", "visible_keys", _m_no_block),
    ("DualCache suffix omitted", "visible_keys", _m_no_suffix),
    ("prefix keys shifted by one position", "visible_keys", _m_prefix_off_by_one),
    ("softmax not normalized", "softmax_weights", _m_unnormalized),
    ("argmax tie to the highest id", "row_confidence", _m_last_argmax),
    ("confidence excludes the top token from the partition", "row_confidence", _m_conf_logit),
    ("append written one position late", "kv_append", _m_append_shift),
    ("write leaves the lengths at pos", "kv_write", _m_write_keeps_length),
    ("write one position late", "kv_write", _m_write_one_late),
    ("LM head with untransposed W", "lm_head", _m_lm_head_transposed),
    ("factor rule <= instead of <", "select_rows", _m_factor_le),
    ("threshold rule without fallback", "select_rows", _m_no_fallback),
]


@pytest.mark.parametrize("label,attr,fn", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, label, attr, fn):
    monkeypatch.setattr(O, attr, fn)
    bad = _failures(P)
    assert bad, f"no pin caught: {label}"


@pytest.mark.parametrize("label,attr,fn", DECODE_MUTATIONS, ids=[m[0] for m in DECODE_MUTATIONS])
def test_planted_decode_mistake_is_caught(monkeypatch, label, attr, fn):
    monkeypatch.setattr(D, attr, fn)
    bad = _failures(DP)
    assert bad, f"no pin caught: {label}"
