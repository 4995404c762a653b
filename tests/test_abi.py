"""The C ABI library loads, exports every declared entry point and validates
its arguments on the host (no kernel is launched by these checks)."""
import ctypes
import os
import re

import pytest

from block_diffusion_decoding_attn_amd import fdl, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "fdl.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fdl_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fdl.LIB_PATH):
        pytest.skip("libfdl.so not built")
    return fdl.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert set(names) == set(fdl.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_strerror(L):
    assert fdl.fdl_version() == 100
    for code in (0, -1, -2, -3, -4):
        assert fdl.fdl_strerror(code) not in ("", "unknown status")
    assert fdl.fdl_strerror(7) == "unknown status"


def _dims(name="qwen2.5-7b_bs4", **over):
    d = fdl.make_dims(synth.get_config(name))
    for k, v in over.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("over,code", [
    ({}, fdl.FDL_OK),
    ({"batch": 0}, fdl.FDL_E_INVAL),
    ({"n_q_heads": 27}, fdl.FDL_E_INVAL),
    ({"sub_block": 5}, fdl.FDL_E_INVAL),
    ({"gen_len": 500}, fdl.FDL_E_INVAL),
    ({"dtype": 7}, fdl.FDL_E_INVAL),
    ({"attn_mode": 3}, fdl.FDL_E_INVAL),
    ({"head_dim": 96}, fdl.FDL_E_UNSUPPORTED),
    ({"prompt_len": -1}, fdl.FDL_E_INVAL),
])
def test_dims_check(L, over, code):
    assert fdl.fdl_dims_check(_dims(**over)) == code


def test_workspace_sizes(L):
    for name in synth.CONFIG_ORDER:
        cfg = synth.get_config(name)
        d = fdl.make_dims(cfg)
        ws = fdl.fdl_block_attn_workspace_size(d)
        rows = cfg.batch * cfg.n_q_heads * cfg.sub_block
        if cfg.dtype == "f32":
            # split partials (m, l, O) per query row
            assert ws == 0 or ws % (rows * (cfg.head_dim + 2) * 4) == 0
        else:
            # per split, KV head and 64-lane wave of 32 rows: the wave's d/2 O values
            # as bf16 pairs, m and l (d/4 + 2 32-bit words per lane)
            pairs = cfg.batch * cfg.n_kv_heads
            g_rows = cfg.n_q_heads // cfg.n_kv_heads * cfg.sub_block
            nw = 2 if g_rows <= 64 else 4 if g_rows <= 128 else 8
            per_split = pairs * nw * 64 * (cfg.head_dim // 4 + 2) * 4
            assert ws == 0 or (ws % per_split == 0 and ws > 0), (name, ws)
        assert fdl.fdl_conf_select_workspace_size(d, cfg.sub_block) >= cfg.batch * cfg.sub_block * 16
    assert fdl.fdl_block_attn_workspace_size(_dims(batch=0)) == 0
    assert fdl.fdl_conf_select_workspace_size(_dims(), 0) == 0
    assert fdl.fdl_conf_select_workspace_size(_dims(), 257) == 0


def test_entry_points_reject_before_launch(L):
    """Invalid scalars or null pointers return an error without launching."""
    d = _dims()
    P = ctypes.c_void_p
    fake = P(16)  # never dereferenced: validation fails first
    by = ctypes.byref
    # block index out of range, sub index out of range, null pointers
    assert L.fdl_block_attn(by(d), 16, 0, fake, fake, fake, None, fake, fake, fake, None, None, 0, None) == -1
    assert L.fdl_block_attn(by(d), 0, 4, fake, fake, fake, None, fake, fake, fake, None, None, 0, None) == -1
    assert L.fdl_block_attn(by(d), 0, 0, None, fake, fake, None, fake, fake, fake, None, None, 0, None) == -1
    assert L.fdl_block_attn(None, 0, 0, fake, fake, fake, None, fake, fake, fake, None, None, 0, None) == -1
    d96 = _dims(head_dim=96)
    assert L.fdl_block_attn(by(d96), 0, 0, fake, fake, fake, None, fake, fake, fake, None, None, 0, None) == -2
    # too many rows per KV head for one workgroup
    dbig = _dims(n_q_heads=28 * 2, n_kv_heads=2, sub_block=32)
    assert L.fdl_block_attn(by(dbig), 0, 0, fake, fake, fake, None, fake, fake, fake, None, None, 0, None) == -2
    # prefill / refresh attention
    assert L.fdl_prefill_attn(by(d), 0, 0, 32, 1, fake, fake, fake, fake, None, None) == -1
    assert L.fdl_prefill_attn(by(d), -1, 32, 32, 1, fake, fake, fake, fake, None, None) == -1
    assert L.fdl_prefill_attn(by(d), 0, 32, 1537, 1, fake, fake, fake, fake, None, None) == -1
    assert L.fdl_prefill_attn(by(d), 0, 32, 32, 2, fake, fake, fake, fake, None, None) == -1
    assert L.fdl_prefill_attn(by(d), 0, 32, 32, 1, None, fake, fake, fake, None, None) == -1
    assert L.fdl_prefill_attn(by(_dims("tiny_fp32")), 0, 32, 32, 1, fake, fake, fake, fake, None, None) == -2
    # lm head
    assert L.fdl_lm_head(by(d), 0, fake, fake, fake, None) == -1
    assert L.fdl_lm_head(by(d), 4, None, fake, fake, None) == -1
    assert L.fdl_lm_head(by(_dims(hidden=3600)), 4, fake, fake, fake, None) == -2
    df = _dims("tiny_fp32")
    assert L.fdl_lm_head(by(df), 65, fake, fake, fake, None) == -2
    # select
    args = [fake, fake, fake, fake]
    assert L.fdl_conf_select(by(d), 0, fake, fake, fake, 0, 0, 0.0, *args, None, None, fake, 1 << 20, None) == -1
    assert L.fdl_conf_select(by(d), 8, fake, fake, None, 0, 0, 0.0, *args, None, None, fake, 1 << 20, None) == -1
    assert L.fdl_conf_select(by(d), 8, fake, fake, fake, 1, 0, 0.0, *args, None, None, fake, 1 << 20, None) == -1
    assert L.fdl_conf_select(by(d), 8, fake, fake, fake, 2, 0, ctypes.c_float(0.0), *args, None, None, fake,
                             1 << 20, None) == -1
    assert L.fdl_conf_select(by(d), 8, fake, fake, fake, 5, 0, 0.0, *args, None, None, fake, 1 << 20, None) == -1
    # append
    assert L.fdl_kv_append(by(d), fake, fake, fake, fake, 0, fake, None) == -1
    assert L.fdl_kv_append(by(d), fake, fake, fake, fake, 1537, fake, None) == -1
    assert L.fdl_kv_append(by(d), fake, fake, fake, fake, 32, None, None) == -1
    # write at a position: inside the cache, with a block to write
    assert L.fdl_kv_write(by(d), fake, fake, fake, fake, -1, 32, fake, None) == -1
    assert L.fdl_kv_write(by(d), fake, fake, fake, fake, 1536 - 31, 32, fake, None) == -1
    assert L.fdl_kv_write(by(d), fake, fake, fake, fake, 0, 0, fake, None) == -1
    assert L.fdl_kv_write(by(d), fake, None, fake, fake, 0, 32, fake, None) == -1
    assert L.fdl_kv_write(None, fake, fake, fake, fake, 0, 32, None, None) == -1


def test_workspace_too_small_rejected(L):
    """A missing or short workspace returns FDL_E_WORKSPACE before any launch."""
    d = _dims()
    P = ctypes.c_void_p
    fake = P(16)
    by = ctypes.byref
    args = [fake, fake, fake, fake]
    # the 7B/bs4 step splits its keys, so block attention needs partials space
    assert fdl.fdl_block_attn_workspace_size(d) > 0
    assert L.fdl_block_attn(by(d), 0, 0, fake, fake, fake, None, fake, fake, fake, None, None, 0, None) == -4
    assert L.fdl_block_attn(by(d), 15, 3, fake, fake, fake, None, fake, fake, fake, None, fake, 64, None) == -4
    need = fdl.fdl_conf_select_workspace_size(d, 8)
    assert L.fdl_conf_select(by(d), 8, fake, fake, fake, 0, 0, 0.0, *args, None, None, fake, need - 1, None) == -4
    assert L.fdl_conf_select(by(d), 8, fake, fake, fake, 0, 0, 0.0, *args, None, None, None, need, None) == -4
    need = fdl.fdl_lm_head_select_workspace_size(d, 8)
    assert need >= 32 * 16
    assert L.fdl_lm_head_select(by(d), 8, fake, fake, None, fake, fake, 0, 0, 0.0, *args, None, None, fake,
                                need - 1, None) == -4
    assert L.fdl_lm_head_select(by(d), 8, fake, fake, None, fake, fake, 0, 0, 0.0, *args, None, None, None,
                                need, None) == -4
    # the long-context shape: the tiled LM head keeps one partial per 256-row weight tile
    dl = _dims("qwen2.5-7b_long_bs16")
    assert fdl.fdl_lm_head_select_workspace_size(dl, 32) >= 16 * 32 * ((152064 + 255) // 256) * 16


def _decode_args(**over):
    fake = 16
    a = fdl.fdl_decode_args(w=fake, gain=2.0, mask_id=10, eos_id=11, prompt=fake, boost_tok=fake, boost_val=fake,
                            tau=fake, mode=0, k=0, factor=1.0, max_blocks=0, k_cache=fake, v_cache=fake, len=fake,
                            tokens=fake, masked=fake, seq_steps=fake, eos_block=fake, counters=fake, trace_cap=0)
    for k, v in over.items():
        setattr(a, k, v)
    return a


def test_decode_slots_and_workspace(L):
    d = _dims()
    nb, subs, S = 512 // 32, 32 // 8, 8
    assert fdl.fdl_decode_step_slots(d, fdl.FDL_SELECT_THRESHOLD, 0, 0) == nb * subs * S
    assert fdl.fdl_decode_step_slots(d, fdl.FDL_SELECT_FACTOR, 0, 2) == 2 * subs * S
    assert fdl.fdl_decode_step_slots(d, fdl.FDL_SELECT_TOPK, 3, 1) == subs * 3
    assert fdl.fdl_decode_step_slots(d, fdl.FDL_SELECT_TOPK, 0, 1) == 0
    assert fdl.fdl_decode_step_slots(d, fdl.FDL_SELECT_THRESHOLD, 0, nb + 1) == 0
    ws = fdl.fdl_decode_workspace_size(d)
    assert ws >= fdl.fdl_block_attn_workspace_size(d) + fdl.fdl_lm_head_select_workspace_size(d, 8)
    assert fdl.fdl_decode_workspace_size(_dims(batch=0)) == 0


def test_decode_rejects_before_launch(L):
    d = _dims()
    by = ctypes.byref
    ws = fdl.fdl_decode_workspace_size(d)
    fake = ctypes.c_void_p(16)

    def call(dims=d, args=None, wsz=ws, w=fake):
        return L.fdl_decode(by(dims), by(args if args is not None else _decode_args()), w, wsz, None)

    assert L.fdl_decode(by(d), None, fake, ws, None) == -1
    assert call(args=_decode_args(w=None)) == -1
    assert call(args=_decode_args(prompt=None)) == -1
    assert call(args=_decode_args(mask_id=152064)) == -1
    assert call(args=_decode_args(eos_id=-1)) == -1
    assert call(args=_decode_args(gain=float("nan"))) == -1
    assert call(args=_decode_args(max_blocks=17)) == -1
    assert call(args=_decode_args(tau=None)) == -1
    assert call(args=_decode_args(mode=1, k=0)) == -1
    assert call(args=_decode_args(mode=2, factor=0.0)) == -1
    assert call(args=_decode_args(trace_meta=16)) == -1           # trace pointers: all or none
    full = dict(trace_meta=16, trace_tokens=16, trace_masked=16, trace_token=16, trace_conf=16)
    slots = fdl.fdl_decode_step_slots(d, 0, 0, 0)
    assert call(args=_decode_args(trace_cap=slots - 1, **full)) == -1
    assert call(dims=_dims(hidden=3520)) == -2                    # stand-in model needs H = Hq * d
    assert call(wsz=ws - 1) == -4
    assert call(w=None) == -4


def test_noalloc_rejects_oversized_problem(L):
    """The allocation-free LM head + select refuses, before any launch, a
    problem whose select partials exceed the library's static scratch."""
    cfg = synth.small_variant(synth.get_config("qwen2.5-7b_long_bs16"), vocab=1 << 24, hidden=64)
    d = fdl.make_dims(cfg)
    assert fdl.fdl_lm_head_select_workspace_size(d, 32) > fdl.FDL_NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    rc = L.fdl_lm_head_select_noalloc(ctypes.byref(d), 32, fake, fake, None, fake, fake, fdl.FDL_SELECT_THRESHOLD,
                                      0, ctypes.c_float(1.0), fake, fake, fake, fake, None, None, None)
    assert rc == fdl.FDL_E_SCRATCH
    assert "scratch" in fdl.fdl_strerror(rc)
