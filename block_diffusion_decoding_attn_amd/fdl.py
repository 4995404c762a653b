"""ctypes binding of libfdl (include/fdl.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Functions keep the C names and take torch tensors that live on the
current HIP device; work is enqueued on torch's current stream.  A missing or
unloadable library raises immediately -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfdl.so")

FDL_OK, FDL_E_INVAL, FDL_E_UNSUPPORTED, FDL_E_HIP, FDL_E_WORKSPACE, FDL_E_SCRATCH = 0, -1, -2, -3, -4, -5
FDL_NOALLOC_SCRATCH_BYTES = 8 << 20
FDL_F32, FDL_BF16 = 0, 1
FDL_ATTN_BLOCK_CAUSAL, FDL_ATTN_DUAL_CACHE = 0, 1
FDL_SELECT_THRESHOLD, FDL_SELECT_TOPK, FDL_SELECT_FACTOR = 0, 1, 2

EXPORTS = (
    "fdl_version", "fdl_strerror", "fdl_dims_check", "fdl_block_attn_workspace_size", "fdl_block_attn",
    "fdl_prefill_attn",
    "fdl_lm_head", "fdl_conf_select_workspace_size", "fdl_conf_select", "fdl_lm_head_select_workspace_size",
    "fdl_lm_head_select", "fdl_lm_head_select_noalloc", "fdl_kv_append", "fdl_kv_write", "fdl_decode_workspace_size", "fdl_decode_step_slots",
    "fdl_decode",
)


class FdlError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed: {code} ({msg})")
        self.code = code


class fdl_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "prompt_len", "gen_len", "block", "sub_block", "n_q_heads", "n_kv_heads", "head_dim",
        "hidden", "vocab", "dtype", "attn_mode")]


class fdl_decode_args(ctypes.Structure):
    _fields_ = [
        ("w", ctypes.c_void_p), ("gain", ctypes.c_float), ("mask_id", ctypes.c_int32), ("eos_id", ctypes.c_int32),
        ("prompt", ctypes.c_void_p), ("boost_tok", ctypes.c_void_p), ("boost_val", ctypes.c_void_p),
        ("tau", ctypes.c_void_p), ("mode", ctypes.c_int32), ("k", ctypes.c_int32), ("factor", ctypes.c_float),
        ("max_blocks", ctypes.c_int32),
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p), ("len", ctypes.c_void_p),
        ("tokens", ctypes.c_void_p), ("masked", ctypes.c_void_p), ("seq_steps", ctypes.c_void_p),
        ("eos_block", ctypes.c_void_p), ("counters", ctypes.c_void_p),
        ("trace_cap", ctypes.c_int32), ("trace_meta", ctypes.c_void_p), ("trace_tokens", ctypes.c_void_p),
        ("trace_masked", ctypes.c_void_p), ("trace_token", ctypes.c_void_p), ("trace_conf", ctypes.c_void_p),
    ]


def make_dims(cfg, batch: Optional[int] = None) -> fdl_dims:
    """fdl_dims from a workload description with the same field names."""
    return fdl_dims(
        batch=cfg.batch if batch is None else batch, prompt_len=cfg.prompt_len, gen_len=cfg.gen_len,
        block=cfg.block, sub_block=cfg.sub_block, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
        head_dim=cfg.head_dim, hidden=cfg.hidden, vocab=cfg.vocab,
        dtype=FDL_F32 if cfg.dtype == "f32" else FDL_BF16,
        attn_mode=FDL_ATTN_DUAL_CACHE if cfg.attn_mode == "dual_cache" else FDL_ATTN_BLOCK_CAUSAL)


_lib = None
_lock = threading.Lock()
_P = ctypes.c_void_p
_I = ctypes.c_int32
_D = ctypes.POINTER(fdl_dims)


def lib() -> ctypes.CDLL:
    """Load libfdl.so once (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                                   "`python -m block_diffusion_decoding_attn_amd.build`")
            L = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_LOCAL)
            L.fdl_version.restype = ctypes.c_int
            L.fdl_strerror.restype = ctypes.c_char_p
            L.fdl_strerror.argtypes = [ctypes.c_int]
            L.fdl_dims_check.argtypes = [_D]
            L.fdl_block_attn_workspace_size.restype = ctypes.c_size_t
            L.fdl_block_attn_workspace_size.argtypes = [_D]
            L.fdl_block_attn.argtypes = [_D, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
            L.fdl_prefill_attn.argtypes = [_D, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P]
            L.fdl_lm_head.argtypes = [_D, _I, _P, _P, _P, _P]
            L.fdl_conf_select_workspace_size.restype = ctypes.c_size_t
            L.fdl_conf_select_workspace_size.argtypes = [_D, _I]
            L.fdl_conf_select.argtypes = [_D, _I, _P, _P, _P, _I, _I, ctypes.c_float, _P, _P, _P, _P, _P, _P, _P,
                                          ctypes.c_size_t, _P]
            L.fdl_lm_head_select_workspace_size.restype = ctypes.c_size_t
            L.fdl_lm_head_select_workspace_size.argtypes = [_D, _I]
            L.fdl_lm_head_select.argtypes = [_D, _I, _P, _P, _P, _P, _P, _I, _I, ctypes.c_float, _P, _P, _P, _P, _P,
                                             _P, _P, ctypes.c_size_t, _P]
            L.fdl_lm_head_select_noalloc.argtypes = [_D, _I, _P, _P, _P, _P, _P, _I, _I, ctypes.c_float, _P, _P, _P,
                                                     _P, _P, _P, _P]
            L.fdl_kv_append.argtypes = [_D, _P, _P, _P, _P, _I, _P, _P]
            L.fdl_kv_write.argtypes = [_D, _P, _P, _P, _P, _I, _I, _P, _P]
            L.fdl_decode_workspace_size.restype = ctypes.c_size_t
            L.fdl_decode_workspace_size.argtypes = [_D]
            L.fdl_decode_step_slots.restype = ctypes.c_int32
            L.fdl_decode_step_slots.argtypes = [_D, _I, _I, _I]
            L.fdl_decode.argtypes = [_D, ctypes.POINTER(fdl_decode_args), _P, ctypes.c_size_t, _P]
            _lib = L
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check(fn: str, rc: int):
    if rc != FDL_OK:
        raise FdlError(fn, rc, lib().fdl_strerror(rc).decode())


def _dtype(d: fdl_dims) -> torch.dtype:
    return torch.float32 if d.dtype == FDL_F32 else torch.bfloat16


def _expect(name, t, shape, dtype):
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name}: expected {tuple(shape)} {dtype}, got {tuple(t.shape)} {t.dtype}")


def fdl_version() -> int:
    return lib().fdl_version()


def fdl_strerror(code: int) -> str:
    return lib().fdl_strerror(code).decode()


def fdl_dims_check(dims: fdl_dims) -> int:
    return lib().fdl_dims_check(ctypes.byref(dims))


def fdl_block_attn_workspace_size(dims: fdl_dims) -> int:
    return lib().fdl_block_attn_workspace_size(ctypes.byref(dims))


def fdl_conf_select_workspace_size(dims: fdl_dims, rows_per_seq: int) -> int:
    return lib().fdl_conf_select_workspace_size(ctypes.byref(dims), rows_per_seq)


def fdl_block_attn(dims: fdl_dims, block_idx: int, sub_idx: int, q, k_cache, v_cache, prefix_len, k_blk, v_blk,
                   out, lse=None, workspace=None, stream=None):
    d = dims
    dt = _dtype(d)
    cap = d.prompt_len + d.gen_len
    _expect("q", q, (d.batch, d.sub_block, d.n_q_heads, d.head_dim), dt)
    _expect("k_cache", k_cache, (d.batch, d.n_kv_heads, cap, d.head_dim), dt)
    _expect("v_cache", v_cache, (d.batch, d.n_kv_heads, cap, d.head_dim), dt)
    _expect("k_blk", k_blk, (d.batch, d.n_kv_heads, d.block, d.head_dim), dt)
    _expect("v_blk", v_blk, (d.batch, d.n_kv_heads, d.block, d.head_dim), dt)
    _expect("out", out, (d.batch, d.sub_block, d.n_q_heads, d.head_dim), dt)
    if prefix_len is not None:
        _expect("prefix_len", prefix_len, (d.batch,), torch.int32)
    if lse is not None:
        _expect("lse", lse, (d.batch, d.n_q_heads, d.sub_block), torch.float32)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().fdl_block_attn(ctypes.byref(d), block_idx, sub_idx, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                              _ptr(prefix_len), _ptr(k_blk), _ptr(v_blk), _ptr(out), _ptr(lse), _ptr(workspace),
                              ws_bytes, _stream(stream))
    _check("fdl_block_attn", rc)
    return out


def fdl_prefill_attn(dims: fdl_dims, q_start: int, n_keys: int, causal: bool, q, k, v, out, lse=None,
                     stream=None):
    d = dims
    dt = _dtype(d)
    cap = d.prompt_len + d.gen_len
    n_q = q.shape[1]
    _expect("q", q, (d.batch, n_q, d.n_q_heads, d.head_dim), dt)
    _expect("k", k, (d.batch, d.n_kv_heads, cap, d.head_dim), dt)
    _expect("v", v, (d.batch, d.n_kv_heads, cap, d.head_dim), dt)
    _expect("out", out, (d.batch, n_q, d.n_q_heads, d.head_dim), dt)
    if lse is not None:
        _expect("lse", lse, (d.batch, d.n_q_heads, n_q), torch.float32)
    rc = lib().fdl_prefill_attn(ctypes.byref(d), q_start, n_q, n_keys, 1 if causal else 0, _ptr(q), _ptr(k),
                                _ptr(v), _ptr(out), _ptr(lse), _stream(stream))
    _check("fdl_prefill_attn", rc)
    return out


def fdl_lm_head(dims: fdl_dims, x, w, logits, stream=None):
    d = dims
    dt = _dtype(d)
    rows = x.shape[0]
    _expect("x", x, (rows, d.hidden), dt)
    _expect("w", w, (d.vocab, d.hidden), dt)
    _expect("logits", logits, (rows, d.vocab), torch.float32)
    rc = lib().fdl_lm_head(ctypes.byref(d), rows, _ptr(x), _ptr(w), _ptr(logits), _stream(stream))
    _check("fdl_lm_head", rc)
    return logits


def fdl_conf_select(dims: fdl_dims, rows_per_seq: int, logits, masked, tau, mode: int, k: int, factor: float,
                    token_out, conf_out, commit_out, n_commit, tokens_inout=None, masked_inout=None,
                    workspace=None, stream=None):
    d = dims
    B, R = d.batch, rows_per_seq
    if logits.dim() == 2:
        _expect("logits", logits, (B * R, d.vocab), torch.float32)
    else:
        _expect("logits", logits, (B, R, d.vocab), torch.float32)
    _expect("masked", masked, (B, R), torch.uint8)
    if tau is not None:
        _expect("tau", tau, (B,), torch.float32)
    _expect("token_out", token_out, (B, R), torch.int32)
    _expect("conf_out", conf_out, (B, R), torch.float32)
    _expect("commit_out", commit_out, (B, R), torch.uint8)
    _expect("n_commit", n_commit, (B,), torch.int32)
    if tokens_inout is not None:
        _expect("tokens_inout", tokens_inout, (B, R), torch.int32)
    if masked_inout is not None:
        _expect("masked_inout", masked_inout, (B, R), torch.uint8)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().fdl_conf_select(ctypes.byref(d), R, _ptr(logits), _ptr(masked), _ptr(tau), mode, k, factor,
                               _ptr(token_out), _ptr(conf_out), _ptr(commit_out), _ptr(n_commit),
                               _ptr(tokens_inout), _ptr(masked_inout), _ptr(workspace), ws_bytes, _stream(stream))
    _check("fdl_conf_select", rc)


def fdl_lm_head_select_workspace_size(dims: fdl_dims, rows_per_seq: int) -> int:
    return lib().fdl_lm_head_select_workspace_size(ctypes.byref(dims), rows_per_seq)


def fdl_lm_head_select(dims: fdl_dims, rows_per_seq: int, x, w, logits, masked, tau, mode: int, k: int,
                       factor: float, token_out, conf_out, commit_out, n_commit, tokens_inout=None,
                       masked_inout=None, workspace=None, stream=None):
    d = dims
    dt = _dtype(d)
    B, R = d.batch, rows_per_seq
    _expect("x", x, (B * R, d.hidden), dt)
    _expect("w", w, (d.vocab, d.hidden), dt)
    if logits is not None:
        _expect("logits", logits, (B * R, d.vocab), torch.float32)
    _expect("masked", masked, (B, R), torch.uint8)
    if tau is not None:
        _expect("tau", tau, (B,), torch.float32)
    _expect("token_out", token_out, (B, R), torch.int32)
    _expect("conf_out", conf_out, (B, R), torch.float32)
    _expect("commit_out", commit_out, (B, R), torch.uint8)
    _expect("n_commit", n_commit, (B,), torch.int32)
    if tokens_inout is not None:
        _expect("tokens_inout", tokens_inout, (B, R), torch.int32)
    if masked_inout is not None:
        _expect("masked_inout", masked_inout, (B, R), torch.uint8)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().fdl_lm_head_select(ctypes.byref(d), R, _ptr(x), _ptr(w), _ptr(logits), _ptr(masked), _ptr(tau),
                                  mode, k, factor, _ptr(token_out), _ptr(conf_out), _ptr(commit_out),
                                  _ptr(n_commit), _ptr(tokens_inout), _ptr(masked_inout), _ptr(workspace), ws_bytes,
                                  _stream(stream))
    _check("fdl_lm_head_select", rc)


def fdl_lm_head_select_noalloc(dims: fdl_dims, rows_per_seq: int, x, w, logits, masked, tau, mode: int, k: int,
                               factor: float, token_out, conf_out, commit_out, n_commit, tokens_inout=None,
                               masked_inout=None, stream=None):
    """fdl_lm_head_select with the library's static scratch instead of a workspace."""
    d = dims
    dt = _dtype(d)
    B, R = d.batch, rows_per_seq
    _expect("x", x, (B * R, d.hidden), dt)
    _expect("w", w, (d.vocab, d.hidden), dt)
    if logits is not None:
        _expect("logits", logits, (B * R, d.vocab), torch.float32)
    _expect("masked", masked, (B, R), torch.uint8)
    if tau is not None:
        _expect("tau", tau, (B,), torch.float32)
    _expect("token_out", token_out, (B, R), torch.int32)
    _expect("conf_out", conf_out, (B, R), torch.float32)
    _expect("commit_out", commit_out, (B, R), torch.uint8)
    _expect("n_commit", n_commit, (B,), torch.int32)
    if tokens_inout is not None:
        _expect("tokens_inout", tokens_inout, (B, R), torch.int32)
    if masked_inout is not None:
        _expect("masked_inout", masked_inout, (B, R), torch.uint8)
    rc = lib().fdl_lm_head_select_noalloc(ctypes.byref(d), R, _ptr(x), _ptr(w), _ptr(logits), _ptr(masked),
                                          _ptr(tau), mode, k, factor, _ptr(token_out), _ptr(conf_out),
                                          _ptr(commit_out), _ptr(n_commit), _ptr(tokens_inout), _ptr(masked_inout),
                                          _stream(stream))
    _check("fdl_lm_head_select_noalloc", rc)


def fdl_kv_append(dims: fdl_dims, k_cache, v_cache, k_new, v_new, length, stream=None):
    d = dims
    dt = _dtype(d)
    cap = d.prompt_len + d.gen_len
    n_new = k_new.shape[2]
    _expect("k_cache", k_cache, (d.batch, d.n_kv_heads, cap, d.head_dim), dt)
    _expect("v_cache", v_cache, (d.batch, d.n_kv_heads, cap, d.head_dim), dt)
    _expect("k_new", k_new, (d.batch, d.n_kv_heads, n_new, d.head_dim), dt)
    _expect("v_new", v_new, (d.batch, d.n_kv_heads, n_new, d.head_dim), dt)
    _expect("len", length, (d.batch,), torch.int32)
    rc = lib().fdl_kv_append(ctypes.byref(d), _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), n_new,
                             _ptr(length), _stream(stream))
    _check("fdl_kv_append", rc)


def fdl_kv_write(dims: fdl_dims, k_cache, v_cache, k_new, v_new, pos: int, length=None, stream=None):
    d = dims
    dt = _dtype(d)
    cap = d.prompt_len + d.gen_len
    n_new = k_new.shape[2]
    _expect("k_cache", k_cache, (d.batch, d.n_kv_heads, cap, d.head_dim), dt)
    _expect("v_cache", v_cache, (d.batch, d.n_kv_heads, cap, d.head_dim), dt)
    _expect("k_new", k_new, (d.batch, d.n_kv_heads, n_new, d.head_dim), dt)
    _expect("v_new", v_new, (d.batch, d.n_kv_heads, n_new, d.head_dim), dt)
    if length is not None:
        _expect("len", length, (d.batch,), torch.int32)
    rc = lib().fdl_kv_write(ctypes.byref(d), _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), pos, n_new,
                            _ptr(length), _stream(stream))
    _check("fdl_kv_write", rc)


def fdl_decode_workspace_size(dims: fdl_dims) -> int:
    return lib().fdl_decode_workspace_size(ctypes.byref(dims))


def fdl_decode_step_slots(dims: fdl_dims, mode: int, k: int, max_blocks: int) -> int:
    return lib().fdl_decode_step_slots(ctypes.byref(dims), mode, k, max_blocks)


def fdl_decode(dims: fdl_dims, w, prompt, boost_tok, boost_val, tau, mode: int, k: int, factor: float,
               mask_id: int, eos_id: int, gain: float, max_blocks: int, k_cache, v_cache, length, tokens, masked,
               seq_steps, eos_block, counters, trace=None, workspace=None, stream=None):
    """trace: None, or a dict of tensors meta [T][2], tokens [T][B][D], masked
    [T][B][D], token [T][B][S], conf [T][B][S]."""
    d = dims
    dt = _dtype(d)
    B, P, L, D, S = d.batch, d.prompt_len, d.gen_len, d.block, d.sub_block
    cap = P + L
    _expect("w", w, (d.vocab, d.hidden), dt)
    if P > 0:
        _expect("prompt", prompt, (B, P), torch.int32)
    _expect("boost_tok", boost_tok, (B, L), torch.int32)
    _expect("boost_val", boost_val, (B, L), torch.float32)
    if tau is not None:
        _expect("tau", tau, (B,), torch.float32)
    _expect("k_cache", k_cache, (B, d.n_kv_heads, cap, d.head_dim), dt)
    _expect("v_cache", v_cache, (B, d.n_kv_heads, cap, d.head_dim), dt)
    _expect("len", length, (B,), torch.int32)
    _expect("tokens", tokens, (B, cap), torch.int32)
    _expect("masked", masked, (B, cap), torch.uint8)
    _expect("seq_steps", seq_steps, (B,), torch.int32)
    _expect("eos_block", eos_block, (B,), torch.int32)
    _expect("counters", counters, (2,), torch.int32)
    a = fdl_decode_args(w=_ptr(w), gain=gain, mask_id=mask_id, eos_id=eos_id, prompt=_ptr(prompt) if P else None,
                        boost_tok=_ptr(boost_tok), boost_val=_ptr(boost_val), tau=_ptr(tau), mode=mode, k=k,
                        factor=factor, max_blocks=max_blocks, k_cache=_ptr(k_cache), v_cache=_ptr(v_cache),
                        len=_ptr(length), tokens=_ptr(tokens), masked=_ptr(masked), seq_steps=_ptr(seq_steps),
                        eos_block=_ptr(eos_block), counters=_ptr(counters), trace_cap=0)
    if trace is not None:
        T = trace["meta"].shape[0]
        _expect("trace meta", trace["meta"], (T, 2), torch.int32)
        _expect("trace tokens", trace["tokens"], (T, B, D), torch.int32)
        _expect("trace masked", trace["masked"], (T, B, D), torch.uint8)
        _expect("trace token", trace["token"], (T, B, S), torch.int32)
        _expect("trace conf", trace["conf"], (T, B, S), torch.float32)
        a.trace_cap = T
        a.trace_meta, a.trace_tokens, a.trace_masked = (_ptr(trace[n]) for n in ("meta", "tokens", "masked"))
        a.trace_token, a.trace_conf = _ptr(trace["token"]), _ptr(trace["conf"])
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().fdl_decode(ctypes.byref(d), ctypes.byref(a), _ptr(workspace), ws_bytes, _stream(stream))
    _check("fdl_decode", rc)
