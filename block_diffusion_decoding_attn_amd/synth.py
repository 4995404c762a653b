"""Seeded synthetic inputs for the cached block-diffusion denoising step.

This module only draws and shapes input tensors; it performs none of the
step's own arithmetic (no attention, no projection, no selection).  Both the
HIP path and the CPU oracle consume exactly the tensors produced here.

Workload shapes follow the Fast-dLLM pages: block size D = 32 and sub-block
size 8 ("Fast-dLLM v2: Efficient Block-Diffusion LLM", Inference Pipeline,
"Sub-block size as a decoding granularity knob"), threshold tau = 0.9
(ibid., Level 2), prompt length P and answer length L ("Fast-dLLM: Reusing
Bidirectional State ...", section 2).  Head counts, hidden and vocabulary
sizes are those of Qwen2.5-1.5B/7B and LLaDA-8B.  The pages measure on
GSM8K/MATH/HumanEval/MBPP with trained checkpoints; seeded Gaussian tensors of
the same shapes stand in for them here.

Every tensor is drawn from its own torch CPU generator whose seed is derived
from (seed, config id, tensor id, index) with numpy's SeedSequence, so any
tensor can be regenerated on its own, on any host, bit for bit.  Values are
drawn in float32 and rounded once to the config's dtype (round to nearest
even for bfloat16).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Tuple

import numpy as np
import torch

# ----------------------------------------------------------------------------
# Workload configurations
# ----------------------------------------------------------------------------

BLOCK_CAUSAL = "block_causal"   # v2: block attends to itself and the cached prefix
DUAL_CACHE = "dual_cache"       # v1 DualCache: prefix cache + fresh block + cached suffix


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int
    dtype: str            # "f32" or "bf16"
    batch: int            # B
    n_q_heads: int        # Hq
    n_kv_heads: int       # Hkv
    head_dim: int         # d
    prompt_len: int       # P
    gen_len: int          # L
    block: int            # D
    sub_block: int        # S, query rows per step (= D for whole-block steps)
    hidden: int           # H
    vocab: int            # V
    attn_mode: str
    tau: Tuple[float, ...] = (0.9,)   # tau choices (one value => every sequence)
    description: str = ""

    @property
    def cap(self) -> int:
        """KV-cache capacity per sequence and head: P + L positions."""
        return self.prompt_len + self.gen_len

    @property
    def n_blocks(self) -> int:
        return self.gen_len // self.block

    @property
    def subs_per_block(self) -> int:
        return self.block // self.sub_block

    @property
    def rows(self) -> int:
        """LM-head rows per step: one per query position of every sequence."""
        return self.batch * self.sub_block

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


CONFIGS: Dict[str, Config] = {
    c.name: c
    for c in [
        Config("tiny_fp32", 0, "f32", 1, 4, 2, 64, 96, 32, 32, 32, 256, 512, BLOCK_CAUSAL,
               description="tiny fp32 single step: 96-token prefix + one 32-token block "
                           "(rows 0-7 committed, 8-31 masked), GQA 4/2, d 64, LM head 256->512"),
        Config("qwen2.5-1.5b_bs1", 1, "bf16", 1, 12, 2, 128, 512, 256, 32, 8, 1536, 151936, BLOCK_CAUSAL,
               description="Qwen2.5-1.5B shapes, batch 1, prompt 512, gen 256, sub-block 8"),
        Config("qwen2.5-7b_bs4", 2, "bf16", 4, 28, 4, 128, 1024, 512, 32, 8, 3584, 152064, BLOCK_CAUSAL,
               description="Qwen2.5-7B shapes, batch 4, prompt 1024, gen 512, sub-block 8"),
        Config("llada-8b_dualcache", 3, "bf16", 1, 32, 32, 128, 512, 1024, 32, 32, 4096, 126464, DUAL_CACHE,
               description="LLaDA-8B-style v1 DualCache, MHA 32 heads, prompt 512, gen 1024, block 32"),
        Config("qwen2.5-7b_long_bs16", 4, "bf16", 16, 28, 4, 128, 4096, 32, 32, 32, 3584, 152064, BLOCK_CAUSAL,
               tau=(0.7, 0.8, 0.9, 0.95),
               description="long-context stress: batch 16, 4096-token prefix cache, one 32-token block"),
    ]
}

CONFIG_ORDER: List[str] = list(CONFIGS)


def get_config(name_or_index) -> Config:
    if isinstance(name_or_index, int):
        return CONFIGS[CONFIG_ORDER[name_or_index]]
    return CONFIGS[name_or_index]


def small_variant(cfg: Config, **over) -> Config:
    """Same structure, smaller sizes (for parity cases the oracle finishes quickly)."""
    return dataclasses.replace(cfg, **over)


# ----------------------------------------------------------------------------
# Seeded draws
# ----------------------------------------------------------------------------

# tensor ids (stable: changing them changes every stored expectation)
T_Q, T_KCACHE, T_VCACHE, T_KBLK, T_VBLK, T_X, T_W = 1, 2, 3, 4, 5, 6, 7
T_BOOST_TOK, T_BOOST_VAL, T_MASK, T_TAU, T_LOGITS, T_KREFRESH, T_VREFRESH = 8, 9, 10, 11, 12, 13, 14


def _gen(seed: int, cfg_id: int, tensor_id: int, index: int = 0) -> torch.Generator:
    state = np.random.SeedSequence([seed, cfg_id, tensor_id, index]).generate_state(2, dtype=np.uint32)
    g = torch.Generator(device="cpu")
    g.manual_seed(int(state[0]) << 32 | int(state[1]))
    return g


def normal(shape, seed, cfg_id, tensor_id, index=0, std=1.0, dtype=torch.bfloat16) -> torch.Tensor:
    """N(0, std^2) float32 draws, rounded once to `dtype`."""
    g = _gen(seed, cfg_id, tensor_id, index)
    t = torch.randn(*shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def uniform(shape, seed, cfg_id, tensor_id, index=0, lo=0.0, hi=1.0) -> torch.Tensor:
    g = _gen(seed, cfg_id, tensor_id, index)
    return torch.rand(*shape, generator=g, dtype=torch.float64) * (hi - lo) + lo


def randint(shape, seed, cfg_id, tensor_id, index, lo, hi) -> torch.Tensor:
    g = _gen(seed, cfg_id, tensor_id, index)
    return torch.randint(lo, hi, shape, generator=g, dtype=torch.int64)


# ----------------------------------------------------------------------------
# Step inputs
# ----------------------------------------------------------------------------

def boost_shift(vocab: int, kind: str) -> float:
    """Offset added to the U(0,12) peaking boost.

    "literal": the boost exactly as the workload states it, U(0,12).  At a
    vocabulary of ~150k the log-partition of N(0,1) logits is ~12.4, so this
    almost never lifts a position above tau = 0.9 and every step commits by
    the fallback.  "calibrated": U(0,12) + ln(V/512), identical at V = 512 and
    giving roughly a quarter of positions above 0.9 at V ~ 150k, the outcome
    the workload describes.
    """
    if kind == "literal":
        return 0.0
    if kind == "calibrated":
        return math.log(vocab / 512.0)
    raise ValueError(kind)


def weights(cfg: Config, seed: int = 0) -> torch.Tensor:
    """LM-head weight W[V][H] ~ N(0, 1/H)."""
    return normal((cfg.vocab, cfg.hidden), seed, cfg.cfg_id, T_W, std=cfg.hidden ** -0.5, dtype=cfg.torch_dtype)


def hidden_rows(cfg: Config, w: torch.Tensor, step: int, seed: int = 0, boost: str = "calibrated",
                rows: int | None = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Final hidden rows X[M][H] for one step, with the peaking boost folded in.

    Each row r draws N(0,1) entries, a target token t_r ~ U{0..V-1} and a boost
    b_r ~ U(0,12) (+ shift).  The row is moved along W[t_r] by
    b_r * W[t_r] / |W[t_r]|^2 so that, before the single rounding to the
    config dtype, its logit for t_r rises by exactly b_r while the other
    logits move only by b_r * cos(W[t_r], W[v]) * |W[v]|/|W[t_r]| (~N(0, b_r^2/H)).
    Returns (x, t, b).
    """
    m = cfg.rows if rows is None else rows
    base = normal((m, cfg.hidden), seed, cfg.cfg_id, T_X, step, dtype=torch.float32).double()
    t = randint((m,), seed, cfg.cfg_id, T_BOOST_TOK, step, 0, cfg.vocab)
    b = uniform((m,), seed, cfg.cfg_id, T_BOOST_VAL, step, 0.0, 12.0) + boost_shift(cfg.vocab, boost)
    wt = w[t].double()
    base += (b / (wt * wt).sum(1)).unsqueeze(1) * wt
    return base.to(cfg.torch_dtype), t, b


def queries(cfg: Config, step: int, seed: int = 0, batch: int | None = None) -> torch.Tensor:
    """Q[B][S][Hq][d] ~ N(0,1)."""
    bsz = cfg.batch if batch is None else batch
    return normal((bsz, cfg.sub_block, cfg.n_q_heads, cfg.head_dim), seed, cfg.cfg_id, T_Q, step,
                  dtype=cfg.torch_dtype)


def kv_cache(cfg: Config, seed: int = 0, fill: int | None = None, batch: int | None = None):
    """K/V cache [B][Hkv][cap][d]; positions >= `fill` are zero (not yet written)."""
    bsz = cfg.batch if batch is None else batch
    shape = (bsz, cfg.n_kv_heads, cfg.cap, cfg.head_dim)
    k = normal(shape, seed, cfg.cfg_id, T_KCACHE, dtype=cfg.torch_dtype)
    v = normal(shape, seed, cfg.cfg_id, T_VCACHE, dtype=cfg.torch_dtype)
    if fill is not None and fill < cfg.cap:
        k[:, :, fill:] = 0
        v[:, :, fill:] = 0
    return k, v


def block_kv(cfg: Config, block_idx: int, seed: int = 0, batch: int | None = None):
    """Fresh K/V of the active block [B][Hkv][D][d]."""
    bsz = cfg.batch if batch is None else batch
    shape = (bsz, cfg.n_kv_heads, cfg.block, cfg.head_dim)
    return (normal(shape, seed, cfg.cfg_id, T_KBLK, block_idx, dtype=cfg.torch_dtype),
            normal(shape, seed, cfg.cfg_id, T_VBLK, block_idx, dtype=cfg.torch_dtype))


def refresh_kv(cfg: Config, block_idx: int, seed: int = 0, batch: int | None = None):
    """Refreshed full-context K/V [B][Hkv][P+L][d] for a v1 DualCache block boundary.

    Stands in for the model's recomputation of every position (the model
    itself is not part of the step)."""
    bsz = cfg.batch if batch is None else batch
    shape = (bsz, cfg.n_kv_heads, cfg.cap, cfg.head_dim)
    return (normal(shape, seed, cfg.cfg_id, T_KREFRESH, block_idx, dtype=cfg.torch_dtype),
            normal(shape, seed, cfg.cfg_id, T_VREFRESH, block_idx, dtype=cfg.torch_dtype))


def masked_rows(cfg: Config, step: int, seed: int = 0) -> torch.Tensor:
    """uint8 masked[B][S]: 1 = position still [MASK] (a commit candidate).

    tiny_fp32: block rows 0-7 committed, 8-31 masked.  Long-context stress: per
    sequence a uniformly random count in 0..24 (0-75% of 32) of committed
    positions, chosen uniformly.  Otherwise every row of the sub-block is
    masked (each sub-block is visited once, fully masked)."""
    B, S = cfg.batch, cfg.sub_block
    m = torch.ones((B, S), dtype=torch.uint8)
    if cfg.name == "tiny_fp32":
        m[:, :8] = 0
    elif cfg.name == "qwen2.5-7b_long_bs16":
        n = randint((B,), seed, cfg.cfg_id, T_MASK, step, 0, 25)
        for bi in range(B):
            g = _gen(seed, cfg.cfg_id, T_MASK, 1000 + step * 64 + bi)
            perm = torch.randperm(S, generator=g)
            m[bi, perm[: int(n[bi])]] = 0
    return m


def taus(cfg: Config, step: int = 0, seed: int = 0) -> torch.Tensor:
    """float32 tau[B]: one value for every sequence, or drawn per sequence."""
    if len(cfg.tau) == 1:
        return torch.full((cfg.batch,), cfg.tau[0], dtype=torch.float32)
    idx = randint((cfg.batch,), seed, cfg.cfg_id, T_TAU, step, 0, len(cfg.tau))
    return torch.tensor([cfg.tau[int(i)] for i in idx], dtype=torch.float32)


def logits_direct(rows: int, vocab: int, step: int, seed: int = 0, cfg_id: int = 99,
                  boost: str = "calibrated") -> torch.Tensor:
    """fp32 logits[rows][V] ~ N(0,1) with the one-token U(0,12) (+shift) boost
    added directly: a select-only input that both sides see bit for bit."""
    l = normal((rows, vocab), seed, cfg_id, T_LOGITS, step, dtype=torch.float32)
    t = randint((rows,), seed, cfg_id, T_BOOST_TOK, step, 0, vocab)
    b = uniform((rows,), seed, cfg_id, T_BOOST_VAL, step, 0.0, 12.0) + boost_shift(vocab, boost)
    l[torch.arange(rows), t] += b.float()
    return l


def schedule(cfg: Config) -> List[Tuple[int, int, bool]]:
    """(block_idx, sub_idx, append_after) for every denoising step of the workload.

    One step per sub-block (each sub-block visited once); the block's K/V is
    appended after its last sub-block.  v1 DualCache: one step per block, the
    cache being refreshed before each block."""
    out = []
    for b in range(cfg.n_blocks):
        for s in range(cfg.subs_per_block):
            out.append((b, s, s == cfg.subs_per_block - 1))
    return out


# ----------------------------------------------------------------------------
# Decode-loop inputs
# ----------------------------------------------------------------------------

T_PROMPT, T_EOS = 15, 16


@dataclasses.dataclass
class DecodeInputs:
    """Inputs of one run of the decode loop (whole generation of a batch).

    prompt [B][P] int32 token ids; boost_tok/boost_val [B][L] the drawn token
    and boost of every generated position (int32 / float32); tau [B] float32;
    eos_at [B] the generated position whose boost targets EOS (>= L: none);
    mask_id / eos_id the two reserved token ids; gain the attention-output
    gain of the stand-in model."""
    prompt: torch.Tensor
    boost_tok: torch.Tensor
    boost_val: torch.Tensor
    tau: torch.Tensor
    eos_at: torch.Tensor
    mask_id: int
    eos_id: int
    gain: float


def reserved_ids(vocab: int) -> Tuple[int, int]:
    """(mask_id, eos_id): the last two ids of the vocabulary."""
    return vocab - 1, vocab - 2


def decode_inputs(cfg: Config, seed: int = 0, boost: str = "calibrated", gain: float = 2.0,
                  eos: bool = True) -> DecodeInputs:
    """Seeded inputs of the decode loop.

    Prompt tokens and the boost targets are uniform over the ordinary ids
    0..V-3; boosts are U(0,12) (+ shift, as for the single-step rows).  With
    eos, each sequence draws eos_at ~ U{0..2L-1}: when it falls inside the
    generation, that position's boost targets EOS with the top boost
    12 (+ shift), so about half of the sequences stop early, at different
    blocks (the padded-batch case)."""
    B, P, L, V = cfg.batch, cfg.prompt_len, cfg.gen_len, cfg.vocab
    mask_id, eos_id = reserved_ids(V)
    prompt = randint((B, P), seed, cfg.cfg_id, T_PROMPT, 0, 0, V - 2).to(torch.int32)
    tok = randint((B, L), seed, cfg.cfg_id, T_BOOST_TOK, 7777, 0, V - 2)
    val = uniform((B, L), seed, cfg.cfg_id, T_BOOST_VAL, 7777, 0.0, 12.0) + boost_shift(V, boost)
    eos_at = randint((B,), seed, cfg.cfg_id, T_EOS, 0, 0, 2 * L) if eos else torch.full((B,), 2 * L)
    for b in range(B):
        p = int(eos_at[b])
        if p < L:
            tok[b, p] = eos_id
            val[b, p] = 12.0 + boost_shift(V, boost)
    return DecodeInputs(prompt, tok.to(torch.int32), val.to(torch.float32), taus(cfg, 0, seed), eos_at,
                        mask_id, eos_id, gain)
