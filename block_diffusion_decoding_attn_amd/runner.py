"""Device buffers and call sequence of a workload's denoising steps.

A step is the whole hot path over one batch: fdl_block_attn, the LM head and
the select (fdl_lm_head_select, or fdl_lm_head then fdl_conf_select) and,
after the last step of a block, fdl_kv_append, which writes the block's K/V at
each sequence's device-side length and advances it.  For the v1 DualCache
workload every block starts instead with the refresh, which rewrites all
P + L cached positions through fdl_kv_write (position 0, len set to P + L in
the same launch); nothing is appended there.

The hidden rows fed to the LM head are synthetic (the transformer layers
between attention and the LM head are not part of the step), so the attention
output and the LM-head input are independent buffers.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import torch

from . import fdl, synth


@dataclasses.dataclass
class StepInputs:
    q: torch.Tensor          # [B][S][Hq][d]
    x: torch.Tensor          # [B*S][H]
    masked: torch.Tensor     # [B][S] uint8
    tau: torch.Tensor        # [B] f32
    block_idx: int
    sub_idx: int
    append_after: bool


class StepRunner:
    """Holds one workload's device state and enqueues its steps.

    select: "threshold" (Algorithm 2), "topk" (fixed count `k`) or "factor".
    fused: LM head and select as one fdl_lm_head_select call (the logits are
    not materialized unless write_logits); otherwise fdl_lm_head then
    fdl_conf_select.
    """

    def __init__(self, cfg: synth.Config, seed: int = 0, boost: str = "calibrated", select: str = "threshold",
                 k: int = 4, factor: float = 1.0, device: str = "cuda", steps: Optional[List[int]] = None,
                 keep_host: bool = False, fused: bool = True, write_logits: bool = False):
        self.cfg, self.seed, self.boost = cfg, seed, boost
        self.fused, self.write_logits = fused, write_logits or not fused
        self.select_mode = {"threshold": fdl.FDL_SELECT_THRESHOLD, "topk": fdl.FDL_SELECT_TOPK,
                            "factor": fdl.FDL_SELECT_FACTOR}[select]
        self.k, self.factor = k, factor
        self.dims = fdl.make_dims(cfg)
        self.dev = torch.device(device)
        self.sched = synth.schedule(cfg)
        self.dual = cfg.attn_mode == synth.DUAL_CACHE
        B, S, cap = cfg.batch, cfg.sub_block, cfg.cap
        dt = cfg.torch_dtype

        self.w_host = synth.weights(cfg, seed)
        self.w = self.w_host.to(self.dev)
        fill = cfg.prompt_len
        kc, vc = synth.kv_cache(cfg, seed, fill=None if self.dual else fill)
        self.kc_host, self.vc_host = (kc, vc) if keep_host else (None, None)
        self.k_cache, self.v_cache = kc.to(self.dev), vc.to(self.dev)
        # per-sequence lengths and the masked rows of every step share one byte
        # buffer, so that reset() is a single copy: [len: B int32, padded to
        # 16 bytes][masked: steps x B x S]
        self.step_ids = list(range(len(self.sched))) if steps is None else list(steps)
        n_steps = len(self.step_ids)
        len_bytes = (4 * B + 15) // 16 * 16
        self.state = torch.zeros((len_bytes + n_steps * B * S,), dtype=torch.uint8, device=self.dev)
        self.len = self.state[:4 * B].view(torch.int32)
        self.len.fill_(fill)

        self.blocks = sorted({self.sched[i][0] for i in self.step_ids})
        self.kb_host: Dict[int, tuple] = {}
        self.k_blk: Dict[int, torch.Tensor] = {}
        self.v_blk: Dict[int, torch.Tensor] = {}
        self.refresh: Dict[int, tuple] = {}
        for b in self.blocks:
            kb, vb = synth.block_kv(cfg, b, seed)
            if keep_host:
                self.kb_host[b] = (kb, vb)
            self.k_blk[b], self.v_blk[b] = kb.to(self.dev), vb.to(self.dev)
            if self.dual:
                kr, vr = synth.refresh_kv(cfg, b, seed)
                self.refresh[b] = (kr.to(self.dev), vr.to(self.dev), (kr, vr) if keep_host else None)
        self.inputs: Dict[int, StepInputs] = {}
        self.host_inputs: Dict[int, StepInputs] = {}
        # masked state of every step: the select updates it in place (committed
        # rows leave the masked set); reset() restores the initial state
        masks = [synth.masked_rows(cfg, i, seed) for i in self.step_ids]
        self.masked_all = self.state[len_bytes:].view(n_steps, B, S)
        self.masked_all.copy_(torch.stack(masks))
        self.state_init = self.state.clone()
        for n, i in enumerate(self.step_ids):
            b, s, app = self.sched[i]
            q = synth.queries(cfg, i, seed)
            x, _, _ = synth.hidden_rows(cfg, self.w_host, i, seed, boost)
            t = synth.taus(cfg, i, seed)
            if keep_host:
                self.host_inputs[i] = StepInputs(q, x, masks[n], t, b, s, app)
            self.inputs[i] = StepInputs(q.to(self.dev), x.to(self.dev), self.masked_all[n], t.to(self.dev), b, s,
                                        app)

        # outputs / workspaces
        self.out = torch.empty((B, S, cfg.n_q_heads, cfg.head_dim), dtype=dt, device=self.dev)
        self.lse = torch.empty((B, cfg.n_q_heads, S), dtype=torch.float32, device=self.dev)
        self.logits = torch.empty((B * S, cfg.vocab), dtype=torch.float32, device=self.dev)
        self.token = torch.empty((B, S), dtype=torch.int32, device=self.dev)
        self.conf = torch.empty((B, S), dtype=torch.float32, device=self.dev)
        self.commit = torch.empty((B, S), dtype=torch.uint8, device=self.dev)
        self.n_commit = torch.empty((B,), dtype=torch.int32, device=self.dev)
        self.tokens = torch.zeros((B, S), dtype=torch.int32, device=self.dev)
        ws_a = fdl.fdl_block_attn_workspace_size(self.dims)
        ws_s = max(fdl.fdl_conf_select_workspace_size(self.dims, S),
                   fdl.fdl_lm_head_select_workspace_size(self.dims, S))
        # the attention workspace starts zeroed: it holds the split counters
        self.ws_attn = torch.zeros((max(ws_a, 16),), dtype=torch.uint8, device=self.dev)
        self.ws_sel = torch.empty((max(ws_s, 16),), dtype=torch.uint8, device=self.dev)

    # -- the step ------------------------------------------------------------
    def reset(self):
        """Back to the start of the schedule: the cache holds only the prompt and
        every step's rows are masked as initially drawn."""
        self.state.copy_(self.state_init)

    def refresh_block(self, b: int):
        """v1 DualCache refresh before block b: rewrite all P + L positions, len = P + L."""
        kr, vr, _ = self.refresh[b]
        fdl.fdl_kv_write(self.dims, self.k_cache, self.v_cache, kr, vr, 0, self.len)

    def attention(self, i: int):
        inp = self.inputs[i]
        fdl.fdl_block_attn(self.dims, inp.block_idx, inp.sub_idx, inp.q, self.k_cache, self.v_cache, None,
                           self.k_blk[inp.block_idx], self.v_blk[inp.block_idx], self.out, self.lse, self.ws_attn)

    def lm_head(self, i: int):
        fdl.fdl_lm_head(self.dims, self.inputs[i].x, self.w, self.logits)

    def select(self, i: int):
        inp = self.inputs[i]
        fdl.fdl_conf_select(self.dims, self.cfg.sub_block, self.logits, inp.masked, inp.tau, self.select_mode,
                            self.k, self.factor, self.token, self.conf, self.commit, self.n_commit, self.tokens,
                            inp.masked, self.ws_sel)

    def lm_head_select(self, i: int):
        inp = self.inputs[i]
        fdl.fdl_lm_head_select(self.dims, self.cfg.sub_block, inp.x, self.w,
                               self.logits if self.write_logits else None, inp.masked, inp.tau, self.select_mode,
                               self.k, self.factor, self.token, self.conf, self.commit, self.n_commit, self.tokens,
                               inp.masked, self.ws_sel)

    def append(self, i: int):
        """Store the finished block b at every sequence's length and advance
        it (fdl_kv_append: one launch for a block's worth of K/V)."""
        b = self.inputs[i].block_idx
        fdl.fdl_kv_append(self.dims, self.k_cache, self.v_cache, self.k_blk[b], self.v_blk[b], self.len)

    def step(self, i: int):
        inp = self.inputs[i]
        if self.dual and inp.sub_idx == 0:
            self.refresh_block(inp.block_idx)
        self.attention(i)
        if self.fused:
            self.lm_head_select(i)
        else:
            self.lm_head(i)
            self.select(i)
        if inp.append_after and not self.dual:
            self.append(i)


class DecodeRunner:
    """Device buffers of one run of the decode loop (fdl_decode): a whole
    generation of the batch from the prompt, with the stand-in model of the
    library (tied embedding w, attention-output gain, per-position boost)."""

    def __init__(self, cfg: synth.Config, seed: int = 0, boost: str = "calibrated", gain: float = 2.0,
                 select: str = "threshold", k: int = 4, factor: float = 1.0, max_blocks: int = 0,
                 trace: bool = True, eos: bool = True, inputs: Optional[synth.DecodeInputs] = None,
                 device: str = "cuda", w_host: Optional[torch.Tensor] = None):
        self.cfg, self.seed = cfg, seed
        self.mode = {"threshold": fdl.FDL_SELECT_THRESHOLD, "topk": fdl.FDL_SELECT_TOPK,
                     "factor": fdl.FDL_SELECT_FACTOR}[select]
        self.select, self.k, self.factor, self.max_blocks = select, k, factor, max_blocks
        self.inp = synth.decode_inputs(cfg, seed, boost, gain, eos) if inputs is None else inputs
        self.dims = fdl.make_dims(cfg)
        dev = self.dev = torch.device(device)
        B, P, L, D, S = cfg.batch, cfg.prompt_len, cfg.gen_len, cfg.block, cfg.sub_block
        cap = cfg.cap
        self.w_host = synth.weights(cfg, seed) if w_host is None else w_host
        self.w = self.w_host.to(dev)
        self.prompt = self.inp.prompt.to(dev)
        self.boost_tok = self.inp.boost_tok.to(dev)
        self.boost_val = self.inp.boost_val.to(dev)
        self.tau = self.inp.tau.to(dev)
        dt = cfg.torch_dtype
        self.k_cache = torch.zeros((B, cfg.n_kv_heads, cap, cfg.head_dim), dtype=dt, device=dev)
        self.v_cache = torch.zeros_like(self.k_cache)
        i32 = dict(dtype=torch.int32, device=dev)
        self.len = torch.zeros((B,), **i32)
        self.tokens = torch.zeros((B, cap), **i32)
        self.masked = torch.zeros((B, cap), dtype=torch.uint8, device=dev)
        self.seq_steps = torch.zeros((B,), **i32)
        self.eos_block = torch.zeros((B,), **i32)
        self.counters = torch.zeros((2,), **i32)
        self.slots = fdl.fdl_decode_step_slots(self.dims, self.mode, k, max_blocks)
        self.trace = None
        if trace:
            T = self.slots
            self.trace = dict(meta=torch.zeros((T, 2), **i32), tokens=torch.zeros((T, B, D), **i32),
                              masked=torch.zeros((T, B, D), dtype=torch.uint8, device=dev),
                              token=torch.zeros((T, B, S), **i32),
                              conf=torch.zeros((T, B, S), dtype=torch.float32, device=dev))
        ws = fdl.fdl_decode_workspace_size(self.dims)
        self.ws = torch.empty((max(ws, 16),), dtype=torch.uint8, device=dev)

    def run(self, stream=None, trace: bool = True):
        """Enqueue one whole generation; trace=False skips the per-step record."""
        fdl.fdl_decode(self.dims, self.w, self.prompt, self.boost_tok, self.boost_val, self.tau, self.mode, self.k,
                       self.factor, self.inp.mask_id, self.inp.eos_id, self.inp.gain, self.max_blocks,
                       self.k_cache, self.v_cache, self.len, self.tokens, self.masked, self.seq_steps,
                       self.eos_block, self.counters, self.trace if trace else None, self.ws, stream)

    def capture(self, trace: bool = True) -> "torch.cuda.CUDAGraph":
        """Record one whole generation (every launch fdl_decode enqueues) in a
        HIP graph; replaying it reruns the generation from the prompt.  The
        loop reinitializes all of its state on the device, and none of its
        launches is a memset, so replays need no host-side reset."""
        side = torch.cuda.Stream(device=self.dev)
        side.wait_stream(torch.cuda.current_stream(self.dev))
        with torch.cuda.stream(side):
            self.run(trace=trace)                     # warm-up outside the capture
        torch.cuda.current_stream(self.dev).wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.run(trace=trace)
        return graph

    def results(self) -> dict:
        """Host copies of the outputs; the trace as a list of per-step dicts."""
        c = self.counters.cpu().numpy()
        out = dict(tokens=self.tokens.cpu().numpy(), masked=self.masked.cpu().numpy(),
                   k_cache=self.k_cache.float().cpu().numpy(), v_cache=self.v_cache.float().cpu().numpy(),
                   length=self.len.cpu().numpy(), seq_steps=self.seq_steps.cpu().numpy(),
                   eos_block=self.eos_block.cpu().numpy(), steps=int(c[0]), blocks_run=int(c[1]), trace=[])
        if self.trace is not None:
            n = min(int(c[0]), self.slots)
            t = {name: v[:n].cpu().numpy() for name, v in self.trace.items()}
            for s in range(n):
                out["trace"].append(dict(block=int(t["meta"][s, 0]), sub=int(t["meta"][s, 1]),
                                         tokens=t["tokens"][s], masked=t["masked"][s].astype(bool),
                                         token=t["token"][s], conf=t["conf"][s]))
        return out
