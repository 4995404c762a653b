"""The allocation-free entry point fdl_lm_head_select_noalloc against
fdl_lm_head_select (same kernels, caller workspace) through the C ABI: two
calls in a row on the library's static scratch, the second with a smaller
input, each compared with the workspace path bit for bit (token ids, commit
sets and counts, confidences, the in-place token/masked updates)."""
import numpy as np
import pytest
import torch

from block_diffusion_decoding_attn_amd import fdl, synth

pytestmark = pytest.mark.gpu


def _call(cfg, R, step, noalloc):
    dev = torch.device("cuda")
    d = fdl.make_dims(cfg)
    w = synth.weights(cfg).to(dev)
    x, _, _ = synth.hidden_rows(cfg, synth.weights(cfg), step, rows=cfg.batch * R)
    x = x.to(dev)
    masked = synth.masked_rows(cfg, step).to(dev)[:, :R].contiguous()
    tau = synth.taus(cfg, step).to(dev)
    B = cfg.batch
    out = dict(token=torch.full((B, R), -7, dtype=torch.int32, device=dev),
               conf=torch.full((B, R), -7.0, dtype=torch.float32, device=dev),
               commit=torch.full((B, R), 7, dtype=torch.uint8, device=dev),
               n_commit=torch.full((B,), -7, dtype=torch.int32, device=dev),
               tokens=torch.full((B, R), -1, dtype=torch.int32, device=dev))
    m = masked.clone()
    args = (d, R, x, w, None, masked, tau, fdl.FDL_SELECT_THRESHOLD, 0, 1.0, out["token"], out["conf"],
            out["commit"], out["n_commit"], out["tokens"], m)
    if noalloc:
        fdl.fdl_lm_head_select_noalloc(*args)
    else:
        ws = torch.empty((fdl.fdl_lm_head_select_workspace_size(d, R),), dtype=torch.uint8, device=dev)
        fdl.fdl_lm_head_select(*args, ws)
    torch.cuda.synchronize()
    out["masked"] = m
    return {k: v.cpu().numpy() for k, v in out.items()}


@pytest.mark.parametrize("first,second", [
    # the long-context shape (tiled LM head, 512 rows), then the 7B/bs4 shape (skinny, 32 rows)
    (("qwen2.5-7b_long_bs16", 32), ("qwen2.5-7b_bs4", 8)),
])
def test_noalloc_matches_workspace_path(first, second):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    for step, (name, R) in enumerate([first, second]):
        cfg = synth.get_config(name)
        d = fdl.make_dims(cfg)
        assert fdl.fdl_lm_head_select_workspace_size(d, R) <= fdl.FDL_NOALLOC_SCRATCH_BYTES
        print(f"noalloc call {step}: {name} rows {cfg.batch * R}", flush=True)
        ref = _call(cfg, R, step, noalloc=False)
        got = _call(cfg, R, step, noalloc=True)
        for key in ref:
            np.testing.assert_array_equal(got[key], ref[key], err_msg=f"{name}: {key}")
        assert (got["n_commit"] >= 1).all()

