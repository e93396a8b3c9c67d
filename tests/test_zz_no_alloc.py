"""dflash_draft_step_noalloc (the draft step for callers that cannot allocate: its
workspace is the library's static per-GPU scratch) against dflash_draft_step with
a caller workspace: drafts and logits bitwise equal, on two calls in a row whose
second has the smaller input (the scratch keeps the first call's contents), at the
MiMo-shaped batch-8 SWA drafter and then the Qwen3-8B-shaped batch-1 drafter, and
again on tiny fp32 / bf16 drafters.  Dims whose workspace exceeds the scratch are
rejected before anything is enqueued."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from block_diffusion_speculative_dflash_amd import binding as bd
from block_diffusion_speculative_dflash_amd import configs, synth
from block_diffusion_speculative_dflash_amd.configs import BF16
from tests.parity import say

pytestmark = pytest.mark.gpu


def _state(wl, d, seed=0):
    """Weights and a prefilled cache (the last min(context, 128) positions)."""
    W = bd.pack_weights(d, synth.make_weights(d, seed=seed, device="cuda"))
    ctx = synth.make_context_lengths(wl, seed=seed) if wl is not None else np.full(d.batch, 100)
    pre = np.minimum(ctx, min(d.window, 128))
    cache = bd.alloc_cache(d, ctx_len=ctx - pre, anchor=synth.make_anchors(d, seed=seed))
    ws = bd.alloc_workspace(d)
    n = int(pre.max())
    for r0 in range(0, n, d.max_inject_rows):
        m = min(d.max_inject_rows, n - r0)
        taps = synth.make_taps(d, m, seed=seed, stream=30_000 + r0, device="cuda")
        rows = torch.as_tensor(np.clip(pre - r0, 0, m), dtype=torch.int32, device="cuda")
        bd.dflash_fuse_inject(d, W, taps, rows, m, True, cache, ws)
    torch.cuda.synchronize()
    return W, cache, ws


def _compare(name, d, W, cache, ws):
    B, k, V = d.batch, d.block_k, d.vocab
    ref_d = torch.empty((B, k), dtype=torch.int32, device="cuda")
    ref_z = torch.empty((B, k, V), dtype=torch.float32, device="cuda")
    bd.dflash_draft_step(d, W, cache, ref_d, ref_z, ws)
    got_d = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    got_z = torch.full((B, k, V), float("nan"), dtype=torch.float32, device="cuda")
    bd.dflash_draft_step_noalloc(d, W, cache, got_d, got_z)
    got_d2 = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    bd.dflash_draft_step_noalloc(d, W, cache, got_d2, None)     # without logits
    torch.cuda.synchronize()
    assert torch.equal(got_d, ref_d) and torch.equal(got_d2, ref_d), f"{name}: drafts differ"
    assert torch.equal(got_z, ref_z), f"{name}: logits differ"
    assert int(cache["dev_error"].item()) == 0
    say(f"[noalloc] {name}: drafts and logits bitwise equal to dflash_draft_step "
        f"(workspace {bd.dflash_workspace_bytes(d) >> 20} MiB of {bd.NOALLOC_SCRATCH_BYTES >> 20})")


@pytest.mark.timeout(600)
def test_noalloc_draft_step_matches_the_workspace_entry_point():
    # full size: the batch-8 drafter (77 MiB of scratch), then the smaller batch-1 one
    for wl in (configs.C3, configs.C2):
        d = wl.dims
        W, cache, ws = _state(wl, d)
        _compare(wl.name, d, W, cache, ws)
        del W, cache, ws
        torch.cuda.empty_cache()
    # tiny drafters: bf16 GQA batch 4, then fp32 batch 1
    for d in (replace(configs.C1.dims, batch=4, n_q_heads=4, n_kv_heads=2, window=64, cache_slots=72, dtype=BF16),
              configs.C1.dims):
        W, cache, ws = _state(None, d)
        _compare(f"tiny {d.dtype} B{d.batch}", d, W, cache, ws)


def test_noalloc_rejects_dims_beyond_the_scratch():
    d = configs.C5.dims
    assert bd.dflash_workspace_bytes(d) > bd.NOALLOC_SCRATCH_BYTES
    import ctypes
    st = bd.lib().dflash_draft_step_noalloc(ctypes.byref(bd.dims_struct(d)), None, None, None, None, None)
    assert st == bd.DFLASH_E_TOO_LARGE
    assert "scratch" in bd.status_string(st)
