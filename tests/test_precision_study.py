"""Why a bf16 drafter computes in fp16: the logit error that 16-bit storage of the
intermediate values costs, measured with the fp64 oracle itself.

The pages fix no compute precision for the drafter.  The oracle's `act_round` hook
rounds the values an implementation stores between its matrix products (normalised
matrix inputs, q/k/v, injected K/V rows, attention output, SwiGLU product) and
everything else stays float64.  At the Qwen3-8B-shaped drafter (hidden 4096, 5
layers, 32/8 heads x 128, SwiGLU 12288, vocab 151936, block 16) with a 512-position
context and the synthetic weights (logit std about 1.28), bf16 storage moves the
logits by about 0.10, twice the 0.05 parity bar, and fp16 storage by about 0.014:
same bytes and the same matrix-core rate, so the GPU path stores fp16.
"""
import numpy as np
import pytest
import torch

from block_diffusion_speculative_dflash_amd import configs, synth
from oracle import dflash_oracle as orc

LOGIT_BAR = 0.05


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).to(torch.bfloat16).to(torch.float64).numpy()


def _fp16(a):
    return np.asarray(a, np.float64).astype(np.float16).astype(np.float64)


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_bf16_storage_misses_the_logit_bar_and_fp16_meets_it():
    d = configs.C2.dims
    n_ctx = 512
    Wt = synth.make_weights(d, seed=0, device="cpu")
    W = {name: t.float().numpy() for name, t in Wt.items()}
    del Wt
    taps = synth.make_taps(d, n_ctx, seed=0, stream=0, device="cpu").float().numpy()
    logits = {}
    for name, rnd in (("exact", None), ("bf16", _bf16), ("fp16", _fp16)):
        st = orc.new_state(d, batch=1, ctx_len=[0], anchor=[123])
        orc.fuse_inject(d, W, st, taps, [n_ctx], commit=True, act_round=rnd)
        logits[name] = orc.draft_step(d, W, st, act_round=rnd)["logits"][0]
    err = {name: float(np.max(np.abs(logits[name] - logits["exact"]))) for name in ("bf16", "fp16")}
    print(f"logit std {logits['exact'].std():.3f}; max |dz|: bf16 storage {err['bf16']:.4f}, "
          f"fp16 storage {err['fp16']:.4f}")
    assert err["bf16"] > LOGIT_BAR
    assert err["fp16"] < LOGIT_BAR / 2
    assert err["bf16"] > 4 * err["fp16"]
