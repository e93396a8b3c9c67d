"""The workloads carry the constants the pages print (tests/golden/page_constants.json)."""
import json
import os

from block_diffusion_speculative_dflash_amd import configs
from block_diffusion_speculative_dflash_amd.configs import planted_mean

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))


def test_every_drafter_fuses_five_taps():
    for w in configs.ALL:
        assert w.dims.n_taps == GOLD["n_taps"]["value"]


def test_block_sizes_windows_and_depths():
    assert configs.C2.dims.block_k == GOLD["block_k_default"]["value"]
    assert configs.C4.dims.block_k == GOLD["block_k_llama31"]["value"]
    for w in (configs.C1, configs.C3, configs.C5):
        assert w.dims.block_k == GOLD["block_k_mimo"]["value"]
    for w in (configs.C3, configs.C5):
        assert w.dims.window == GOLD["swa_window"]["value"]
        assert w.dims.cache_slots == w.dims.window + w.dims.block_k
    assert configs.C5.context == GOLD["context_256k"]["value"]
    lo, hi = GOLD["draft_layers"]["value"]
    for w in configs.ALL[1:]:
        assert lo <= w.dims.n_layers <= hi


def test_planted_geometric_means_reproduce_the_pages_acceptance():
    means = GOLD["accept_means_mimo"]["value"]
    for q, key in zip(configs.C3.sub_runs, ("code", "math", "agent")):
        assert abs(planted_mean(("geometric", q), 8) - means[key]) < 5e-4
    assert abs(planted_mean(configs.C2.accept, 16) - GOLD["accept_mean_dflash_qwen3"]["value"]) < 5e-4


def test_full_attention_windows_cover_the_reachable_context():
    for w in configs.ALL:
        d = w.dims
        assert d.cache_slots >= d.window + d.block_k
        if w.prefill == w.context:                       # full attention
            reach = w.context + max(w.rewind, 9) * (d.block_k + 1)
            assert d.window >= min(reach, w.context + (w.rewind or 9) * (d.block_k + 1))
