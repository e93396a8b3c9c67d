"""Shapes of the DFlash block draft-and-verify step and the five workloads.

The drafter (DFlash, "Block Diffusion for Flash Speculative Decoding", as described
on the zhihu answer "如何评价小米6月9日发布的MiMo-V2.5-Pro-UltraSpeed模式", §5.1-§5.4)
fuses hidden states tapped from 5 target layers, injects the fused feature into
every draft layer's K/V, and fills a block of k positions (one visible anchor plus
k-1 mask positions) in a single forward pass. The MiMo deployment (hotdry blog
"MiMo-V2.5 speculative decoding draft scheduling", engineering checklist) fixes
block size 8, a sliding window of 128 tokens and a 256k context.

Each workload below is a synthetic stand-in with the shapes of a named model
family; weights are random (no trained checkpoint exists here).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

F32 = "f32"
BF16 = "bf16"


@dataclass(frozen=True)
class Dims:
    """Static shapes of one drafter instance (mirrors ``dflash_dims`` in dflash.h).

    window      W: how many committed positions before the block each query sees.
    sink        s: the first s positions stay visible to every query after they
                leave the window (attention sink; 0 = plain sliding window).
    cache_slots C: slots per (layer, sequence, kv head): s sink slots, then a ring
                of C - s >= W + k slots, so the k+1 tentative rows of one round
                never overwrite a row that the next round's window still needs.
    max_inject_rows: the largest per-sequence row count one fuse_inject call may
                carry (sizes the workspace); at least k + 1.
    """

    batch: int
    block_k: int
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    n_taps: int
    tap_dim: int
    window: int
    cache_slots: int
    dtype: str
    max_inject_rows: int
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    sink: int = 0

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    def with_batch(self, batch: int) -> "Dims":
        return replace(self, batch=batch)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes plus the state the decode starts from.

    context:     logical committed length at the first block step (C4: the upper
                 end of a ragged range [context_lo, context]).
    prefill:     how many positions before ``context`` are actually injected
                 (all of them for full attention, the last W for SWA).
    accept:      ("geometric", q) -> planted accepted length min(G, k) with
                 P(G >= j) = q**j, or ("uniform", None) -> uniform on 0..k, or
                 ("each", None) -> every value 0..k in turn (tiny parity runs).
    rewind:      full-attention workloads restore the committed length every
                 ``rewind`` steps so the context stays at its nominal size.
    """

    name: str
    dims: Dims
    context: int
    prefill: int
    accept: Tuple[str, Optional[float]]
    context_lo: Optional[int] = None
    rewind: int = 0
    sub_runs: Tuple[float, ...] = field(default_factory=tuple)
    description: str = ""


def _qwen_like(batch, k, layers, ffn, vocab, window, slots, max_inject):
    return Dims(batch=batch, block_k=k, n_layers=layers, hidden=4096, n_q_heads=32,
                n_kv_heads=8, head_dim=128, ffn=ffn, vocab=vocab, n_taps=5,
                tap_dim=4096, window=window, cache_slots=slots, dtype=BF16,
                max_inject_rows=max_inject)


def tiny_fp32(window: int = 128 + 9 * 9, slots: Optional[int] = None,
              dtype: str = F32, block_k: int = 8, batch: int = 1) -> Dims:
    """Tiny fp32 drafter: 1 layer, hidden 256, 4x64 MHA, SwiGLU 683, vocab 1024."""
    slots = window + block_k if slots is None else slots
    return Dims(batch=batch, block_k=block_k, n_layers=1, hidden=256, n_q_heads=4,
                n_kv_heads=4, head_dim=64, ffn=683, vocab=1024, n_taps=5,
                tap_dim=256, window=window, cache_slots=slots, dtype=dtype,
                max_inject_rows=max(block_k + 1, 64))


# Tiny fp32 (CPU-seconds): batch 1, context 128, block 8.  Full attention: the
# window covers the 128 prefilled positions plus 9 rounds of k+1 growth.
C1 = Workload("tiny_fp32_b1_k8", tiny_fp32(), context=128, prefill=128,
              accept=("each", None), rewind=0,
              description="tiny fp32 drafter, batch 1, context 128, block 8")

# Qwen3-8B-shaped drafter, batch 1, block 16, full-attention context 4096; the
# context is restored every 8 steps, so the window covers 4096 + 8*17.
C2 = Workload("qwen3_8b_b1_k16_ctx4096",
              _qwen_like(1, 16, 5, 12288, 151936, 4096 + 8 * 17, 4096 + 8 * 17 + 16, 64),
              context=4096, prefill=4096, accept=("geometric", 0.87072), rewind=8,
              description="Qwen3-8B-shaped 5-layer drafter, batch 1, block 16, context 4096")

# MiMo-style all-SWA drafter, batch 8, block 8, window 128 over a logical 65536
# context; the ring holds 128 + 8 slots.
C3 = Workload("mimo_swa_b8_k8_w128_ctx65536",
              _qwen_like(8, 8, 5, 12288, 151936, 128, 136, 64),
              context=65536, prefill=128, accept=("geometric", 0.94664),
              sub_runs=(0.94664, 0.91846, 0.85920),
              description="MiMo-style SWA drafter, batch 8, block 8, window 128, logical 65536")

# LLaMA-3.1-8B-shaped drafter, batch 64, block 10, 8 layers, ragged full-attention
# context uniform in 512..2048 (restored every 8 steps).
C4 = Workload("llama31_8b_b64_k10_ragged2048",
              Dims(batch=64, block_k=10, n_layers=8, hidden=4096, n_q_heads=32,
                   n_kv_heads=8, head_dim=128, ffn=14336, vocab=128256, n_taps=5,
                   tap_dim=4096, window=2048 + 8 * 11, cache_slots=2048 + 8 * 11 + 10,
                   dtype=BF16, max_inject_rows=64),
              context=2048, context_lo=512, prefill=2048, accept=("geometric", 0.84772),
              rewind=8,
              description="LLaMA-3.1-8B-shaped 8-layer drafter, batch 64, block 10, ragged 512..2048")

# Long-context throughput: batch 256, block 8, SWA 128 over a logical 262144
# context, per-sequence accepted lengths uniform on 0..8.
C5 = Workload("longctx_swa_b256_k8_w128_ctx262144",
              _qwen_like(256, 8, 5, 12288, 151936, 128, 136, 16),
              context=262144, prefill=128, accept=("uniform", None),
              description="SWA drafter, batch 256, block 8, window 128, logical 262144")

WORKLOADS = {w.name: w for w in (C1, C2, C3, C4, C5)}
ALL = (C1, C2, C3, C4, C5)


def planted_mean(accept: Tuple[str, Optional[float]], k: int) -> float:
    """Expected planted accepted length for an ``accept`` spec at block size k."""
    kind, q = accept
    if kind == "geometric":
        return float(sum(q ** j for j in range(1, k + 1)))
    if kind in ("uniform", "each"):
        return k / 2.0
    raise ValueError(kind)
