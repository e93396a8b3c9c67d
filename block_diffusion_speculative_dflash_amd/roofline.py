"""Algorithmic bytes and FLOPs of one block step (draft + inject + verify).

Counted: every weight matrix once per call that uses it (so the K/V rows of w_qkv
count in both the injection and the draft), the committed K/V window each layer
reads, the new K/V rows, the taps, the embedding row of each anchor, and tokens.
Not counted: activations between kernels (fusible) and, for greedy steps, logits
(never written).  A sampled step adds the drafter's logits (written once by the LM
head, its log-sum-exp partials), the target's logits (read once by the verify) and
the residual row of each sequence (target and draft rows re-read).
"""
from __future__ import annotations

from dataclasses import dataclass

from .configs import BF16, Dims

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
MFMA_FP32_PEAK_TFLOPS = 157.3


@dataclass
class StepCost:
    bytes_total: float
    flops_total: float
    bytes_weights: float
    bytes_kv_read: float
    bytes_kv_write: float
    bytes_taps: float
    head_bytes: float   # final-norm + LM-head + argmax kernel, per launch
    head_flops: float


def step_cost(d: Dims, mean_ctx: float, sampled: bool = False) -> StepCost:
    e = 2 if d.dtype == BF16 else 4
    B, k, L, D = d.batch, d.block_k, d.n_layers, d.hidden
    Hq, Hkv, dh, F, V = d.n_q_heads, d.n_kv_heads, d.head_dim, d.ffn, d.vocab
    kv_rows = 2 * Hkv * dh
    p_fuse = D * d.n_taps * d.tap_dim
    p_inject = L * kv_rows * D
    p_layer = (Hq + 2 * Hkv) * dh * D + D * Hq * dh + 2 * F * D + D * F
    p_head = V * D
    weights = (p_fuse + p_inject + L * p_layer + p_head + 2 * L * D + 3 * D) * e
    n_ctx = min(mean_ctx, d.window)
    kv_read = L * B * n_ctx * kv_rows * e
    kv_write = L * B * (k + 1) * kv_rows * e
    taps = B * (k + 1) * d.n_taps * d.tap_dim * e
    tokens = B * (k + (k + 1) * 3 + 4) * 4 + B * D * e
    rows_d, rows_i = B * k, B * (k + 1)
    flops = (2 * rows_d * (L * p_layer + p_head) + 4 * rows_d * L * Hq * dh * (n_ctx + k)
             + 2 * rows_i * (p_fuse + p_inject))
    # LM head: weights, normalised rows, sum-of-squares partials, and one 8-byte argmax
    # key per row and 64-column tile (the streaming head's tiling; the tiled head at
    # >= 128 rows writes 4x or 2x fewer); the finalisation kernel reads the keys back
    # (the drafts it writes are counted with the tokens)
    n_col = (V + 63) // 64
    keys = rows_d * n_col * 8
    head_bytes = p_head * e + rows_d * D * e + rows_d * 4 * ((D + 63) // 64) + keys
    extra = keys
    if sampled:
        logits_out = rows_d * V * 4 + rows_d * n_col * 8
        head_bytes += logits_out
        extra += logits_out + rows_d * n_col * 8 + rows_d * 4 + B * (k + 1) * V * 4 + 2 * B * V * 4
    return StepCost(weights + kv_read + kv_write + taps + tokens + extra, flops, weights, kv_read,
                    kv_write, taps, head_bytes, 2.0 * rows_d * p_head)


# HBM traffic of the LM-head kernel measured with hardware counters (FETCH_SIZE and
# WRITE_SIZE per dispatch, each scaled by what the counter reads for a device copy of
# 1 GiB: fetch x2.000, write x1.000), keyed by workload name.  A figure holds only for
# the kernel sources it was taken with ("stream": the weight-streaming GEMM of batches
# up to 127 rows, "tiled": the tiled MFMA GEMM); `measured_head_traffic` returns None
# otherwise.  The tiled heads' counters include activation re-reads that the MALL
# serves: an XCD's 32 resident workgroups cover all row tiles of a few weight columns
# at a time, so every such group of columns reads the whole activation block again
# (at batch 256: 8 row tiles x 4 columns, 16 MB of activations per 4 x 2 MB of weights,
# 3.0x the weights-once bytes with perfect L2 sharing; measured 3.13x; batch 64: 1.59x).
HEAD_TRAFFIC = {
    "qwen3_8b_b1_k16_ctx4096": {
        "sources": "stream",
        "source_sha256": "11ca99f1acfd4e50841a081a7d55c24729ee9b979fad5a0839fd123ba6b31827",
        "bytes": 1256521742,
    },
    "mimo_swa_b8_k8_w128_ctx65536": {
        "sources": "stream",
        "source_sha256": "11ca99f1acfd4e50841a081a7d55c24729ee9b979fad5a0839fd123ba6b31827",
        "bytes": 1289927564,
    },
    "llama31_8b_b64_k10_ragged2048": {
        "sources": "tiled",
        "source_sha256": "073c58b133674e906753f916bcada0a7bf0841c737c67027e9c7deb9a51cfe62",
        "bytes": 1695407743,
    },
    "longctx_swa_b256_k8_w128_ctx262144": {
        "sources": "tiled",
        "source_sha256": "073c58b133674e906753f916bcada0a7bf0841c737c67027e9c7deb9a51cfe62",
        "bytes": 4070146558,
    },
}
# every source of each GEMM's translation unit (besides HIP's own)
_KERNEL_SOURCES = {
    "stream": ("gemm.hip", "gemm_body.h", "gemm.h", "common.h", "epilogue.h", "philox.h"),
    "tiled": ("gemm_tiled.hip", "gemm.h", "common.h", "epilogue.h", "philox.h"),
}


def kernel_source_sha256(kind: str = "stream") -> str:
    import hashlib
    import os
    h = hashlib.sha256()
    base = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    for f in _KERNEL_SOURCES[kind]:
        with open(os.path.join(base, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_head_traffic(workload: str):
    rec = HEAD_TRAFFIC.get(workload)
    if rec is None or rec["source_sha256"] != kernel_source_sha256(rec["sources"]):
        return None
    return rec["bytes"]
