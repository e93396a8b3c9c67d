"""Binding of libdflash_harness.so: the benchmark's target stand-in.

The target model's verify forward needs trained weights, so benchmarks plant the
target's tokens from the device drafts instead (a per-step table of accepted
lengths a* decides how many drafts each sequence gets accepted).  Not part of the
C-ABI library; only tests and the benchmark load it.
"""
from __future__ import annotations

import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
HARNESS_PATH = os.path.join(PKG, "libdflash_harness.so")
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(HARNESS_PATH):
            raise RuntimeError(f"{HARNESS_PATH} is missing: build it first")
        L = ctypes.CDLL(HARNESS_PATH)
        P, I = ctypes.c_void_p, ctypes.c_int
        L.dflash_harness_plant.argtypes = [P, P, P, P, P, I, P, P, P, P, P, I, I, I, P]
        L.dflash_harness_plant.restype = ctypes.c_int
        L.dflash_harness_plant_logits.argtypes = [P, P, P, P, I, P, P, P, P, P, P, P, P, I, I, I, P]
        L.dflash_harness_plant_logits.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(t):
    return None if t is None else t.data_ptr()


def plant(draft: torch.Tensor, target: torch.Tensor, a_star_tab: torch.Tensor,
          fill_tab: torch.Tensor, step_counter: torch.Tensor, accept_len: torch.Tensor,
          accept_total: torch.Tensor, vocab: int, stream=None, block_len=None, n_rows=None,
          kb_total=None) -> None:
    """target[b] <- planted tokens for step step_counter % n_tab of the tables (a*
    clipped to block_len[b] when given, and n_rows[b] <- block_len[b] + 1);
    accept_total += sum(accept_len) (the previous step's); step_counter += 1."""
    B, k = draft.shape
    n_tab = a_star_tab.shape[0]
    s = (torch.cuda.current_stream() if stream is None else stream).cuda_stream
    st = lib().dflash_harness_plant(draft.data_ptr(), target.data_ptr(), a_star_tab.data_ptr(),
                                    fill_tab.data_ptr(), step_counter.data_ptr(), n_tab,
                                    accept_len.data_ptr(), accept_total.data_ptr(), _p(block_len), _p(n_rows),
                                    _p(kb_total), B, k, vocab, s)
    if st != 0:
        raise RuntimeError(f"dflash_harness_plant failed ({st})")


def plant_logits(draft: torch.Tensor, target: torch.Tensor, a_star_tab: torch.Tensor,
                 step_counter: torch.Tensor, saved_idx: torch.Tensor, saved_val: torch.Tensor,
                 accept_len: torch.Tensor, accept_total: torch.Tensor, rng_step=None, stream=None,
                 block_len=None, n_rows=None, kb_total=None) -> None:
    """Sampled-verification stand-in: restore last step's planted logits, plant
    +1e4 / -1e4 on the drafted tokens so that a* drafts are accepted, advance
    rng_step (if given), accept_total += sum(accept_len), step_counter += 1."""
    B, k = draft.shape
    V = target.shape[-1]
    s = (torch.cuda.current_stream() if stream is None else stream).cuda_stream
    st = lib().dflash_harness_plant_logits(draft.data_ptr(), target.data_ptr(), a_star_tab.data_ptr(),
                                           step_counter.data_ptr(), a_star_tab.shape[0], saved_idx.data_ptr(),
                                           saved_val.data_ptr(), accept_len.data_ptr(), accept_total.data_ptr(),
                                           _p(rng_step), _p(block_len), _p(n_rows), _p(kb_total), B, k, V, s)
    if st != 0:
        raise RuntimeError(f"dflash_harness_plant_logits failed ({st})")


class RoundLoop:
    """The decode round the benchmark times, on resident device buffers:
    draft step -> target stand-in planted on the device from the drafts (table of
    planted accepted lengths a*) -> tentative injection of the k+1 new rows ->
    verification (greedy, or rejection sampling at temperature > 0) -> optionally
    the block-size controller.  Every launch goes to the current stream, so a round
    runs eagerly or inside a HIP-graph capture alike; nothing in a round touches the
    host.  The sampled path reads its random-number step from a device word that
    the stand-in advances every round, so replays of one captured graph draw new
    numbers."""

    def __init__(self, d, W, cache, ws, a_tab, fill, seed: int = 0, temperature: float = 0.0,
                 adaptive: bool = False, persistent: bool = False, device="cuda"):
        from . import binding as bd
        from . import synth
        self.bd, self.d, self.W, self.cache, self.ws = bd, d, W, cache, ws
        B, k, V = d.batch, d.block_k, d.vocab
        self.n_tab = int(a_tab.shape[0])
        self.a_tab_d = torch.as_tensor(a_tab, dtype=torch.int32, device=device)
        self.fill_d = torch.as_tensor(fill, dtype=torch.int32, device=device)
        self.step_ctr = torch.zeros(1, dtype=torch.int32, device=device)
        self.acc_total = torch.zeros(1, dtype=torch.int64, device=device)
        self.draft = torch.zeros((B, k), dtype=torch.int32, device=device)
        self.target = torch.zeros((B, k + 1), dtype=torch.int32, device=device)
        self.accept = torch.zeros(B, dtype=torch.int32, device=device)
        self.out_tok = torch.zeros((B, k + 1), dtype=torch.int32, device=device)
        self.n_rows_step = torch.full((B,), k + 1, dtype=torch.int32, device=device)
        self.n_rows_in = torch.full((B,), k + 1, dtype=torch.int32, device=device)
        self.sampled = temperature > 0
        self.adaptive = adaptive
        self.persistent = persistent  # greedy draft step as one persistent kernel per layer
        if adaptive:
            # controller state: every sequence starts at the full block with the average at theta_up
            self.aparams = bd.adapt_params()
            cache["block_len"] = torch.full((B,), k, dtype=torch.int32, device=device)
            self.ema = torch.full((B,), self.aparams.theta_up, dtype=torch.float32, device=device)
            self.off_left = torch.zeros(B, dtype=torch.int32, device=device)
            self.kb_total = torch.zeros(1, dtype=torch.int64, device=device)  # block rows drafted
        self.blk = cache.get("block_len")
        if self.sampled:
            # sampled target stand-in: resident filler logits, planted per round from the drafts
            self.tgt_logits = synth.make_logits((B, k + 1, V), seed=seed, stream=31_337, device=device)
            self.saved_idx = torch.full((B, k + 1), -1, dtype=torch.int32, device=device)
            self.saved_val = torch.zeros((B, k + 1), dtype=torch.float32, device=device)
            self.logits = torch.empty((B, k, V), dtype=torch.float32, device=device)
            self.lse = torch.empty((B, k), dtype=torch.float32, device=device)
            self.rng_step = torch.zeros(1, dtype=torch.int64, device=device)
            self.smp = bd.sampling_struct(temperature, seed + 1, 0, step_dev=self.rng_step)

    def round(self, taps) -> None:
        """Enqueue one decode round; taps [B, k+1, n_taps, d_t] are the target's tapped
        hidden states of the k+1 positions it verified."""
        bd, d, W, cache, ws = self.bd, self.d, self.W, self.cache, self.ws
        k, V = d.block_k, d.vocab
        ad = self.adaptive
        n_rows = self.n_rows_in if ad else self.n_rows_step
        if self.sampled:
            bd.dflash_draft_step_sampled(d, W, cache, self.smp, self.draft, self.logits, self.lse, ws)
            plant_logits(self.draft, self.tgt_logits, self.a_tab_d, self.step_ctr, self.saved_idx, self.saved_val,
                         self.accept, self.acc_total, self.rng_step, block_len=self.blk,
                         n_rows=self.n_rows_in if ad else None, kb_total=self.kb_total if ad else None)
            bd.dflash_fuse_inject(d, W, taps, n_rows, k + 1, False, cache, ws)
            bd.dflash_verify_sampled(d, self.smp, self.draft, self.logits, self.lse, self.tgt_logits, cache,
                                     self.accept, self.out_tok, ws)
        else:
            if self.persistent:
                bd.dflash_draft_step_persistent(d, W, cache, self.draft, None, ws)
            else:
                bd.dflash_draft_step(d, W, cache, self.draft, None, ws)
            plant(self.draft, self.target, self.a_tab_d, self.fill_d, self.step_ctr, self.accept, self.acc_total,
                  V, block_len=self.blk, n_rows=self.n_rows_in if ad else None,
                  kb_total=self.kb_total if ad else None)
            bd.dflash_fuse_inject(d, W, taps, n_rows, k + 1, False, cache, ws)
            bd.dflash_verify_commit(d, self.draft, self.target, cache, self.accept, self.out_tok)
        if ad:
            bd.dflash_adapt_block_len(d, self.aparams, self.accept, cache, self.ema, self.off_left)

    def restart(self, ctx_len) -> None:
        """Back to table entry 0 with the given committed lengths (after warm-up or
        capture rounds consumed entries)."""
        self.cache["ctx_len"].copy_(ctx_len)
        self.step_ctr.zero_()
        self.acc_total.zero_()
        self.accept.zero_()
        if self.adaptive:
            self.blk.fill_(self.d.block_k)
            self.ema.fill_(self.aparams.theta_up)
            self.off_left.zero_()
            self.kb_total.zero_()
        if self.sampled:
            self.rng_step.zero_()
