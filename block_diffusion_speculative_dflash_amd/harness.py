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
