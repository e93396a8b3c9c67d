"""ctypes binding of libdflash (include/dflash.h): argument marshalling only.

Each function has the C entry point's name and arguments; torch tensors supply
device pointers and the current HIP stream.  Every computation runs in the HIP
library; there is no fallback, and loading fails loudly if the library is absent.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

from .configs import BF16, Dims

PKG = os.path.dirname(os.path.abspath(__file__))
# DFLASH_LIBRARY: another build of the same library (the host-sanitized test build)
LIB_PATH = os.environ.get("DFLASH_LIBRARY") or os.path.join(PKG, "libdflash.so")

DFLASH_OK, DFLASH_E_INVALID, DFLASH_E_UNSUPPORTED, DFLASH_E_WORKSPACE, DFLASH_E_HIP = 0, -1, -2, -3, -4
DFLASH_E_TOO_LARGE = -5
NOALLOC_SCRATCH_BYTES = 96 << 20
DEVERR_TOKEN, DEVERR_ROWS, DEVERR_CTXLEN, DEVERR_RANGE, DEVERR_BLOCK, DEVERR_OVERFLOW, DEVERR_TIMEOUT = \
    1, 2, 4, 8, 16, 32, 64

_INT_FIELDS = ("batch", "block_k", "n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim",
               "ffn", "vocab", "n_taps", "tap_dim", "window", "cache_slots", "dtype",
               "max_inject_rows")
WEIGHT_FIELDS = ("fuse_w", "fuse_norm", "embed", "mask_embed", "attn_norm", "w_qkv", "w_o",
                 "mlp_norm", "w_gate_up", "w_down", "final_norm", "lm_head", "packed")


class DflashDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in _INT_FIELDS] + [("rms_eps", ctypes.c_float),
                                                            ("rope_theta", ctypes.c_float),
                                                            ("sink", ctypes.c_int32)]


class DflashWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_FIELDS]


class DflashCache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("ctx_len", ctypes.c_void_p),
                ("anchor", ctypes.c_void_p), ("dev_error", ctypes.c_void_p), ("block_len", ctypes.c_void_p)]


class DflashAdaptParams(ctypes.Structure):
    _fields_ = [("alpha", ctypes.c_float), ("theta_down", ctypes.c_float), ("theta_off", ctypes.c_float),
                ("theta_up", ctypes.c_float), ("cooldown", ctypes.c_int32)]


class DflashSampling(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("reserved", ctypes.c_uint32),
                ("seed", ctypes.c_uint64), ("step", ctypes.c_uint64), ("step_dev", ctypes.c_void_p)]


class DFlashError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")
        self.status = status


_lib: Optional[ctypes.CDLL] = None

EXPORTED = ("dflash_workspace_bytes", "dflash_status_string", "dflash_packed_bytes",
            "dflash_pack_weights", "dflash_fuse_inject", "dflash_draft_step",
            "dflash_verify_commit", "dflash_draft_step_timed", "dflash_draft_step_sampled",
            "dflash_draft_step_sampled_timed", "dflash_verify_sampled", "dflash_adapt_block_len",
            "dflash_debug_poison", "dflash_draft_step_noalloc", "dflash_draft_step_persistent")
POISON_RING, POISON_WORKSPACE = 1, 2


def lib() -> ctypes.CDLL:
    """The loaded libdflash.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m block_diffusion_speculative_dflash_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I, S = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    L.dflash_workspace_bytes.argtypes = [ctypes.POINTER(DflashDims)]
    L.dflash_workspace_bytes.restype = S
    L.dflash_status_string.argtypes = [ctypes.c_int]
    L.dflash_status_string.restype = ctypes.c_char_p
    L.dflash_packed_bytes.argtypes = [ctypes.POINTER(DflashDims)]
    L.dflash_packed_bytes.restype = S
    L.dflash_pack_weights.argtypes = [ctypes.POINTER(DflashDims), ctypes.POINTER(DflashWeights), P, S,
                                      P, P]
    L.dflash_pack_weights.restype = ctypes.c_int
    L.dflash_fuse_inject.argtypes = [ctypes.POINTER(DflashDims), ctypes.POINTER(DflashWeights), P, P,
                                     I, I, ctypes.POINTER(DflashCache), P, S, P]
    L.dflash_fuse_inject.restype = ctypes.c_int
    L.dflash_draft_step.argtypes = [ctypes.POINTER(DflashDims), ctypes.POINTER(DflashWeights),
                                    ctypes.POINTER(DflashCache), P, P, P, S, P]
    L.dflash_draft_step.restype = ctypes.c_int
    L.dflash_draft_step_persistent.argtypes = L.dflash_draft_step.argtypes
    L.dflash_draft_step_persistent.restype = ctypes.c_int
    L.dflash_draft_step_timed.argtypes = L.dflash_draft_step.argtypes + [P, P]
    L.dflash_draft_step_timed.restype = ctypes.c_int
    L.dflash_verify_commit.argtypes = [ctypes.POINTER(DflashDims), P, P, ctypes.POINTER(DflashCache),
                                       P, P, P]
    L.dflash_verify_commit.restype = ctypes.c_int
    L.dflash_draft_step_sampled.argtypes = [ctypes.POINTER(DflashDims), ctypes.POINTER(DflashWeights),
                                            ctypes.POINTER(DflashCache), ctypes.POINTER(DflashSampling),
                                            P, P, P, P, S, P]
    L.dflash_draft_step_sampled.restype = ctypes.c_int
    L.dflash_draft_step_sampled_timed.argtypes = L.dflash_draft_step_sampled.argtypes + [P, P]
    L.dflash_draft_step_sampled_timed.restype = ctypes.c_int
    L.dflash_verify_sampled.argtypes = [ctypes.POINTER(DflashDims), ctypes.POINTER(DflashSampling),
                                        P, P, P, P, ctypes.POINTER(DflashCache), P, P, P, S, P]
    L.dflash_verify_sampled.restype = ctypes.c_int
    L.dflash_adapt_block_len.argtypes = [ctypes.POINTER(DflashDims), ctypes.POINTER(DflashAdaptParams), P,
                                         ctypes.POINTER(DflashCache), P, P, P]
    L.dflash_adapt_block_len.restype = ctypes.c_int
    L.dflash_debug_poison.argtypes = [ctypes.POINTER(DflashDims), ctypes.POINTER(DflashCache), P, S, I, P]
    L.dflash_debug_poison.restype = ctypes.c_int
    L.dflash_draft_step_noalloc.argtypes = [ctypes.POINTER(DflashDims), ctypes.POINTER(DflashWeights),
                                            ctypes.POINTER(DflashCache), P, P, P]
    L.dflash_draft_step_noalloc.restype = ctypes.c_int
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().dflash_status_string(int(status)).decode()


# ----------------------------------------------------------------------------- structs
def dims_struct(d: Dims) -> DflashDims:
    vals = {n: getattr(d, n) for n in _INT_FIELDS if n != "dtype"}
    vals["dtype"] = 1 if d.dtype == BF16 else 0
    return DflashDims(**vals, rms_eps=d.rms_eps, rope_theta=d.rope_theta, sink=d.sink)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libdflash must be contiguous")
    return t.data_ptr()


def weights_struct(W: Dict[str, torch.Tensor]) -> DflashWeights:
    return DflashWeights(**{n: _ptr(W.get(n)) for n in WEIGHT_FIELDS})


def cache_struct(cache: Dict[str, torch.Tensor]) -> DflashCache:
    return DflashCache(k=_ptr(cache["k"]), v=_ptr(cache["v"]), ctx_len=_ptr(cache["ctx_len"]),
                       anchor=_ptr(cache["anchor"]), dev_error=_ptr(cache["dev_error"]),
                       block_len=_ptr(cache.get("block_len")))


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(fn: str, status: int) -> None:
    if status != DFLASH_OK:
        raise DFlashError(fn, status)


# ----------------------------------------------------------------------------- entry points
def dflash_workspace_bytes(dims: Dims) -> int:
    n = lib().dflash_workspace_bytes(ctypes.byref(dims_struct(dims)))
    if n == 0:
        raise DFlashError("dflash_workspace_bytes", DFLASH_E_INVALID)
    return int(n)


def dflash_packed_bytes(dims: Dims) -> int:
    n = lib().dflash_packed_bytes(ctypes.byref(dims_struct(dims)))
    if n == 0:
        raise DFlashError("dflash_packed_bytes", DFLASH_E_INVALID)
    return int(n)


def dflash_pack_weights(dims: Dims, weights, packed: torch.Tensor, dev_error: torch.Tensor,
                        stream=None) -> None:
    ds, ws = dims_struct(dims), weights_struct(weights)
    st = lib().dflash_pack_weights(ctypes.byref(ds), ctypes.byref(ws), _ptr(packed),
                                   packed.numel() * packed.element_size(), _ptr(dev_error),
                                   _stream(stream))
    _check("dflash_pack_weights", st)


def pack_weights(dims: Dims, weights: Dict[str, torch.Tensor], device="cuda") -> Dict[str, torch.Tensor]:
    """Add the packed GEMM copy (dflash_pack_weights) to a weight dict, in place."""
    packed = torch.empty(dflash_packed_bytes(dims), dtype=torch.uint8, device=device)
    err = torch.zeros(1, dtype=torch.uint32, device=device)
    dflash_pack_weights(dims, weights, packed, err)
    torch.cuda.synchronize()
    if int(err.item()) != 0:
        raise DFlashError("dflash_pack_weights (weight outside the fp16 range)", int(err.item()))
    weights["packed"] = packed
    return weights


def dflash_fuse_inject(dims: Dims, weights, taps: torch.Tensor, n_rows: torch.Tensor, n_max: int,
                       commit: bool, cache, workspace: torch.Tensor, stream=None) -> None:
    ds, ws, cs = dims_struct(dims), weights_struct(weights), cache_struct(cache)
    st = lib().dflash_fuse_inject(ctypes.byref(ds), ctypes.byref(ws), _ptr(taps), _ptr(n_rows),
                                  int(n_max), int(bool(commit)), ctypes.byref(cs), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream))
    _check("dflash_fuse_inject", st)


def dflash_draft_step(dims: Dims, weights, cache, draft: torch.Tensor,
                      logits_out: Optional[torch.Tensor], workspace: torch.Tensor, stream=None) -> None:
    ds, ws, cs = dims_struct(dims), weights_struct(weights), cache_struct(cache)
    st = lib().dflash_draft_step(ctypes.byref(ds), ctypes.byref(ws), ctypes.byref(cs), _ptr(draft),
                                 _ptr(logits_out), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream))
    _check("dflash_draft_step", st)


def dflash_draft_step_persistent(dims: Dims, weights, cache, draft: torch.Tensor,
                                 logits_out: Optional[torch.Tensor], workspace: torch.Tensor, stream=None) -> None:
    ds, ws, cs = dims_struct(dims), weights_struct(weights), cache_struct(cache)
    st = lib().dflash_draft_step_persistent(ctypes.byref(ds), ctypes.byref(ws), ctypes.byref(cs), _ptr(draft),
                                            _ptr(logits_out), _ptr(workspace),
                                            workspace.numel() * workspace.element_size(), _stream(stream))
    _check("dflash_draft_step_persistent", st)


def dflash_draft_step_noalloc(dims: Dims, weights, cache, draft: torch.Tensor,
                              logits_out: Optional[torch.Tensor], stream=None) -> None:
    ds, ws, cs = dims_struct(dims), weights_struct(weights), cache_struct(cache)
    st = lib().dflash_draft_step_noalloc(ctypes.byref(ds), ctypes.byref(ws), ctypes.byref(cs), _ptr(draft),
                                         _ptr(logits_out), _stream(stream))
    _check("dflash_draft_step_noalloc", st)


def dflash_draft_step_timed(dims: Dims, weights, cache, draft: torch.Tensor,
                            logits_out: Optional[torch.Tensor], workspace: torch.Tensor,
                            head_begin: int, head_end: int, stream=None) -> None:
    ds, ws, cs = dims_struct(dims), weights_struct(weights), cache_struct(cache)
    st = lib().dflash_draft_step_timed(ctypes.byref(ds), ctypes.byref(ws), ctypes.byref(cs),
                                       _ptr(draft), _ptr(logits_out), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(),
                                       _stream(stream), head_begin, head_end)
    _check("dflash_draft_step_timed", st)


def dflash_verify_commit(dims: Dims, draft: torch.Tensor, target: torch.Tensor, cache,
                         accept_len: torch.Tensor, out_tokens: torch.Tensor, stream=None) -> None:
    ds, cs = dims_struct(dims), cache_struct(cache)
    st = lib().dflash_verify_commit(ctypes.byref(ds), _ptr(draft), _ptr(target), ctypes.byref(cs),
                                    _ptr(accept_len), _ptr(out_tokens), _stream(stream))
    _check("dflash_verify_commit", st)


def sampling_struct(temperature: float, seed: int, step: int,
                    step_dev: Optional[torch.Tensor] = None) -> DflashSampling:
    """Sampling parameters; step_dev (one int64 device word) makes the kernels read
    the step at run time, for graph replays."""
    return DflashSampling(temperature=float(temperature), reserved=0, seed=int(seed) & (2**64 - 1),
                          step=int(step) & (2**64 - 1), step_dev=_ptr(step_dev))


def dflash_draft_step_sampled(dims: Dims, weights, cache, sampling: DflashSampling, draft: torch.Tensor,
                              logits_out: torch.Tensor, lse_out: torch.Tensor, workspace: torch.Tensor,
                              stream=None) -> None:
    ds, ws, cs = dims_struct(dims), weights_struct(weights), cache_struct(cache)
    st = lib().dflash_draft_step_sampled(ctypes.byref(ds), ctypes.byref(ws), ctypes.byref(cs),
                                         ctypes.byref(sampling), _ptr(draft), _ptr(logits_out), _ptr(lse_out),
                                         _ptr(workspace), workspace.numel() * workspace.element_size(),
                                         _stream(stream))
    _check("dflash_draft_step_sampled", st)


def dflash_draft_step_sampled_timed(dims: Dims, weights, cache, sampling: DflashSampling,
                                    draft: torch.Tensor, logits_out: torch.Tensor, lse_out: torch.Tensor,
                                    workspace: torch.Tensor, head_begin: int, head_end: int,
                                    stream=None) -> None:
    ds, ws, cs = dims_struct(dims), weights_struct(weights), cache_struct(cache)
    st = lib().dflash_draft_step_sampled_timed(ctypes.byref(ds), ctypes.byref(ws), ctypes.byref(cs),
                                               ctypes.byref(sampling), _ptr(draft), _ptr(logits_out),
                                               _ptr(lse_out), _ptr(workspace),
                                               workspace.numel() * workspace.element_size(),
                                               _stream(stream), head_begin, head_end)
    _check("dflash_draft_step_sampled_timed", st)


def dflash_verify_sampled(dims: Dims, sampling: DflashSampling, draft: torch.Tensor, draft_logits: torch.Tensor,
                          draft_lse: torch.Tensor, target_logits: torch.Tensor, cache, accept_len: torch.Tensor,
                          out_tokens: torch.Tensor, workspace: torch.Tensor, stream=None) -> None:
    ds, cs = dims_struct(dims), cache_struct(cache)
    st = lib().dflash_verify_sampled(ctypes.byref(ds), ctypes.byref(sampling), _ptr(draft), _ptr(draft_logits),
                                     _ptr(draft_lse), _ptr(target_logits), ctypes.byref(cs), _ptr(accept_len),
                                     _ptr(out_tokens), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(stream))
    _check("dflash_verify_sampled", st)


def adapt_params(alpha: float = 0.25, theta_down: float = 4.0, theta_off: float = 2.0,
                 theta_up: float = 6.0, cooldown: int = 16) -> DflashAdaptParams:
    return DflashAdaptParams(alpha=alpha, theta_down=theta_down, theta_off=theta_off, theta_up=theta_up,
                             cooldown=cooldown)


def dflash_adapt_block_len(dims: Dims, params: DflashAdaptParams, accept_len: torch.Tensor, cache,
                           ema: torch.Tensor, off_left: torch.Tensor, stream=None) -> None:
    ds, cs = dims_struct(dims), cache_struct(cache)
    st = lib().dflash_adapt_block_len(ctypes.byref(ds), ctypes.byref(params), _ptr(accept_len), ctypes.byref(cs),
                                      _ptr(ema), _ptr(off_left), _stream(stream))
    _check("dflash_adapt_block_len", st)


def dflash_debug_poison(dims: Dims, cache, workspace: Optional[torch.Tensor], what: int, stream=None) -> None:
    ds = dims_struct(dims)
    cs = cache_struct(cache) if cache is not None else None
    st = lib().dflash_debug_poison(ctypes.byref(ds), ctypes.byref(cs) if cs is not None else None,
                                   _ptr(workspace),
                                   0 if workspace is None else workspace.numel() * workspace.element_size(),
                                   int(what), _stream(stream))
    _check("dflash_debug_poison", st)


# ----------------------------------------------------------------------------- buffers
def alloc_cache(dims: Dims, device="cuda", ctx_len=None, anchor=None) -> Dict[str, torch.Tensor]:
    """Caller-owned decode state: K/V rings (fp16 for bf16 drafters, fp32 for fp32
    drafters), committed lengths, anchors, error word."""
    dt = cache_dtype(dims)
    shape = (dims.n_layers, dims.batch, dims.n_kv_heads, dims.cache_slots, dims.head_dim)
    B = dims.batch

    def ints(v):
        if v is None:
            return torch.zeros(B, dtype=torch.int32, device=device)
        return torch.as_tensor(v, dtype=torch.int32).reshape(B).to(device)

    return {"k": torch.zeros(shape, dtype=dt, device=device),
            "v": torch.zeros(shape, dtype=dt, device=device),
            "ctx_len": ints(ctx_len), "anchor": ints(anchor),
            "dev_error": torch.zeros(1, dtype=torch.uint32, device=device)}


def cache_dtype(dims: Dims) -> torch.dtype:
    return torch.float16 if dims.dtype == BF16 else torch.float32


def alloc_workspace(dims: Dims, device="cuda") -> torch.Tensor:
    """Zero-filled workspace of dflash_workspace_bytes(dims) bytes."""
    return torch.zeros(dflash_workspace_bytes(dims), dtype=torch.uint8, device=device)
