"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/dflash.h declares, and rejects bad arguments on the host before anything
is enqueued (so no device is touched)."""
import ctypes
import os
import re
from dataclasses import replace

import pytest

from block_diffusion_speculative_dflash_amd import binding as bd
from block_diffusion_speculative_dflash_amd import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash.h")

needs_lib = pytest.mark.skipif(not os.path.exists(bd.LIB_PATH), reason="libdflash.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_\w+)\s*\(", text)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("dflash_fuse_inject", "dflash_draft_step", "dflash_verify_commit"):
        assert n in names


@needs_lib
def test_library_exports_every_declared_symbol():
    L = bd.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    assert set(bd.EXPORTED) <= set(declared_functions())


@needs_lib
def test_status_strings_and_workspace_query():
    assert bd.status_string(0) == "ok"
    assert "workspace" in bd.status_string(bd.DFLASH_E_WORKSPACE)
    for w in configs.ALL:
        n = bd.dflash_workspace_bytes(w.dims)
        assert n > 0 and n % 256 == 0
        assert bd.dflash_packed_bytes(w.dims) > 0
    L = bd.lib()
    bad = bd.dims_struct(replace(configs.C1.dims, block_k=0))
    assert L.dflash_workspace_bytes(ctypes.byref(bad)) == 0
    bad = bd.dims_struct(replace(configs.C1.dims, n_kv_heads=3))
    assert L.dflash_workspace_bytes(ctypes.byref(bad)) == 0
    bad = bd.dims_struct(replace(configs.C1.dims, cache_slots=configs.C1.dims.window))
    assert L.dflash_workspace_bytes(ctypes.byref(bad)) == 0
    bad = bd.dims_struct(replace(configs.C1.dims, sink=-1))
    assert L.dflash_workspace_bytes(ctypes.byref(bad)) == 0
    d = configs.C1.dims                            # sink slots come on top of window + k
    bad = bd.dims_struct(replace(d, sink=2, cache_slots=d.window + d.block_k + 1))
    assert L.dflash_workspace_bytes(ctypes.byref(bad)) == 0
    good = bd.dims_struct(replace(d, sink=2, cache_slots=d.window + d.block_k + 2))
    assert L.dflash_workspace_bytes(ctypes.byref(good)) > 0


FAKE = 0x10000  # 16-byte aligned host integer, never dereferenced: validation fails first


def _weights(ptr=FAKE):
    return bd.DflashWeights(**{n: ptr for n in bd.WEIGHT_FIELDS})


def _cache(ptr=FAKE):
    return bd.DflashCache(k=ptr, v=ptr, ctx_len=ptr, anchor=ptr, dev_error=ptr)


@needs_lib
def test_invalid_arguments_are_rejected_on_the_host():
    # every call below must fail host validation; the pointers are fake, so never
    # run this where a GPU could receive a launch by mistake
    import torch
    if torch.cuda.is_available():
        pytest.skip("fake-pointer validation probe runs on CPU-only hosts")
    L = bd.lib()
    d = bd.dims_struct(configs.C2.dims)
    w, c = _weights(), _cache()
    ws = bd.dflash_workspace_bytes(configs.C2.dims)
    by = ctypes.byref
    # bad dims
    bad = bd.dims_struct(replace(configs.C2.dims, head_dim=96))
    assert L.dflash_draft_step(by(bad), by(w), by(c), FAKE, None, FAKE, ws, None) == bd.DFLASH_E_INVALID
    # NULL or misaligned packed weights, NULL norm gain
    w0 = _weights()
    w0.packed = None
    assert L.dflash_draft_step(by(d), by(w0), by(c), FAKE, None, FAKE, ws, None) == bd.DFLASH_E_INVALID
    w0.packed = FAKE + 2
    assert L.dflash_draft_step(by(d), by(w0), by(c), FAKE, None, FAKE, ws, None) == bd.DFLASH_E_INVALID
    w0 = _weights()
    w0.final_norm = None
    assert L.dflash_draft_step(by(d), by(w0), by(c), FAKE, None, FAKE, ws, None) == bd.DFLASH_E_INVALID
    # pack: missing source matrix, small destination, NULL error word
    w0 = _weights()
    w0.lm_head = None
    pb = bd.dflash_packed_bytes(configs.C2.dims)
    assert L.dflash_pack_weights(by(d), by(w0), FAKE, pb, FAKE, None) == bd.DFLASH_E_INVALID
    assert L.dflash_pack_weights(by(d), by(w), FAKE, pb - 1, FAKE, None) == bd.DFLASH_E_INVALID
    assert L.dflash_pack_weights(by(d), by(w), FAKE, pb, None, None) == bd.DFLASH_E_INVALID
    # workspace missing or too small
    assert L.dflash_draft_step(by(d), by(w), by(c), FAKE, None, None, ws, None) == bd.DFLASH_E_WORKSPACE
    assert L.dflash_draft_step(by(d), by(w), by(c), FAKE, None, FAKE, ws - 1, None) == bd.DFLASH_E_WORKSPACE
    # fuse_inject: n_max out of range, bad commit flag, small workspace
    assert L.dflash_fuse_inject(by(d), by(w), FAKE, FAKE, 0, 0, by(c), FAKE, ws, None) == bd.DFLASH_E_INVALID
    assert L.dflash_fuse_inject(by(d), by(w), FAKE, FAKE, 65, 0, by(c), FAKE, ws, None) == bd.DFLASH_E_INVALID
    assert L.dflash_fuse_inject(by(d), by(w), FAKE, FAKE, 17, 2, by(c), FAKE, ws, None) == bd.DFLASH_E_INVALID
    assert L.dflash_fuse_inject(by(d), by(w), FAKE, FAKE, 17, 0, by(c), FAKE, 100, None) == bd.DFLASH_E_WORKSPACE
    # verify: NULL outputs, misaligned target
    assert L.dflash_verify_commit(by(d), FAKE, FAKE, by(c), None, FAKE, None) == bd.DFLASH_E_INVALID
    assert L.dflash_verify_commit(by(d), FAKE, FAKE + 1, by(c), FAKE, FAKE, None) == bd.DFLASH_E_INVALID
    # block size beyond one wavefront
    bad = bd.dims_struct(replace(configs.C2.dims, block_k=64, max_inject_rows=80))
    assert L.dflash_verify_commit(by(bad), FAKE, FAKE, by(c), FAKE, FAKE, None) == bd.DFLASH_E_INVALID


@needs_lib
def test_sampled_calls_reject_bad_arguments_on_the_host():
    import torch
    if torch.cuda.is_available():
        pytest.skip("fake-pointer validation probe runs on CPU-only hosts")
    L = bd.lib()
    d = bd.dims_struct(configs.C2.dims)
    w, c = _weights(), _cache()
    ws = bd.dflash_workspace_bytes(configs.C2.dims)
    by = ctypes.byref
    good = bd.sampling_struct(0.8, 1, 2)
    bad_samplings = [bd.sampling_struct(t, 1, 2) for t in (0.0, -1.0, float("nan"), float("inf"))]
    r = bd.sampling_struct(0.8, 1, 2)
    r.reserved = 1
    bad_samplings.append(r)
    for sm in bad_samplings:
        assert L.dflash_draft_step_sampled(by(d), by(w), by(c), by(sm), FAKE, FAKE, FAKE, FAKE, ws,
                                           None) == bd.DFLASH_E_INVALID
        assert L.dflash_verify_sampled(by(d), by(sm), FAKE, FAKE, FAKE, FAKE, by(c), FAKE, FAKE, FAKE, ws,
                                       None) == bd.DFLASH_E_INVALID
    assert L.dflash_draft_step_sampled(by(d), by(w), by(c), None, FAKE, FAKE, FAKE, FAKE, ws,
                                       None) == bd.DFLASH_E_INVALID
    # logits and lse outputs are required; lse must be 4-byte aligned
    assert L.dflash_draft_step_sampled(by(d), by(w), by(c), by(good), FAKE, None, FAKE, FAKE, ws,
                                       None) == bd.DFLASH_E_INVALID
    assert L.dflash_draft_step_sampled(by(d), by(w), by(c), by(good), FAKE, FAKE, None, FAKE, ws,
                                       None) == bd.DFLASH_E_INVALID
    assert L.dflash_draft_step_sampled(by(d), by(w), by(c), by(good), FAKE, FAKE, FAKE + 2, FAKE, ws,
                                       None) == bd.DFLASH_E_INVALID
    assert L.dflash_draft_step_sampled(by(d), by(w), by(c), by(good), FAKE, FAKE, FAKE, FAKE, ws - 1,
                                       None) == bd.DFLASH_E_WORKSPACE
    # verify: NULL inputs / outputs, logits rows not 16-byte aligned, small workspace
    args = [FAKE] * 4
    for j in range(4):
        a = list(args)
        a[j] = None
        assert L.dflash_verify_sampled(by(d), by(good), *a, by(c), FAKE, FAKE, FAKE, ws,
                                       None) == bd.DFLASH_E_INVALID
    assert L.dflash_verify_sampled(by(d), by(good), FAKE, FAKE + 4, FAKE, FAKE, by(c), FAKE, FAKE, FAKE, ws,
                                   None) == bd.DFLASH_E_INVALID
    assert L.dflash_verify_sampled(by(d), by(good), FAKE, FAKE, FAKE, FAKE + 8, by(c), FAKE, FAKE, FAKE, ws,
                                   None) == bd.DFLASH_E_INVALID
    assert L.dflash_verify_sampled(by(d), by(good), FAKE, FAKE, FAKE, FAKE, by(c), None, FAKE, FAKE, ws,
                                   None) == bd.DFLASH_E_INVALID
    assert L.dflash_verify_sampled(by(d), by(good), FAKE, FAKE, FAKE, FAKE, by(c), FAKE, FAKE, FAKE, ws - 1,
                                   None) == bd.DFLASH_E_WORKSPACE


@needs_lib
def test_block_length_calls_reject_bad_arguments_on_the_host():
    import torch
    if torch.cuda.is_available():
        pytest.skip("fake-pointer validation probe runs on CPU-only hosts")
    L = bd.lib()
    d = bd.dims_struct(configs.C2.dims)
    by = ctypes.byref
    c = _cache()
    c.block_len = FAKE
    good = bd.adapt_params()
    bad = [bd.adapt_params(alpha=0.0), bd.adapt_params(alpha=1.5), bd.adapt_params(cooldown=0),
           bd.adapt_params(theta_down=float("nan")), bd.adapt_params(theta_up=float("inf"))]
    for p in bad:
        assert L.dflash_adapt_block_len(by(d), by(p), FAKE, by(c), FAKE, FAKE, None) == bd.DFLASH_E_INVALID
    assert L.dflash_adapt_block_len(by(d), None, FAKE, by(c), FAKE, FAKE, None) == bd.DFLASH_E_INVALID
    assert L.dflash_adapt_block_len(by(d), by(good), None, by(c), FAKE, FAKE, None) == bd.DFLASH_E_INVALID
    assert L.dflash_adapt_block_len(by(d), by(good), FAKE, by(c), None, FAKE, None) == bd.DFLASH_E_INVALID
    assert L.dflash_adapt_block_len(by(d), by(good), FAKE, by(c), FAKE, FAKE + 2, None) == bd.DFLASH_E_INVALID
    c0 = _cache()                                   # the controller needs block_len
    assert L.dflash_adapt_block_len(by(d), by(good), FAKE, by(c0), FAKE, FAKE, None) == bd.DFLASH_E_INVALID
    # a misaligned block_len is rejected by every call that reads it
    c2 = _cache()
    c2.block_len = FAKE + 1
    ws = bd.dflash_workspace_bytes(configs.C2.dims)
    assert L.dflash_draft_step(by(d), by(_weights()), by(c2), FAKE, None, FAKE, ws, None) == bd.DFLASH_E_INVALID
    assert L.dflash_verify_commit(by(d), FAKE, FAKE, by(c2), FAKE, FAKE, None) == bd.DFLASH_E_INVALID


EXTREMES = (0, 1, -1, 63, 64, 65, 2 ** 16, 2 ** 24 + 1, 2 ** 30, 2 ** 31 - 1, -2 ** 31)


@needs_lib
@pytest.mark.parametrize("base", ["C2", "C5"])
def test_size_queries_survive_extreme_dims(base):
    """Every dims field at the edges of int32 (one at a time, then all at once): the
    size queries return 0 (rejected) or a 256-byte multiple, and nothing in the host
    arithmetic overflows (the host-sanitized build aborts on signed overflow)."""
    L = bd.lib()
    by = ctypes.byref
    ref = bd.dims_struct(getattr(configs, base).dims)
    names = [n for n, _ in bd.DflashDims._fields_ if n not in ("rms_eps", "rope_theta")]

    def check(s):
        n = L.dflash_workspace_bytes(by(s))
        p = L.dflash_packed_bytes(by(s))
        assert n % 256 == 0 and (n == 0) == (p == 0), (n, p)

    for name in names:
        for v in EXTREMES:
            s = bd.DflashDims.from_buffer_copy(ref)
            setattr(s, name, v)
            check(s)
    for name in ("rms_eps", "rope_theta"):
        for v in (float("nan"), float("inf"), -1.0, 0.0, 3.0e38):
            s = bd.DflashDims.from_buffer_copy(ref)
            setattr(s, name, v)
            check(s)
    for v in (2 ** 31 - 1, 2 ** 24 + 1, 2 ** 16):
        s = bd.DflashDims.from_buffer_copy(ref)
        for name in names:
            if name != "dtype":
                setattr(s, name, v)
        check(s)
