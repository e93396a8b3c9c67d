"""Side-by-side runner: the HIP library (through its C ABI) and the fp64 oracle on
the same seeded inputs, step by step, with the parity rules:

* fp32 drafters: logits normwise max|z_gpu - z_ref| / max|z_ref| <= 1e-4; drafts
  bit-exact wherever the oracle's top-1/top-2 margin is >= 1e-3;
* bf16 drafters: max |z_gpu - z_ref| <= 0.05; drafts bit-exact wherever the
  oracle's margin is >= 0.1;
* greedy verification is integer work, so for every sampled sequence the accepted
  length, emitted tokens, committed length and anchor the GPU produced from its
  own drafts and the planted target tokens must equal what the oracle's
  verify_commit makes of those same drafts and tokens, with no margin gate;
* accepted lengths, emitted tokens, committed lengths and anchors also bit-exact
  against the oracle's own trajectory for every sequence whose deciding positions
  (0 .. min(a, k-1)) all pass the margin gate; K/V rows of the committed window
  within the logit tolerance.
The oracle plants the target tokens from its own drafts; a sequence whose GPU
accepted length differs at a low-margin position is re-synchronised to the
oracle's committed length and anchor (counted as excluded).
"""
from __future__ import annotations

import sys
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

from block_diffusion_speculative_dflash_amd import binding as bd
from block_diffusion_speculative_dflash_amd import synth
from block_diffusion_speculative_dflash_amd.configs import BF16, Dims
from oracle import dflash_oracle as orc


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_weights(W) -> dict:
    """Exact host copies (float32 holds every bf16 value) of the device weights."""
    return {k: v.float().cpu().numpy() for k, v in W.items() if k != "packed"}


@dataclass
class Tol:
    margin: float
    logit_abs: Optional[float]
    logit_rel: Optional[float]

    @staticmethod
    def for_dims(d: Dims) -> "Tol":
        return Tol(0.1, 0.05, None) if d.dtype == BF16 else Tol(1e-3, None, 1e-4)

    def logit_ok(self, err_abs: float, ref_max: float) -> bool:
        if self.logit_abs is not None:
            return err_abs <= self.logit_abs
        return err_abs <= self.logit_rel * ref_max


@dataclass
class StepReport:
    logit_err: float
    logit_ref_max: float
    logits_ok: bool
    drafts_checked: int
    drafts_total: int
    draft_mismatch: int
    seqs_checked: int
    seqs_excluded: int
    state_mismatch: int
    kv_err: float
    kv_ref_max: float
    kv_ok: bool
    accept: List[int] = field(default_factory=list)
    seqs_verified: int = 0       # sequences whose verify/commit was compared with no gate
    verify_mismatch: int = 0     # ... and disagreed with the oracle's verify_commit

    @property
    def ok(self) -> bool:
        return (self.logits_ok and self.draft_mismatch == 0 and self.state_mismatch == 0 and self.kv_ok
                and self.verify_mismatch == 0)


def integer_state(ctx_len, anchor, dims) -> "orc.State":
    """Oracle state carrying only the integer part (committed lengths, anchors):
    the K/V rings are empty arrays, which verify_commit's rollback indexes freely."""
    n = len(ctx_len)
    ring = np.empty((1, n, 1, dims.cache_slots, 0))
    return orc.State(ring, ring.copy(), np.array(ctx_len, np.int64), np.array(anchor, np.int64))


@dataclass
class SampledReport:
    logit_err: float
    logit_ref_max: float
    logits_ok: bool
    lse_err: float
    lse_ok: bool
    drafts_checked: int
    drafts_total: int
    draft_mismatch: int
    seqs_checked: int
    seqs_excluded: int
    state_mismatch: int
    kv_err: float
    kv_ok: bool
    accept: List[int] = field(default_factory=list)

    @property
    def ok(self) -> bool:
        return (self.logits_ok and self.lse_ok and self.draft_mismatch == 0 and self.state_mismatch == 0
                and self.kv_ok)


class ParityRun:
    def __init__(self, dims: Dims, W, ctx_start: Sequence[int], anchors: Sequence[int],
                 prefill_rows: Sequence[int], sample: Optional[Sequence[int]] = None, seed: int = 0,
                 check_kv: bool = True, poison: bool = False, persistent: bool = False):
        """poison: before every library call fill the workspace's scratch with NaN, and
        after every verification the ring slots no window reaches (dflash_debug_poison),
        so any read of stale memory shows in the results."""
        self.d, self.W, self.seed, self.check_kv, self.poison = dims, W, seed, check_kv, poison
        self.persistent = persistent  # greedy draft steps through dflash_draft_step_persistent
        self.last = {}
        self.Wn = oracle_weights(W)
        if "packed" not in W:
            bd.pack_weights(dims, W)
        self.tol = Tol.for_dims(dims)
        B = dims.batch
        self.sample = list(range(B)) if sample is None else list(sample)
        ctx_start = np.asarray(ctx_start, np.int64)
        pre = np.asarray(prefill_rows, np.int64)
        anchors = np.asarray(anchors, np.int64)
        p0 = ctx_start - pre
        s = self.sample
        self.cache = bd.alloc_cache(dims, ctx_len=p0, anchor=anchors)
        self.ws = bd.alloc_workspace(dims)
        self.st = orc.new_state(dims, batch=len(s), ctx_len=p0[s], anchor=anchors[s])
        n_max = dims.max_inject_rows
        if dims.sink > 0 and int(p0.min()) >= dims.sink:
            # attention sink: positions 0..s-1 are injected first, then the prefill
            # continues at p0 (both sides), as a long context would have left them
            sink_taps = synth.make_taps(dims, dims.sink, seed=seed, stream=10_000, device="cuda")
            say(f"[parity] sink rows 0..{dims.sink - 1} (B={B})")
            self.cache["ctx_len"].zero_()
            sr = torch.full((B,), dims.sink, dtype=torch.int32, device="cuda")
            self._poison()
            bd.dflash_fuse_inject(dims, W, sink_taps, sr, dims.sink, True, self.cache, self.ws)
            self.cache["ctx_len"].copy_(torch.as_tensor(p0, dtype=torch.int32))
            torch.cuda.synchronize()
            self.st.ctx_len[:] = 0
            orc.fuse_inject(dims, self.Wn, self.st, sink_taps[s].float().cpu().numpy(),
                            np.full(len(s), dims.sink), commit=True)
            self.st.ctx_len[:] = p0[s]
        n_pre = int(pre.max())
        if n_pre > 0:
            taps = synth.make_taps(dims, n_pre, seed=seed, stream=0, device="cuda")
            say(f"[parity] prefill {n_pre} rows in chunks of {n_max} (B={B})")
            for r0 in range(0, n_pre, n_max):
                chunk = taps[:, r0:r0 + n_max].contiguous()
                n_rows = torch.as_tensor(np.clip(pre - r0, 0, chunk.shape[1]), dtype=torch.int32).cuda()
                self._poison()
                bd.dflash_fuse_inject(dims, W, chunk, n_rows, chunk.shape[1], True, self.cache, self.ws)
            torch.cuda.synchronize()
        if n_pre > 0:
            orc.fuse_inject(dims, self.Wn, self.st, taps[s].float().cpu().numpy(), pre[s], commit=True)
        self.step_idx = 0

    def dev_error(self) -> int:
        return int(self.cache["dev_error"].item())

    def _poison(self, ring: bool = False) -> None:
        if self.poison:
            bd.dflash_debug_poison(self.d, self.cache, self.ws,
                                   bd.POISON_WORKSPACE | (bd.POISON_RING if ring else 0))

    def _kv_error(self):
        """Largest |K/V| error over the committed window rows of the sampled sequences."""
        d, s = self.d, self.sample
        kv_err, kv_max = 0.0, 0.0
        if self.check_kv:
            kc = self.cache["k"][:, s].float().cpu().numpy()
            vc = self.cache["v"][:, s].float().cpu().numpy()
            for j in range(len(s)):
                P = int(self.st.ctx_len[j])
                slots = np.array([orc.slot_of(d, int(p)) for p in orc.window_positions(d, P)], dtype=np.int64)
                for ring, cache_np in ((self.st.k_ring, kc), (self.st.v_ring, vc)):
                    ref = ring[:, j][:, :, slots]
                    got = cache_np[:, j][:, :, slots]
                    kv_err = max(kv_err, float(np.max(np.abs(got - ref))) if ref.size else 0.0)
                    kv_max = max(kv_max, float(np.max(np.abs(ref))) if ref.size else 0.0)
        return kv_err, kv_max

    def _set_block_len(self, block_len):
        """Per-sequence block lengths of this round (None: k for all); returns the host
        array of every sequence's k_b."""
        d = self.d
        if block_len is None:
            self.cache.pop("block_len", None)
            return np.full(d.batch, d.block_k, np.int64)
        kb = np.asarray(block_len, dtype=np.int64)
        self.cache["block_len"] = torch.as_tensor(kb, dtype=torch.int32, device="cuda")
        return kb

    def _inject_block(self, kb=None):
        """Tentative K/V rows of the k_b+1 positions the target just processed (both sides)."""
        d, k, s = self.d, self.d.block_k, self.sample
        kb = np.full(d.batch, k, np.int64) if kb is None else np.asarray(kb, np.int64)
        taps = synth.make_taps(d, k + 1, seed=self.seed, stream=1 + self.step_idx, device="cuda")
        n_rows = torch.as_tensor(kb + 1, dtype=torch.int32, device="cuda")
        self._poison()
        bd.dflash_fuse_inject(d, self.W, taps, n_rows, k + 1, False, self.cache, self.ws)
        orc.fuse_inject(d, self.Wn, self.st, taps[s].float().cpu().numpy(), kb[s] + 1, commit=False)

    def step_sampled(self, a_star: Sequence[int], temperature: float, seed: int = 1234,
                     soft: float = 0.0, block_len=None) -> "SampledReport":
        """One sampled round: dflash_draft_step_sampled, tentative injection,
        dflash_verify_sampled, against the oracle's draft forward, Gumbel-max drafts
        and rejection-sampling verification with the same seed and step.

        The logits and log-sum-exps are checked against the logit tolerance; each
        decision is then compared where its distance from the threshold exceeds what
        the measured errors can move it: err_s = max |z_gpu - z_ref| / T, err_l = max
        |lse_gpu - lse_ref|; drafts where the perturbed top-2 gap >= 2 err_s + 1e-3;
        a sequence's verification where every acceptance score |log p - log q - log u|
        >= err_s + err_l + 1e-3 (the target logits are the same values on both sides)
        and the emitted draw's gap >= 2 (err_s + err_l) slack + 1e-3."""
        from oracle import sampling as sp
        d, W, s = self.d, self.W, self.sample
        B, k, V = d.batch, d.block_k, d.vocab
        T = float(temperature)
        step = self.step_idx
        smp = bd.sampling_struct(T, seed, step)
        kb = self._set_block_len(block_len)
        a_star = np.minimum(np.asarray(a_star, np.int64), kb)
        say(f"[parity] sampled step {step}: draft_step_sampled B={B} k={k} V={V} T={T} kb={list(kb[:8])}")
        draft = torch.empty((B, k), dtype=torch.int32, device="cuda")
        logits = torch.empty((B, k, V), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, k), dtype=torch.float32, device="cuda")
        self._poison()
        bd.dflash_draft_step_sampled(d, W, self.cache, smp, draft, logits, lse, self.ws)
        torch.cuda.synchronize()
        self.last = {"draft": draft.clone(), "logits": logits.clone(), "lse": lse.clone()}
        o = orc.draft_step(d, self.Wn, self.st, block_len=kb[s])
        zr = o["logits"]
        sd = sp.sample_drafts(zr, T, seed, step, seq_ids=s, block_len=kb[s])
        xr, gap, lse_r = sd["draft"], sd["gap"], sd["lse"]
        live = np.arange(k)[None, :] < kb[s][:, None]               # rows inside each block
        zg = logits[s].cpu().numpy().astype(np.float64)
        dg = draft[s].cpu().numpy().astype(np.int64)
        err = float(np.max(np.abs(zg - zr)[live])) if live.any() else 0.0
        ref_max = float(np.max(np.abs(zr[live]))) if live.any() else 1.0
        lse_err = float(np.max(np.abs(lse[s].cpu().numpy() - lse_r)[live])) if live.any() else 0.0
        assert np.all(dg[~live] == -1), "drafts past a block must read -1"
        tol_z = self.tol.logit_abs if self.tol.logit_abs is not None else self.tol.logit_rel * ref_max
        err_s = err / T
        thr = 2 * err_s + 1e-3
        gate = gap >= thr
        mism = int(np.sum((dg != xr) & gate))

        # target stand-in: planted from the oracle's drafts and logits where sampled
        x_all = draft.cpu().numpy().astype(np.int64)
        x_all[s] = xr
        z_all = logits.clone()
        z_all[s] = torch.as_tensor(np.nan_to_num(zr), dtype=torch.float32, device="cuda")
        fill = synth.make_logits((B, k + 1, V), seed=self.seed, stream=7919 * (step + 1), device="cuda")
        tgt = synth.plant_target_logits(z_all, x_all, np.asarray(a_star), fill, soft=soft, seed=step).contiguous()
        say(f"[parity] sampled step {step}: fuse_inject + verify_sampled")
        self._inject_block(kb)
        acc = torch.empty(B, dtype=torch.int32, device="cuda")
        out = torch.empty((B, k + 1), dtype=torch.int32, device="cuda")
        self._poison()
        bd.dflash_verify_sampled(d, smp, draft, logits, lse, tgt, self.cache, acc, out, self.ws)
        torch.cuda.synchronize()
        self.last.update(accept=acc.clone(), out=out.clone())
        r = sp.verify_sampled(xr, zr, tgt[s].cpu().numpy().astype(np.float64), T, seed, step, seq_ids=s,
                              block_len=kb[s])
        sp.commit_sampled(d, self.st, r, block_len=kb[s])

        acc_g, out_g = acc[s].cpu().numpy(), out[s].cpu().numpy()
        ctx_g, anc_g = self.cache["ctx_len"][s].cpu().numpy(), self.cache["anchor"][s].cpu().numpy()
        checked = excluded = state_mism = 0
        for j, b in enumerate(s):
            a_ref = int(r["accept_len"][j])
            dq = err_s + lse_err
            ok = (all(gap[j, i] >= thr for i in range(0, min(a_ref, int(kb[b]) - 1) + 1))
                  and r["accept_margin"][j] >= dq + 1e-3
                  and r["emit_gap"][j] >= 2 * dq * r["emit_slack"][j] + 1e-3)
            if ok:
                checked += 1
                same = (acc_g[j] == a_ref and np.array_equal(out_g[j], r["out_tokens"][j])
                        and ctx_g[j] == self.st.ctx_len[j] and anc_g[j] == self.st.anchor[j])
                state_mism += int(not same)
            else:
                excluded += 1
                self.cache["ctx_len"][b] = int(self.st.ctx_len[j])
                self.cache["anchor"][b] = int(self.st.anchor[j])
        # rolled-back rows (after any re-synchronisation of the committed lengths)
        self._poison(ring=True)
        kv_err, kv_max = self._kv_error()
        self.step_idx += 1
        # log-sum-exp is 1-Lipschitz in the max norm: |d lse| <= max |dz| / T
        rep = SampledReport(err, ref_max, self.tol.logit_ok(err, ref_max), lse_err, lse_err <= tol_z / T + 1e-5,
                            int(gate.sum()), gate.size, mism, checked, excluded, state_mism, kv_err,
                            self.tol.logit_ok(kv_err, max(kv_max, 1e-30)), list(map(int, acc_g)))
        say(f"[parity] sampled step {step}: logit_err={err:.3g} lse_err={lse_err:.3g} drafts "
            f"{rep.drafts_checked}/{rep.drafts_total} gated, mismatches {mism}; seqs checked {checked}, "
            f"excluded {excluded}, state mismatches {state_mism}; kv_err={kv_err:.3g} accept={rep.accept[:8]}")
        return rep

    def step(self, a_star: Sequence[int], block_len=None) -> StepReport:
        d, W, s = self.d, self.W, self.sample
        B, k, V = d.batch, d.block_k, d.vocab
        kb = self._set_block_len(block_len)
        a_star = np.minimum(np.asarray(a_star, np.int64), kb)
        say(f"[parity] step {self.step_idx}: draft_step B={B} k={k} V={V} kb={list(kb[:8])}")
        ctx_before = self.cache["ctx_len"][s].cpu().numpy()
        anc_before = self.cache["anchor"][s].cpu().numpy()
        draft = torch.empty((B, k), dtype=torch.int32, device="cuda")
        logits = torch.empty((B, k, V), dtype=torch.float32, device="cuda")
        self._poison()
        if self.persistent:
            bd.dflash_draft_step_persistent(d, W, self.cache, draft, logits, self.ws)
        else:
            bd.dflash_draft_step(d, W, self.cache, draft, logits, self.ws)
        torch.cuda.synchronize()
        self.last = {"draft": draft.clone(), "logits": logits.clone()}
        o = orc.draft_step(d, self.Wn, self.st, block_len=kb[s])
        zg = logits[s].cpu().numpy().astype(np.float64)
        dg = draft[s].cpu().numpy().astype(np.int64)
        zr, dr, mr = o["logits"], o["draft"], o["margin"]
        live = np.arange(k)[None, :] < kb[s][:, None]               # rows inside each block
        err = float(np.max(np.abs(zg - zr)[live])) if live.any() else 0.0
        ref_max = float(np.max(np.abs(zr[live]))) if live.any() else 1.0
        gate = (mr >= self.tol.margin) & live
        mism = int(np.sum((dg != dr) & gate)) + int(np.sum(dg[~live] != -1))

        # target stand-in: planted from the oracle's drafts for sampled sequences
        fill = synth.target_fill(k, 1, B, seed=self.seed + 7919 * (self.step_idx + 1))[0]
        a_star = np.asarray(a_star, np.int64)
        T = synth.plant_targets(np.maximum(draft.cpu().numpy(), 0), a_star, fill, V)
        T[s] = synth.plant_targets(np.maximum(dr, 0), a_star[s], fill[s], V)
        taps = synth.make_taps(d, k + 1, seed=self.seed, stream=1 + self.step_idx, device="cuda")
        n_rows = torch.as_tensor(kb + 1, dtype=torch.int32, device="cuda")
        say(f"[parity] step {self.step_idx}: fuse_inject + verify_commit")
        self._poison()
        bd.dflash_fuse_inject(d, W, taps, n_rows, k + 1, False, self.cache, self.ws)
        acc = torch.empty(B, dtype=torch.int32, device="cuda")
        out = torch.empty((B, k + 1), dtype=torch.int32, device="cuda")
        Tt = torch.as_tensor(T, dtype=torch.int32).cuda()
        bd.dflash_verify_commit(d, draft, Tt, self.cache, acc, out)
        torch.cuda.synchronize()
        self.last.update(accept=acc.clone(), out=out.clone())
        orc.fuse_inject(d, self.Wn, self.st, taps[s].float().cpu().numpy(), kb[s] + 1, commit=False)
        r = orc.verify_commit(d, self.st, np.maximum(dr, 0), T[s], block_len=kb[s])

        acc_g = acc[s].cpu().numpy()
        out_g = out[s].cpu().numpy()
        ctx_g = self.cache["ctx_len"][s].cpu().numpy()
        anc_g = self.cache["anchor"][s].cpu().numpy()
        # verify/commit of the GPU's own drafts against the same targets, every
        # sampled sequence, no margin gate (integer work: must be bit-exact)
        ist = integer_state(ctx_before, anc_before, d)
        ri = orc.verify_commit(d, ist, dg, T[s], block_len=kb[s])
        verify_mism = 0
        for j in range(len(s)):
            same = (acc_g[j] == ri["accept_len"][j] and np.array_equal(out_g[j], ri["out_tokens"][j])
                    and ctx_g[j] == ist.ctx_len[j] and anc_g[j] == ist.anchor[j])
            verify_mism += int(not same)
        checked = excluded = state_mism = 0
        for j, b in enumerate(s):
            a_ref = int(r["accept_len"][j])
            deciding = range(0, min(a_ref, int(kb[b]) - 1) + 1)
            if all(mr[j, i] >= self.tol.margin for i in deciding):
                checked += 1
                same = (acc_g[j] == a_ref and np.array_equal(out_g[j], r["out_tokens"][j])
                        and ctx_g[j] == self.st.ctx_len[j] and anc_g[j] == self.st.anchor[j])
                state_mism += int(not same)
            else:
                excluded += 1
                self.cache["ctx_len"][b] = int(self.st.ctx_len[j])
                self.cache["anchor"][b] = int(self.st.anchor[j])

        # rolled-back rows (after any re-synchronisation of the committed lengths)
        self._poison(ring=True)
        kv_err, kv_max = self._kv_error()
        self.step_idx += 1
        rep = StepReport(err, ref_max, self.tol.logit_ok(err, ref_max), int(gate.sum()), gate.size,
                         mism, checked, excluded, state_mism, kv_err, kv_max,
                         self.tol.logit_ok(kv_err, max(kv_max, 1e-30)), list(map(int, acc_g)),
                         len(s), verify_mism)
        say(f"[parity] step {self.step_idx - 1}: logit_err={err:.3g} (ref max {ref_max:.3g}) "
            f"drafts {rep.drafts_checked}/{rep.drafts_total} gated, mismatches {mism}; "
            f"verify on own drafts {len(s) - verify_mism}/{len(s)} exact; "
            f"seqs checked {checked}, excluded {excluded}, state mismatches {state_mism}; "
            f"kv_err={kv_err:.3g} accept={rep.accept[:8]}")
        return rep
