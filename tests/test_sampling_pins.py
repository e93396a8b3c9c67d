"""Pins of the sampled-verification oracle (CPU only).

* Philox4x64-10 against numpy's own implementation of the generator (numpy adds
  one to the 256-bit counter before each block, with carry across the words), and
  the order of the 32-bit values against numpy's 32-bit stream;
* the counter layout: no two draws of a family share a (counter, value) pair;
* the Gumbel-max law: draws follow softmax(s) (chi-square);
* the whole rejection-sampling rule is lossless: on a tiny prefix-dependent model,
  the first two emitted tokens follow the target's autoregressive law (chi-square);
* closed forms: row 0 is accepted with probability sum_v min(p_v, q_v), and after
  a rejection the emitted token follows (p - q)+ normalised;
* T -> 0 gives greedy verification exactly; p = q accepts the whole block; a draft
  the target gives zero probability is always rejected.
"""
import numpy as np
import pytest
from scipy import stats

from oracle import dflash_oracle as orc
from oracle import sampling as sp
from tests.helpers import tiny_dims

P_MIN = 1e-4  # chi-square acceptance level (seeded, so each test is deterministic)


def _u64(x):
    return np.array(x, dtype=np.uint64)


@pytest.mark.parametrize("key", [[0, 0], [1, 2], [0xDEADBEEFCAFEBABE, 12345], [2**64 - 1, 2**63]])
def test_philox_matches_numpy(key):
    rng = np.random.default_rng(5)
    ctrs = [[0, 0, 0, 0], [5, 0, 0, 0], [2**64 - 2, 7, 9, 11], [2**64 - 1, 2**64 - 1, 3, 0]]
    ctrs += [[int(x) for x in rng.integers(0, 2**63, size=4, dtype=np.int64)] for _ in range(6)]
    for c in ctrs:
        ref = [int(x) for x in np.random.Philox(key=_u64(key), counter=_u64(c)).random_raw(4)]
        v = (c[0] | c[1] << 64 | c[2] << 128 | c[3] << 192) + 1
        nxt = [(v >> (64 * j)) & (2**64 - 1) for j in range(4)]
        assert sp.philox4x64(nxt, key) == ref
        blk = sp.philox4x64_np(*[_u64(w) for w in nxt], key)
        assert [int(x) for x in blk] == ref


def test_philox_vectorised_matches_numpy_stream():
    key = [0x0123456789ABCDEF, 77]
    raw = np.random.Philox(key=_u64(key), counter=_u64([0, 0, 0, 0])).random_raw(4 * 300)
    blk = sp.philox4x64_np(np.arange(1, 301, dtype=np.uint64), 0, 0, 0, key)
    assert np.array_equal(blk.reshape(-1), raw)


def test_u32_order_matches_numpy_32bit_stream():
    key = [7, 3]
    g = np.random.Generator(np.random.Philox(key=_u64(key), counter=_u64([0, 0, 0, 0])))
    ref = g.integers(0, 2**32, size=16, dtype=np.uint32, endpoint=False).astype(np.uint64)
    blk = sp.philox4x64_np(_u64([1, 2]), 0, 0, 0, key)
    got = np.concatenate([sp.u32_of(blk[j], np.arange(8)) for j in range(2)])
    assert np.array_equal(got, ref)


def test_uniform_is_open_and_centred():
    u = sp.uniform(np.array([0, 2**32 - 1], dtype=np.uint64))
    assert 0 < u[0] < 1e-9 and 1 - 1e-9 < u[1] < 1
    assert u[0] + u[1] == 1.0
    g = sp.gumbel(np.array([0, 2**31, 2**32 - 1], dtype=np.uint64))
    assert np.all(np.isfinite(g)) and g[0] < g[1] < g[2]
    assert abs(g[1] - (-np.log(np.log(2.0)))) < 1e-8


def test_draw_counters_never_collide():
    seen = set()
    for m in range(24):
        for v in range(256):
            c0 = 16 * (v >> 5) + (v & 15)
            key = (c0, m >> 2, 2 * (m & 3) + ((v >> 4) & 1))
            assert key not in seen
            seen.add(key)
    seen = set()
    for v in range(512):
        key = (v >> 3, v & 7)
        assert key not in seen
        seen.add(key)


def test_draft_noise_matches_scalar_definition():
    for m, v in [(0, 0), (5, 17), (6, 33), (13, 1000), (70, 151935)]:
        c = [16 * (v >> 5) + (v & 15), m >> 2, 9, 0]
        w = sp.philox4x64(c, [4, sp.STREAM_DRAFT])
        e = 2 * (m & 3) + ((v >> 4) & 1)
        h = (w[e // 2] >> (32 * (e & 1))) & 0xFFFFFFFF
        assert sp.draft_noise(4, 9, m, v + 1)[v] == -np.log(-np.log((h + 0.5) * 2.0**-32))


def _chi2_p(counts, probs):
    counts = np.asarray(counts, dtype=np.float64)
    exp = np.asarray(probs, dtype=np.float64) * counts.sum()
    return stats.chisquare(counts, exp).pvalue


def gumbel_law_pvalues(n: int):
    """Chi-square p-values of Gumbel-max draws (draft and emit noise) against softmax."""
    z = np.array([0.3, -1.0, 2.0, 0.0, 1.1, -0.4])
    T = 0.7
    p = np.exp(sp.log_softmax(z, T))
    counts = np.zeros(6)
    for step in range(n):
        counts[sp.gumbel_max(z / T, sp.draft_noise(11, step, 3, 6))[0]] += 1
    c2 = np.zeros(6)
    for step in range(n // 2):
        c2[sp.gumbel_max(z / T, sp.emit_noise(12, step, 1, 6))[0]] += 1
    return _chi2_p(counts, p), _chi2_p(c2, p)


def test_gumbel_max_draws_follow_softmax():
    assert min(gumbel_law_pvalues(12000)) > P_MIN


def test_gumbel_max_excludes_minus_inf():
    s = np.array([-np.inf, 0.0, -np.inf, 1.0])
    for step in range(200):
        y, _ = sp.gumbel_max(s, sp.emit_noise(1, step, 0, 4))
        assert y in (1, 3)


# a tiny "model": logits tables indexed by the prefix of generated tokens
V_T, K_T = 3, 2


def _tables(seed):
    rng = np.random.default_rng(seed)
    tgt, drf = {}, {}
    prefixes = [()] + [(a,) for a in range(V_T)] + [(a, b) for a in range(V_T) for b in range(V_T)]
    for pre in prefixes:
        tgt[pre] = rng.normal(0, 1.2, V_T)
        for i in range(K_T):
            drf[(pre, i)] = rng.normal(0, 1.2, V_T)
    return tgt, drf


def _first_two(tgt, drf, T, seed, trial):
    gen = []
    r = 0
    while len(gen) < 2:
        pre = tuple(gen)
        step = 8 * trial + r
        z = np.array([drf[(pre, i)] for i in range(K_T)])[None]
        x = sp.sample_drafts(z, T, seed, step)["draft"][0]
        t = np.array([tgt[(pre + tuple(int(v) for v in x[:i]))[:2]] for i in range(K_T + 1)])[None]
        res = sp.verify_sampled(x[None], z, t, T, seed, step)
        a = int(res["accept_len"][0])
        gen += [int(v) for v in res["out_tokens"][0, :a + 1]]
        r += 1
    return gen[0], gen[1]


def lossless_pvalue(n: int, seed: int = 3, T: float = 0.9) -> float:
    tgt, drf = _tables(seed)
    counts = np.zeros((V_T, V_T))
    for trial in range(n):
        t1, t2 = _first_two(tgt, drf, T, seed, trial)
        counts[t1, t2] += 1
    p1 = np.exp(sp.log_softmax(tgt[()], T))
    law = np.array([[p1[a] * np.exp(sp.log_softmax(tgt[(a,)], T))[b] for b in range(V_T)] for a in range(V_T)])
    return _chi2_p(counts.reshape(-1), law.reshape(-1))


def test_rejection_sampling_is_lossless():
    assert lossless_pvalue(6000) > P_MIN


def acceptance_checks(n: int = 6000, seed: int = 8) -> bool:
    """Row-0 acceptance rate vs sum min(p, q), and the law after a rejection."""
    rng = np.random.default_rng(seed)
    V, T = 5, 1.3
    z = rng.normal(0, 1.5, (1, 1, V))
    t = rng.normal(0, 1.5, (1, 2, V))
    p = np.exp(sp.log_softmax(t[0, 0], T))
    q = np.exp(sp.log_softmax(z[0, 0], T))
    alpha = float(np.sum(np.minimum(p, q)))
    acc = 0
    rej = np.zeros(V)
    for step in range(n):
        x = sp.sample_drafts(z, T, seed, step)["draft"]
        r = sp.verify_sampled(x, z, t, T, seed, step)
        if r["accept_len"][0] == 1:
            acc += 1
        else:
            rej[r["emitted"][0]] += 1
    sd = np.sqrt(alpha * (1 - alpha) / n)
    resid = np.maximum(p - q, 0)
    live = resid > 0
    return (abs(acc / n - alpha) < 4.5 * sd and not np.any(rej[~live]) and
            _chi2_p(rej[live], resid[live] / resid.sum()) > P_MIN)


def test_acceptance_rate_and_residual_law():
    assert acceptance_checks()


def greedy_limit_ok(seed: int = 4) -> bool:
    """At T -> 0 the sampled rule is greedy verification: drafts are argmaxes and the
    accept length / emitted tokens equal the greedy oracle's."""
    rng = np.random.default_rng(seed)
    n, k, V, T = 6, 4, 12, 1e-5
    z = np.round(rng.normal(0, 2, (n, k, V)), 2) + rng.permutation(V) * 1e-3
    t = np.round(rng.normal(0, 2, (n, k + 1, V)), 2) + rng.permutation(V) * 1e-3
    # plant agreement on a prefix of every sequence
    for j in range(n):
        for i in range(j % (k + 1)):
            t[j, i] = z[j, i]
    d = sp.sample_drafts(z, T, seed, 1)
    if not np.array_equal(d["draft"], np.argmax(z, axis=-1)):
        return False
    r = sp.verify_sampled(d["draft"], z, t, T, seed, 1)
    dims = tiny_dims(block_k=k, batch=n, vocab=V)
    st = orc.new_state(dims, batch=n, ctx_len=[20] * n)
    g = orc.verify_commit(dims, st, d["draft"], np.argmax(t, axis=-1))
    return (np.array_equal(r["accept_len"], g["accept_len"]) and
            np.array_equal(r["out_tokens"], g["out_tokens"]))


def test_zero_temperature_limit_is_greedy():
    assert greedy_limit_ok()


def test_equal_distributions_accept_everything():
    rng = np.random.default_rng(6)
    z = rng.normal(0, 1, (3, 5, 9))
    t = np.concatenate([z, rng.normal(0, 1, (3, 1, 9))], axis=1)
    for step in range(40):
        x = sp.sample_drafts(z, 0.8, 2, step)["draft"]
        assert np.all(sp.verify_sampled(x, z, t, 0.8, 2, step)["accept_len"] == 5)


def test_zero_probability_draft_is_rejected_there():
    rng = np.random.default_rng(7)
    z = rng.normal(0, 1, (2, 4, 9))
    for step in range(30):
        x = sp.sample_drafts(z, 1.0, 5, step)["draft"]
        t = np.concatenate([z, rng.normal(0, 1, (2, 1, 9))], axis=1)
        r_at = [1, 3]
        for j in range(2):
            t[j, r_at[j], x[j, r_at[j]]] = -1e4
        r = sp.verify_sampled(x, z, t, 1.0, 5, step)
        assert list(r["accept_len"]) == r_at
        for j in range(2):
            assert r["emitted"][j] != x[j, r_at[j]]
            assert list(r["out_tokens"][j, :r_at[j]]) == list(x[j, :r_at[j]])


def test_commit_moves_state_like_greedy():
    dims = tiny_dims(block_k=3, batch=2)
    st = orc.new_state(dims, batch=2, ctx_len=[10, 20])
    sp.commit_sampled(dims, st, {"accept_len": np.array([0, 3]), "emitted": np.array([5, 9])})
    assert list(st.ctx_len) == [11, 24] and list(st.anchor) == [5, 9]
