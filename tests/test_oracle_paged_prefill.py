"""Pins for the oracle's paged prefill (CPU only).

``oracle.prefill_paged`` is attention of each sequence's newest Nq tokens against its whole
cached history, with the causal diagonal aligned to the bottom right (query i at position
L - Nq + i). It is pinned by reductions to cases pinned elsewhere — Nq = L is ordinary
causal attention, Nq = 1 is single-query decode — by a pure-Python brute force over ragged
lengths (including Nq > L, whose first rows see no key), and by the shared-prefix identity:
merging the partial over a prefix with the partial over the rest equals the whole.
Planted alignment mistakes must fail one of these pins.
"""

import math

import numpy as np
import pytest

import oracle


def brute_prefill(q, ks, vs, scale, causal):
    """Pure Python, no max subtraction, math.fsum; positions written out per query."""
    B, Hq, nq, d = q.shape
    out = np.zeros((B, Hq, nq, d))
    ms = np.full((B, Hq, nq), -math.inf)
    ls = np.zeros((B, Hq, nq))
    for b in range(B):
        L = ks[b].shape[1]
        g = Hq // ks[b].shape[0]
        for h in range(Hq):
            kk, vv = ks[b][h // g], vs[b][h // g]
            for i in range(nq):
                pos = L - nq + i
                keys = [j for j in range(L) if not causal or j <= pos]
                if not keys:
                    continue
                s = {j: scale * math.fsum(float(q[b, h, i, t]) * float(kk[j, t]) for t in range(d))
                     for j in keys}
                e = {j: math.exp(s[j]) for j in keys}
                z = math.fsum(e.values())
                mx = max(s.values())
                out[b, h, i] = [math.fsum(e[j] * float(vv[j, c]) for j in keys) / z for c in range(d)]
                ms[b, h, i] = mx
                ls[b, h, i] = z * math.exp(-mx)
    return out, ms, ls


def _draw(rng, lens, Hq, Hkv, nq, d):
    q = rng.standard_normal((len(lens), Hq, nq, d))
    ks = [rng.standard_normal((Hkv, L, d)) for L in lens]
    vs = [rng.standard_normal((Hkv, L, d)) for L in lens]
    return q, ks, vs


def pin_full_chunk_is_causal_attention(fn):
    """Nq = L for every sequence: query i sits at position i, the ordinary causal case."""
    rng = np.random.default_rng(41)
    L, Hq, Hkv, d = 13, 4, 2, 5
    q, ks, vs = _draw(rng, [L, L], Hq, Hkv, L, d)
    o, m, l = fn(q, ks, vs, 0.45, True)
    k = np.stack(ks)
    v = np.stack(vs)
    o_ref, m_ref, l_ref = oracle.attention(q, k, v, 0.45, True)
    np.testing.assert_allclose(o, o_ref, atol=1e-13)
    np.testing.assert_allclose(m, m_ref, atol=1e-13)
    np.testing.assert_allclose(l, l_ref, rtol=1e-12)


def pin_single_query_is_decode(fn):
    """Nq = 1: the one query is the newest token and sees every key, as in decode."""
    rng = np.random.default_rng(42)
    lens = [1, 7, 30]
    q, ks, vs = _draw(rng, lens, 4, 1, 1, 6)
    for causal in (True, False):
        o, m, l = fn(q, ks, vs, 0.6, causal)
        o_ref, m_ref, l_ref = oracle.decode(q[:, :, 0], ks, vs, 0.6)
        np.testing.assert_allclose(o[:, :, 0], o_ref, atol=1e-13)
        np.testing.assert_allclose(m[:, :, 0], m_ref, atol=1e-13)
        np.testing.assert_allclose(l[:, :, 0], l_ref, rtol=1e-12)


def pin_brute_ragged(fn):
    """Ragged lengths, Nq below, at and above L; GQA 2:1; both mask settings."""
    rng = np.random.default_rng(43)
    lens = [3, 5, 9, 0]
    q, ks, vs = _draw(rng, lens, 4, 2, 5, 3)
    for causal in (True, False):
        o, m, l = fn(q, ks, vs, 0.7, causal)
        ob, mb, lb = brute_prefill(q, ks, vs, 0.7, causal)
        np.testing.assert_allclose(o, ob, atol=1e-12)
        np.testing.assert_array_equal(np.isinf(m), np.isinf(mb))
        fin = np.isfinite(mb)
        np.testing.assert_allclose(m[fin], mb[fin], atol=1e-12)
        np.testing.assert_allclose(l, lb, rtol=1e-11)
    # L = 3 < Nq = 5 (causal): the first two queries see no key
    o, m, l = fn(q, ks, vs, 0.7, True)
    assert np.all(o[0, :, :2] == 0) and np.all(m[0, :, :2] == -np.inf) and np.all(l[0, :, :2] == 0)
    assert np.all(l[0, :, 2:] > 0)
    # L = 0: nothing to attend to
    assert np.all(o[3] == 0) and np.all(l[3] == 0)


def pin_shared_prefix_merge(fn):
    """Keys split into a prefix of P tokens and the rest: every query (all positions >= P)
    sees the whole prefix, so its partial is the unmasked one; the rest is again a paged
    prefill with bottom-right alignment. Merging the two equals the whole."""
    rng = np.random.default_rng(44)
    lens, P, nq = [20, 27], 11, 6
    q, ks, vs = _draw(rng, lens, 2, 2, nq, 4)
    o, m, l = fn(q, ks, vs, 0.5, True)
    pre = fn(q, [k[:, :P] for k in ks], [v[:, :P] for v in vs], 0.5, False)
    suf = fn(q, [k[:, P:] for k in ks], [v[:, P:] for v in vs], 0.5, True)
    R = q.shape[0] * q.shape[1] * nq
    om, mm, lm = oracle.merge(np.stack([pre[0].reshape(R, -1), suf[0].reshape(R, -1)]),
                              np.stack([pre[1].reshape(R), suf[1].reshape(R)]),
                              np.stack([pre[2].reshape(R), suf[2].reshape(R)]))
    np.testing.assert_allclose(om, o.reshape(R, -1), atol=1e-13)
    np.testing.assert_allclose(mm, m.reshape(R), atol=1e-13)
    np.testing.assert_allclose(lm, l.reshape(R), rtol=1e-12)


PINS = (pin_full_chunk_is_causal_attention, pin_single_query_is_decode, pin_brute_ragged,
        pin_shared_prefix_merge)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_prefill_paged_pins(pin):
    pin(oracle.prefill_paged)


def _mutant(kind):
    """A copy of the definition with one planted mistake in the query positions."""
    def fn(q, ks, vs, scale, causal):
        B, Hq, nq, d = q.shape
        out = np.zeros((B, Hq, nq, d))
        ms = np.full((B, Hq, nq), -np.inf)
        ls = np.zeros((B, Hq, nq))
        for b in range(B):
            L = ks[b].shape[1]
            g = Hq // ks[b].shape[0]
            if kind == "top_left":
                pos = np.arange(nq)
            elif kind == "off_by_one":
                pos = L - nq + np.arange(nq) - 1
            elif kind == "strict":
                pos = L - nq + np.arange(nq) - 0.5
            else:
                pos = L - nq + np.arange(nq)
            for h in range(Hq):
                s = scale * (q[b, h] @ ks[b][h // g].T)
                allowed = (np.arange(L)[None, :] <= pos[:, None]) if causal else np.ones(s.shape, bool)
                sm = np.where(allowed, s, -np.inf)
                m = sm.max(axis=1) if L else np.full(nq, -np.inf)
                sh = np.where(np.isfinite(m), m, 0.0)
                p = np.where(allowed, np.exp(sm - sh[:, None]), 0.0)
                l = p.sum(axis=1)
                out[b, h] = np.where(l[:, None] > 0, (p @ vs[b][h // g]) / np.where(l > 0, l, 1)[:, None], 0)
                ms[b, h], ls[b, h] = m, l
        return out, ms, ls
    return fn


@pytest.mark.parametrize("kind", ["top_left", "off_by_one", "strict"])
def test_prefill_pins_catch_alignment_mistakes(kind):
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(_mutant(kind))
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught {kind!r}"


def test_prefill_mutant_harness_passes_when_correct():
    for pin in PINS:
        pin(_mutant("none"))


def test_varlen_queries_reduce_to_single_sequences():
    """With per-sequence query counts, each sequence's rows equal prefill_paged on that
    sequence alone with Nq = its count; the rows past it are empty; counts all equal to Nq
    give the uniform result."""
    rng = np.random.default_rng(45)
    lens, Nq = [9, 14, 5, 0], 6
    q, ks, vs = _draw(rng, lens, 4, 2, Nq, 3)
    q_lens = [6, 3, 0, 2]
    for causal in (True, False):
        o, m, l = oracle.prefill_paged(q, ks, vs, 0.8, causal, q_lens=q_lens)
        for b, n in enumerate(q_lens):
            ob, mb, lb = oracle.prefill_paged(q[b:b + 1, :, :n], ks[b:b + 1], vs[b:b + 1], 0.8, causal)
            np.testing.assert_allclose(o[b, :, :n], ob[0], atol=1e-13)
            np.testing.assert_allclose(l[b, :, :n], lb[0], rtol=1e-12)
            assert np.all(o[b, :, n:] == 0) and np.all(l[b, :, n:] == 0) and np.all(m[b, :, n:] == -np.inf)
        ou, mu, lu = oracle.prefill_paged(q, ks, vs, 0.8, causal, q_lens=[Nq] * 4)
        o0, m0, l0 = oracle.prefill_paged(q, ks, vs, 0.8, causal)
        np.testing.assert_array_equal(ou, o0)
        np.testing.assert_array_equal(lu, l0)
    # a planted mistake: positions from Nq instead of the sequence's own count
    o_bad = np.zeros_like(o)
    for b, n in enumerate(q_lens):
        if n:
            ob, _, _ = oracle.prefill_paged(q[b:b + 1], ks[b:b + 1], vs[b:b + 1], 0.8, True)
            o_bad[b, :, :n] = ob[0, :, :n]
    o, _, _ = oracle.prefill_paged(q, ks, vs, 0.8, True, q_lens=q_lens)
    assert not np.allclose(o_bad, o)
