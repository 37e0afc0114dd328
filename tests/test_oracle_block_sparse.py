"""Pins for the oracle's block-sparse attention (CPU only).

``oracle.attention_block_sparse`` admits key j for query i iff key block j // bk is listed
for query block i // bq (and j <= i when causal). It is pinned by reductions — listing every
block gives dense attention, listing the lower block triangle under the causal mask gives
causal attention, both pinned elsewhere — by a pure-Python brute force that expands the
block lists into an element mask on its own, by the merge of disjoint block sets (the union
of their keys), and by rows whose lists are empty. Planted mistakes in the block mapping
must fail one of these pins.
"""

import math

import numpy as np
import pytest

import oracle


def csr(rows):
    """Compressed rows from a list of key-block lists."""
    offsets = np.zeros(len(rows) + 1, dtype=np.int32)
    offsets[1:] = np.cumsum([len(r) for r in rows])
    indices = np.asarray([j for r in rows for j in r], dtype=np.int32)
    return offsets, indices


def brute(q, k, v, scale, causal, rows, bq, bk):
    B, Hq, N, d = q.shape
    g = Hq // k.shape[1]
    nqb = -(-N // bq)
    nkb = -(-N // bk)
    out = np.zeros((B, Hq, N, d))
    ms = np.full((B, Hq, N), -math.inf)
    ls = np.zeros((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            for i in range(N):
                listed = set(j for j in rows[(b * Hq + h) * nqb + i // bq] if 0 <= j < nkb)
                keys = [j for j in range(N) if j // bk in listed and (not causal or j <= i)]
                if not keys:
                    continue
                s = {j: scale * math.fsum(float(q[b, h, i, t]) * float(k[b, h // g, j, t])
                                          for t in range(d)) for j in keys}
                e = {j: math.exp(s[j]) for j in keys}
                z = math.fsum(e.values())
                mx = max(s.values())
                out[b, h, i] = [math.fsum(e[j] * float(v[b, h // g, j, c]) for j in keys) / z
                                for c in range(d)]
                ms[b, h, i] = mx
                ls[b, h, i] = z * math.exp(-mx)
    return out, ms, ls


def _draw(seed, B, Hq, Hkv, N, d):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, Hq, N, d)), rng.standard_normal((B, Hkv, N, d)),
            rng.standard_normal((B, Hkv, N, d)))


def pin_all_blocks_is_dense(fn):
    q, k, v = _draw(51, 2, 4, 2, 11, 5)
    bq, bk = 4, 3
    nqb, nkb = 3, 4
    rows = [list(range(nkb))] * (2 * 4 * nqb)
    for causal in (False, True):
        o, m, l = fn(q, k, v, 0.5, causal, *csr(rows), bq, bk)
        o_ref, m_ref, l_ref = oracle.attention(q, k, v, 0.5, causal)
        np.testing.assert_allclose(o, o_ref, atol=1e-13)
        np.testing.assert_allclose(m, m_ref, atol=1e-13)
        np.testing.assert_allclose(l, l_ref, rtol=1e-12)


def pin_lower_triangle_is_causal(fn):
    """Blocks (qb, kb) with kb * bk <= the block's last row, under the causal mask."""
    q, k, v = _draw(52, 1, 2, 1, 13, 4)
    bq, bk = 4, 2
    nqb, nkb = 4, 7
    rows = [[kb for kb in range(nkb) if kb * bk <= min(13, (qb + 1) * bq) - 1]
            for _ in range(2) for qb in range(nqb)]
    o, m, l = fn(q, k, v, 0.8, True, *csr(rows), bq, bk)
    o_ref, m_ref, l_ref = oracle.attention(q, k, v, 0.8, True)
    np.testing.assert_allclose(o, o_ref, atol=1e-13)
    np.testing.assert_allclose(l, l_ref, rtol=1e-12)


def pin_brute(fn):
    """Random block lists (with repeats of nothing, out-of-range entries and empty rows),
    GQA 2:1, both mask settings."""
    q, k, v = _draw(53, 2, 4, 2, 10, 3)
    bq, bk = 3, 2
    nqb, nkb = 4, 5
    rng = np.random.default_rng(54)
    rows = []
    for r in range(2 * 4 * nqb):
        sel = sorted(rng.choice(nkb, size=int(rng.integers(0, nkb + 1)), replace=False).tolist())
        if r % 5 == 0:
            sel = sel + [nkb + 2, -1]  # entries that name no key block
        rows.append(sel)
    rows[4] = []  # head 1, query block 0 (rows 0..2)
    for causal in (False, True):
        o, m, l = fn(q, k, v, 0.6, causal, *csr(rows), bq, bk)
        ob, mb, lb = brute(q, k, v, 0.6, causal, rows, bq, bk)
        np.testing.assert_allclose(o, ob, atol=1e-12)
        np.testing.assert_array_equal(np.isinf(m), np.isinf(mb))
        fin = np.isfinite(mb)
        np.testing.assert_allclose(m[fin], mb[fin], atol=1e-12)
        np.testing.assert_allclose(l, lb, rtol=1e-11)
    # an empty row list: its queries see nothing
    o, m, l = fn(q, k, v, 0.6, False, *csr(rows), bq, bk)
    assert np.all(o[0, 1, 0:3] == 0) and np.all(l[0, 1, 0:3] == 0)


def pin_disjoint_sets_merge(fn):
    """Two disjoint block sets per row, merged, equal the block-sparse result over their
    union."""
    q, k, v = _draw(55, 1, 2, 2, 12, 4)
    bq, bk = 4, 2
    nqb, nkb = 3, 6
    rng = np.random.default_rng(56)
    left, right, union = [], [], []
    for _ in range(2 * nqb):
        perm = rng.permutation(nkb).tolist()
        cut = int(rng.integers(1, nkb))
        left.append(sorted(perm[:cut]))
        right.append(sorted(perm[cut:]))
        union.append(sorted(perm))
    a = fn(q, k, v, 0.7, False, *csr(left), bq, bk)
    b = fn(q, k, v, 0.7, False, *csr(right), bq, bk)
    u = fn(q, k, v, 0.7, False, *csr(union), bq, bk)
    R = 2 * 12
    om, mm, lm = oracle.merge(np.stack([a[0].reshape(R, -1), b[0].reshape(R, -1)]),
                              np.stack([a[1].reshape(R), b[1].reshape(R)]),
                              np.stack([a[2].reshape(R), b[2].reshape(R)]))
    np.testing.assert_allclose(om, u[0].reshape(R, -1), atol=1e-13)
    np.testing.assert_allclose(lm, u[2].reshape(R), rtol=1e-12)


PINS = (pin_all_blocks_is_dense, pin_lower_triangle_is_causal, pin_brute, pin_disjoint_sets_merge)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_block_sparse_pins(pin):
    pin(oracle.attention_block_sparse)


def _mutant(kind):
    """A copy of the definition with one planted mistake in the block mapping."""
    def fn(q, k, v, scale, causal, offsets, indices, bq, bk):
        B, Hq, N, d = q.shape
        g = Hq // k.shape[1]
        nqb, nkb = -(-N // bq), -(-N // bk)
        out = np.zeros((B, Hq, N, d))
        ms = np.full((B, Hq, N), -np.inf)
        ls = np.zeros((B, Hq, N))
        for b in range(B):
            for h in range(Hq):
                blocks = np.zeros((nqb, nkb), bool)
                for qb in range(nqb):
                    r = (b * Hq + h) * nqb + qb
                    if kind == "row_of_next_head":
                        r = ((b * Hq + h + 1) % (B * Hq)) * nqb + qb
                    sel = np.asarray(indices[offsets[r]:offsets[r + 1]], int)
                    sel = sel[(sel >= 0) & (sel < nkb)]
                    if kind == "shifted_block":
                        sel = np.clip(sel + 1, 0, nkb - 1)
                    blocks[qb, sel] = True
                rows_b = np.arange(N) // (bk if kind == "swapped_sizes" else bq)
                keys_b = np.arange(N) // (bq if kind == "swapped_sizes" else bk)
                allowed = blocks[np.minimum(rows_b, nqb - 1)][:, np.minimum(keys_b, nkb - 1)]
                if causal:
                    allowed &= np.arange(N)[None, :] <= np.arange(N)[:, None]
                s = scale * (q[b, h] @ k[b, h // g].T)
                sm = np.where(allowed, s, -np.inf)
                m = sm.max(axis=1)
                sh = np.where(np.isfinite(m), m, 0.0)
                p = np.where(allowed, np.exp(sm - sh[:, None]), 0.0)
                l = p.sum(axis=1)
                out[b, h] = np.where(l[:, None] > 0, (p @ v[b, h // g]) / np.where(l > 0, l, 1)[:, None], 0)
                ms[b, h], ls[b, h] = m, l
        return out, ms, ls
    return fn


@pytest.mark.parametrize("kind", ["row_of_next_head", "shifted_block", "swapped_sizes"])
def test_block_sparse_pins_catch_mapping_mistakes(kind):
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(_mutant(kind))
        except (AssertionError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught {kind!r}"


def test_block_sparse_mutant_harness_passes_when_correct():
    for pin in PINS:
        pin(_mutant("none"))
