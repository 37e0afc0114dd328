"""Pins for the float64 CPU oracle (CPU only).

The oracle is checked against things other than itself: the values the worked example on
"FlashAttention, explained." prints, closed forms, invariants that hold in exact arithmetic,
and a brute-force route (pure Python, ``math.exp`` without max subtraction, ``math.fsum``)
that shares no code with it. A final group plants plausible mistakes into copies of the
oracle's definition and checks that at least one pin fails for each, so the pins are known
to bite.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle


# ----------------------------------------------------------------------------------------
# Brute force: a different route to the same definition, for tiny inputs only.
# ----------------------------------------------------------------------------------------

def brute_head(q, k, v, scale, causal):
    """Pure-Python exact attention without max subtraction, summed with math.fsum."""
    n, nk, dv = len(q), len(k), len(v[0])
    out, ms, ls = [], [], []
    for i in range(n):
        keys = [j for j in range(nk) if (not causal or j <= i)]
        if not keys:
            out.append([0.0] * dv)
            ms.append(-math.inf)
            ls.append(0.0)
            continue
        s = {j: scale * math.fsum(float(q[i][t]) * float(k[j][t]) for t in range(len(q[i])))
             for j in keys}
        e = {j: math.exp(s[j]) for j in keys}
        z = math.fsum(e.values())
        mx = max(s.values())
        out.append([math.fsum(e[j] * float(v[j][c]) for j in keys) / z for c in range(dv)])
        ms.append(mx)
        ls.append(z * math.exp(-mx))
    return np.array(out), np.array(ms), np.array(ls)


def load_golden(golden_dir):
    with open(os.path.join(golden_dir, "worked_example.json")) as f:
        return json.load(f)


# ----------------------------------------------------------------------------------------
# Pins, written against callables so the mutation tests below can reuse them.
# Each returns None on success and raises AssertionError on failure.
# ----------------------------------------------------------------------------------------

def pin_worked_example(head, g):
    row = np.array(g["row"])
    d = row.size
    q = row[None, :]
    eye = np.eye(d)
    o, m, l = head(q, eye, eye, 1.0, False)
    tol = 0.5 * 10.0 ** -g["printed_decimals"]
    np.testing.assert_allclose(o[0], g["weights"], atol=tol, rtol=0)
    assert abs(m[0] - g["m"]) <= 1e-12
    assert abs(l[0] - g["l"]) <= tol


def pin_rows_sum_to_one(head):
    rng = np.random.default_rng(11)
    for causal in (False, True):
        q = rng.standard_normal((9, 5))
        k = rng.standard_normal((9, 5))
        ones = np.ones((9, 3))
        o, _, _ = head(q, k, ones, 0.7, causal)
        np.testing.assert_allclose(o, 1.0, atol=1e-12, rtol=0)


def pin_uniform_scores(head):
    rng = np.random.default_rng(12)
    n, d = 10, 4
    v = rng.standard_normal((n, d))
    k = rng.standard_normal((n, d))
    q = np.zeros((n, d))
    o, m, l = head(q, k, v, 0.3, False)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), atol=1e-12)
    np.testing.assert_allclose(l, n, atol=1e-12)
    np.testing.assert_allclose(m, 0.0, atol=0)
    o, _, l = head(q, k, v, 0.3, True)
    prefix = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(o, prefix, atol=1e-12)
    np.testing.assert_allclose(l, np.arange(1, n + 1), atol=1e-12)


def pin_causal_row0(head):
    rng = np.random.default_rng(13)
    q, k, v = (rng.standard_normal((6, 3)) for _ in range(3))
    o, m, l = head(q, k, v, 1.3, True)
    assert np.array_equal(o[0], v[0])
    assert l[0] == 1.0
    assert m[0] == 1.3 * float(q[0] @ k[0])


def pin_brute(head):
    rng = np.random.default_rng(14)
    for n, d, causal, scale in ((1, 1, False, 1.0), (5, 3, False, 0.41), (7, 8, True, 0.9),
                                (16, 8, True, 1 / math.sqrt(8)), (12, 2, False, 2.5)):
        q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
        v = rng.standard_normal((n, d + 1))
        ob, mb, lb = brute_head(q.tolist(), k.tolist(), v.tolist(), scale, causal)
        o, m, l = head(q, k, v, scale, causal)
        np.testing.assert_allclose(o, ob, atol=1e-13, rtol=1e-12)
        np.testing.assert_allclose(m, mb, atol=1e-13, rtol=1e-12)
        np.testing.assert_allclose(l, lb, atol=1e-13, rtol=1e-12)


def pin_two_keys(head):
    q = np.array([[0.5, -1.0]])
    k = np.array([[1.0, 2.0], [-3.0, 0.25]])
    v = np.array([[1.0, 0.0, 2.0], [0.0, 1.0, -4.0]])
    scale = 0.8
    s0, s1 = scale * (q[0] @ k[0]), scale * (q[0] @ k[1])
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    o, _, _ = head(q, k, v, scale, False)
    np.testing.assert_allclose(o[0], w0 * v[0] + (1 - w0) * v[1], atol=1e-15)


def pin_one_hot_and_no_overflow(head):
    rng = np.random.default_rng(15)
    n, d = 8, 4
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    q = k[5:6] * 1.0
    scores = k @ q[0]
    assert int(np.argmax(scores)) == 5
    o, m, l = head(q, k, v, 1e4, False)
    np.testing.assert_allclose(o[0], v[5], atol=1e-12)
    assert np.isfinite(m).all() and abs(l[0] - 1.0) < 1e-12
    # scores around 1e3 overflow exp() unless the maximum is subtracted first
    q2 = np.full((1, 2), 30.0)
    k2 = np.array([[20.0, 20.0], [19.0, 20.0]])
    o, m, l = head(q2, k2, v[:2], 1.0, False)
    w0 = 1.0 / (1.0 + math.exp(-30.0))
    assert np.isfinite(o).all()
    np.testing.assert_allclose(o[0], w0 * v[0] + (1 - w0) * v[1], atol=1e-12)


def pin_key_shift(head):
    rng = np.random.default_rng(16)
    q, k, v = (rng.standard_normal((7, 5)) for _ in range(3))
    c = rng.standard_normal(5)
    for causal in (False, True):
        o1, _, _ = head(q, k, v, 0.6, causal)
        o2, _, _ = head(q, k + c[None, :], v, 0.6, causal)
        np.testing.assert_allclose(o1, o2, atol=1e-12)


def pin_key_permutation(head):
    rng = np.random.default_rng(17)
    q, k, v = (rng.standard_normal((9, 4)) for _ in range(3))
    perm = rng.permutation(9)
    o1, m1, l1 = head(q, k, v, 0.5, False)
    o2, m2, l2 = head(q, k[perm], v[perm], 0.5, False)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l1, l2, atol=1e-12)


HEAD_PINS = (pin_rows_sum_to_one, pin_uniform_scores, pin_causal_row0, pin_brute,
             pin_two_keys, pin_one_hot_and_no_overflow, pin_key_shift, pin_key_permutation)


# ----------------------------------------------------------------------------------------
# The oracle against its pins
# ----------------------------------------------------------------------------------------

def test_worked_example_head(golden_dir):
    pin_worked_example(oracle.attention_head, load_golden(golden_dir))


def test_worked_example_online(golden_dir):
    """The two-block walk of the worked example, through the running (m, l, O) update."""
    g = load_golden(golden_dir)
    eye = np.eye(len(g["row"]))
    blocks = g["blocks"]
    vals = [eye[:len(blocks[0])], eye[len(blocks[0]):]]
    o, m, l, trace = oracle.online_softmax(blocks, vals)
    tol = 0.5 * 10.0 ** -g["printed_decimals"]
    assert trace[0][0] == g["m_after_first_block"]
    np.testing.assert_allclose(trace[0][1], 1.0 + math.exp(-1.0), atol=1e-15)
    assert m == g["m"]
    assert abs(l - g["l"]) <= tol
    np.testing.assert_allclose(o, g["weights"], atol=tol, rtol=0)
    # the rescale factor e^(2-3) is the page's correction of every old term
    np.testing.assert_allclose(trace[1][1], trace[0][1] * math.exp(2 - 3) + math.exp(0) + math.exp(-3),
                               atol=1e-15)


def test_worked_example_merge(golden_dir):
    """Two partials over keys {0, 1} and {2, 3}, merged, give the whole-row weights."""
    g = load_golden(golden_dir)
    row = np.array(g["row"])
    eye = np.eye(4)
    parts = []
    for keys in ([0, 1], [2, 3]):
        # scores against unit-vector keys are the row entries themselves
        o, m, l = oracle.attention_head(row[None, :], eye[keys], eye[keys], 1.0, False)
        parts.append((o[0], m[0], l[0]))
    o_parts = np.stack([p[0] for p in parts])[:, None, :]
    m_parts = np.array([[p[1]] for p in parts])
    l_parts = np.array([[p[2]] for p in parts])
    o, m, l = oracle.merge(o_parts, m_parts, l_parts)
    tol = 0.5 * 10.0 ** -g["printed_decimals"]
    np.testing.assert_allclose(o[0], g["weights"], atol=tol, rtol=0)
    assert m[0] == g["m"] and abs(l[0] - g["l"]) <= tol


@pytest.mark.parametrize("pin", HEAD_PINS, ids=lambda p: p.__name__)
def test_head_pins(pin):
    pin(oracle.attention_head)


def test_probs_rows_sum_to_one():
    rng = np.random.default_rng(21)
    q, k = rng.standard_normal((12, 6)), rng.standard_normal((12, 6))
    for causal in (False, True):
        p = oracle.attention_probs(q, k, 0.4, causal)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)
        if causal:
            assert np.all(np.triu(p, 1) == 0)
        # P V reproduces the oracle's O
        v = rng.standard_normal((12, 3))
        o, _, _ = oracle.attention_head(q, k, v, 0.4, causal)
        np.testing.assert_allclose(p @ v, o, atol=1e-12)


def test_live_demo_streaming():
    """The streaming demo on "FlashAttention": 8 tokens, causal, 2x2 tiles.

    Each query row is streamed tile by tile through the running update, skipping the tiles
    above the diagonal; the result equals the whole-row softmax.
    """
    rng = np.random.default_rng(22)
    n, d, tile = 8, 4, 2
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    o_ref, m_ref, l_ref = oracle.attention_head(q, k, v, 0.5, True)
    for i in range(n):
        s_blocks, v_blocks = [], []
        qb = i // tile
        for kb in range(qb + 1):  # tiles strictly above the diagonal are never touched
            j = np.arange(kb * tile, (kb + 1) * tile)
            j = j[j <= i]
            s_blocks.append(0.5 * (k[j] @ q[i]))
            v_blocks.append(v[j])
        o, m, l, _ = oracle.online_softmax(s_blocks, v_blocks)
        np.testing.assert_allclose(o, o_ref[i], atol=1e-13)
        assert abs(m - m_ref[i]) <= 1e-13 and abs(l - l_ref[i]) <= 1e-13


def test_online_random_tilings():
    rng = np.random.default_rng(23)
    for _ in range(20):
        n, d = rng.integers(1, 40), rng.integers(1, 9)
        s = rng.standard_normal(n) * 3
        v = rng.standard_normal((n, d))
        cuts = np.sort(rng.choice(np.arange(1, n + 1), size=min(n, 4), replace=False))
        cuts = np.unique(np.concatenate([[0], cuts, [n]]))
        sb = [s[a:b] for a, b in zip(cuts[:-1], cuts[1:])]
        vb = [v[a:b] for a, b in zip(cuts[:-1], cuts[1:])]
        o, m, l, _ = oracle.online_softmax(sb, vb)
        o_ref, m_ref, l_ref = oracle.attention_head(s[None, :], np.eye(n), v, 1.0, False)
        np.testing.assert_allclose(o, o_ref[0], atol=1e-13)
        assert abs(m - m_ref[0]) <= 1e-13 and abs(l - l_ref[0]) <= 1e-12


def test_empty_row_conventions():
    o, m, l = oracle.attention_head(np.ones((1, 2)), np.zeros((0, 2)), np.zeros((0, 3)), 1.0, False)
    assert np.all(o == 0) and m[0] == -np.inf and l[0] == 0
    o, m, l = oracle.merge(np.zeros((2, 1, 3)), np.full((2, 1), -np.inf), np.zeros((2, 1)))
    assert np.all(o == 0) and m[0] == -np.inf and l[0] == 0
    # an empty partial carries no weight, whatever its O holds
    o, m, l = oracle.merge(np.array([[[1.0, 2.0]], [[np.nan, np.nan]]]), np.array([[0.5], [-np.inf]]),
                           np.array([[2.0], [0.0]]))
    np.testing.assert_array_equal(o, [[1.0, 2.0]])
    assert m[0] == 0.5 and l[0] == 2.0


def test_closed_forms_small_n():
    rng = np.random.default_rng(24)
    v = rng.standard_normal((1, 5))
    o, m, l = oracle.attention_head(rng.standard_normal((1, 5)), rng.standard_normal((1, 5)), v, 0.3,
                                    False)
    np.testing.assert_array_equal(o[0], v[0])


def test_gqa_equals_repeated_mha():
    rng = np.random.default_rng(25)
    B, Hq, Hkv, N, d = 2, 6, 2, 11, 4
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    o1, m1, l1 = oracle.attention(q, k, v, 0.5, True)
    k_rep = np.repeat(k, Hq // Hkv, axis=1)
    v_rep = np.repeat(v, Hq // Hkv, axis=1)
    o2, m2, l2 = oracle.attention(q, k_rep, v_rep, 0.5, True)
    np.testing.assert_array_equal(o1, o2)
    # and each head of the multi-head call is the single-head definition
    for b in range(B):
        for h in range(Hq):
            o, _, _ = brute_head(q[b, h].tolist(), k_rep[b, h].tolist(), v_rep[b, h].tolist(), 0.5, True)
            np.testing.assert_allclose(o1[b, h], o, atol=1e-12)


def test_scale_folding():
    rng = np.random.default_rng(26)
    q, k, v = (rng.standard_normal((6, 4)) for _ in range(3))
    o1, m1, l1 = oracle.attention_head(q, k, v, 0.37, True)
    o2, m2, l2 = oracle.attention_head(0.37 * q, k, v, 1.0, True)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(m1, m2, atol=1e-13)


def test_row_blocks_and_rows_do_not_change_result():
    rng = np.random.default_rng(27)
    q, k, v = (rng.standard_normal((37, 4)) for _ in range(3))
    o1, m1, l1 = oracle.attention_head(q, k, v, 0.5, True, row_block=256)
    o2, m2, l2 = oracle.attention_head(q, k, v, 0.5, True, row_block=5)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    rows = np.array([36, 0, 17])
    o3, m3, l3 = oracle.attention_head(q, k, v, 0.5, True, rows=rows)
    np.testing.assert_allclose(o3, o1[rows], atol=1e-14)


def test_decode_is_last_row_of_causal_prefill():
    rng = np.random.default_rng(28)
    Hq, Hkv, d = 4, 2, 8
    lens = [1, 9, 23]
    q = rng.standard_normal((len(lens), Hq, d))
    ks = [rng.standard_normal((Hkv, L, d)) for L in lens]
    vs = [rng.standard_normal((Hkv, L, d)) for L in lens]
    o, m, l = oracle.decode(q, ks, vs, 0.35)
    for b, L in enumerate(lens):
        for h in range(Hq):
            qq = rng.standard_normal((L, d))
            qq[-1] = q[b, h]
            op, mp, lp = oracle.attention_head(qq, ks[b][h // 2], vs[b][h // 2], 0.35, True)
            np.testing.assert_allclose(o[b, h], op[-1], atol=1e-13)
            assert abs(m[b, h] - mp[-1]) < 1e-13 and abs(l[b, h] - lp[-1]) < 1e-12


def _partials(q, k, v, scale, bounds):
    parts = [oracle.attention_head(q, k[a:b], v[a:b], scale, False) for a, b in bounds]
    return (np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]),
            np.stack([p[2] for p in parts]))


def test_merge_any_partition_equals_unsplit():
    rng = np.random.default_rng(29)
    n, d = 50, 6
    q = rng.standard_normal((5, d))
    k, v = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    o_ref, m_ref, l_ref = oracle.attention_head(q, k, v, 0.8, False)
    for splits in (1, 2, 7, 50):
        edges = np.linspace(0, n, splits + 1).astype(int)
        o, m, l = oracle.merge(*_partials(q, k, v, 0.8, list(zip(edges[:-1], edges[1:]))))
        np.testing.assert_allclose(o, o_ref, atol=1e-13)
        np.testing.assert_allclose(m, m_ref, atol=1e-13)
        np.testing.assert_allclose(l, l_ref, rtol=1e-12)
    # uneven partition with an empty chunk
    bounds = [(0, 3), (3, 3), (3, 40), (40, 50)]
    o, m, l = oracle.merge(*_partials(q, k, v, 0.8, bounds))
    np.testing.assert_allclose(o, o_ref, atol=1e-13)


def test_merge_associative():
    rng = np.random.default_rng(30)
    n, d = 30, 4
    q = rng.standard_normal((3, d))
    k, v = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    o3, m3, l3 = _partials(q, k, v, 1.1, [(0, 10), (10, 20), (20, 30)])
    flat = oracle.merge(o3, m3, l3)
    left = oracle.merge(o3[:2], m3[:2], l3[:2])
    nested = oracle.merge(np.stack([left[0], o3[2]]), np.stack([left[1], m3[2]]),
                          np.stack([left[2], l3[2]]))
    for a, b in zip(flat, nested):
        np.testing.assert_allclose(a, b, atol=1e-13)


# ----------------------------------------------------------------------------------------
# Planted mistakes: every mutant of the definition must fail at least one pin.
# ----------------------------------------------------------------------------------------

def _mutant_head(kind):
    def head(q, k, v, scale, causal):
        q, k, v = np.asarray(q, float), np.asarray(k, float), np.asarray(v, float)
        n, nk = q.shape[0], k.shape[0]
        sc = 1.0 if kind == "no_scale" else scale
        s = sc * (q @ k.T)
        if kind == "transposed":
            s = sc * (k @ q.T) if n == nk else s  # S^T used as if it were S
        i = np.arange(n)[:, None]
        j = np.arange(nk)[None, :]
        if causal:
            allowed = (j < i) if kind == "strict_causal" else (j <= i + 1 if kind == "loose_causal" else j <= i)
        else:
            allowed = np.ones((n, nk), bool)
        s = np.where(allowed, s, -np.inf)
        m = s.max(axis=1)
        m = np.where(np.isfinite(m), m, 0.0)
        if kind == "plus_max":
            p = np.where(allowed, np.exp(s + m[:, None]), 0.0)
        elif kind == "m_unscaled":
            p = np.where(allowed, np.exp(s - m[:, None]), 0.0)
            m = m / sc
        else:
            p = np.where(allowed, np.exp(s - m[:, None]), 0.0)
        l = p.sum(axis=1)
        vv = k if kind == "k_for_v" else v
        if kind == "k_for_v" and k.shape[1] != v.shape[1]:
            vv = np.concatenate([k, k], axis=1)[:, :v.shape[1]]
        num = p @ vv
        if kind == "no_normalise":
            return num, m, l
        if kind == "sum_shifted":
            l = l + 1e-3
        return num / np.where(l > 0, l, 1)[:, None], m, l
    return head


MUTANTS = ("no_scale", "transposed", "strict_causal", "loose_causal", "plus_max", "m_unscaled",
           "k_for_v", "no_normalise", "sum_shifted")


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_catch_planted_mistakes(kind, golden_dir):
    head = _mutant_head(kind)
    g = load_golden(golden_dir)
    caught = []
    for pin in (lambda h: pin_worked_example(h, g),) + HEAD_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(head)
        except (AssertionError, FloatingPointError, ValueError):
            caught.append(pin)
    assert caught, f"no pin caught the planted mistake {kind!r}"


def test_correct_head_passes_the_mutant_harness(golden_dir):
    head = _mutant_head("none")
    g = load_golden(golden_dir)
    pin_worked_example(head, g)
    for pin in HEAD_PINS:
        pin(head)


def test_merge_mutants_are_caught():
    rng = np.random.default_rng(31)
    q = rng.standard_normal((4, 5))
    k, v = rng.standard_normal((20, 5)), rng.standard_normal((20, 5))
    o_ref, _, _ = oracle.attention_head(q, k, v, 0.7, False)
    parts = _partials(q, k, v, 0.7, [(0, 6), (6, 20)])

    def no_l(o_p, m_p, l_p):
        return oracle.merge(o_p, m_p, np.ones_like(l_p))

    def no_rescale(o_p, m_p, l_p):
        return oracle.merge(o_p, np.zeros_like(m_p), l_p)

    for bad in (no_l, no_rescale):
        o, _, _ = bad(*parts)
        assert not np.allclose(o, o_ref, atol=1e-6)
    o, _, _ = oracle.merge(*parts)
    np.testing.assert_allclose(o, o_ref, atol=1e-13)


def test_gqa_mapping_mutant_is_caught():
    rng = np.random.default_rng(32)
    B, Hq, Hkv, N, d = 1, 4, 2, 5, 3
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    o, _, _ = oracle.attention(q, k, v, 1.0, False)
    # interleaved mapping h % Hkv is a plausible mistake; consecutive groups are the reading
    wrong = np.stack([oracle.attention_head(q[0, h], k[0, h % Hkv], v[0, h % Hkv], 1.0, False)[0]
                      for h in range(Hq)])
    assert not np.allclose(o[0], wrong)
    right = np.stack([oracle.attention_head(q[0, h], k[0, h // 2], v[0, h // 2], 1.0, False)[0]
                      for h in range(Hq)])
    np.testing.assert_array_equal(o[0], right)
