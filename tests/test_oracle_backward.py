"""Pins for the oracle's attention backward (CPU only).

``oracle.attention_backward`` gives dQ, dK, dV of O = softmax(scale q k^T + M) v. It is
pinned by central finite differences of the forward oracle (a different route: it never
forms dS), by the closed form D_i = sum_j P_ij dP_ij that the recomputation relies on, by
the grouped-query rule (a shared key/value head receives the sum of its query heads'
gradients, checked against separate single-head problems), and by the causal structure
(the last key is seen only by the last query). Planted mistakes — a dropped D, a missing
scale on dQ, dK from the untransposed dS, V's gradient through P instead of P^T — must fail
one of these pins.
"""

import numpy as np
import pytest

import oracle


def loss(q, k, v, dout, scale, causal):
    o, _, _ = oracle.attention(q, k, v, scale, causal)
    return float((o * dout).sum())


def fd_grad(fn, x, idx, eps=1e-6):
    xp = x.copy()
    xm = x.copy()
    xp[idx] += eps
    xm[idx] -= eps
    return (fn(xp) - fn(xm)) / (2 * eps)


def _draw(seed, B, Hq, Hkv, N, d):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, Hq, N, d)), rng.standard_normal((B, Hkv, N, d)),
            rng.standard_normal((B, Hkv, N, d)), rng.standard_normal((B, Hq, N, d)))


def pin_finite_differences(bwd):
    for causal in (False, True):
        q, k, v, do = _draw(61 + causal, 1, 4, 2, 6, 3)
        scale = 0.7
        dq, dk, dv = bwd(q, k, v, do, scale, causal)
        rng = np.random.default_rng(62)
        for which, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            for _ in range(6):
                idx = tuple(int(rng.integers(s)) for s in x.shape)

                def f(xx, which=which):
                    args = {"q": q, "k": k, "v": v}
                    args[which] = xx
                    return loss(args["q"], args["k"], args["v"], do, scale, causal)

                num = fd_grad(f, x, idx)
                assert abs(num - g[idx]) <= 1e-7 * max(1.0, abs(num)), (which, idx, num, g[idx])


def pin_d_identity(bwd):
    """dQ computed with D = rowsum(dO * O) equals the form with sum_j P_ij dP_ij."""
    q, k, v, do = _draw(63, 1, 1, 1, 7, 4)
    dq, _, _ = bwd(q, k, v, do, 0.5, True)
    p = oracle.attention_probs(q[0, 0], k[0, 0], 0.5, True)
    dp = do[0, 0] @ v[0, 0].T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    np.testing.assert_allclose(dq[0, 0], 0.5 * ds @ k[0, 0], atol=1e-12)


def pin_gqa_sums_heads(bwd):
    q, k, v, do = _draw(64, 1, 4, 2, 5, 3)
    dq, dk, dv = bwd(q, k, v, do, 0.9, False)
    for kh in range(2):
        acc_k = np.zeros_like(dk[0, kh])
        acc_v = np.zeros_like(dv[0, kh])
        for h in (2 * kh, 2 * kh + 1):
            sq, sk, sv = bwd(q[:, h:h + 1], k[:, kh:kh + 1], v[:, kh:kh + 1], do[:, h:h + 1], 0.9, False)
            np.testing.assert_allclose(dq[0, h], sq[0, 0], atol=1e-12)
            acc_k += sk[0, 0]
            acc_v += sv[0, 0]
        np.testing.assert_allclose(dk[0, kh], acc_k, atol=1e-12)
        np.testing.assert_allclose(dv[0, kh], acc_v, atol=1e-12)


def pin_causal_last_key(bwd):
    """Under the causal mask only the last query sees the last key: dV of the last key is
    P_{N-1,N-1} dO_{N-1}, and changing any earlier query's dO leaves it unchanged."""
    q, k, v, do = _draw(65, 1, 1, 1, 6, 2)
    _, _, dv = bwd(q, k, v, do, 1.0, True)
    p = oracle.attention_probs(q[0, 0], k[0, 0], 1.0, True)
    np.testing.assert_allclose(dv[0, 0, -1], p[-1, -1] * do[0, 0, -1], atol=1e-12)
    do2 = do.copy()
    do2[0, 0, :-1] += 3.0
    _, _, dv2 = bwd(q, k, v, do2, 1.0, True)
    np.testing.assert_allclose(dv2[0, 0, -1], dv[0, 0, -1], atol=1e-12)


PINS = (pin_finite_differences, pin_d_identity, pin_gqa_sums_heads, pin_causal_last_key)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_backward_pins(pin):
    pin(oracle.attention_backward)


def _mutant(kind):
    def bwd(q, k, v, dout, scale, causal):
        B, Hq, N, d = q.shape
        Hkv = k.shape[1]
        g = Hq // Hkv
        dq = np.zeros_like(q)
        dk = np.zeros_like(k)
        dv = np.zeros_like(v)
        for b in range(B):
            for h in range(Hq):
                kh = h // g
                p = oracle.attention_probs(q[b, h], k[b, kh], scale, causal)
                o = p @ v[b, kh]
                dvv = (p if kind == "dv_untransposed" else p.T) @ dout[b, h]
                dp = dout[b, h] @ v[b, kh].T
                dd = (dout[b, h] * o).sum(axis=1)
                ds = p * (dp - (0 if kind == "no_d" else dd[:, None]))
                dq[b, h] = (1.0 if kind == "dq_unscaled" else scale) * (ds @ k[b, kh])
                dk[b, kh] += scale * ((ds if kind == "dk_untransposed" else ds.T) @ q[b, h])
                dv[b, kh] += dvv
        return dq, dk, dv
    return bwd


@pytest.mark.parametrize("kind", ["no_d", "dq_unscaled", "dk_untransposed", "dv_untransposed"])
def test_backward_pins_catch_mistakes(kind):
    caught = []
    for pin in PINS:
        try:
            pin(_mutant(kind))
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught {kind!r}"


def test_backward_mutant_harness_passes_when_correct():
    for pin in PINS:
        pin(_mutant("none"))
