"""fa_merge on the GPU against the float64 oracle (parity tests, through the C ABI)."""

import numpy as np
import pytest

import oracle
import exact_tiled_attention_24_amd as fa
from helpers import assert_close, cuda_device, log_case, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return cuda_device()


def make_partials(S, R, d, seed, empty_frac=0.0):
    """Partials of real attention over disjoint key chunks (so the merge is meaningful)."""
    rng = np.random.default_rng(seed)
    n = S * 9
    q = rng.standard_normal((R, 16))
    k = rng.standard_normal((n, 16))
    v = rng.standard_normal((n, d))
    edges = np.linspace(0, n, S + 1).astype(int)
    parts = [oracle.attention_head(q, k[a:b], v[a:b], 0.5, False) for a, b in zip(edges[:-1], edges[1:])]
    o_p = np.stack([p[0] for p in parts]).astype(np.float32)
    m_p = np.stack([p[1] for p in parts]).astype(np.float32)
    l_p = np.stack([p[2] for p in parts]).astype(np.float32)
    if empty_frac:
        dead = rng.random((S, R)) < empty_frac
        o_p[dead] = np.nan  # an empty partial's O is never read
        m_p[dead] = -np.inf
        l_p[dead] = 0.0
    return o_p, m_p, l_p


@pytest.mark.parametrize("S,R,d,empty", [(1, 7, 128, 0.0), (3, 50, 64, 0.0), (32, 256, 128, 0.3), (3, 11, 99, 0.2),
                                         (5, 9, 100, 0.5), (3000, 4, 128, 0.1)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_merge_random(S, R, d, empty, out, dev):
    import torch

    log_case(f"fa_merge S={S} R={R} d={d} empty={empty} out={out}")
    o_p, m_p, l_p = make_partials(S, R, d, seed=S * 1000 + R, empty_frac=empty)
    t = [torch.from_numpy(a).to(dev) for a in (o_p, m_p, l_p)]
    o, m, l = fa.fa_merge(*t, out_dtype=torch.float32 if out == "f32" else torch.bfloat16,
                          return_stats=True)
    torch.cuda.synchronize()
    o_ref, m_ref, l_ref = oracle.merge(o_p, m_p, l_p)
    got = to_np(o)
    if out == "f32":
        # inputs are float32 partials: compare against the exact merge of those values
        np.testing.assert_allclose(got, o_ref, atol=1e-5)
    else:
        assert_close(got, o_ref, "bf16", "merged O")
    live = l_ref > 0
    np.testing.assert_allclose(to_np(m)[live], m_ref[live], atol=1e-6)
    np.testing.assert_allclose(to_np(l)[live], l_ref[live], rtol=1e-5)
    assert np.all(got[~live] == 0) and np.all(to_np(l)[~live] == 0)


def test_merge_worked_example(dev):
    """Partials over keys {0, 1} and {2, 3} of the row [2, 1, 3, 0] merge into its softmax."""
    import torch

    log_case("fa_merge worked example")
    row = np.array([2.0, 1.0, 3.0, 0.0])
    eye = np.eye(4)
    parts = [oracle.attention_head(row[None, :], eye[ks], eye[ks], 1.0, False) for ks in ([0, 1], [2, 3])]
    o_p = np.stack([p[0] for p in parts]).astype(np.float32)
    m_p = np.stack([p[1] for p in parts]).astype(np.float32)
    l_p = np.stack([p[2] for p in parts]).astype(np.float32)
    o, m, l = fa.fa_merge(*[torch.from_numpy(a).to(dev) for a in (o_p, m_p, l_p)], return_stats=True)
    np.testing.assert_allclose(to_np(o)[0], [0.2369, 0.0871, 0.6439, 0.0321], atol=5e-5)
    np.testing.assert_allclose(to_np(m)[0], 3.0, atol=0)
    np.testing.assert_allclose(to_np(l)[0], 1.5530, atol=5e-5)
