"""The entry points inside a captured HIP graph, replayed with new inputs (through the C ABI).

A captured launch keeps its arguments, so every replay of the decode runs with the same call
tag on the same completion words; each replay must still merge its chunks and equal an eager
call on the same inputs, bit for bit. Between replays the test writes new query values
(eager work on the stream) and synchronises, as a serving loop would.
"""

import numpy as np
import pytest

import oracle
import exact_tiled_attention_24_amd as fa
from exact_tiled_attention_24_amd import inputs as gen
from helpers import assert_close, cuda_device, log_case, to_np

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module")
def dev():
    return cuda_device()


def new_q(shape, rep, dev):
    import torch

    rng = np.random.default_rng(7000 + rep)
    return gen.to_torch(rng.standard_normal(shape).astype(np.float32), "bf16", dev)


@pytest.mark.parametrize("noalloc", [False, True])
def test_decode_graph_replays(noalloc, dev):
    import torch

    x = gen.decode_inputs(3, 16, 4, 128, 16, seed=808, lens=[1000, 4097, 33],
                          max_pages_per_seq=260)
    log_case(f"decode graph replays noalloc={noalloc}")
    q = gen.to_torch(x.q, "bf16", dev)
    kc, vc = gen.to_torch(x.k_cache, "bf16", dev), gen.to_torch(x.v_cache, "bf16", dev)
    table = torch.from_numpy(x.block_table).to(dev)
    lens = torch.from_numpy(x.lens.astype(np.int32)).to(dev)
    out = torch.empty_like(q)
    splits = 3  # several chunks per sequence: the merge runs on every replay
    B, Hq, d = q.shape
    ws = torch.empty(max(16, fa.fa_decode_workspace_bytes(B, Hq, d, 16, x.max_seq_len, splits)),
                     dtype=torch.uint8, device=dev)

    def call():
        if noalloc:
            fa.fa_decode_splitk_noalloc(q, kc, vc, table, lens, x.max_seq_len, out, scale=x.scale,
                                        num_splits=splits)
        else:
            fa.fa_decode_splitk(q, kc, vc, table, lens, x.max_seq_len, scale=x.scale,
                                num_splits=splits, out=out, workspace=ws)

    call()  # eager first (per-device set-up happens outside the capture)
    torch.cuda.synchronize()
    first = out.clone()
    ref, _, _ = oracle.decode(x.q, x.k_seqs, x.v_seqs, x.scale)
    assert_close(to_np(first), ref, "bf16", "eager O")

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        q.copy_(new_q(tuple(q.shape), rep, dev))
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        want = fa.fa_decode_splitk(q, kc, vc, table, lens, x.max_seq_len, scale=x.scale,
                                   num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"replay {rep} differs from an eager call"
    del g


def test_fwd_graph_replays(dev):
    import torch

    x = gen.fwd_inputs(1, 4, 4, 1000, 128, 909, causal=True)
    log_case("fa_fwd graph replays B1 H4 N1000 d128 causal")
    q, k, v = (gen.to_torch(t, "bf16", dev) for t in (x.q, x.k, x.v))
    out = torch.empty_like(q)
    fa.fa_fwd(q, k, v, scale=x.scale, causal=True, out=out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.fa_fwd(q, k, v, scale=x.scale, causal=True, out=out)
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        q.copy_(new_q(tuple(q.shape), rep, dev))
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        want = fa.fa_fwd(q, k, v, scale=x.scale, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"replay {rep} differs from an eager call"
    del g
