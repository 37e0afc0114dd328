"""Calls on two streams at once (through the C ABI).

fa_fwd keeps no state between calls and fa_decode_splitk keeps its partials and completion
words in the caller's workspace, so calls enqueued on two streams of one device, each with
its own outputs (and workspace), may overlap in time; each must equal the same call made
alone, bit for bit.
"""

import numpy as np
import pytest

import exact_tiled_attention_24_amd as fa
from exact_tiled_attention_24_amd import inputs as gen
from helpers import cuda_device, log_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return cuda_device()


def test_fwd_on_two_streams(dev):
    import torch

    log_case("fa_fwd on two streams B2 H8 N2000 d128 causal / B1 H16 N1500 d64 causal")
    xa = gen.fwd_inputs(2, 8, 8, 2000, 128, 1201, causal=True)
    xb = gen.fwd_inputs(1, 16, 16, 1500, 64, 1202, causal=True)
    ta = [gen.to_torch(t, "bf16", dev) for t in (xa.q, xa.k, xa.v)]
    tb = [gen.to_torch(t, "bf16", dev) for t in (xb.q, xb.k, xb.v)]
    want_a = fa.fa_fwd(*ta, scale=xa.scale, causal=True)
    want_b = fa.fa_fwd(*tb, scale=xb.scale, causal=True)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)
    oa, ob = torch.empty_like(ta[0]), torch.empty_like(tb[0])
    for _ in range(3):
        oa.fill_(float("nan"))
        ob.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(sa):
            for _ in range(4):
                fa.fa_fwd(*ta, scale=xa.scale, causal=True, out=oa)
        with torch.cuda.stream(sb):
            for _ in range(4):
                fa.fa_fwd(*tb, scale=xb.scale, causal=True, out=ob)
        torch.cuda.synchronize()
        assert torch.equal(oa, want_a), "stream a differs from the call alone"
        assert torch.equal(ob, want_b), "stream b differs from the call alone"


def test_decode_on_two_streams(dev):
    import torch

    log_case("fa_decode_splitk on two streams, a workspace each")
    xs = [gen.decode_inputs(3, 16, 4, 128, 16, seed=1301 + i, lens=[1000 + 700 * i, 4097, 33 + i],
                            max_pages_per_seq=300) for i in range(2)]
    ups = []
    for x in xs:
        ups.append((gen.to_torch(x.q, "bf16", dev), gen.to_torch(x.k_cache, "bf16", dev),
                    gen.to_torch(x.v_cache, "bf16", dev), torch.from_numpy(x.block_table).to(dev),
                    torch.from_numpy(x.lens.astype(np.int32)).to(dev)))
    splits = 3
    wants = [fa.fa_decode_splitk(*u, x.max_seq_len, scale=x.scale, num_splits=splits)
             for u, x in zip(ups, xs)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=dev) for _ in range(2)]
    outs = [torch.empty_like(u[0]) for u in ups]
    wss = [torch.empty(max(16, fa.fa_decode_workspace_bytes(3, 16, 128, 16, x.max_seq_len, splits)),
                       dtype=torch.uint8, device=dev) for x in xs]
    for _ in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                for _ in range(6):
                    fa.fa_decode_splitk(*ups[i], xs[i].max_seq_len, scale=xs[i].scale,
                                        num_splits=splits, out=outs[i], workspace=wss[i])
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i], wants[i]), f"stream {i} differs from the call alone"
