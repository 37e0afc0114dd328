"""fa_decode_splitk_noalloc against fa_decode_splitk on the GPU (through the C ABI).

The allocation-free entry point runs the same kernel with its completion words and partials
in the library's static per-device scratch. Two calls in a row, the second smaller than the
first: each must equal the workspace entry point's output bit for bit and match the oracle.
"""

import numpy as np
import pytest

import oracle
import exact_tiled_attention_24_amd as fa
from exact_tiled_attention_24_amd import inputs as gen
from helpers import assert_close, cuda_device, log_case, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return cuda_device()


def upload(x, dev):
    import torch

    return (gen.to_torch(x.q, "bf16", dev), gen.to_torch(x.k_cache, "bf16", dev),
            gen.to_torch(x.v_cache, "bf16", dev), torch.from_numpy(x.block_table).to(dev),
            torch.from_numpy(x.lens.astype(np.int32)).to(dev))


@pytest.mark.parametrize("splits", [0, 3])
def test_noalloc_matches_workspace_entry_point(splits, dev):
    import torch

    big = gen.config_decode_inputs(gen.CONFIGS[5])
    small = gen.decode_inputs(3, 16, 4, 128, 16, seed=606, lens=[1000, 4097, 33],
                              max_pages_per_seq=260)
    for name, x in (("workload 5", big), ("small", small)):
        log_case(f"fa_decode_splitk_noalloc {name} splits={splits}")
        q, kc, vc, table, lens = upload(x, dev)
        want = fa.fa_decode_splitk(q, kc, vc, table, lens, x.max_seq_len, scale=x.scale,
                                   num_splits=splits)
        out = torch.full_like(q, float("nan"))
        got = fa.fa_decode_splitk_noalloc(q, kc, vc, table, lens, x.max_seq_len, out,
                                          scale=x.scale, num_splits=splits)
        torch.cuda.synchronize()
        assert got is out
        assert torch.equal(out, want), f"{name}: differs from fa_decode_splitk"
        ref, _, _ = oracle.decode(x.q, x.k_seqs, x.v_seqs, x.scale)
        assert_close(to_np(out), ref, "bf16", f"{name} O")
        del q, kc, vc, table, lens, want, out
        torch.cuda.empty_cache()
