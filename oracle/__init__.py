"""Plain float64 CPU oracle for exact attention, paged prefill and decode, and partial merge.

This package is TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it. The product (the HIP library in
``exact_tiled_attention_24_amd`` and its Python binding) never imports, links or calls it,
and it imports nothing from the product.

Every function is written from the definitions on the pages, in float64 numpy, with no
blocking over keys, fusion or reordering beyond what the definition states. Each function
is pinned by the CPU tests in ``tests/test_oracle.py`` against values the pages print,
closed forms, invariants and a brute-force route that shares no code with it. All functions
here are pinned; none is "parity unpinned".
"""

from .attention import (  # noqa: F401
    attention,
    attention_backward,
    attention_block_sparse,
    attention_head,
    attention_probs,
    decode,
    merge,
    online_softmax,
    prefill_paged,
)
