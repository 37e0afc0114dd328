"""Exact tiled attention for MI355X (gfx950): FlashAttention forward, paged split-K decode
and (m, l, O) partial merge as hand-written HIP kernels behind a C ABI (libfa.so)."""
