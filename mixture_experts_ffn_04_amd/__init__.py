"""MI355X-native MoE FFN layer forward (router, expert permutation, grouped
SwiGLU expert GEMMs, weighted combine, shared expert) behind a C ABI.

The compute runs in hand-written HIP kernels for gfx950 in libmoe_ffn.so;
`api` marshals torch tensors to that library and `workloads` draws seeded
synthetic inputs.  The library is loaded on first use and a missing or
unloadable library raises at that point.
"""
