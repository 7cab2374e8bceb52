"""CPU oracle for the sparsely-gated MoE layer forward pass.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import anything from this package. The product path (the
HIP library and its Python binding) never calls it and never falls back to it.

The oracle is plain numpy in fp64, written from the pages, sharing no code,
tables or constants with the HIP path:

  philox.py  counter-based Gaussian noise: Philox4x64-10 (Salmon et al., SC'11)
             and the Box-Muller transform, from their published definitions.
  moe.py     the layer: router (noisy top-k or Switch top-1), capacity,
             stable slots, per-token expert FFN loop, combine plus residual,
             importance / load / Switch auxiliary terms.

Every function is pinned by a CPU test against something other than itself
(values the pages print, closed forms, brute force, library routines it does
not use). See the module docstrings for the passages each step follows.
"""
