"""CPU oracle for the LatentMoE layer forward (MXFP4 weights, MXFP8 activations).

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, fp64 reference the
GPU library is checked against.  It shares no code with the GPU path and never
imports it.  Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import or run anything here; the product path must
never route through it.

Modules
-------
``mx``     MX element codecs (E2M1, E4M3, E8M0), the block quantiser, packing,
           and the fp64 / exact-integer MX matmul.
``moe``    the layer, step by step: quantise, latent down-projection, sigmoid
           router with top-k and normalised gates, stable expert dispatch,
           SwiGLU experts, gate-weighted combine, up-projection, shared experts;
           plus a brute-force "all experts, then mask" variant.
``weights``oracle-side quantisation of the seeded synthetic weights.
``balance``Quantile Balancing of the selection bias (a reading of the pages;
           its pins check the reading's consequences, not printed values).

Pins (what the oracle is checked against; see ``tests/test_oracle_*.py``)
-------------------------------------------------------------------------
* codec tables against the E2M1 magnitudes printed on "Kimi K3: 2.8 Trillion
  Parameters, Four Bits at a Time" (section "Four bits from the start") and
  against PyTorch's float8_e4m3fn / float4_e2m1fn_x2 / float8_e8m0fnu decoders;
* the MXFP4 rows of that page's quantisation experiment (seed 7);
* the tokens-per-expert list of that page's MoE data-path toy (seed 0);
* exact-integer MX matmul, brute-force dense-mask layer, single-expert
  reduction against an independent PyTorch fp64 MLP, and the invariants;
* the bfloat16 rounding against PyTorch's fp32 -> bfloat16 cast (ties of both
  parities, overflow, subnormals), and the higher-precision map's top-1 layer
  against a PyTorch pipeline with its own casts.

Layer outputs as a whole have no printed value on the pages: beyond the pins
above their parity is checked by construction (brute force, invariants), not
against a published number.
"""

from . import mx, moe, weights  # noqa: F401
