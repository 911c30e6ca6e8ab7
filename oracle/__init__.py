"""CPU oracle for the Kimi-K3-style MXFP8 x MXFP4 MoE expert layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or run anything here.  The
product path (the HIP library and its Python binding) never imports this
package, and this package never imports the product path.

The oracle is plain NumPy in float64.  It follows the pages' method step by
step (routing, MXFP8 activation quantisation, permutation, FC1 grouped GEMM,
SiTU, requantisation, FC2 grouped GEMM, top-k combine) with no blocking,
fusion or reordering beyond what the definitions state.  Every function names
the passage it follows; the readings taken where the pages are silent are
listed in the function docstrings.

Pinning status (what each function is checked against, in
``tests/test_oracle_*.py``):

* codecs: OCP MX closed forms (E4M3 extremes, E2M1 magnitudes), torch's
  independent float8_e4m3fn / float8_e8m0fnu conversions, exhaustive
  brute-force nearest-value search over every bf16 pattern; the report-only
  bf16 rounding against torch's bfloat16 conversion and exact rationals;
* route: brute-force sort, the bias-free special case (top-k of the logits),
  constructed ties, weight invariants;
* permute: brute-force per-expert scan;
* FC1 / FC2 / layer: independent per-token brute force (``oracle.brute``),
  one-hot layout probes (nibble order, gate/up halves, scale indexing),
  integer special cases; the report-only accumulators and |product| sums
  against each other and the triangle inequality;
* SiTU: limits and identities of the closed form;
* combine / expert-parallel masking: linearity and the shard-sum invariant.

"Parity unpinned": beyond these definitions no page prints an input/output
value of the layer, so the absolute output numbers of a full-size case rest
on the pinned pieces above, not on a printed example.
"""
from .codecs import (  # noqa: F401
    E4M3_MAX,
    e2m1_decode,
    e4m3_decode,
    e4m3_encode,
    e8m0_decode,
    mx_exponent,
    mxfp8_quantize,
    mxfp8_dequantize,
    mxfp4_dequantize,
)
from .layer import (  # noqa: F401
    route,
    quant_x,
    permute,
    situ,
    fc1_situ_requant,
    fc2,
    combine,
    oracle_layer,
    oracle_tokens,
)
