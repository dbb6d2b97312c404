"""CPU oracle for the grouped 4:8 / E2M1 / E4M3 expert GEMM path.

TEST INFRASTRUCTURE ONLY.  Plain, slow, float64 numpy code that states what
the hot path computes, so that the HIP library can be checked against it.
Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import it; the library itself never does, and this package
imports nothing from the library.

Source: Hardware-Native Joint Sparse-Quantization for Trillion-Scale
Mixture-of-Experts (paper summary page, paperlayer.ai):
  * "3.4 Implementation details" -- E2M1 values, sparse metadata and one
    (U)E4M3 scale per 32 logical weights are packed; the grouped GEMM runs
    every routing-dependent expert problem in one launch.
  * "A Sparse-quantized representation" (Feasible set, Blackwell paired 4:8
    NVFP4, Storage layout) -- groups of eight keep four values, 16 kept
    values share a scale block, zero is on the value grid.
  * "D.1 Implementation details" / "D.3 End-to-end serving benchmark" --
    dispatch before the first expert GEMM, SwiGLU between gate/up and down,
    token combination weighted by the router.

Every function's docstring names the passage it follows.  Readings taken
where the pages are silent are listed in `READINGS` below.

Pins: every function here is pinned by the `-m "not gpu"` tests in
tests/test_oracle_*.py against closed forms, a library cast, brute force on
tiny inputs, invariances and hand-derived fixtures in tests/golden/.
"""
from .formats import (E2M1_VALUES, E4M3_VALUES, bf16_round, e2m1_decode,
                      e2m1_encode, e4m3_decode, e4m3_encode)
from .pack import PackedExpert, decode, quantize, support
from .paired import (PAIRS, PackedPairedExpert, decode_paired, paired_pattern,
                     paired_support, pattern_mask, quantize_paired)
from .route import route
from .moe import (grouped_gemm, moe_chain, permute, silu, swiglu, unpermute,
                  expert_gemm)
from .w4a4 import (PackedActivations, decode_activations, quantize_activations,
                   w4a4_expert_gemm)

READINGS = {
    "format": "unconstrained 4:8: any 4 of 8 kept, 8-bit mask per group "
              "(bit i <-> position 8g+i), 4 E2M1 nibbles per group in "
              "ascending position, lower position in the low nibble",
    "support": "keep the 4 largest |w| of each group; equal |w| -> lower "
               "position wins; a kept value that rounds to 0 stays kept",
    "global_scale": "one fp32 scale per expert matrix, g = amax/(6*448) "
                    "(g = 1 when amax = 0)",
    "block_scale": "s = E4M3_RNE_satfinite(amax_32 / (6*g)) in fp32, one per "
                   "32 logical = 16 kept weights",
    "values": "q = E2M1_RNE_sat(w / (s*g)) in fp32; zero is +0; s*g == 0 -> 0",
    "swiglu": "gate = first N/2 output columns, up = second N/2; "
              "h = silu(gate) * up, stored as bf16",
    "combine": "out[t] = sum_j w[t,j] * Y[row of (t,j)], j ascending",
    "paired_index": "paired 4:8 pattern index p in [0,6) numbers the kept pair "
                    "couples (0,1) (0,2) (0,3) (1,2) (1,3) (2,3); two per byte, "
                    "even group in the low nibble",
    "paired_support": "keep the two pairs with the largest fp32 |w_2i|+|w_2i+1|; "
                      "equal sums -> lower pair index",
    "paired_values": "kept values quantised exactly as the 4:8 format",
    "act_blocks": "W4A4: activations quantized to E2M1 with one E4M3 scale per 32 "
                  "consecutive K positions (the weights' scale blocks)",
    "act_row_scale": "W4A4: one fp32 scale per activation row, g_t = amax_t/(6*448) "
                     "(g_t = 1 when amax_t = 0); s = E4M3(amax_32/(6 g_t)), "
                     "q = E2M1(x/(s g_t)), all in fp32 with ties to even",
    "act_codes": "W4A4: two codes per byte, position 2i in the low nibble",
}
