"""CPU oracle for the block-scaled FP8 GEMM with a global-amax epilogue.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only the test suite, the smoke check and the benchmark's CPU-baseline leg may
call it.  It shares no code, table or constant generator with the HIP library.

What it computes ("GEMM + Amax (SM100)", section "Equations"):

    A_hat[m,k,l] = dec(A[m,k,l]) * 2^(SFA(m, k // sf, l) - 127)
    B_hat[n,k,l] = dec(B[n,k,l]) * 2^(SFB(n, k // sf, l) - 127)
    C[m,n,l]     = sum_k A_hat[m,k,l] * B_hat[n,k,l]
    Amax         = max_{m,n,l} |C[m,n,l]|

in float64, where every decoded product is exact.  Modules:

* ``codecs``    -- E4M3 / E5M2 / E8M0 decoders built from the bit definitions.
* ``sf_atom``   -- expansion of the scale-factor atom layout (page section
                   "Shapes" and the physical-shape paragraph of "Using JAX
                   arrays") into one scale per (row, K-block).
* ``gemm_amax`` -- dequantisation, the fp64 contraction, the |A|.|B| bound
                   used by the tolerance, and the amax.
* ``mx_quantize`` -- MX block quantisation of float32 data into codes and
                   E8M0 scales in the atom layout (the step that produces
                   the GEMM's inputs).
* ``proj_rope`` -- the projection page's per-head RoPE and dual-direction
                   MXFP8 quantisation of the GEMM output.

Every function has a pin in ``tests/test_oracle_*.py``; see each module's
header for which pin covers it.
"""

from .codecs import (decode, decode_e4m3, decode_e5m2, decode_e8m0, decode_e2m1, unpack_e2m1, element_codes,
                     bytes_per_row, FMT_E4M3, FMT_E5M2, FMT_E2M1)
from .sf_atom import sf_physical_shape, sf_logical_shape, sf_logical_view, expand_scales
from .gemm_amax import (dequantize, gemm_amax, gemm_amax_loops, gemm_rows, gemm_entries,
                        gemm_row_blocks, amax_of)
from .mx_quantize import mx_quantize, block_max, block_exponent, encode_rne, place_scales, pack_e2m1
from .proj_rope import rope, proj_rope_mxfp8

__all__ = [
    "decode", "decode_e4m3", "decode_e5m2", "decode_e8m0", "decode_e2m1", "unpack_e2m1", "element_codes",
    "bytes_per_row", "FMT_E4M3", "FMT_E5M2", "FMT_E2M1",
    "sf_physical_shape", "sf_logical_shape", "sf_logical_view", "expand_scales",
    "dequantize", "gemm_amax", "gemm_amax_loops", "gemm_rows", "gemm_entries", "gemm_row_blocks", "amax_of",
    "mx_quantize", "block_max", "block_exponent", "encode_rne", "place_scales", "pack_e2m1",
    "rope", "proj_rope_mxfp8",
]
