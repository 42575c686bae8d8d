"""CPU oracle for the hybrid linear temporal attention forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the test suite, the smoke check of the
entry module and the CPU-baseline leg of the benchmark use it.  It shares no
code with the HIP path; the only module both sides use is the seeded input
generator (``workloads``), which holds none of the method's arithmetic.

Everything here is plain, slow and written to be checked by eye against the
source paper, "Kairos: A Regret-Aware Native World-Action Model Stack for
Physical AI" (arXiv 2606.16533, HTML v3):

* ``gdn``    -- the gated delta rule of Sec. 2.2.1 (Eq. 1-6 and the read-out of
               step 4), token by token in fp64; plus the chunkwise (WY / UT)
               re-association of the same recurrence, used only as a second
               formulation that the tests compare against the first;
* ``window`` -- the sliding-window attention of Eq. 7 and the dilated variant
               of Eq. 8 as naive masked softmax in fp64, a literal
               rearrange-then-SWA form of Eq. 8, and a scalar brute force;
* ``fp8``    -- an OCP FP8 E4M3 quantiser with per-64-token-block absmax
               scales, written from the format definition;
* ``fp4``    -- the same for the 4-bit path (OCP FP4 E2M1 codes);
* ``hlta``   -- the gated combination of the three branches;
* ``rope``   -- rotary position embedding of the windowed branches' q and k
               at each branch's (group) positions;
* ``prologue`` -- the inputs of the gated delta rule from raw keys and gate
               logits (L2 normalisation, sigmoids of Eq. 1 and Eq. 4, and the
               rescaling that turns the printed Eq. 6 into the canonical form).

Readings of points the paper leaves open are listed in each function's
docstring.  Every function is pinned by tests against closed forms,
invariants, brute force or library routines (torch's scaled-dot-product
attention, torch's float8_e4m3fn cast).
"""
from .gdn import gdn_recurrent, gdn_literal_eq6, gdn_chunked
from .window import (windowed_attention, windowed_attention_rows, window_bruteforce,
                     dswa_reshape, frame_index_maps)
from .fp8 import e4m3_round, e4m3_encode, e4m3_decode, fp8_quantize_blocks, E4M3_MAX
from .fp4 import (e2m1_round, e2m1_encode, e2m1_decode, fp4_pack, fp4_unpack, fp4_quantize_blocks,
                  E2M1_MAX)
from .hlta import hlta, hlta_rows, sigmoid, quantize_frames
from .prologue import l2_normalize, gdn_prologue
from .rope import rope, rope_angles, branch_positions

__all__ = [
    "gdn_recurrent", "gdn_literal_eq6", "gdn_chunked",
    "windowed_attention", "windowed_attention_rows", "window_bruteforce", "dswa_reshape",
    "frame_index_maps",
    "e4m3_round", "e4m3_encode", "e4m3_decode", "fp8_quantize_blocks", "E4M3_MAX",
    "e2m1_round", "e2m1_encode", "e2m1_decode", "fp4_pack", "fp4_unpack", "fp4_quantize_blocks",
    "E2M1_MAX",
    "hlta", "hlta_rows", "sigmoid", "quantize_frames", "l2_normalize", "gdn_prologue",
    "rope", "rope_angles", "branch_positions",
]
