"""Every planted oracle mistake must be caught by at least one pin.

The mistakes are compiled into separate oracle builds (ORACLE_MUTANT=n in
qmv_oracle.c), on the CPU only:
  1 e2m1 sign dropped          2 nibbles swapped          3 3-bit scale of the
  wrong half-block             4 2-bit codebook shifted   5 3-bit codes read
  MSB-first                    6 E8M0 bias 128            7 fp16 bias off by one
  8 out-of-range ids wrap instead of giving zero rows   9 gate and up
  swapped in SwiGLU            10 sigmoid(g) * u in place of silu(g) * u
  11 combine weights shifted by one slot   12 combine drops the last slot
  13 q8 quantizer rounds ties away from zero   14 q8 quantizer uses the
  unrounded scale   15 combine drops the router weights' signs.
The idea of requiring a sign-dropped decode to fail comes from mlxcel issue
#2178, Acceptance Criteria.
"""
import pytest

import oracle
import oracle_pins as pins

# the cheap pins first; the exhaustive ones only run if those all passed
ORDER = [pins.check_hand_worked, pins.check_codebooks_match_pages, pins.check_e2m1_table,
         pins.check_e8m0_library, pins.check_unpackers_agree, pins.check_gather_semantics,
         pins.check_unit_scale_exact, pins.check_block_factored, pins.check_fp16_exhaustive,
         pins.check_bf16_exhaustive, pins.check_random_blocks_exact, pins.check_mxfp4_one_hot, pins.check_swiglu, pins.check_combine, pins.check_combine_signed, pins.check_q8_hand_worked, pins.check_f2h_library, pins.check_q8_invariants]


@pytest.mark.parametrize("mutant", range(1, 16))
def test_mutant_is_caught(mutant):
    o = oracle.load(mutant)
    caught = []
    for check in ORDER:
        try:
            check(o)
        except AssertionError:
            caught.append(check.__name__)
            break
    assert caught, f"mutant {mutant} passed every pin"
