"""The library's quantisers (host code, no GPU) against the oracle's.

3 bits: the levels the specification of this path fixes and the fp32
midpoints the oracle decides
with.  4 bits: the library runs its own Lloyd iteration (positive half, by
symmetry, from another start); it must land on the oracle's pinned codebook,
with identical fp32 thresholds (the decisions are taken in fp32 on both
sides), and its f16 level operands must sit within the stated relative error.
"""

import numpy as np
import pytest

from oracle import isoquant4_oracle as O4
from oracle import isoquant_oracle as O

iq = pytest.importorskip("compressed_space_attention_amd.isoquant",
                         reason="libisoquant.so not built")


def test_three_bit_codebook_is_the_specified_one():
    levels, thr, alpha = iq.codebook(3)
    assert np.array_equal(levels, O.CENTROIDS)
    assert np.array_equal(thr, O.THRESHOLDS_F32)
    assert alpha == pytest.approx(1.7670845, abs=1e-7)


def test_four_bit_levels_match_the_oracle_iteration():
    levels, thr, _ = iq.codebook(4)
    want = O4.centroids4()
    assert np.max(np.abs(levels - want)) < 1e-12
    assert np.array_equal(levels, -levels[::-1])             # exactly symmetric
    assert np.array_equal(thr, O4.thresholds4_f32())          # the same fp32 decisions
    assert thr[7] == 0.0


def test_four_bit_f16_level_operands():
    """alpha * level rounded to f16 stays within 1e-4 (relative) of the exact
    product for every magnitude (plain f16 rounding of the levels: up to
    2^-11 = 4.9e-4)."""
    levels, _, alpha = iq.codebook(4)
    assert 1.0 <= alpha < 2.0
    mags = alpha * levels[8:]
    err = np.abs(mags.astype(np.float16).astype(np.float64) - mags) / mags
    assert np.max(err) < 1e-4
