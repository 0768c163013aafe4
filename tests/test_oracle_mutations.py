"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in the oracle (on the CPU, by monkeypatching a
single function) and checks that at least one pin of test_oracle_pins fails.
"""

import math

import numpy as np
import pytest

from oracle import isoquant_oracle as O
from tests import test_oracle_pins as P


def _fails(*checks):
    for fn, args in checks:
        try:
            fn(*args)
        except AssertionError:
            return True
    return False


def _quat_mul_sign_flip(a, b):
    aw, ax, ay, az = (float(t) for t in a)
    bw, bx, by, bz = (float(t) for t in b)
    return np.array([aw * bw - ax * bx - ay * by - az * bz,
                     aw * bx + ax * bw - ay * bz - az * by,      # planted: + ay*bz -> -
                     aw * by - ax * bz + ay * bw + az * bx,
                     aw * bz + ax * by - ay * bx + az * bw])


def _so4_no_conjugate(q_left, q_right):
    a = O.quat_normalize(q_left)
    p = O.quat_normalize(q_right)                                  # planted: no conj
    m = np.empty((4, 4))
    for j in range(4):
        e = np.zeros(4)
        e[j] = 1.0
        m[:, j] = O.quat_mul(O.quat_mul(a, e), p)
    return m


def _forward_transposed_blocks(x, blocks):
    return _orig["forward_rotate"](x, np.swapaxes(blocks, -1, -2))


def _inverse_transposed_blocks(z, blocks):
    return _orig["inverse_rotate"](z, np.swapaxes(blocks, -1, -2))


def _forward_unnormalised(x, blocks):
    return _orig["forward_rotate"](x, blocks) * math.sqrt(O.HEAD_DIM)


def _dequant_no_norm(codes, norm16):
    return O.CENTROIDS[np.asarray(codes)] / math.sqrt(O.HEAD_DIM) * np.ones_like(
        O.fp16_bits_to_float(norm16))[..., None]


def _position_wrong_lane(coord):
    g, r = divmod(coord, 32)
    b, s = divmod(r, 8)                                            # planted: lanes swapped
    return g, b, 3 * s


_orig = {"forward_rotate": O.forward_rotate, "inverse_rotate": O.inverse_rotate}

MUTATIONS = {
    "hamilton_sign": [("quat_mul", _quat_mul_sign_flip)],
    "missing_conjugate": [("so4_block", _so4_no_conjugate)],
    "blocks_transposed": [("forward_rotate", _forward_transposed_blocks),
                          ("inverse_rotate", _inverse_transposed_blocks)],
    "wht_unnormalised": [("forward_rotate", _forward_unnormalised)],
    "norm_dropped": [("dequantize_rotated", _dequant_no_norm)],
    "pack_lane_swap": [("_bit_position", _position_wrong_lane)],
}

PINS = [
    (P.test_block_equals_left_times_right_isoclinic_closed_form, ()),
    (P.test_conjugation_matches_scipy_3d_rotation, ()),
    (P.test_round_trip_dot_products_and_dense_equivalence, ()),
    (P.test_quantiser_closed_form_orientation, ("left",)),
    (P.test_quantiser_closed_form_orientation, ("right",)),
    (P.test_distortion_sanity_on_gaussian_vectors, ()),
    (P.test_decode_equals_plain_attention_on_materialised_kv, ()),
]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    for attr, fn in MUTATIONS[name]:
        monkeypatch.setattr(O, attr, fn)
    pins = list(PINS)
    if name == "pack_lane_swap":
        pins = [(P.test_pack_worked_examples, c) for c in P._golden_pack_cases()]
    assert _fails(*pins), f"no pin caught the planted mistake {name!r}"
