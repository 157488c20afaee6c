"""The accuracy margin of the W4A8 decode kernel's operand form, on the CPU.

The decode kernel feeds each INT4 weight q = v - 8s to the FP8 matrix instruction as two
exact parts, v as the E4M3 subnormal code v * 2^-9 and the sign part, both scaled by 2^9
(oracle.fp8_truncation_bound with split=2).  On the W4A8 workload's activation
distribution (N(0,1) rows quantized to E4M3) the instruction's truncation bound H for
that form stays far below 1e-5 * S, so the plain parity bar holds with margin whatever
the signs of the individual losses.
"""
import numpy as np

import datagen
import oracle


def test_decode_workload_meets_the_plain_bar_by_the_bound():
    d = datagen.make_shape("w4a8", 16, 256, 8192, seed=5)
    ref, S = oracle.run("w4a8", d)
    H = oracle.fp8_truncation_bound("w4a8", d, split=2)
    assert (H <= 0.3 * 1e-5 * S).all(), float((H / (1e-5 * S)).max())
    # the E4M3 form of v charges less on the same inputs
    assert (oracle.fp8_truncation_bound("w4a8", d, split=True) <= H).all()
