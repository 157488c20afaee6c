"""Pins for the oracle's FP6 (E3M2) re-encoded W4A8 weight layout.

Checked against the E3M2 format (each code decoded here from its bit fields), against
the instruction's K pairing measured on gfx950 with one set bit per operand position
(lane 0: K 0..15 and 32..47; lane 17: 64..79 and 96..111; lane 33: 16..31 and 48..63;
lane 63: 80..95 and 112..127), as a bijection on the weights, and by the padding rule
and the scales shared with w4a8_prepack.
"""
import numpy as np
import pytest

import datagen
import oracle


def decode_e3m2(c):
    """Value of a 6-bit E3M2 code: sign bit 5, exponent field bits 4..2 (bias 3),
    mantissa bits 1..0; field 0 is subnormal (m/4 * 2^-2)."""
    s, E, m = (c >> 5) & 1, (c >> 2) & 7, c & 3
    v = 2.0 ** (E - 3) * (1 + m / 4) if E else 2.0 ** -2 * (m / 4)
    return -v if s else v


def lane_codes(Bp6, G32, KG, g32, kg, h, lane):
    """The 32 codes of lane `lane`, half h, in block (g32, kg)."""
    blk = Bp6.reshape(G32, KG, 3072)[g32, kg]
    lo = blk[1024 * h + 16 * lane:1024 * h + 16 * lane + 16]
    hi = blk[2048 + 16 * lane + 8 * h:2048 + 16 * lane + 8 * h + 8]
    word = int.from_bytes(bytes(lo) + bytes(hi), "little")
    return [(word >> (6 * e)) & 63 for e in range(32)]


def test_e3m2_codes_from_the_format():
    for q in range(-8, 8):
        assert decode_e3m2(oracle.e3m2_code(q)) == q
    for q in (9, 11, 13, 15, 17, 29, 32):
        with pytest.raises(ValueError):
            oracle.e3m2_code(q)
    # exact integers up to the largest finite value 28 = 2^4 * 1.75
    for q in (10, 12, 14, 16, 20, 24, 28):
        assert decode_e3m2(oracle.e3m2_code(q)) == q
    assert oracle.e3m2_code(1) == 0b001100 and oracle.e3m2_code(-8) == 0b111000
    assert oracle.e3m2_code(7) == 0b010111 and oracle.e3m2_code(28) == 0b011111
    # every positive code decodes to a distinct, increasing value
    vals = [decode_e3m2(c) for c in range(32)]
    assert all(a < b for a, b in zip(vals, vals[1:]))


MEASURED_K = {0: list(range(0, 16)) + list(range(32, 48)), 17: list(range(64, 80)) + list(range(96, 112)),
              33: list(range(16, 32)) + list(range(48, 64)), 63: list(range(80, 96)) + list(range(112, 128))}


def test_lane_k_order_matches_the_measured_pairing():
    N, K = 32, 256
    k = np.arange(K)
    q = np.tile(((k % 16) - 8).astype(np.int8), (N, 1))          # element k holds (k % 16) - 8
    B = datagen.pack_nibbles(q.view(np.uint8) & np.uint8(15))
    Bp6, _ = oracle.w4a8_prepack_fp6(B, np.zeros((N, K // 128), np.uint16))
    assert Bp6.size == 1 * 2 * 3072
    for kg in range(2):
        for h in range(2):
            for lane, ks in MEASURED_K.items():
                got = [decode_e3m2(c) for c in lane_codes(Bp6, 1, 2, 0, kg, h, lane)]
                assert got == [((128 * kg + kk) % 16) - 8 for kk in ks]


def test_lane_row_and_half():
    N, K = 64, 128
    rows = np.arange(N)
    q = np.repeat(((rows % 16) - 8).astype(np.int8)[:, None], K, axis=1)   # row n holds (n % 16) - 8
    q[rows // 16 % 2 == 1] = np.repeat((7 - rows[rows // 16 % 2 == 1] % 8).astype(np.int8)[:, None], K, axis=1)
    B = datagen.pack_nibbles(q.view(np.uint8) & np.uint8(15))
    Bp6, _ = oracle.w4a8_prepack_fp6(B, np.zeros((N, 1), np.uint16))
    for g32 in range(2):
        for h in range(2):
            for lane in range(64):
                row = 32 * g32 + 16 * h + lane % 16
                assert {decode_e3m2(c) for c in lane_codes(Bp6, 2, 1, g32, 0, h, lane)} == {q[row, 0]}


def test_every_weight_once_and_padding():
    N, K = 40, 384
    rng = np.random.default_rng(5)
    q = rng.integers(-8, 8, (N, K)).astype(np.int8)
    B = datagen.pack_nibbles(q.view(np.uint8) & np.uint8(15))
    sB = datagen.bf16_bits(rng.uniform(0.005, 0.05, (N, K // 128)).astype(np.float32))
    Bp6, Sp = oracle.w4a8_prepack_fp6(B, sB)
    G32, KG = 2, 3
    assert Bp6.size == G32 * KG * 3072
    seen = np.full((32 * G32, K), 99, np.int16)
    slot_base = {s: 64 * (s & 1) + 16 * (s >> 1) for s in range(4)}
    for g32 in range(G32):
        for kg in range(KG):
            for h in range(2):
                for lane in range(64):
                    row, s = 32 * g32 + 16 * h + lane % 16, lane // 16
                    for e, c in enumerate(lane_codes(Bp6, G32, KG, g32, kg, h, lane)):
                        kk = 128 * kg + slot_base[s] + e + (0 if e < 16 else 16)
                        assert seen[row, kk] == 99
                        seen[row, kk] = decode_e3m2(c)
    assert np.array_equal(seen[:N], q)
    assert not seen[N:].any()
    _, Sp4 = oracle.w4a8_prepack(B, sB)
    assert np.array_equal(Sp.view(np.uint32), Sp4.view(np.uint32))
