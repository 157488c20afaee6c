"""Pins for the oracle's pre-packed W4A8 weight layout (a nibble permutation plus the
bf16 -> fp32 widening of the group scales).

Checked by hand-derived contents (a lane holds its row and K slot; byte 4w+j holds
elements 8w+j and 8w+j+4), as a bijection on the nibbles, by the padding rule, and
by the exact value of every widened scale.
"""
import numpy as np

import datagen
import oracle


def test_lane_row_slot_and_nibble_order():
    N, K = 16, 256
    # Mark every nibble with the low 4 bits of its K index: element k holds k % 16.
    k = np.arange(K)
    codes = np.tile((k % 16).astype(np.uint8), (N, 1))
    B = datagen.pack_nibbles(codes)
    sB = np.zeros((N, K // 128), np.uint16)
    Bp, _ = oracle.w4a8_prepack(B, sB)
    Bp = Bp.reshape(1, 2, 64, 16)               # [g16][kg][lane][byte]
    for kg in range(2):
        for l in range(64):
            slot = l // 16
            for w in range(4):
                for j in range(4):
                    lo = (128 * kg + 32 * slot + 8 * w + j) % 16
                    hi = (128 * kg + 32 * slot + 8 * w + j + 4) % 16
                    assert Bp[0, kg, l, 4 * w + j] == lo | (hi << 4)
    # Mark nibbles with their row instead: lane l holds row l % 16.
    rows = np.repeat(np.arange(N, dtype=np.uint8)[:, None], K, axis=1)
    Bp, _ = oracle.w4a8_prepack(datagen.pack_nibbles(rows), sB)
    lanes = np.arange(64) % 16
    assert np.array_equal(Bp.reshape(2, 64, 16)[0], np.repeat((lanes | lanes << 4)[:, None], 16, axis=1))


def test_nibbles_are_a_permutation():
    N, K = 48, 512
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 16, (N, K), dtype=np.uint8)
    Bp, _ = oracle.w4a8_prepack(datagen.pack_nibbles(codes), np.zeros((N, K // 128), np.uint16))
    nibs = np.concatenate([Bp & 15, Bp >> 4])
    assert Bp.size == N * K // 2
    assert np.array_equal(np.bincount(nibs, minlength=16), np.bincount(codes.ravel(), minlength=16))
    # per row group and K group, the multiset of nibbles is preserved
    Bq = Bp.reshape(N // 16, K // 128, 1024)
    for g in range(N // 16):
        for kg in range(K // 128):
            got = np.sort(np.concatenate([Bq[g, kg] & 15, Bq[g, kg] >> 4]))
            want = np.sort(codes[16 * g:16 * g + 16, 128 * kg:128 * kg + 128].ravel())
            assert np.array_equal(got, want)


def test_scales_and_padding():
    N, K = 20, 384
    rng = np.random.default_rng(2)
    q = rng.integers(-8, 8, (N, K)).astype(np.int8)
    B = datagen.pack_nibbles(q.view(np.uint8) & np.uint8(15))
    sB = datagen.bf16_bits(rng.uniform(0.005, 0.05, (N, K // 128)).astype(np.float32))
    Bp, Sp = oracle.w4a8_prepack(B, sB)
    assert Bp.size == 2 * 3 * 1024 and Sp.size == 3 * 32
    Sp = Sp.reshape(3, 32)
    want = (sB.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(Sp[:, :N], want.T)
    assert np.all(Sp[:, N:] == 0)
    pad = Bp.reshape(2, 3, 64, 16)[1][:, np.arange(64) % 16 >= N - 16]
    assert not pad.any()
