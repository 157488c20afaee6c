"""Pins for the oracle's pre-packed decode-weight layout (a byte permutation).

Checked against element-by-element loops over the layout's defining formula, against
its inverse (every byte of B and sfB appears exactly once, in the place the formula
names), and against the padding rule for ragged N and K.
"""
import numpy as np
import pytest

import oracle


def loops(B, sfB):
    """The layout by explicit loops over (g, s, lane, byte) and (g, c, lane, i)."""
    N, half = B.shape
    K = 2 * half
    G, KT = -(-N // 16), K // 128
    KC = -(-KT // 4)
    Bp = np.zeros(G * KT * 1024, np.uint8)
    Sp = np.zeros(G * KC * 256, np.uint8)
    for g in range(G):
        for s in range(KT):
            for l in range(64):
                r, slot = l % 16, l // 16
                for b in range(16):
                    row = 16 * g + r
                    Bp[((g * KT + s) * 64 + l) * 16 + b] = B[row, 64 * s + 16 * slot + b] if row < N else 0
        for c in range(KC):
            for l in range(64):
                r, slot = l % 16, l // 16
                for i in range(4):
                    row, step = 16 * g + r, 4 * c + i
                    Sp[((g * KC + c) * 64 + l) * 4 + i] = sfB[row, 4 * step + slot] if (row < N and step < KT) else 127
    return Bp, Sp


@pytest.mark.parametrize("shape", [(16, 512), (37, 384), (5, 128), (48, 1280)])
def test_matches_loops(shape):
    N, K = shape
    rng = np.random.default_rng(N + K)
    B = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    sfB = rng.integers(0, 256, (N, K // 32), dtype=np.uint8)
    Bp, Sp = oracle.gemv_prepack(B, sfB)
    Bl, Sl = loops(B, sfB)
    assert np.array_equal(Bp, Bl)
    assert np.array_equal(Sp, Sl)


def test_every_byte_once():
    # Distinct values mark every source byte; the packed arrays hold each exactly once
    # (plus padding), so no byte is dropped or duplicated.
    N, K = 32, 1024
    B = np.arange(N * K // 2, dtype=np.int64).reshape(N, K // 2)
    Bp, _ = oracle.gemv_prepack((B % 251).astype(np.uint8), np.zeros((N, K // 32), np.uint8))
    assert Bp.size == N * K // 2
    # reconstruct through the inverse index map and compare
    G, KT = N // 16, K // 128
    idx = np.arange(Bp.size)
    b, l, s, g = idx % 16, (idx // 16) % 64, (idx // 1024) % KT, idx // (1024 * KT)
    rows, cols = 16 * g + l % 16, 64 * s + 16 * (l // 16) + b
    assert np.array_equal(np.sort(rows * (K // 2) + cols), np.arange(N * K // 2))
    assert np.array_equal(Bp, (B[rows, cols] % 251).astype(np.uint8))


def test_padding():
    N, K = 3, 640            # one partial row group, KT = 5 (one partial scale chunk)
    B = np.full((N, K // 2), 0xAB, np.uint8)
    sfB = np.full((N, K // 32), 200, np.uint8)
    Bp, Sp = oracle.gemv_prepack(B, sfB)
    Bp = Bp.reshape(1, 5, 64, 16)
    Sp = Sp.reshape(1, 2, 64, 4)
    lanes = np.arange(64)
    real = lanes % 16 < N
    assert np.all(Bp[0][:, real] == 0xAB) and np.all(Bp[0][:, ~real] == 0)
    assert np.all(Sp[0, 0][real] == 200) and np.all(Sp[0, 0][~real] == 127)
    assert np.all(Sp[0, 1][real, 0] == 200)            # step 4 exists
    assert np.all(Sp[0, 1][:, 1:] == 127)              # steps 5..7 do not


def test_lane_holds_its_row_and_k_slot():
    """By hand: in the 16x16x128 instruction's operand a lane l holds weight row l % 16
    and K slot l // 16 (elements 32*slot .. 32*slot + 31 of the step).  Mark B's bytes
    with their row, then with their 16-byte chunk within the step, then with the step."""
    N, K = 16, 256
    rows = np.repeat(np.arange(N, dtype=np.uint8)[:, None], K // 2, axis=1)
    chunk = np.tile((np.arange(K // 2) // 16 % 4).astype(np.uint8), (N, 1))
    step = np.tile((np.arange(K // 2) // 64).astype(np.uint8), (N, 1))
    sf = np.zeros((N, K // 32), np.uint8)
    lane = np.repeat(np.arange(64), 16)
    for s in range(2):
        bp_r = oracle.gemv_prepack(rows, sf)[0].reshape(2, 1024)[s]
        bp_c = oracle.gemv_prepack(chunk, sf)[0].reshape(2, 1024)[s]
        bp_s = oracle.gemv_prepack(step, sf)[0].reshape(2, 1024)[s]
        assert np.array_equal(bp_r, lane % 16)
        assert np.array_equal(bp_c, lane // 16)
        assert np.all(bp_s == s)
    # scales: sfB[r][4*step + slot] = 16*step + 4*slot + (r % 4) marks (step, slot, row)
    sf = np.array([[(16 * (j // 4) + 4 * (j % 4) + r % 4) for j in range(K // 32)] for r in range(N)], np.uint8)
    Sp = oracle.gemv_prepack(rows, sf)[1].reshape(1, 64, 4)    # one chunk of 4 steps (2 real)
    for l in range(64):
        for i in range(4):
            want = 16 * i + 4 * (l // 16) + (l % 16) % 4 if i < 2 else 127
            assert Sp[0, l, i] == want
