"""Pins of the oracle's packed byte layout against hand-built bytes.

The layout is the library's interface (each section of a tensor's packed block
starts at a multiple of 256 bytes): 1-bit sign bits then scales; 2-bit codes,
then the group minima, then the group steps; 2:16 value pairs then index bytes;
low rank INT4 factors U then V as two's-complement nibbles (element t of the
row-major matrix in nibble t, even t low), then the column scales of U and of
V. INT4 factors: "Accelerating Parallel Diffusion Model Serving with Residual
Compression", Key designs / Low-rank strategy for extreme compression; the
quantisers: Main experiment table. Every expected byte below is written out by
hand, not produced by the oracle.
"""
import numpy as np

import oracle


def test_int4_nibbles_by_hand():
    # rank 8: one row 0..7 and one row of negatives
    q = np.array([[0, 1, 2, 3, 4, 5, 6, 7],
                  [-1, -2, -3, -4, -5, -6, -7, 0]], np.int8)
    want = [0x10, 0x32, 0x54, 0x76,      # 1 in the high nibble of byte 0, 0 low
            0xEF, 0xCD, 0xAB, 0x09]      # -1 = 0xF low, -2 = 0xE high, ..., -7 = 0x9 low, 0 high
    assert oracle._pack_int4(q).tolist() == want
    assert np.array_equal(oracle._unpack_int4(np.array(want, np.uint8), 16).reshape(2, 8), q)
    # the extremes -7 and 7 in both halves of a byte
    assert oracle._pack_int4(np.array([-7, 7, 7, -7], np.int8)).tolist() == [0x79, 0x97]


def test_int4_rank48_rows_are_contiguous_nibble_runs():
    # rank 48: row i holds elements 48 i .. 48 i + 47, i.e. bytes 24 i .. 24 i + 23
    q = np.zeros((3, 48), np.int8)
    q[1, 0] = -1          # element 48 -> byte 24, low nibble
    q[1, 47] = 3          # element 95 -> byte 47, high nibble
    q[2, 1] = 7           # element 97 -> byte 48, high nibble
    b = oracle._pack_int4(q)
    assert b.size == 72
    nz = {i: int(v) for i, v in enumerate(b) if v}
    assert nz == {24: 0x0F, 47: 0x30, 48: 0x70}


def test_q2_sections_by_hand():
    # one 128-element group: codes, then mn at byte 256, then d at byte 512
    r = np.zeros(128, np.float32)
    r[0], r[1], r[5], r[127] = -1.0, 2.0, 1.0, 0.0    # mn -1, mx 2, d 1
    o = oracle.compress_tensor("q2", r.reshape(1, 128), np.zeros((1, 128), np.float32), group=128)
    pk = o["packed"]
    assert pk.size == 768
    # codes: q = round(r - mn): r=-1 -> 0, 2 -> 3, 0 -> 1, 1 -> 2
    #   byte 0: elements 0..3 = 0, 3, 1, 1 -> 0b01_01_11_00
    #   byte 1: elements 4..7 = 1, 2, 1, 1 -> 0b01_01_10_01
    assert pk[0] == 0b01011100 and pk[1] == 0b01011001
    assert np.all(pk[2:31] == 0b01010101) and pk[31] == 0b01010101
    assert not pk[32:256].any()
    assert pk[256:260].view(np.float32)[0] == -1.0 and not pk[260:512].any()
    assert pk[512:516].view(np.float32)[0] == 1.0 and not pk[516:].any()


def test_q1_sections_by_hand():
    r = np.full(64, -0.5, np.float32)
    r[[0, 8, 63]] = 0.5
    o = oracle.compress_tensor("q1", r.reshape(1, 64), np.zeros((1, 64), np.float32), group=64)
    pk = o["packed"]
    assert pk.size == 512
    assert pk[:8].tolist() == [0x01, 0x01, 0, 0, 0, 0, 0, 0x80]
    assert not pk[8:256].any()
    assert pk[256:260].view(np.float32)[0] == 0.5 and not pk[260:].any()


def test_nm_sections_by_hand():
    r = np.zeros(16, np.float32)
    r[3], r[9] = -2.0, 1.5
    o = oracle.compress_tensor("nm", r.reshape(1, 16), np.zeros((1, 16), np.float32))
    pk = o["packed"]
    assert pk.size == 512
    # bf16 of -2.0 = 0xC000, of 1.5 = 0x3FC0, little-endian, ascending index order
    assert pk[:4].tolist() == [0x00, 0xC0, 0xC0, 0x3F]
    assert pk[256] == (3 | (9 << 4)) and not pk[257:].any()


def test_lowrank_sections_by_hand():
    # n = 2 rows, m = 2 cols, rank 8: U nibbles (8 B) | V nibbles (8 B) | sU | sV
    U = [0x21, 0, 0, 0, 0x0F, 0, 0, 0]       # U[0][:2] = 1, 2 ; U[1][0] = -1
    V = [0x03, 0, 0, 0, 0x90, 0, 0, 0]       # V[0][0] = 3 ; V[1][1] = -7
    su = np.array([0.5, 0.25] + [0] * 6, np.float32)
    sv = np.array([2.0, 1.0] + [0] * 6, np.float32)
    pk = np.zeros(4 * 256, np.uint8)
    pk[0:8] = U
    pk[256:264] = V
    pk[512:544] = su.view(np.uint8)
    pk[768:800] = sv.view(np.uint8)
    assert oracle.tensor_bytes("lr", 2, 2, rank=8) == pk.size
    c = oracle.decode_tensor("lr", pk, 2, 2, rank=8)
    # Uq = [[0.5, 0.5], [-0.5, 0]] (first two columns), Vq = [[6, 0], [0, -7]]
    want = np.array([[0.5 * 6, 0.5 * -7], [-0.5 * 6, 0.0]])
    assert np.array_equal(c, want)
