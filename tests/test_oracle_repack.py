"""Pins of the oracle's interleaved pre-tiled layout (repack / unrepack)."""

import numpy as np
import pytest

import oracle
import synth
from conftest import read_golden


def _single_entry_case(bits, K, N, G, kind, row, col):
    codes = np.zeros((K, N), np.uint8)
    zeros = np.zeros((K // G, N), np.uint8)
    scales = np.zeros((K // G, N), np.uint16)
    if kind == "code":
        codes[row, col] = 0xA if bits == 4 else 0xA5
    elif kind == "zero":
        zeros[row, col] = 0xB if bits == 4 else 0xB7
    else:
        scales[row, col] = 0x1234
    x = np.zeros((1, K), np.uint16)
    return synth.gen.pack_case(bits, codes, zeros, scales, x, G)


@pytest.mark.parametrize("entry", read_golden("packed_layout_positions.txt"))
def test_layout_positions_hand_worked(entry):
    kind, bits, K, N, G, row, col, byte, shift = entry[0], *map(int, entry[1:])
    c = _single_entry_case(bits, K, N, G, kind, row, col)
    buf = oracle.repack(bits, c.qweight, c.qzeros, c.scales, K, N, G)
    nz = np.flatnonzero(buf)
    if kind == "scale":
        assert list(nz) == [byte, byte + 1]
        assert buf[byte] == 0x34 and buf[byte + 1] == 0x12
    else:
        val = {("code", 4): 0xA, ("code", 8): 0xA5, ("zero", 4): 0xB, ("zero", 8): 0xB7}[(kind, bits)]
        assert list(nz) == [byte]
        assert buf[byte] == (val << shift) & 0xFF


@pytest.mark.parametrize("bits,K,N,G", [
    (4, 64, 128, 32), (4, 256, 200, 128), (4, 384, 64, 384), (4, 192, 8, 64), (4, 160, 24, 160),
    (8, 64, 128, 32), (8, 256, 100, 256), (8, 128, 4, 64), (8, 96, 72, 32), (8, 512, 40, 256),
])
def test_repack_roundtrip_and_size(bits, K, N, G):
    c = synth.make_inputs(bits, 1, K, N, G, seed=(31, K, N))
    buf = oracle.repack(bits, c.qweight, c.qzeros, c.scales, K, N, G)
    nblk = -(-N // 16)
    rec, tile = (40, 1024) if bits == 4 else (48, 2048)
    meta = -(-(K // G) * rec // 16) * 16
    assert buf.size == nblk * (meta + -(-K // 128) * tile)
    codes, zeros, scales = oracle.unrepack(bits, buf, K, N, G)
    assert np.array_equal(codes, c.codes)
    assert np.array_equal(zeros, c.zeros)
    assert np.array_equal(scales, c.scales)
    if bits == 4:
        assert np.array_equal(oracle.pack_w4(codes), c.qweight)


def test_repack_padding_columns_are_zero():
    # N = 72 leaves 8 padding columns in the last 16-column block; their
    # codes, zeros and scales must be 0 so a consumer can read whole blocks.
    bits, K, N, G = 4, 96, 72, 32
    c = synth.make_inputs(bits, 1, K, N, G, seed=(32,))
    full = synth.gen.pack_case(bits, np.pad(c.codes, ((0, 0), (0, 8))), np.pad(c.zeros, ((0, 0), (0, 8))),
                               np.pad(c.scales, ((0, 0), (0, 8))), c.x, G)
    a = oracle.repack(bits, c.qweight, c.qzeros, c.scales, K, N, G)
    b = oracle.repack(bits, full.qweight, full.qzeros, full.scales, K, 80, G)
    assert np.array_equal(a, b)


def test_repack_is_a_bijection_on_code_positions():
    # Every (row, column) code lands on its own nibble: distinct positions.
    bits, K, N, G = 4, 64, 64, 32
    seen = set()
    for row in range(0, K, 3):
        for col in range(0, N, 5):
            c = _single_entry_case(bits, K, N, G, "code", row, col)
            buf = oracle.repack(bits, c.qweight, c.qzeros, c.scales, K, N, G)
            (pos,) = np.flatnonzero(buf)
            nib = 0 if buf[pos] & 0x0F else 1
            assert (pos, nib) not in seen
            seen.add((pos, nib))


@pytest.mark.parametrize("bits,K,N,G", [(4, 100, 64, 100), (4, 64, 12, 32), (8, 64, 64, 48), (4, 0, 64, 32),
                                       (4, 384, 64, 96), (8, 640, 64, 320)])
def test_layout_rejects_invalid_shapes(bits, K, N, G):
    assert oracle.packed_bytes(bits, K, N, G) == 0


def test_gate_up_order_hand_derived():
    # N = 32: two blocks of (8 gate, 8 up); N = 48: halves of 24, three blocks
    assert oracle.gate_up_order(32).tolist() == (list(range(0, 8)) + list(range(16, 24))
                                                 + list(range(8, 16)) + list(range(24, 32)))
    assert oracle.gate_up_order(48).tolist() == (list(range(0, 8)) + list(range(24, 32)) + list(range(8, 16))
                                                 + list(range(32, 40)) + list(range(16, 24)) + list(range(40, 48)))
    o = oracle.gate_up_order(14336 * 2)
    assert sorted(o.tolist()) == list(range(28672))          # a permutation
    with pytest.raises(ValueError):
        oracle.gate_up_order(40)


@pytest.mark.parametrize("bits,K,N,G", [(4, 256, 48, 128), (4, 160, 112, 32), (8, 384, 32, 384), (8, 128, 80, 64)])
def test_gate_up_repack_roundtrip(bits, K, N, G):
    c = synth.make_inputs(bits, 1, K, N, G, seed=(71, bits, N))
    packed = oracle.repack_gate_up(bits, c.qweight, c.qzeros, c.scales, K, N, G)
    assert packed.size == oracle.packed_bytes(bits, K, N, G)
    codes, zeros, scales = oracle.unrepack(bits, packed, K, N, G)
    order = oracle.gate_up_order(N)
    assert np.array_equal(codes, c.codes[:, order])
    assert np.array_equal(zeros, c.zeros[:, order])
    assert np.array_equal(scales, c.scales[:, order])


@pytest.mark.parametrize("bits,K,N,G", [(4, 256, 48, 128), (8, 128, 80, 64), (4, 96, 112, 32)])
def test_gate_up_repack_equals_repack_of_permuted_codes(bits, K, N, G):
    """The word shortcut of repack_gate_up against a checkpoint rebuilt from
    column-permuted codes, zeros and scales by the generator's own packer."""
    c = synth.make_inputs(bits, 1, K, N, G, seed=(81, bits, N))
    order = oracle.gate_up_order(N)
    cp = synth.gen.pack_case(bits, c.codes[:, order], c.zeros[:, order], c.scales[:, order], c.x, G)
    want = oracle.repack(bits, cp.qweight, cp.qzeros, cp.scales, K, N, G)
    assert np.array_equal(oracle.repack_gate_up(bits, c.qweight, c.qzeros, c.scales, K, N, G), want)
