"""Pins of the oracle's compressed-tensors pack-quantized ingest (CPU only).

The unpacking is pinned by hand-computed words (tests/golden), by a second
route that reads the words' bytes through a little-endian memory view, and
by the inverse packing over every byte value at every position. The scale
conversion is pinned by values whose fp32 form is known exactly.
"""
import numpy as np
import pytest

import oracle
from golden_io import pack_quantized_cases


def _signed(words):
    return np.array([w - (1 << 32) if w >= 1 << 31 else w for w in words], np.int64)


def test_hand_computed_words():
    cases = pack_quantized_cases()
    assert len(cases) >= 6
    words = _signed([w for w, _ in cases]).astype(np.int32)[:, None]
    got = oracle.unpack_pack_quantized(words)
    assert got.dtype == np.int8 and got.shape == (len(cases), 4)
    for (w, qs), row in zip(cases, got):
        assert row.tolist() == qs, hex(w)


def test_matches_little_endian_byte_view():
    rng = np.random.default_rng(5)
    words = rng.integers(-(1 << 31), 1 << 31, size=(37, 24), dtype=np.int64).astype(np.int32)
    bytes_le = np.ascontiguousarray(words.astype("<i4")).view(np.uint8).reshape(37, 96)
    expect = (bytes_le.astype(np.int16) - 128).astype(np.int8)
    assert np.array_equal(oracle.unpack_pack_quantized(words), expect)


@pytest.mark.parametrize("pos", [0, 1, 2, 3])
def test_every_value_at_every_position_round_trips(pos):
    q = np.zeros((256, 4), np.int64)
    q[:, pos] = np.arange(-128, 128)
    # pack_to_int32 of the page: uint8 (q + 128), four per word, element j in byte j
    words = sum(((q[:, j] + 128) & 0xFF) << (8 * j) for j in range(4))
    words = np.where(words >= 1 << 31, words - (1 << 32), words).astype(np.int32)[:, None]
    assert np.array_equal(oracle.unpack_pack_quantized(words), q.astype(np.int8))


def test_scale_conversion_exact():
    f32 = np.array([1.0, 0.0078125, 3.0e-5, 1e-40], np.float32)
    assert np.array_equal(oracle.scale_to_f32(f32, "f32").view(np.uint32), f32.view(np.uint32))
    # bf16 bit patterns: 1.0, 2^-7, smallest subnormal 2^-133, -3.0
    bf = np.array([0x3F80, 0x3C00, 0x0001, 0xC040], np.uint16)
    assert oracle.scale_to_f32(bf, "bf16").tolist() == [1.0, 2.0**-7, 2.0**-133, -3.0]
    # fp16 bit patterns: 1.0, 2^-14 (smallest normal), 2^-24 (smallest subnormal), 65504
    h = np.array([0x3C00, 0x0400, 0x0001, 0x7BFF], np.uint16)
    assert oracle.scale_to_f32(h, "f16").tolist() == [1.0, 2.0**-14, 2.0**-24, 65504.0]
