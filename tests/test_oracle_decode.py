"""Pins of the oracle's storage decoding (fp16 and Q4_0).

- fp16: the oracle's bit-level decoder against numpy's float16 -> float64
  conversion for all 65536 bit patterns (a library routine).
- Q4_0 (hada.io README summary, quantisation section: INT4 weights in Q4_0;
  block = fp16 scale s + 32 four-bit codes q, w = (q - 8) * s): hand-built
  blocks with closed-form values: all codes 8 give zeros, scale 1 gives
  q - 8 in -8..7 at the positions the stated nibble reading fixes, scales
  2^-k are exact.
"""
import numpy as np
import pytest

from oracle import oracle as O


def test_half_all_bit_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([O.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.signbit(O.half_to_double(0x8000)) and not np.signbit(O.half_to_double(0x0000))


def _block_row(d, code_bytes, scales_bits):
    """One Q4_0 row assembled by hand: d/2 code bytes then d/32 little-endian fp16 scales."""
    assert len(code_bytes) == d // 2 and len(scales_bits) == d // 32
    sc = np.array(scales_bits, dtype=np.uint16).view(np.uint8)
    return np.concatenate([np.array(code_bytes, dtype=np.uint8), sc])[None, :]


def test_q4_0_all_eight_is_zero():
    d = 256
    row = _block_row(d, [0x88] * (d // 2), [0x3C00] * (d // 32))   # s = 1.0
    w = O.load_row(row, d, 0, q4=True)
    assert np.array_equal(w, np.zeros(d))


def test_q4_0_scale_one_values_and_nibble_positions():
    d = 256
    # byte t of block j: low nibble = t, high nibble = 15 - t
    code = []
    for j in range(d // 32):
        code += [t | ((15 - t) << 4) for t in range(16)]
    row = _block_row(d, code, [0x3C00] * (d // 32))
    w = O.load_row(row, d, 0, q4=True)
    for j in range(d // 32):
        for t in range(16):
            assert w[32 * j + t] == t - 8            # low nibble -> element t of the block
            assert w[32 * j + 16 + t] == 7 - t       # high nibble -> element t + 16
    assert set(w.tolist()) == set(range(-8, 8))


@pytest.mark.parametrize("k", [0, 1, 3, 10, 14])
def test_q4_0_power_of_two_scales_exact(k):
    d = 256
    s_bits = int(np.float16(2.0 ** -k).view(np.uint16))
    code = [(t % 16) | (((t * 7) % 16) << 4) for t in range(d // 2)]
    row = _block_row(d, code, [s_bits] * (d // 32))
    w = O.load_row(row, d, 0, q4=True)
    for idx in range(d // 2):
        j, t = divmod(idx, 16)
        lo, hi = code[idx] & 15, code[idx] >> 4
        assert w[32 * j + t] == (lo - 8) * 2.0 ** -k
        assert w[32 * j + t + 16] == (hi - 8) * 2.0 ** -k


def test_q4_0_per_block_scales():
    d = 512
    scales = [float(2 ** (j % 5) * (-1 if j % 3 == 0 else 1)) for j in range(d // 32)]
    bits = [int(np.float16(s).view(np.uint16)) for s in scales]
    row = _block_row(d, [0x9F] * (d // 2), bits)   # low 15 -> +7, high 9 -> +1
    w = O.load_row(row, d, 0, q4=True)
    for j, s in enumerate(scales):
        assert np.all(w[32 * j:32 * j + 16] == 7 * s)
        assert np.all(w[32 * j + 16:32 * j + 32] == 1 * s)


def test_float_rows_decode_as_stored():
    rng = np.random.default_rng(0)
    a32 = rng.standard_normal((3, 64)).astype(np.float32)
    a16 = a32.astype(np.float16)
    for i in range(3):
        assert np.array_equal(O.load_row(a32, 64, i), a32[i].astype(np.float64))
        assert np.array_equal(O.load_row(a16, 64, i), a16[i].astype(np.float64))
