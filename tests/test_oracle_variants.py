"""Pins of the oracle's ablation variants (BF16): top-15 + sentinel and top-8
with 3-bit codes, the two designs the pages measure against the top-16 codec
(technical summary, "Decision de Diseno" and "Resultados").  Checked against
what the definitions fix: exhaustive round trips, the escape sets and their
order from an independent numpy evaluation, hand-worked streams, the closed
form of the stream size, and error paths."""
import numpy as np
import pytest

import kvsynth
import oracle as O

V = [O.SENTINEL, O.TOP8]
CB = np.array([127, 126, 128, 125, 129, 124, 130, 123, 131, 122, 132, 121, 133, 120, 134, 119], np.uint8)


def _all_patterns():
    x = np.arange(65536, dtype=np.uint16)
    # cross a chunk boundary with a ragged tail
    return np.concatenate([x, x[::-7][:12345]])


@pytest.mark.parametrize("v", V)
def test_exhaustive_round_trip(v):
    x = _all_patterns()
    for cb in (CB, np.arange(16, dtype=np.uint8), np.arange(240, 256, dtype=np.uint8)):
        s = O.variant_compress(v, x, cb)
        assert np.array_equal(O.variant_decompress(v, s, x.size), x)


@pytest.mark.parametrize("v", V)
def test_escape_sets_and_order_against_numpy(v):
    x = kvsynth.to_numpy_bits(kvsynth.random_bits(3 * 65536 - 77, O.BF16, seed=5, sigma=2.0))
    cbs = np.stack([O.calibrate(O.BF16, x[i::3]) for i in range(3)])
    seg = 65536
    s = O.variant_compress(v, x, cbs, seg)
    e = (x >> 7) & 0xFF
    used = 15 if v == O.SENTINEL else 8
    chunk_cb = np.minimum(np.arange(x.size) // 65536, 2)
    member = np.array([e[i] in cbs[chunk_cb[i]][:used] for i in range(x.size)])
    esc_idx = np.nonzero(~member)[0]
    E = int(np.frombuffer(s[16:24].tobytes(), "<u8")[0])
    assert E == esc_idx.size
    n = x.size
    K = 3
    C = -(-n // 65536)
    a = lambda z: -(-z // 256) * 256
    n0 = a(64 + 16 * K + 8 * (C + 1))
    code_bytes = -(-n // 2) if v == O.SENTINEL else 3 * -(-n // 8)
    n1 = n0 + a(code_bytes)
    p = n1 + a(n)
    assert s.size == O.variant_stream_size(v, n, K, E) == p + (1 if v == O.SENTINEL else 3) * E
    if v == O.SENTINEL:
        # values in element order; sentinel nibbles exactly at the escapes
        assert np.array_equal(s[p:p + E], e[esc_idx].astype(np.uint8))
        nib = np.empty(n, np.uint8)
        nib[0::2] = s[n0:n0 + (n + 1) // 2] & 0xF
        nib[1::2] = s[n0:n0 + n // 2] >> 4
        assert np.array_equal(np.nonzero(nib == 15)[0], esc_idx)
    else:
        rec = s[p:p + 3 * E].reshape(-1, 3).astype(np.int64)
        pos = rec[:, 0] | (rec[:, 1] << 8)
        assert np.array_equal(pos, esc_idx % 65536)
        assert np.array_equal(rec[:, 2], e[esc_idx])
        # codes: 3 bits each, element j of a group at bits 3j
        g = s[n0:n0 + code_bytes].reshape(-1, 3).astype(np.int64)
        word = g[:, 0] | (g[:, 1] << 8) | (g[:, 2] << 16)
        codes = ((word[:, None] >> (3 * np.arange(8))) & 7).reshape(-1)[:n]
        want = np.array([list(cbs[chunk_cb[i]][:8]).index(e[i]) if member[i] else 0 for i in range(n)])
        assert np.array_equal(codes, want)


def _u64(v):
    return list(int(v).to_bytes(8, "little"))


def _hand_input():
    # x0: +, exp 127, mant 5 -> code 0; x1: -, exp 130, mant 0x7F -> code 6;
    # x2: +, exp 119 (entry 15: escape in both variants), mant 1;
    # x3: -, exp 200 (not in the codebook), mant 0x40; x4: +, exp 123 -> code 7
    return np.array([0x3F85, 0xC17F, 0x3B81, 0xE440, 0x3D80], np.uint16)


def test_hand_worked_sentinel_stream():
    s = O.variant_compress(O.SENTINEL, _hand_input(), CB)
    head = [0x53, 0x5A, 0x31, 0x00, 1, 0, 1, 16] + _u64(5) + _u64(2) + _u64(770) + [1, 0, 0, 0, 1, 0, 0, 0] + _u64(5)
    head += [1] + [0] * 15  # variant byte
    want = np.zeros(770, np.uint8)
    want[:64] = head
    want[64:80] = CB
    want[80:96] = _u64(0) + _u64(2)
    want[256:259] = [0x60, 0xFF, 0x07]            # codes 0,6 | 15,15 | 7
    want[512:517] = [0x05, 0xFF, 0x01, 0xC0, 0x00]  # sign|mantissa
    want[768:770] = [119, 200]                     # raw exponents, element order
    assert np.array_equal(s, want)


def test_hand_worked_top8_stream():
    s = O.variant_compress(O.TOP8, _hand_input(), CB)
    head = [0x53, 0x5A, 0x31, 0x00, 1, 0, 1, 16] + _u64(5) + _u64(2) + _u64(774) + [1, 0, 0, 0, 1, 0, 0, 0] + _u64(5)
    head += [2] + [0] * 15
    want = np.zeros(774, np.uint8)
    want[:64] = head
    want[64:80] = CB
    want[80:96] = _u64(0) + _u64(2)
    want[256:259] = [0x30, 0x70, 0x00]             # 0 | 6<<3 | 0<<6 | 0<<9 | 7<<12
    want[512:517] = [0x05, 0xFF, 0x01, 0xC0, 0x00]
    want[768:774] = [2, 0, 119, 3, 0, 200]         # (position, exponent) records
    assert np.array_equal(s, want)


@pytest.mark.parametrize("v", V)
def test_variant_streams_are_not_main_streams(v):
    x = _hand_input()
    s = O.variant_compress(v, x, CB)
    assert O.decompress_rc(s, O.BF16, x.size)[0] == O.E_CORRUPT       # main decoder rejects it
    other = O.TOP8 if v == O.SENTINEL else O.SENTINEL
    assert O.variant_decompress_rc(other, s, x.size)[0] == O.E_CORRUPT
    main = O.compress(O.BF16, x, CB)
    assert O.variant_decompress_rc(v, main, x.size)[0] == O.E_CORRUPT


def test_sentinel_count_must_match_offsets():
    x = _hand_input()
    s = O.variant_compress(O.SENTINEL, x, CB).copy()
    s[256] = 0x6F  # x0 becomes a sentinel: 3 sentinels, 2 values
    assert O.variant_decompress_rc(O.SENTINEL, s, x.size)[0] == O.E_CORRUPT
    s = O.variant_compress(O.SENTINEL, x, CB)
    assert O.variant_decompress_rc(O.SENTINEL, s[:-1], x.size)[0] == O.E_CORRUPT  # truncated


def test_top8_record_checks():
    x = _hand_input()
    s = O.variant_compress(O.TOP8, x, CB).copy()
    s[768], s[771] = 3, 2  # positions out of order
    assert O.variant_decompress_rc(O.TOP8, s, x.size)[0] == O.E_CORRUPT
    s = O.variant_compress(O.TOP8, x, CB).copy()
    s[771] = 5  # position past the chunk's end (n = 5)
    assert O.variant_decompress_rc(O.TOP8, s, x.size)[0] == O.E_CORRUPT


@pytest.mark.parametrize("v", V)
def test_empty_and_tiny(v):
    for n in (0, 1, 7, 8, 9):
        x = (np.arange(n, dtype=np.uint16) * 4099) & 0xFFFF
        s = O.variant_compress(v, x, CB)
        assert np.array_equal(O.variant_decompress(v, s, n), x)
