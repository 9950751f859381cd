"""Pins of the CPU oracle against what the SplitZip pages and plain mathematics fix.

None of these checks re-types the oracle's own formulas: each compares the
oracle with float semantics (numpy frexp), an independent numpy computation
of a definition (codebook membership, escape sets), brute force, a hand-worked
stream, the explainer's worked example, or the pages' ratio limits.

Pages: "SplitZip: Ultra Fast Lossless KV Compression for Disaggregated LLM
Serving" (arXiv 2605.01708v2): the Spanish technical summary [TS], the English
explainer [EX] and the authors' abstract [AB].
"""
import itertools
import math
import os

import numpy as np
import pytest

import kvsynth
import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
CHUNK = 65536


def _exp_bf16(x):
    return (x.astype(np.uint32) >> 7) & 0xFF


def _exp_e5m2(x):
    return (x.astype(np.uint32) >> 2) & 0x1F


def _records(stream, n_escapes):
    """Escape records decoded from the tail of the stream (the section is the
    last 3E bytes)."""
    tail = stream[len(stream) - 3 * n_escapes:].reshape(-1, 3).astype(np.int64)
    return tail[:, 0] | (tail[:, 1] << 8), tail[:, 2]


def _hdr_u64(stream, off):
    return int(np.frombuffer(stream[off:off + 8].tobytes(), dtype="<u8")[0])


# ---------------------------------------------------------------- round trips
@pytest.mark.parametrize("cbname", ["calibrated", "excludes_0_255", "includes_0_255"])
def test_bf16_all_patterns_roundtrip(cbname):
    """Every one of the 65,536 BF16 bit patterns (+-0, subnormals, +-Inf, NaN
    payloads included) decodes bit-exactly ([AB]: tensors are preserved
    bitwise; [TS] Estrategia de Decodificacion / Correccion)."""
    allp = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    rng = np.random.default_rng(7)
    # three chunks and a ragged tail: every pattern, shuffled, then a prefix again
    x = np.concatenate([rng.permutation(allp), rng.permutation(allp), allp[: 12345]])
    if cbname == "calibrated":
        cb = O.calibrate(O.BF16, x)
    elif cbname == "excludes_0_255":
        cb = np.arange(120, 136, dtype=np.uint8)
    else:
        cb = np.array([0, 255] + list(range(120, 134)), dtype=np.uint8)
    s = O.compress(O.BF16, x, cb)
    y = O.decompress(s, O.BF16, x.size)
    assert np.array_equal(y, x)
    # each exponent value occurs 256 times among the 65,536 patterns
    member = np.isin(_exp_bf16(x), cb.astype(np.uint32))
    assert _hdr_u64(s, 16) == int((~member).sum())


@pytest.mark.parametrize("cbname", ["calibrated", "excludes_0_31", "includes_0_31"])
def test_e5m2_all_patterns_roundtrip(cbname):
    """All 256 E5M2 patterns round-trip bit-exactly ([TS] Contribuciones Clave 4; [AB])."""
    allp = np.arange(256, dtype=np.uint8)
    rng = np.random.default_rng(8)
    x = np.concatenate([rng.permutation(allp) for _ in range(600)])  # 153,600: 3 chunks, ragged
    if cbname == "calibrated":
        cb = O.calibrate(O.E5M2, x)
    elif cbname == "excludes_0_31":
        cb = np.arange(8, 24, dtype=np.uint8)
    else:
        cb = np.array([0, 31] + list(range(8, 22)), dtype=np.uint8)
    s = O.compress(O.E5M2, x, cb)
    assert np.array_equal(O.decompress(s, O.E5M2, x.size), x)
    member = np.isin(_exp_e5m2(x), cb.astype(np.uint32))
    assert _hdr_u64(s, 16) == int((~member).sum())


@pytest.mark.parametrize("dtype", [O.BF16, O.E5M2])
@pytest.mark.parametrize("n", [0, 1, 2, 3, 7, 8, 9, 15, 16, 17, 65535, 65536, 65537, 131073])
def test_sizes_roundtrip(dtype, n):
    """Empty, odd, partial-group and partial-chunk sizes round-trip, and the
    stream has the closed-form length."""
    x = kvsynth.to_numpy_bits(kvsynth.random_bits(n, dtype, seed=n + 11))
    cb = O.calibrate(dtype, x[: max(1, n // 2)])
    s = O.compress(dtype, x, cb)
    assert np.array_equal(O.decompress(s, dtype, n), x)
    E = _hdr_u64(s, 16)
    assert len(s) == O.stream_size(dtype, n, 1, E)


# --------------------------------------------------- field split vs float math
def test_bf16_split_matches_float_semantics():
    """The exponent an escape record carries and the sign|mantissa byte are the
    IEEE fields of the value ([EX] "1. The 'Note' Structure"; [TS] Preservacion
    de Signo/Mantisa): for a normal BF16 value v = (-1)^s 2^(e-127) (1 + m/128).
    A codebook disjoint from the data's exponents makes every element escape,
    so the records expose every exponent."""
    rng = np.random.default_rng(3)
    mags = 2.0 ** rng.integers(-20, 21, size=4000) * (1 + rng.integers(0, 128, size=4000) / 128.0)
    vals = (mags * np.where(rng.random(4000) < 0.5, -1.0, 1.0)).astype(np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)  # exact: 7 mantissa bits only
    cb = np.arange(0, 16, dtype=np.uint8)  # exponents 0..15 never occur here
    s = O.compress(O.BF16, bits, cb)
    E = _hdr_u64(s, 16)
    assert E == bits.size
    pos, ev = _records(s, E)
    assert np.array_equal(pos, np.arange(bits.size))
    fr_m, fr_e = np.frexp(np.abs(vals.astype(np.float64)))  # |v| = fr_m 2^fr_e, fr_m in [0.5, 1)
    assert np.array_equal(ev, fr_e - 1 + 127)
    # sign|mantissa section: N1 = N0 + A(ceil(n/2)); N0 = A(64 + 16 + 16)
    n0 = 256
    n1 = n0 + ((bits.size + 1) // 2 + 255) // 256 * 256
    sm = s[n1:n1 + bits.size].astype(np.int64)
    mant = np.round((2 * fr_m - 1) * 128).astype(np.int64)
    sign = (vals < 0).astype(np.int64)
    assert np.array_equal(sm, (sign << 7) | mant)


def test_e5m2_split_matches_float_semantics():
    """E5M2: v = (-1)^s 2^(e-15) (1 + m/4) for normal values; escape values are e."""
    import torch
    rng = np.random.default_rng(4)
    e = rng.integers(1, 31, size=3000)
    m = rng.integers(0, 4, size=3000)
    sgn = rng.random(3000) < 0.5
    vals = np.where(sgn, -1.0, 1.0) * 2.0 ** (e - 15) * (1 + m / 4.0)
    bits = torch.from_numpy(vals.astype(np.float32)).to(torch.float8_e5m2).view(torch.uint8).numpy()
    back = torch.from_numpy(bits).view(torch.float8_e5m2).to(torch.float64).numpy()
    assert np.array_equal(back, vals)  # exactly representable
    present = set(np.unique(e).tolist())
    cb = np.array([v for v in range(32) if v not in present][:16], dtype=np.uint8)
    cb = np.concatenate([cb, np.array([v for v in range(32) if v not in cb][: 16 - cb.size], np.uint8)])
    s = O.compress(O.E5M2, bits, cb)
    E = _hdr_u64(s, 16)
    pos, ev = _records(s, E)
    esc_mask = ~np.isin(e, cb.astype(np.int64))
    assert np.array_equal(pos, np.nonzero(esc_mask)[0])
    assert np.array_equal(ev, e[esc_mask])
    assert np.array_equal(O.decompress(s, O.E5M2, bits.size), bits)


# -------------------------------------------------------------- calibration
def _bruteforce_top16(exps, V):
    vals, counts = np.unique(exps, return_counts=True)
    cnt = dict(zip(vals.tolist(), counts.tolist()))
    universe = list(range(V))
    best = None
    # candidates: any 16-subset of the values present plus the smallest absent ones
    present = sorted(cnt)
    absent = [v for v in universe if v not in cnt]
    pool = present + absent[: max(0, 16 - len(present)) + 2]
    for sub in itertools.combinations(pool, 16):
        covered = sum(cnt.get(v, 0) for v in sub)
        key = (-covered, sum(sub))
        if best is None or key < best[0]:
            best = (key, set(sub))
    return best[1], cnt


@pytest.mark.parametrize("seed", range(12))
def test_calibrate_matches_bruteforce(seed):
    """The codebook is the top-16 exponent set by frequency ([TS] Codificacion
    de Longitud Fija; [AB] offline top-16 codebook): it maximizes coverage
    (= minimizes escapes), and on ties takes the lower exponents.  Checked
    against an exhaustive search over all 16-subsets on tiny inputs."""
    rng = np.random.default_rng(seed)
    k = int(rng.integers(3, 21))
    values = rng.choice(256, size=k, replace=False)
    counts = rng.integers(1, 6, size=k)  # small counts -> many ties
    exps = np.repeat(values, counts)
    x = ((rng.integers(0, 2, size=exps.size) << 15) | (exps << 7) | rng.integers(0, 128, size=exps.size)).astype(np.uint16)
    cb = O.calibrate(O.BF16, x)
    want, cnt = _bruteforce_top16(exps, 256)
    assert set(cb.tolist()) == want
    # code order: non-increasing count, equal counts in ascending exponent
    keys = [(-cnt.get(v, 0), v) for v in cb.tolist()]
    assert keys == sorted(keys)
    assert len(set(cb.tolist())) == 16


def test_calibrate_e5m2_fill_and_ties():
    """Fewer than 16 distinct exponents: the missing slots take the lowest
    unseen exponents; the codebook always has 16 distinct entries."""
    x = np.array([(20 << 2), (20 << 2) | 1, (3 << 2), (25 << 2) | 0x80], dtype=np.uint8)
    cb = O.calibrate(O.E5M2, x)
    assert cb.tolist()[:3] == [20, 3, 25]
    assert cb.tolist()[3:] == [v for v in range(32) if v not in (20, 3, 25)][:13]


def test_zero_escapes_when_at_most_16_exponents():
    """A tensor with <= 16 distinct exponents, calibrated on itself, has no
    escapes, and its stream is the dense part only."""
    rng = np.random.default_rng(5)
    exps = rng.choice(np.arange(100, 140), size=16, replace=False)
    n = 3 * CHUNK + 77
    e = rng.choice(exps, size=n)
    x = ((rng.integers(0, 2, size=n) << 15) | (e << 7) | rng.integers(0, 128, size=n)).astype(np.uint16)
    cb = O.calibrate(O.BF16, x)
    s = O.compress(O.BF16, x, cb)
    assert _hdr_u64(s, 16) == 0
    assert len(s) == O.stream_size(O.BF16, n, 1, 0)
    assert np.array_equal(O.decompress(s, O.BF16, n), x)


# ------------------------------------------------------------ escape stream
@pytest.mark.parametrize("dtype", [O.BF16, O.E5M2])
def test_escapes_and_codes_match_definition(dtype):
    """With K per-segment codebooks: every element whose exponent is in its
    chunk's codebook gets the index of that entry as its 4-bit code, two codes
    per byte with the even element low ([TS] Codificacion de Longitud Fija);
    every other element is an escape record (chunk-relative 16-bit position,
    raw exponent) in element order, with code 0 ([TS] Flujo de Escape)."""
    rng = np.random.default_rng(9)
    seg = 2 * CHUNK
    K = 3
    n = K * seg - 4321
    x = kvsynth.to_numpy_bits(kvsynth.random_bits(n, dtype, seed=99, sigma=1.5))
    V = 256 if dtype == O.BF16 else 32
    ex = _exp_bf16(x) if dtype == O.BF16 else _exp_e5m2(x)
    cbs = []
    for k in range(K):
        part = x[k * seg:(k + 1) * seg]
        cbs.append(O.calibrate(dtype, part[: 5000]))
    cbs[1] = rng.permutation(cbs[1])  # code order is whatever the codebook says
    cbs = np.stack(cbs)
    s = O.compress(dtype, x, cbs, segment_elems=seg)
    assert np.array_equal(O.decompress(s, dtype, n), x)
    seg_of = np.arange(n) // seg
    table = np.full((K, V), -1, dtype=np.int64)
    for k in range(K):
        table[k, cbs[k]] = np.arange(16)
    code = table[seg_of, ex]
    esc = code < 0
    E = _hdr_u64(s, 16)
    assert E == int(esc.sum()) == O.count_escapes(dtype, x, cbs, seg)
    pos, val = _records(s, E)
    idx = np.nonzero(esc)[0]
    assert np.array_equal(pos, idx % CHUNK)
    assert np.array_equal(val, ex[esc])
    nib = np.where(esc, 0, code)
    nib = np.concatenate([nib, np.zeros(n % 2, dtype=np.int64)])
    packed = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)
    C = -(-n // CHUNK)
    n0 = (64 + 16 * K + 8 * (C + 1) + 255) // 256 * 256
    assert np.array_equal(s[n0:n0 + packed.size], packed)
    # per-chunk exclusive offsets
    offs = np.frombuffer(s[64 + 16 * K:64 + 16 * K + 8 * (C + 1)].tobytes(), dtype="<u8")
    per_chunk = np.bincount(idx // CHUNK, minlength=C)
    assert np.array_equal(offs, np.concatenate([[0], np.cumsum(per_chunk)]))


def test_explainer_position50_golden():
    """[EX] "3. The SplitZip Strategy", 'The Rare List': the rare exponent at
    position #50 becomes one escape note (50, 99)."""
    spec = {}
    with open(os.path.join(GOLDEN, "explainer_position50.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                key, _, val = line.partition(" ")
                spec.setdefault(key, []).append(val)
    n = int(spec["n"][0])
    e = np.full(n, int(spec["exponent_default"][0]))
    p, v = map(int, spec["exponent_at"][0].split())
    e[p] = v
    sm = (np.arange(n) * 37) % 256
    x = (((sm >> 7) << 15) | (e << 7) | (sm & 0x7F)).astype(np.uint16)
    lo, hi, reps = map(int, spec["calib_exponents"][0].split())
    calib = (np.repeat(np.arange(lo, hi + 1), reps) << 7).astype(np.uint16)
    cb = O.calibrate(O.BF16, calib)
    assert set(cb.tolist()) == set(range(lo, hi + 1))
    s = O.compress(O.BF16, x, cb)
    E = _hdr_u64(s, 16)
    assert E == int(spec["expect_escapes"][0])
    pos, val = _records(s, E)
    rp, rv = map(int, spec["expect_record"][0].split())
    assert pos.tolist() == [rp] and val.tolist() == [rv]
    assert np.array_equal(O.decompress(s, O.BF16, n), x)


# ------------------------------------------------------------ exact bytes
def test_hand_worked_bf16_stream():
    """Five BF16 values, one codebook, worked out by hand from the stream
    layout (header 64 B, codebook, offsets, 256-B aligned sections)."""
    # 1.0 = 0x3F80 (e 127, m 0), -2.0 = 0xC000 (s 1, e 128), 1.5 = 0x3FC0
    # (e 127, m 0x40), 0.0 = 0x0000 (e 0), 3.0 = 0x4040 (e 128, m 0x40)
    x = np.array([0x3F80, 0xC000, 0x3FC0, 0x0000, 0x4040], dtype=np.uint16)
    cb = np.array([127, 128] + list(range(100, 114)), dtype=np.uint8)  # 0 is not a member
    s = O.compress(O.BF16, x, cb)
    exp = np.zeros(771, dtype=np.uint8)
    exp[0:4] = [0x53, 0x5A, 0x31, 0x00]        # magic "SZ1\0"
    exp[4:6] = [1, 0]                          # version 1
    exp[6] = 1                                 # BF16
    exp[7] = 16                                # 65536-element chunks
    exp[8] = 5                                 # n = 5
    exp[16] = 1                                # one escape
    exp[24:26] = [0x03, 0x03]                  # total 771 = 0x303
    exp[32] = 1                                # one chunk
    exp[36] = 1                                # one codebook
    exp[40] = 5                                # segment = n
    exp[64:80] = cb                            # codebook
    exp[80:88] = 0                             # off[0] = 0
    exp[88] = 1                                # off[1] = 1
    # nibbles at 256: codes 0,1,0,(esc)0,1 -> 0x10, 0x00, 0x01
    exp[256:259] = [0x10, 0x00, 0x01]
    # sign|mantissa at 512: 0x00, 0x80, 0x40, 0x00, 0x40
    exp[512:517] = [0x00, 0x80, 0x40, 0x00, 0x40]
    # escape record at 768: position 3, exponent 0
    exp[768:771] = [3, 0, 0]
    assert np.array_equal(s, exp)


def test_hand_worked_e5m2_stream():
    """Nine E5M2 values: one full group of 8 sign|mantissa triples in 3 bytes
    and a partial second group."""
    # e5m2 byte = s<<7 | e<<2 | m ; values chosen with exponents 15 and 16
    x = np.array([(15 << 2) | 0, 0x80 | (16 << 2) | 1, (15 << 2) | 2, (15 << 2) | 3,
                  (16 << 2) | 0, 0x80 | (15 << 2) | 1, (16 << 2) | 2, 0x80 | (16 << 2) | 3,
                  0x80 | (7 << 2) | 1], dtype=np.uint8)
    cb = np.array([15, 16] + list(range(17, 31)), dtype=np.uint8)  # exponent 7 escapes
    s = O.compress(O.E5M2, x, cb)
    # sign|mantissa triples s3 = s<<2|m: 0,5,2,3,0,5,2,7 | 5
    g0 = sum(t << (3 * j) for j, t in enumerate([0, 5, 2, 3, 0, 5, 2, 7]))
    g1 = 5
    assert len(s) == 768 + 3
    assert s[6] == 2
    # codes: e=15->0, 16->1, ..., the last element (e=7) escapes with code 0
    codes = [0, 1, 0, 0, 1, 0, 1, 1, 0]
    want_nib = [codes[0] | codes[1] << 4, codes[2] | codes[3] << 4, codes[4] | codes[5] << 4,
                codes[6] | codes[7] << 4, codes[8]]
    assert list(s[256:261]) == want_nib
    assert list(s[512:518]) == [g0 & 255, (g0 >> 8) & 255, g0 >> 16, g1, 0, 0]
    assert list(s[768:771]) == [8, 0, 7]


# ------------------------------------------------------------ pages' ratios
def test_ratio_limits_from_pages():
    """[TS] Resultados: the BF16 ratio tends to 16/12 = 1.33x as escapes vanish;
    [TS] Contribuciones Clave 4 and [AB]: E5M2 gains up to 1.14x (= 8/7)."""
    n = 1 << 22
    rng = np.random.default_rng(6)
    x = ((rng.integers(0, 2, size=n) << 15) | (127 << 7) | rng.integers(0, 128, size=n)).astype(np.uint16)
    s = O.compress(O.BF16, x, O.calibrate(O.BF16, x))
    r = 2 * n / len(s)
    assert 16 / 12 * (1 - 1e-3) < r < 16 / 12
    assert round(r, 2) == 1.33
    y = ((rng.integers(0, 2, size=n) << 7) | (17 << 2) | rng.integers(0, 4, size=n)).astype(np.uint8)
    s8 = O.compress(O.E5M2, y, O.calibrate(O.E5M2, y))
    r8 = n / len(s8)
    assert 8 / 7 * (1 - 1e-3) < r8 < 8 / 7
    assert round(r8, 2) == 1.14
    # at an escape rate of 0.16% the size is 12 + 24 * 0.0016 bits per value,
    # i.e. about 1.329x, "approaching 1.33x"
    E = int(0.0016 * n)
    r_eps = 2 * n / O.stream_size(O.BF16, n, 1, E)
    assert abs(r_eps - 16 / (12 + 24 * 0.0016)) < 1e-3


def test_closed_form_size_is_dense_plus_escapes_plus_headers():
    """Stream size = n/2 + n + 3 * escapes + headers (BF16), where headers are
    the 64-B header, codebooks, chunk offsets and < 256 B of padding per
    section."""
    for n, K in [(1, 1), (1000, 1), (CHUNK * 5 + 3, 3), (CHUNK * 64, 64)]:
        C = -(-n // CHUNK)
        for E in [0, 1, n // 3, n]:
            S = O.stream_size(O.BF16, n, K, E)
            dense = -(-n // 2) + n + 3 * E
            hdr = 64 + 16 * K + 8 * (C + 1)
            assert hdr <= S - dense < hdr + 3 * 256
            S8 = O.stream_size(O.E5M2, n, K, E)
            dense8 = -(-n // 2) + 3 * (-(-n // 8)) + 3 * E
            assert hdr <= S8 - dense8 < hdr + 3 * 256


# ------------------------------------------------------------ error paths
def test_error_paths():
    x = ((np.arange(1000) * 997) % 65536).astype(np.uint16)  # many exponents -> escapes
    cb = O.calibrate(O.BF16, x[:50])
    assert O.compress_rc(3, x, cb)[0] == O.E_INVALID
    bad = cb.copy()
    bad[5] = bad[4]
    assert O.compress_rc(O.BF16, x, bad)[0] == O.E_CODEBOOK
    assert O.compress_rc(O.E5M2, x.astype(np.uint8), np.arange(20, 36, dtype=np.uint8))[0] == O.E_CODEBOOK
    assert O.compress_rc(O.BF16, x, cb, capacity=100)[0] == O.E_CAPACITY
    # K > 1 needs 65536-multiple segments that cover n
    two = np.stack([cb, cb])
    assert O.compress_rc(O.BF16, x, two, segment_elems=1000)[0] == O.E_INVALID
    assert O.compress_rc(O.BF16, x, two, segment_elems=CHUNK)[0] == O.OK
    s = O.compress(O.BF16, x, cb)
    n = x.size
    assert O.validate(s, O.BF16, n) == O.OK
    assert O.validate(s, O.E5M2, n) == O.E_CORRUPT
    assert O.validate(s, O.BF16, n + 1) == O.E_CORRUPT
    assert O.validate(s[:-1], O.BF16, n) == O.E_CORRUPT           # truncated
    for off, val in [(0, 0x54), (4, 2), (7, 15), (50, 1)]:        # magic, version, chunk log2, reserved
        t = s.copy(); t[off] = val
        assert O.validate(t, O.BF16, n) == O.E_CORRUPT
    E = _hdr_u64(s, 16)
    assert E > 2
    t = s.copy(); t[len(t) - 3 * E] = 0xE8; t[len(t) - 3 * E + 1] = 0x03   # position 1000 >= n
    assert O.validate(t, O.BF16, n) == O.E_CORRUPT
    t = s.copy(); t[len(t) - 3] = t[len(t) - 6]; t[len(t) - 2] = t[len(t) - 5]  # repeated position
    assert O.validate(t, O.BF16, n) == O.E_CORRUPT
    t = s.copy(); t[64 + 16] = 1                                           # off[0] != 0
    assert O.validate(t, O.BF16, n) == O.E_CORRUPT
    t = s.copy(); t[64 + 16 + 8] ^= 1                                      # off[C] != E
    assert O.validate(t, O.BF16, n) == O.E_CORRUPT
    t = s.copy(); t[64 + 3] = t[64 + 2]                                    # duplicate codebook entry
    assert O.validate(t, O.BF16, n) == O.E_CORRUPT
    assert O.decompress_rc(s[:-1], O.BF16, n)[0] == O.E_CORRUPT


def test_calibrate_invalid():
    with pytest.raises(ValueError):
        O.calibrate(7, np.zeros(4, dtype=np.uint16))


def test_calibrate_extreme_exponents():
    """The all-ones exponent (Inf/NaN) and zero exponent (zero/subnormal) are
    ordinary codebook candidates: the most frequent values win whatever they are."""
    x = np.concatenate([np.full(50, 0x7F80 | 3), np.full(40, 0x0001), np.full(30, 0x3F80),
                        np.arange(16) << 7]).astype(np.uint16)
    cb = O.calibrate(O.BF16, x)
    assert cb.tolist()[:3] == [255, 0, 127]
    y = np.concatenate([np.full(9, 0x7F), np.full(7, 0x01), np.full(5, 31 << 2)]).astype(np.uint8)
    assert O.calibrate(O.E5M2, y).tolist()[:2] == [31, 0]
