"""Pins of the oracle's blockwise quantizer, packing and double quantization.

Brute force over exact rationals, an exhaustive fp16 sweep, constructed ties,
closed-form sizes from the QLoRA page's double-quantization arithmetic, and a
round trip through weights placed on codebook points.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import quant as Q

BITS = [2, 3, 4, 8]


def brute_code(w, a, L):
    """argmin_i |w - L_i a| over exact rationals, ties to the lower index."""
    fw, fa = Fraction(float(w)), Fraction(float(a))
    best, bi = None, None
    for i, lv in enumerate(L):
        d = abs(fw - Fraction(float(lv)) * fa)
        if best is None or d < best:
            best, bi = d, i
    return bi


@pytest.mark.parametrize("bits", BITS)
def test_codes_match_exact_argmin(bits):
    rng = np.random.default_rng(100 + bits)
    L = oracle.quantile_codebook(bits)
    nblk = 6 if bits < 8 else 2
    w = (rng.standard_normal((nblk, 64)) * rng.choice([1e-3, 0.02, 1.0, 300.0], size=(nblk, 1))).astype(np.float32)
    a = np.abs(w).max(axis=1).astype(np.float32)
    codes = Q.nearest_codes(w, a, L)
    for j in range(nblk):
        for e in range(64):
            assert codes[j, e] == brute_code(w[j, e], a[j], L), (j, e)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_codes_exhaustive_fp16_sweep(bits):
    """Every finite fp16 in [-1, 1] in blocks whose absmax is exactly 1.0.

    With a = 1, |w - L_i| is exact in float64 (fp16 minus fp32), so an argmin of
    distances (first minimum = lower index) is an independent exact reference.
    """
    allh = np.arange(1 << 16, dtype=np.uint16).view(np.float16)
    vals = allh[np.isfinite(allh) & (np.abs(allh.astype(np.float32)) <= 1.0)].astype(np.float32)
    if bits == 8:
        vals = vals[::7]
    per = 63
    nblk = -(-vals.size // per)
    blocks = np.zeros((nblk, 64), dtype=np.float32)
    blocks[:, 0] = 1.0
    flat = np.zeros(nblk * per, dtype=np.float32)
    flat[: vals.size] = vals
    blocks[:, 1:] = flat.reshape(nblk, per)
    a = np.abs(blocks).max(axis=1).astype(np.float32)
    assert np.all(a == 1.0)
    L = oracle.quantile_codebook(bits)
    codes = Q.nearest_codes(blocks, a, L)
    dist = np.abs(blocks.astype(np.float64)[:, :, None] - L.astype(np.float64)[None, None, :])
    ref = np.argmin(dist, axis=2)
    assert np.array_equal(codes, ref.astype(np.uint8))


@pytest.mark.parametrize("bits", BITS)
def test_ties_go_to_lower_index(bits):
    L = oracle.quantile_codebook(bits)
    n = L.size
    tested = 0
    for a in [2.0, 0.5, 1.0, 8.0]:
        for i in range(n - 1):
            mid = (float(L[i]) + float(L[i + 1])) * a / 2.0
            if float(np.float32(mid)) != mid or abs(mid) > a:
                continue
            blk = np.zeros((1, 64), dtype=np.float32)
            blk[0, 0] = a
            blk[0, 1] = mid
            codes = Q.nearest_codes(blk, np.array([a], np.float32), L)
            assert codes[0, 1] == i, (a, i)
            tested += 1
    assert tested >= 4  # at least the middle pair (mid == 0) for each a


@pytest.mark.parametrize("bits", BITS)
def test_special_values(bits):
    L = oracle.quantile_codebook(bits)
    n = L.size
    blk = np.zeros((3, 64), dtype=np.float32)
    blk[0, 0], blk[0, 1], blk[0, 2], blk[0, 3] = 0.75, -0.75, 0.0, -0.0
    a = np.abs(blk).max(axis=1).astype(np.float32)
    c = Q.nearest_codes(blk, a, L)
    assert c[0, 0] == n - 1 and c[0, 1] == 0
    assert c[0, 2] == n // 2 - 1 and c[0, 3] == n // 2 - 1  # +-0 tie between the middle pair
    assert np.all(c[1] == 0) and np.all(c[2] == 0)  # absmax 0 -> every code 0


@pytest.mark.parametrize("bits", BITS)
def test_error_within_half_gap(bits):
    rng = np.random.default_rng(7)
    L = oracle.quantile_codebook(bits).astype(np.float64)
    w = (rng.standard_normal((200, 64)) * 0.02).astype(np.float32)
    a = np.abs(w).max(axis=1).astype(np.float32)
    c = Q.nearest_codes(w, a, L.astype(np.float32)).astype(np.int64)
    r = w.astype(np.float64) / a[:, None]
    hi = np.searchsorted(L, r, side="right").clip(1, L.size - 1)
    gap = L[hi] - L[hi - 1]
    err = np.abs(w - L[c] * a[:, None])
    assert np.all(err <= 0.5 * gap * a[:, None] * (1 + 1e-12))


@pytest.mark.parametrize("bits", BITS)
def test_packing_layout(bits):
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 1 << bits, size=(5, 64), dtype=np.uint8)
    packed = Q.pack_codes(codes, bits)
    assert packed.size == 5 * 8 * bits
    for j in range(5):
        big = int.from_bytes(packed[8 * bits * j: 8 * bits * (j + 1)].tobytes(), "little")
        for e in range(64):
            assert (big >> (bits * e)) & ((1 << bits) - 1) == codes[j, e]
    assert np.array_equal(Q.unpack_codes(packed, bits, 5), codes)


def test_packing_nibble_order():
    codes = np.tile(np.arange(16, dtype=np.uint8), 4)[None, :]
    packed = Q.pack_codes(codes, 4)
    assert packed[0] == 0x10 and packed[1] == 0x32 and packed[7] == 0xFE


@pytest.mark.parametrize("bits", BITS)
def test_bits_per_param(bits, page_value):
    rows, cols = 4096, 4096
    cb, qb, kb = oracle.qweight_sizes(rows, cols, bits)
    total_bits = 8 * (cb + qb + kb)
    per_param = Fraction(total_bits, rows * cols)
    assert per_param == bits + Fraction(8, 64) + Fraction(32, 64 * 256)
    overhead = float(per_param - bits)
    assert abs(overhead - page_value("double_quant_overhead_bits")) < 5e-4
    # first-level constants of 16 bits, not double-quantized: 16/64 bits per parameter
    assert Fraction(16, 64) == Fraction(page_value("single_quant_overhead_bits_16bit_consts")).limit_denominator(8)
    # saving against float32 first-level constants (32/64) is about 0.37 bits
    assert abs((32 / 64 - overhead) - page_value("double_quant_saving_bits")) < 5e-3
    if bits == 4:
        assert cb == rows * cols * page_value("nf4_weight_bytes_per_param")


def test_65b_memory_figures(page_value):
    params = 65e9
    fp16_gb = 2 * params / 1e9
    assert abs(fp16_gb - page_value("params_65b_fp16_gb")) / page_value("params_65b_fp16_gb") < 0.02
    per_param_bits = 4 + 8 / 64 + 32 / (64 * 256)
    nf4_gb = params * per_param_bits / 8 / 1e9
    assert nf4_gb < page_value("params_65b_qlora_gb")  # weights are part of the ~40 GB total


def _round_f32_fraction(q: Fraction) -> float:
    """Round a positive rational to float32 (nearest, ties even) by integer arithmetic."""
    if q == 0:
        return 0.0
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    e = max(e, -126)
    scaled = q / Fraction(2) ** (e - 23)  # mantissa in [2^23, 2^24) for normals
    m = scaled.numerator // scaled.denominator
    rem = scaled - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    return float(Fraction(m) * Fraction(2) ** (e - 23))


def test_double_quant_exact():
    rng = np.random.default_rng(11)
    nblk = 256 * 3 + 37  # three full groups and a tail group
    a = np.abs(rng.standard_normal(nblk) * 0.05).astype(np.float32)
    a[5] = 0.0
    a[256:512] = 0.0  # an all-zero group
    a[600] = a[600] * 40  # an outlier block
    q8, step = Q.double_quantize(a)
    assert step.dtype == np.float32 and step.size == 4 and q8.size == nblk
    for h in range(4):
        g = a[256 * h: 256 * (h + 1)].max()
        assert float(step[h]) == _round_f32_fraction(Fraction(float(g)) / 255)
    for j in range(nblk):
        s = Fraction(float(step[j // 256]))
        fa = Fraction(float(a[j]))
        best = min(range(256), key=lambda m: (abs(fa - m * s), m))
        assert q8[j] == best, j
        assert abs(fa - q8[j] * s) <= s / 2


def test_round_trip_on_codebook_points():
    """Weights on scaled codebook points with representable scales come back bit-exact."""
    rng = np.random.default_rng(5)
    for bits in BITS:
        L = oracle.quantile_codebook(bits)
        ngrp = 3
        nblk = 256 * ngrp
        w = np.zeros((nblk, 64), dtype=np.float32)
        for h in range(ngrp):
            s = np.float32(int(rng.integers(1 << 15, 1 << 16)) * 2.0 ** -26)  # 16 significant bits
            ms = rng.integers(1, 256, size=256)
            ms[rng.integers(0, 256)] = 255
            for jj in range(256):
                j = 256 * h + jj
                ap = np.float32(ms[jj] * s)  # exact: 8 x 16 bits
                idx = rng.integers(0, L.size, size=64)
                w[j] = (L[idx] * ap).astype(np.float32)
                w[j, rng.integers(0, 64)] = ap * (1 if rng.integers(0, 2) else -1)
        qw = oracle.quantize(w.reshape(-1), "f32", bits)
        back = oracle.dequantize(qw.codes, qw.absmax_q8, qw.absmax_c, bits, w.size)
        assert np.array_equal(back.view(np.uint32), w.reshape(-1).view(np.uint32)), bits


def test_zero_block_dequantizes_to_negative_zero():
    w = np.zeros(64 * 4, dtype=np.float32)
    w[64:128] = 0.01
    qw = oracle.quantize(w, "f32", 4)
    back = oracle.dequantize(qw.codes, qw.absmax_q8, qw.absmax_c, 4, w.size)
    assert np.all(back[:64] == 0) and np.all(np.signbit(back[:64]))  # level -1 times +0


def test_tail_block_and_group():
    rng = np.random.default_rng(9)
    numel = 64 * 300 + 17
    w = (rng.standard_normal(numel) * 0.02).astype(np.float16)
    qw = oracle.quantize(w, "f16", 4)
    assert qw.absmax.size == 301 and qw.absmax_c.size == 2 and qw.codes.size == 301 * 32
    assert qw.absmax[-1] == np.abs(w[64 * 300:].astype(np.float32)).max()
    assert np.all(qw.code_matrix[-1, 17:] == 0)
    back = oracle.dequantize(qw.codes, qw.absmax_q8, qw.absmax_c, 4, numel)
    assert back.size == numel


def test_nonfinite_rejected():
    w = np.zeros(128, dtype=np.float32)
    w[77] = np.inf
    with pytest.raises(ValueError):
        oracle.quantize(w, "f32", 4)


def test_bf16_widening():
    bits16 = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x4049], dtype=np.uint16)
    f = oracle.widen(bits16, "bf16")
    assert f.tolist()[:4] == [1.0, -1.0, 0.0, -0.0] and abs(f[4] - 3.140625) == 0


def _round_f32_signed(q: Fraction) -> float:
    """Round any rational to float32 (nearest, ties even): round-to-nearest is symmetric in sign."""
    if q < 0:
        return -_round_f32_fraction(-q)
    return _round_f32_fraction(q)


@pytest.mark.parametrize("bits", BITS)
def test_dequantize_two_roundings(bits):
    """Dequantization is fl32(L[c] * fl32(m * s)): two float32 roundings in that order (QLoRA page,
    "2. Double Quantization": the block constant is dequantized first, then scales the level).

    Steps with 24 significant bits make m * s inexact, so a single rounding fl32(L * m * s) differs on
    some elements; the reference is built from exact rationals, independently of numpy's float32.
    """
    rng = np.random.default_rng(300 + bits)
    L = oracle.quantile_codebook(bits)
    nblk = 256 * 2
    step = np.array([np.float32((int(rng.integers(1 << 23, 1 << 24)) | 1) * 2.0 ** -30) for _ in range(2)],
                    dtype=np.float32)
    q8 = rng.integers(0, 256, size=nblk).astype(np.uint8)
    codes = rng.integers(0, 1 << bits, size=(nblk, 64)).astype(np.uint8)
    packed = Q.pack_codes(codes, bits)
    got_a = Q.dequantize_scales(q8, step)
    got_w = oracle.dequantize(packed, q8, step, bits, nblk * 64).reshape(nblk, 64)
    differs = 0
    for j in range(nblk):
        s = Fraction(float(step[j // 256]))
        a1 = _round_f32_fraction(int(q8[j]) * s)
        assert float(got_a[j]) == a1, j
        for e in range(0, 64, 5 if bits == 8 else 3):
            lv = Fraction(float(L[codes[j, e]]))
            two = _round_f32_signed(lv * Fraction(a1))
            one = _round_f32_signed(lv * int(q8[j]) * s)
            assert float(got_w[j, e]) == two, (j, e)
            differs += two != one
    assert differs > 0  # the sample tells the two orders apart
