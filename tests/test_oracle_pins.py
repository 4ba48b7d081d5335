"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test checks one oracle step against something other than its own code:
hand-worked fixtures, exact rational arithmetic, an integer special case, a
library fp64 product, or exhaustive enumeration.  A dropped term, a wrong
sign, a transposed operand or a wrong group index fails at least one of them.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from conftest import read_golden

# ----------------------------------------------------------------------------
# Unpack: the AWQ nibble order
# ----------------------------------------------------------------------------


def test_unpack_matches_hand_worked_words():
    rows = read_golden("awq_nibble_order.txt")
    words = np.array([[int(r[0], 16)] for r in rows], dtype=np.uint32)
    expect = np.array([[int(v) for v in r[1:]] for r in rows], dtype=np.uint8)
    assert np.array_equal(oracle.unpack_w4(words), expect)


def test_pack_unpack_bijection_random_words():
    rng = np.random.default_rng(1)
    words = rng.integers(0, 2**32, size=(37, 11), dtype=np.uint64).astype(np.uint32)
    codes = oracle.unpack_w4(words)
    assert codes.max() <= 15
    assert np.array_equal(oracle.pack_w4(codes), words)


def test_generator_packer_and_oracle_unpacker_agree():
    # synth packs with its own constant; the oracle unpacks with its own.
    rng = np.random.default_rng(2)
    codes = rng.integers(0, 16, size=(19, 64), dtype=np.uint8)
    assert np.array_equal(oracle.unpack_w4(synth.pack_awq_w4(codes)), codes)


# ----------------------------------------------------------------------------
# bf16 rounding
# ----------------------------------------------------------------------------


def test_bf16_rounding_hand_worked_values():
    rows = read_golden("bf16_rne.txt")
    vals = np.array([float.fromhex(r[0]) for r in rows])
    expect = np.array([int(r[1], 16) for r in rows], dtype=np.uint16)
    got = oracle.f64_to_bf16(vals)
    assert [hex(v) for v in got] == [hex(v) for v in expect]


def _rne_bf16_exact(v: float) -> int:
    """Round with exact rationals: nearest of the two neighbouring bf16 values."""
    fr = Fraction(v)
    sign = 0x8000 if (v < 0 or (v == 0 and np.signbit(v))) else 0
    a = abs(fr)
    if a == 0:
        return sign
    e = 0
    while a >= 2 ** (e + 1):
        e += 1
    while a < 2 ** e:
        e -= 1
    q = Fraction(2) ** max(e - 7, -133)
    n = a / q
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    r = lo * q
    if r >= 2**128:
        return sign | 0x7F80
    f = np.array([float(r)], dtype=np.float32).view(np.uint32)[0]
    return sign | int(f >> 16)


def test_bf16_rounding_against_exact_rationals():
    rng = np.random.default_rng(3)
    # values built to sit on and next to rounding ties, across many binades
    base = rng.integers(0, 2**8, size=400) * 2 + 1                  # odd: exact ties at 9 bits
    exps = rng.integers(-140, 120, size=400)
    ties = np.ldexp(base.astype(np.float64) + 256 * 2, exps - 9)    # 9-significant-bit values
    nudged = ties * (1 + rng.choice([-1, 1], size=400) * 2.0**-40)
    randoms = rng.standard_normal(400) * np.exp2(rng.integers(-60, 60, size=400))
    vals = np.concatenate([ties, nudged, randoms, -ties])
    got = oracle.f64_to_bf16(vals)
    want = np.array([_rne_bf16_exact(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, want)


def test_bf16_rounding_matches_torch_on_fp32_inputs():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(4)
    f = (rng.standard_normal(20000) * np.exp2(rng.integers(-30, 30, 20000))).astype(np.float32)
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f64_to_bf16(f.astype(np.float64)), want)


# ----------------------------------------------------------------------------
# fp16 (IEEE binary16): the format of the scales and activations of many AWQ
# checkpoints
# ----------------------------------------------------------------------------


def test_f16_decode_exhaustive_matches_numpy():
    # every one of the 65536 bit patterns against numpy's own float16
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_to_f32(b)
    want = b.view(np.float16).astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))  # signed zeros too


def test_f16_rounding_hand_worked_values():
    rows = read_golden("f16_rne.txt")
    vals = np.array([float.fromhex(r[0]) for r in rows])
    expect = np.array([int(r[1], 16) for r in rows], dtype=np.uint16)
    got = oracle.f64_to_f16(vals)
    assert [hex(v) for v in got] == [hex(v) for v in expect]


def _rne_f16_exact(v: float) -> int:
    """Round with exact rationals to the nearest fp16 value (ties to even);
    encode it with numpy (exact, the value has <= 11 significant bits)."""
    fr = Fraction(v)
    neg = v < 0 or (v == 0 and np.signbit(v))
    a = abs(fr)
    if a == 0:
        return 0x8000 if neg else 0
    e = 0
    while a >= 2 ** (e + 1):
        e += 1
    while a < 2 ** e:
        e -= 1
    q = Fraction(2) ** max(e - 10, -24)
    n = a / q
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    r = lo * q
    if r >= 2**16:
        return 0xFC00 if neg else 0x7C00
    h = np.array([float(r)], dtype=np.float64).astype(np.float16).view(np.uint16)[0]
    return int(h) | (0x8000 if neg else 0)


def test_f16_rounding_against_exact_rationals():
    rng = np.random.default_rng(33)
    base = rng.integers(0, 2**11, size=400) * 2 + 1                 # odd: exact ties at 12 bits
    exps = rng.integers(-30, 16, size=400)
    ties = np.ldexp(base.astype(np.float64) + 2**11 * 2, exps - 12)  # 12-significant-bit values
    nudged = ties * (1 + rng.choice([-1, 1], size=400) * 2.0**-40)
    randoms = rng.standard_normal(400) * np.exp2(rng.integers(-28, 17, size=400))
    vals = np.concatenate([ties, nudged, randoms, -ties])
    got = oracle.f64_to_f16(vals)
    want = np.array([_rne_f16_exact(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, want)


def test_f16_rounding_matches_numpy_on_doubles():
    rng = np.random.default_rng(34)
    v = rng.standard_normal(50000) * np.exp2(rng.integers(-30, 18, 50000))
    assert np.array_equal(oracle.f64_to_f16(v), v.astype(np.float16).view(np.uint16))


def _all_finite_f16_patterns():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return b[np.isfinite(b.view(np.float16))]


def test_dequant_w8_f16_scales_exhaustive_exactness():
    # Every finite fp16 scale times every difference q - z in [-255, 255]:
    # 8 + 11 significant bits fit fp32's 24, so the fp32 product is exact.
    sb = _all_finite_f16_patterns()
    d = np.arange(-255, 256)
    K, N, G = d.size, sb.size, 1
    q = np.maximum(d, 0).astype(np.uint8)
    z = np.maximum(-d, 0).astype(np.uint8)
    qweight = np.repeat(q[:, None], N, axis=1)
    zeros = np.repeat(z[:, None], N, axis=1)
    scales = np.repeat(sb[None, :], K, axis=0)
    w = oracle.dequant(8, qweight, zeros, scales, K, N, G, dtype="f16")
    exact = d[:, None].astype(np.float64) * sb.view(np.float16).astype(np.float64)[None, :]
    assert np.array_equal(w.astype(np.float64), exact)


def test_dequant_w4_f16_scales_exhaustive_exactness():
    sb = _all_finite_f16_patterns()
    qz = np.array([(q, z) for q in range(16) for z in range(16)])
    K, N = qz.shape[0], 64
    sbs = sb[: (sb.size // N) * N].reshape(-1, N)
    for chunk in np.array_split(np.arange(sbs.shape[0]), 8):
        s = sbs[chunk]
        R = s.shape[0]
        codes = np.tile(np.repeat(qz[:, 0:1], N, axis=1), (R, 1)).astype(np.uint8)
        zeros = np.tile(np.repeat(qz[:, 1:2], N, axis=1), (R, 1)).astype(np.uint8)
        scales = np.repeat(s, K, axis=0)
        w = oracle.dequant(4, synth.pack_awq_w4(codes), synth.pack_awq_w4(zeros), scales, R * K, N, 1,
                           dtype="f16")
        exact = (codes.astype(np.float64) - zeros) * scales.view(np.float16).astype(np.float64)
        assert np.array_equal(w.astype(np.float64), exact)


# ----------------------------------------------------------------------------
# Dequantization: (q - z) * s in fp32 is exact
# ----------------------------------------------------------------------------


def _all_finite_bf16_patterns():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = synth.bf16_bits_to_f32(b)
    return b[np.isfinite(f)]


def test_dequant_w8_exhaustive_exactness():
    # Every finite bf16 scale times every difference q - z in [-255, 255].
    sb = _all_finite_bf16_patterns()
    d = np.arange(-255, 256)
    K, N, G = d.size, sb.size, 1
    q = np.maximum(d, 0).astype(np.uint8)
    z = np.maximum(-d, 0).astype(np.uint8)
    qweight = np.repeat(q[:, None], N, axis=1)
    zeros = np.repeat(z[:, None], N, axis=1)
    scales = np.repeat(sb[None, :], K, axis=0)
    w = oracle.dequant(8, qweight, zeros, scales, K, N, G)
    exact = d[:, None].astype(np.float64) * synth.bf16_bits_to_f32(sb)[None, :].astype(np.float64)
    finite = np.abs(exact) <= np.finfo(np.float32).max
    assert np.array_equal(w[finite].astype(np.float64), exact[finite])
    assert np.all(np.isinf(w[~finite]))


def test_dequant_w4_exhaustive_exactness():
    sb = _all_finite_bf16_patterns()
    qz = np.array([(q, z) for q in range(16) for z in range(16)])
    K, N = qz.shape[0], 64
    sbs = sb[: (sb.size // N) * N].reshape(-1, N)
    for chunk in np.array_split(np.arange(sbs.shape[0]), 8):
        s = sbs[chunk]                                   # [R][N] scales
        R = s.shape[0]
        # row k = (r, pair) ; G = 1 so every row has its own zero/scale
        codes = np.tile(np.repeat(qz[:, 0:1], N, axis=1), (R, 1)).astype(np.uint8)
        zeros = np.tile(np.repeat(qz[:, 1:2], N, axis=1), (R, 1)).astype(np.uint8)
        scales = np.repeat(s, K, axis=0)
        w = oracle.dequant(4, synth.pack_awq_w4(codes), synth.pack_awq_w4(zeros), scales,
                           R * K, N, 1)
        exact = ((codes.astype(np.float64) - zeros) * synth.bf16_bits_to_f32(scales).astype(np.float64))
        finite = np.abs(exact) <= np.finfo(np.float32).max
        assert np.array_equal(w[finite].astype(np.float64), exact[finite])


def test_dequant_group_index_and_column_selection():
    c = synth.make_inputs(4, 1, 96, 24, 32, seed=(5,))
    w_all = oracle.dequant(4, c.qweight, c.qzeros, c.scales, c.K, c.N, c.G)
    s = synth.bf16_bits_to_f32(c.scales).astype(np.float64)
    k = np.arange(c.K)
    expect = (c.codes.astype(np.float64) - c.zeros[k // c.G]) * s[k // c.G]
    assert np.array_equal(w_all.astype(np.float64), expect)
    cols = np.array([23, 0, 7, 8, 16])
    w_sel = oracle.dequant(4, c.qweight, c.qzeros, c.scales, c.K, c.N, c.G, cols=cols)
    assert np.array_equal(w_sel, w_all[:, cols])


# ----------------------------------------------------------------------------
# Linear: brute force, special cases, library product, scaling
# ----------------------------------------------------------------------------


def _exact_y(c):
    """Exact rational y[m][n] from the definition, for tiny cases."""
    xs = [[Fraction(float(v)) for v in row] for row in synth.bf16_bits_to_f32(c.x)]
    ss = [[Fraction(float(v)) for v in row] for row in synth.bf16_bits_to_f32(c.scales)]
    y = []
    for m in range(c.M):
        row = []
        for n in range(c.N):
            acc = Fraction(0)
            for k in range(c.K):
                g = k // c.G
                acc += xs[m][k] * (int(c.codes[k, n]) - int(c.zeros[g, n])) * ss[g][n]
            row.append(acc)
        y.append(row)
    return y


@pytest.mark.parametrize("bits,M,K,N,G,seed", [
    (4, 1, 32, 8, 32, 11), (4, 3, 64, 16, 32, 12), (4, 2, 64, 16, 64, 13),
    (8, 1, 32, 8, 32, 14), (8, 3, 64, 12, 64, 15), (8, 2, 64, 16, 16, 16),
])
def test_linear_tiny_against_exact_rationals(bits, M, K, N, G, seed):
    c = synth.make_inputs(bits, M, K, N, G, seed=(seed,))
    y64 = oracle.awq_linear(c)
    exact = _exact_y(c)
    # fp64 holds these sums exactly (<= 64 terms of <= 24 significant bits
    # spanning well under 53 bits), so equality is exact
    for m in range(M):
        for n in range(N):
            assert Fraction(float(y64[m, n])) == exact[m][n]
    got_bf16 = oracle.f64_to_bf16(y64)
    want_bf16 = np.array([[_rne_bf16_exact(float(exact[m][n])) for n in range(N)] for m in range(M)])
    assert np.array_equal(got_bf16, want_bf16.astype(np.uint16))


@pytest.mark.parametrize("bits", [4, 8])
def test_linear_q_equals_zero_gives_zero(bits):
    c = synth.make_inputs(bits, 4, 256, 48, 64, seed=(21,))
    codes = c.zeros[np.arange(c.K) // c.G]
    cz = synth.gen.pack_case(bits, codes, c.zeros, c.scales, c.x, c.G)
    y = oracle.awq_linear(cz)
    assert np.all(y == 0.0)


@pytest.mark.parametrize("bits,K", [(4, 1024), (8, 512)])
def test_linear_unit_scale_reduces_to_integer_gemm(bits, K):
    rng = np.random.default_rng(22)
    M, N, G = 5, 64, 128
    codes = rng.integers(0, 1 << bits, size=(K, N), dtype=np.uint8)
    zval = 8 if bits == 4 else 128
    zeros = np.full((K // G, N), zval, dtype=np.uint8)
    scales = np.full((K // G, N), 0x3F80, dtype=np.uint16)       # bf16 1.0
    xi = rng.integers(-2, 3, size=(M, K))
    x = synth.f32_to_bf16_bits(xi.astype(np.float32))
    c = synth.gen.pack_case(bits, codes, zeros, scales, x, G)
    y = oracle.awq_linear(c)
    want = xi.astype(np.int64) @ (codes.astype(np.int64) - zval)
    assert np.array_equal(y, want.astype(np.float64))


@pytest.mark.parametrize("bits,K", [(4, 1024), (8, 512)])
def test_linear_f16_unit_scale_reduces_to_integer_gemm(bits, K):
    rng = np.random.default_rng(27)
    M, N, G = 5, 64, 128
    codes = rng.integers(0, 1 << bits, size=(K, N), dtype=np.uint8)
    zval = 8 if bits == 4 else 128
    zeros = np.full((K // G, N), zval, dtype=np.uint8)
    scales = np.full((K // G, N), 0x3C00, dtype=np.uint16)       # fp16 1.0
    xi = rng.integers(-2, 3, size=(M, K))
    x = xi.astype(np.float16).view(np.uint16)
    c = synth.gen.pack_case(bits, codes, zeros, scales, x, G, dtype="f16")
    y = oracle.awq_linear(c)
    want = xi.astype(np.int64) @ (codes.astype(np.int64) - zval)
    assert np.array_equal(y, want.astype(np.float64))


@pytest.mark.parametrize("bits,M,K,N,G,seed", [(4, 2, 64, 16, 32, 41), (8, 3, 64, 8, 64, 42)])
def test_linear_f16_tiny_against_exact_rationals(bits, M, K, N, G, seed):
    c = synth.make_inputs(bits, M, K, N, G, seed=(seed,), dtype="f16")
    y64 = oracle.awq_linear(c)
    xs = [[Fraction(float(v)) for v in row] for row in c.x.view(np.float16)]
    q = c.codes.astype(int)
    z = c.zeros.astype(int)
    s = c.scales.view(np.float16)
    for m in range(M):
        for n in range(N):
            e = sum(xs[m][k] * (q[k, n] - z[k // G, n]) * Fraction(float(s[k // G, n])) for k in range(K))
            assert Fraction(float(y64[m, n])) == e
            assert int(oracle.f64_to_f16(np.array([y64[m, n]]))[0]) == _rne_f16_exact(float(e))


def test_linear_f16_and_bf16_agree_where_the_values_coincide():
    # x and scales with at most 8 significant bits inside fp16's normal range
    # are the same numbers in both formats: the two decodings must give the
    # same fp64 sums, bit for bit.
    rng = np.random.default_rng(43)
    M, K, N, G = 3, 256, 40, 64
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    zeros = rng.integers(0, 16, size=(K // G, N), dtype=np.uint8)
    xv = np.ldexp(rng.integers(-255, 256, size=(M, K)).astype(np.float64), rng.integers(-12, 0, size=(M, K)))
    sv = np.ldexp(rng.integers(128, 256, size=(K // G, N)).astype(np.float64), rng.integers(-14, -6, size=(K // G, N)))
    cb = synth.gen.pack_case(4, codes, zeros, synth.f32_to_bf16_bits(sv), synth.f32_to_bf16_bits(xv), G)
    ch = synth.gen.pack_case(4, codes, zeros, synth.f32_to_f16_bits(sv), synth.f32_to_f16_bits(xv), G, dtype="f16")
    assert np.array_equal(synth.bf16_bits_to_f32(cb.x), ch.x.view(np.float16).astype(np.float32))
    yb, yh = oracle.awq_linear(cb), oracle.awq_linear(ch)
    assert np.any(yb != 0) and np.array_equal(yb, yh)


def test_per_channel_equals_repeated_group_metadata():
    # G = K (one scale/zero per column) must equal G = 32 with that metadata repeated.
    c = synth.make_inputs(8, 3, 256, 40, 256, seed=(23,))
    y_pc = oracle.awq_linear(c)
    reps = c.K // 32
    c32 = synth.gen.pack_case(8, c.codes, np.repeat(c.zeros, reps, axis=0),
                              np.repeat(c.scales, reps, axis=0), c.x, 32)
    assert np.array_equal(oracle.awq_linear(c32), y_pc)


@pytest.mark.parametrize("bits,M,K,N,G", [(4, 4, 512, 96, 128), (8, 2, 256, 64, 256)])
def test_linear_matches_library_fp64_product(bits, M, K, N, G):
    c = synth.make_inputs(bits, M, K, N, G, seed=(24,))
    y = oracle.awq_linear(c)
    w = oracle.dequant(bits, c.qweight, c.qzeros, c.scales, K, N, G).astype(np.float64)
    ref = synth.bf16_bits_to_f32(c.x).astype(np.float64) @ w
    rms = np.sqrt(np.mean(ref**2, axis=1, keepdims=True))
    assert np.all(np.abs(y - ref) <= 1e-12 * np.maximum(np.abs(ref), rms))


def test_linear_scales_with_power_of_two_inputs():
    c = synth.make_inputs(4, 2, 256, 32, 128, seed=(25,))
    y = oracle.awq_linear(c)
    x4 = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(c.x) * np.float32(4.0))
    c4 = synth.gen.pack_case(4, c.codes, c.zeros, c.scales, x4, c.G)
    assert np.array_equal(oracle.awq_linear(c4), 4.0 * y)


def test_linear_sampled_rows_and_columns_match_full():
    c = synth.make_inputs(4, 6, 256, 128, 128, seed=(26,))
    y = oracle.awq_linear(c)
    rows, cols = np.array([5, 0, 3]), np.array([127, 1, 64, 9])
    assert np.array_equal(oracle.awq_linear(c, cols=cols, rows=rows), y[rows][:, cols])


# ----------------------------------------------------------------------------
# SiLU product of a fused [gate | up] layer
# ----------------------------------------------------------------------------


def test_silu_closed_forms():
    # sigmoid(ln k) = k / (k + 1), so silu(ln k) = ln k * k / (k + 1)
    ks = np.array([3.0, 1.0 / 3.0, 7.0, 1.0])
    g = np.log(ks)
    got = oracle.silu_mul(g, np.ones_like(g))
    want = g * ks / (ks + 1.0)
    assert np.all(np.abs(got - want) <= 4e-16 * np.abs(want) + 1e-300)
    # the limits: silu(v) -> v as v -> +inf, -> -0 as v -> -inf, with no NaN
    far = oracle.silu_mul(np.array([800.0, -800.0, 40.0]), np.ones(3))
    assert far[0] == 800.0 and far[1] == 0.0 and np.signbit(far[1]) and far[2] == 40.0


def test_silu_mul_scales_the_up_operand_only():
    # silu(ln 3) * 2 is 1.5 ln 3; swapping the operands would give silu(2) ln 3
    got = oracle.silu_mul(np.array([np.log(3.0)]), np.array([2.0]))
    assert abs(got[0] - 1.5 * np.log(3.0)) <= 4e-16 * got[0]
    rng = np.random.default_rng(41)
    g, u = rng.normal(0, 4, 64), rng.normal(0, 4, 64)
    assert np.array_equal(oracle.silu_mul(g, u), oracle.silu_mul(g, np.ones(64)) * u)


def test_silu_matches_tanh_form():
    # sigmoid(v) = (1 + tanh(v / 2)) / 2: a second route through a library routine
    v = np.random.default_rng(42).uniform(-30, 30, 4096)
    want = v * (1.0 + np.tanh(v / 2.0)) / 2.0
    got = oracle.silu_mul(v, np.ones_like(v))
    # at large negative v, 1 + tanh(v / 2) cancels: that form is good to
    # about eps * |v| there, absolutely
    assert np.all(np.abs(got - want) <= 1e-14 * np.abs(want) + 1e-15 * np.abs(v))


@pytest.mark.parametrize("bits", [4, 8])
def test_silu_mul_pairs_column_n_with_n_plus_half(bits):
    # gate columns 0..7, up columns 8..15; exact sums from the definition
    c = synth.make_inputs(bits, 2, 64, 16, 32, seed=(43, bits))
    exact = _exact_y(c)
    got = oracle.awq_linear_silu_mul(c)
    assert got.shape == (2, 8)
    for m in range(2):
        for n in range(8):
            g, u = float(exact[m][n]), float(exact[m][n + 8])
            want = g * (1.0 + np.tanh(g / 2.0)) / 2.0 * u
            assert abs(got[m, n] - want) <= 1e-13 * max(abs(want), 1e-30)
    # sampled rows and columns agree with the full result
    sub = oracle.awq_linear_silu_mul(c, cols=np.array([7, 0, 3]), rows=np.array([1]))
    assert np.array_equal(sub, got[[1]][:, [7, 0, 3]])
