"""Pins for the CPU oracle: each check rests on something other than the
oracle's own formulas.

* torch's float8_e4m3fn dtype: an independent implementation of the OCP E4M3
  format (decode of all 256 codes; round-to-nearest-even cast of in-range
  values).
* brute-force nearest search over all E4M3 values in exact rational
  arithmetic (Python ``fractions``), ties resolved to the even code.
* hand-worked 32-element blocks (derivations in the comments).
* closed forms and invariants: the scale characterisation
  2^8 <= amax * 2^-X < 2^9, exact round trips of small integers and powers
  of two, the round-trip error bound, scale invariance, transposition.
* exact integer arithmetic for dbias and the GEMM.
"""

import math
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def bf16_bits(values):
    """Exact float values (representable in BF16) -> BF16 bit patterns."""
    f = np.asarray(values, dtype=np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(((bits.astype(np.uint32)) << 16).view(np.float32), f), "not exact in BF16"
    return bits


def block_row(values):
    """One 32-element rowwise block (rest zero) as a [1, 32] BF16 array."""
    v = list(values) + [0.0] * (32 - len(values))
    return bf16_bits(np.array(v, dtype=np.float64).reshape(1, 32))


# ----------------------------------------------------------- E4M3 / E8M0

def torch_e4m3_values():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_decode_matches_torch_for_all_codes():
    ours = oracle.e4m3_decode(np.arange(256))
    ref = torch_e4m3_values()
    nan_o, nan_r = np.isnan(ours), np.isnan(ref)
    assert np.array_equal(nan_o, nan_r)
    assert list(np.nonzero(nan_o)[0]) == [0x7F, 0xFF]
    assert np.array_equal(ours[~nan_o], ref[~nan_r])
    # signed zero is kept as a distinct code
    assert math.copysign(1.0, ours[0x80]) == -1.0


def test_e4m3_landmarks():
    d = oracle.e4m3_decode
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert d(0x08) == 2.0 ** -6          # smallest normal
    assert d(0x01) == 2.0 ** -9          # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert d(0x38) == 1.0
    pos = oracle.e4m3_decode(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0)      # codes 0..0x7E are strictly increasing
    assert np.isfinite(oracle.e4m3_decode(np.arange(256))).sum() == 254


def test_e8m0_decode_is_the_shifted_exponent():
    # "frost(gemm): Add Rubin kernel pipelines", ue8m0 readback nitpick: the
    # byte shifted into the fp32 exponent field is the scale value.
    for b in range(1, 255):
        as_f32 = np.array([b << 23], dtype=np.uint32).view(np.float32)[0]
        assert oracle.e8m0_decode(b) == float(as_f32)
    # Byte 0: OCP gives 2^-127 (the page's readback would give 0.0).
    assert oracle.e8m0_decode(0) == 2.0 ** -127
    assert np.isnan(oracle.e8m0_decode(255))


POS_CODES = [(c, Fraction(float(v))) for c, v in enumerate(torch_e4m3_values()[:0x7F])]


def brute_force_encode(v: Fraction, negative: bool) -> int:
    """Nearest E4M3 value by exhaustive search; ties go to the even code;
    magnitudes from 448 up saturate to 448; the sign bit is always kept."""
    a = abs(v)
    if a >= 448:
        code = 0x7E
    else:
        best = None
        for c, val in POS_CODES:
            d = abs(val - a)
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                best = (d, c)
        code = best[1]
    return code | (0x80 if negative else 0)


def _encode_cases():
    vals = []
    pos = [float(v) for _, v in POS_CODES]
    for a, b in zip(pos[:-1], pos[1:]):
        mid = (a + b) / 2
        vals += [a, mid, math.nextafter(mid, 0.0), math.nextafter(mid, 1e9), b]
    vals += [447.0, 448.0, 449.0, 463.0, 464.0, 465.0, 479.0, 480.0, 500.0, 511.0, 1e30]
    vals += [2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -11, 2.0 ** -40, 0.0]
    rng = random.Random(7)
    for _ in range(3000):
        vals.append(rng.uniform(0, 512) * 2.0 ** rng.randint(-12, 0))
    out = []
    for v in vals:
        out += [v, -v]
    out.append(-0.0)
    return out


def test_e4m3_encode_matches_brute_force_nearest_even():
    cases = _encode_cases()
    got = oracle.e4m3_encode(np.array(cases))
    for v, g in zip(cases, got):
        want = brute_force_encode(Fraction(v), math.copysign(1.0, v) < 0)
        assert int(g) == want, (v, hex(int(g)), hex(want))


def test_e4m3_encode_matches_torch_cast_on_all_bf16_scalings():
    # Every finite BF16 pattern, scaled by powers of two; torch's cast is RNE
    # and agrees with saturation wherever |v| <= 448.
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]
    x = oracle.bf16_value(bits)
    for k in (-133, -127, -100, -40, -9, -6, 0, 3, 8, 40, 119, 127):
        v = np.ldexp(x, k)
        with np.errstate(over="ignore"):
            f32 = v.astype(np.float32)
        keep = np.isfinite(f32) & (np.abs(v) <= 448.0) & (f32.astype(np.float64) == v)
        ours = oracle.e4m3_encode(v[keep])
        ref = torch.from_numpy(f32[keep]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(ours, ref), k
        # out of range: saturation keeps the sign
        big = np.abs(v) > 448.0
        if big.any():
            sat = oracle.e4m3_encode(v[big])
            assert np.all((sat & 0x7F) == 0x7E)
            assert np.array_equal(sat >> 7, (v[big] < 0).astype(np.uint8))


# ----------------------------------------------------- hand-worked blocks

# Each row: block values (rest of the 32 are zero), expected scale byte,
# expected codes of the listed values, expected dequantized values.
WORKED = [
    # amax 5 -> floor(log2 5) = 2 -> X = -6 -> byte 121.  x*64: 64 -> 1.0*2^6;
    # -0.30078125*64 = -19.25 -> 10*2 = 20 (0xDA); 160 = 1.25*2^7; 192 = 1.5*2^7;
    # 2^-4 = 1.0*2^-4 (exp field 3); 320 = 1.25*2^8.
    ([1.0, -0.30078125, 2.5, 0.0, 3.0, 2.0 ** -10, 5.0], 0x79,
     [0x68, 0xDA, 0x72, 0x00, 0x74, 0x18, 0x7A],
     [1.0, -0.3125, 2.5, 0.0, 3.0, 2.0 ** -10, 5.0]),
    # amax 7.5 -> X = -6; 7.5*64 = 480 saturates to 448 -> 7.0.
    ([7.5, 1.0], 0x79, [0x7E, 0x68], [7.0, 1.0]),
    # amax 500 -> floor(log2) = 8 -> X = 0 -> byte 127; 448 exact; 500 saturates.
    ([448.0, 1.0, 500.0], 0x7F, [0x7E, 0x38, 0x7E], [448.0, 1.0, 448.0]),
    # amax 1 -> X = -8 -> byte 119; x*256: 2^-8 -> 2 * 2^-9; 2^-10 is a tie
    # between 0 and 2^-9 -> even (0); 3*2^-11 = 0.75 * 2^-9 -> 1 * 2^-9.
    ([1.0, 2.0 ** -16, 2.0 ** -18, 3 * 2.0 ** -19], 0x77,
     [0x78, 0x02, 0x00, 0x01], [1.0, 2.0 ** -16, 0.0, 2.0 ** -17]),
    # all-subnormal block: 2^-130 -> X = -138 clamps to -127 (byte 0);
    # 2^-130 * 2^127 = 2^-3 (exp field 4) -> dequantizes exactly.
    ([2.0 ** -130] * 32, 0x00, [0x20] * 32, [2.0 ** -130] * 32),
    # all zero -> byte 0
    ([0.0] * 32, 0x00, [0x00] * 32, [0.0] * 32),
]


@pytest.mark.parametrize("case", range(len(WORKED)))
def test_worked_block(case):
    vals, byte, codes, deq = WORKED[case]
    x = block_row(vals)
    q, s = oracle.quantize_rowwise(x)
    assert s[0, 0] == byte
    assert list(q[0, :len(codes)]) == codes
    assert np.all(q[0, len(vals):] == 0)
    d = oracle.dequantize(q, s)[0, :len(deq)]
    assert list(d) == deq


def test_worked_block_max_bf16():
    # max BF16 = (2 - 2^-7) * 2^127 -> floor(log2) = 127 -> X = 119 -> byte 246;
    # scaled value 510 saturates to 448 -> 448 * 2^119; 1.0 * 2^-119 -> +0.
    x = np.zeros((1, 32), dtype=np.uint16)
    x[0, 0] = workloads.BF16_MAX_BITS
    x[0, 1:] = 0x3F80
    q, s = oracle.quantize_rowwise(x)
    assert s[0, 0] == 0xF6
    assert q[0, 0] == 0x7E and np.all(q[0, 1:] == 0)
    assert oracle.dequantize(q, s)[0, 0] == 448.0 * 2.0 ** 119


def test_signed_zero_and_negative_underflow_keep_sign():
    x = block_row([-0.0, 1.0, -(2.0 ** -20), 2.0 ** -20])
    q, s = oracle.quantize_rowwise(x)
    assert s[0, 0] == 0x77
    assert q[0, 0] == 0x80 and q[0, 2] == 0x80 and q[0, 3] == 0x00
    xz = block_row([-0.0])
    qz, sz = oracle.quantize_rowwise(xz)
    assert sz[0, 0] == 0 and qz[0, 0] == 0x80


def test_scaled_tie_encodings():
    # encoder on pre-scaled values: ties to even at both ends of the range
    v = np.array([2.0 ** -10, 3 * 2.0 ** -10, 17.0, 19.0, 464.0, 465.0, 240.0, 248.0])
    assert list(oracle.e4m3_encode(v)) == [0x00, 0x02, 0x58, 0x5A, 0x7E, 0x7E, 0x77, 0x78]


# --------------------------------------------------- closed-form invariants

def _random_blocks(n, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 32)).astype(np.float32)
    x *= np.ldexp(np.float32(1), rng.integers(-140, 120, size=(n, 1))).astype(np.float32)
    bits = workloads.f32_to_bf16_bits(x)
    bits[(bits & 0x7F80) == 0x7F80] = 0x3F80
    sub = rng.random((n, 32)) < 0.05
    bits[sub] = (rng.integers(0, 2, sub.sum()).astype(np.uint16) << 15) | \
        rng.integers(0, 128, sub.sum()).astype(np.uint16)
    bits[rng.random(n) < 0.02] = 0
    return bits


def test_scale_characterisation():
    bits = _random_blocks(20000, 1)
    q, s = oracle.quantize_rowwise(bits)
    x = oracle.bf16_value(bits)
    amax = np.abs(x).max(axis=1)
    X = s[:, 0].astype(np.int64) - 127
    scaled = np.ldexp(amax, -X)
    nz = amax > 0
    clamped = nz & (amax < 2.0 ** -119)
    free = nz & ~clamped
    assert np.all((scaled[free] >= 256) & (scaled[free] < 512))
    assert np.all(s[clamped, 0] == 0) and np.all(scaled[clamped] < 256)
    assert np.all(s[~nz, 0] == 0)
    assert clamped.sum() > 0 and free.sum() > 0 and (~nz).sum() > 0


def test_round_trip_bound():
    bits = _random_blocks(20000, 2)
    q, s = oracle.quantize_rowwise(bits)
    x = oracle.bf16_value(bits)
    d = oracle.dequantize(q, s)
    X = np.repeat(s.astype(np.int64) - 127, 32, axis=1)
    v = np.ldexp(np.abs(x), -X)                 # scaled magnitude
    err = np.abs(x - d)
    sat = v >= 448
    normal = (v >= 2.0 ** -6) & ~sat
    sub = (v < 2.0 ** -6)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(normal, np.abs(x), 1.0)))
    assert np.all(err[normal] <= np.ldexp(1.0, (e[normal] - 4).astype(np.int64)))
    assert np.all(err[sub] <= np.ldexp(1.0, X[sub] - 10))
    assert np.all(np.abs(d[sat]) == np.ldexp(448.0, X[sat]))
    assert np.all(err[sat] < np.abs(x[sat]) / 8)
    assert np.array_equal(np.signbit(d), np.signbit(x))


def test_small_integers_and_powers_of_two_round_trip_exactly():
    rng = np.random.default_rng(3)
    for k in (-100, -20, 0, 7, 60, 110):
        ints = rng.integers(-14, 15, size=(64, 32)).astype(np.float64)
        ints[:, 0] = rng.choice([-14, 14, 9, -8, 1, 3], size=64)
        x = bf16_bits(np.ldexp(ints, k))
        q, s = oracle.quantize_rowwise(x)
        assert np.array_equal(oracle.dequantize(q, s), np.ldexp(ints, k))
        pw = np.ldexp(1.0, k - np.arange(18))
        xp = block_row(list(pw))
        qp, sp = oracle.quantize_rowwise(xp)
        assert np.array_equal(oracle.dequantize(qp, sp)[0, :18], pw)
    # 15 needs 480 at the chosen scale and saturates to 14
    q, s = oracle.quantize_rowwise(block_row([15.0, 1.0]))
    assert oracle.dequantize(q, s)[0, 0] == 14.0
    # 2^-18 below the top power sits on the 2^-10 tie and goes to zero
    q, s = oracle.quantize_rowwise(block_row([1.0, 2.0 ** -18]))
    assert q[0, 1] == 0


def test_scale_invariance():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((512, 64)).astype(np.float32)
    bits = workloads.f32_to_bf16_bits(x)
    q0, s0 = oracle.quantize_rowwise(bits)
    for k in (-30, -1, 1, 17, 60):
        bk = workloads.f32_to_bf16_bits(np.ldexp(oracle.bf16_value(bits), k).astype(np.float32))
        qk, sk = oracle.quantize_rowwise(bk)
        assert np.array_equal(qk, q0)
        assert np.array_equal(sk.astype(int), s0.astype(int) + k)


def test_colwise_is_rowwise_of_transpose():
    bits = workloads.wide_range_bf16((96, 160), 5, n_maxbf16=3, n_subnormal=40,
                                     n_subnormal_blocks=2)
    qT, sT = oracle.quantize_colwise(bits)
    qr, sr = oracle.quantize_rowwise(np.ascontiguousarray(bits.T))
    assert np.array_equal(qT, qr) and np.array_equal(sT, sr)
    assert qT.shape == (160, 96) and sT.shape == (160, 3)


def test_quantize_block_by_brute_force():
    # whole-block check in exact rationals: X is the unique integer with
    # 2^8 <= amax * 2^-X < 2^9 (clamped to >= -127), codes by nearest search
    bits = _random_blocks(300, 6)
    q, s = oracle.quantize_rowwise(bits)
    for i in range(bits.shape[0]):
        vals = [Fraction(float(v)) for v in oracle.bf16_value(bits[i])]
        amax = max(abs(v) for v in vals)
        if amax == 0:
            X = -127
            want_byte = 0
        else:
            X = -140
            while not (amax / Fraction(2) ** X < 512):
                X += 1
            X = max(X, -127)
            want_byte = X + 127
        assert s[i, 0] == want_byte
        for j, v in enumerate(vals):
            neg = bits[i, j] >> 15 == 1
            assert q[i, j] == brute_force_encode(v / Fraction(2) ** X, neg), (i, j)


def test_dbias_exact_on_integers():
    rng = np.random.default_rng(8)
    ints = rng.integers(-256, 257, size=(96, 64))
    x = bf16_bits(ints.astype(np.float64))
    got = oracle.dbias(x)
    want = ints.sum(axis=0)
    assert np.array_equal(got.astype(np.int64), want)


def test_dbias_is_rounded_once():
    # 2^24 followed by 4096 ones: the exact sum 2^24 + 4096 is a float32, but a
    # float32 running sum would stay at 2^24 (2^24 + 1 ties to even).
    col = np.ones(4097)
    col[0] = 2.0 ** 24
    x = bf16_bits(np.stack([col, -col], axis=1))
    got = oracle.dbias(x)
    assert got[0] == 2.0 ** 24 + 4096 and got[1] == -(2.0 ** 24 + 4096)


def test_dbias_matches_correctly_rounded_sum():
    bits = workloads.student_t_bf16((128, 64), 9)
    got = oracle.dbias(bits)
    x = oracle.bf16_value(bits)
    for c in range(64):
        exact = np.float32(math.fsum(x[:, c]))
        assert got[c] == exact


# ------------------------------------------------------------------ GEMM

def test_gemm_identity_gives_transposed_dequantized_b():
    a = bf16_bits(np.eye(256))
    b = workloads.normal_bf16((256, 256), 1)
    qa, sa = oracle.quantize_rowwise(a)
    qb, sb = oracle.quantize_rowwise(b)
    c = oracle.gemm_tn(qa, sa, qb, sb)
    assert np.array_equal(c, oracle.dequantize(qb, sb).T)


def test_gemm_all_ones():
    x = bf16_bits(np.ones((64, 256)))
    q, s = oracle.quantize_rowwise(x)
    assert np.all(oracle.gemm_tn(q, s, q, s) == 256.0)


def test_gemm_small_integers_exact():
    rng = np.random.default_rng(10)
    A = rng.integers(-14, 15, size=(96, 384))
    B = rng.integers(-14, 15, size=(64, 384))
    qa, sa = oracle.quantize_rowwise(bf16_bits(A.astype(np.float64)))
    qb, sb = oracle.quantize_rowwise(bf16_bits(B.astype(np.float64)))
    c = oracle.gemm_tn(qa, sa, qb, sb)
    assert np.array_equal(c, (A @ B.T).astype(np.float64))


def test_gemm_tiny_brute_force_rationals():
    rng = np.random.default_rng(11)
    M, N, K = 4, 5, 96
    qa = rng.integers(0, 256, size=(M, K)).astype(np.uint8)
    qb = rng.integers(0, 256, size=(N, K)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x30
    qb[(qb & 0x7F) == 0x7F] = 0x31
    sa = rng.integers(100, 150, size=(M, K // 32)).astype(np.uint8)
    sb = rng.integers(100, 150, size=(N, K // 32)).astype(np.uint8)
    vals = {c: Fraction(float(v)) for c, v in enumerate(torch_e4m3_values()) if not math.isnan(v)}
    c = oracle.gemm_tn(qa, sa, qb, sb)
    for m in range(M):
        for n in range(N):
            exact = sum(vals[int(qa[m, k])] * Fraction(2) ** (int(sa[m, k // 32]) - 127) *
                        vals[int(qb[n, k])] * Fraction(2) ** (int(sb[n, k // 32]) - 127)
                        for k in range(K))
            mag = sum(abs(vals[int(qa[m, k])] * vals[int(qb[n, k])]) *
                      Fraction(2) ** (int(sa[m, k // 32]) + int(sb[n, k // 32]) - 254)
                      for k in range(K))
            assert abs(Fraction(c[m, n]) - exact) <= mag * Fraction(K, 2 ** 52)


def test_gemm_row_panels_equal_the_whole_product():
    """Panel-wise evaluation gives the same entries (within the fp64 summation
    error bound), including a partial last panel, and exactly on integers."""
    qa, sa = oracle.quantize_rowwise(workloads.normal_bf16((200, 384), 16))
    qb, sb = oracle.quantize_rowwise(workloads.normal_bf16((72, 384), 17))
    whole = oracle.gemm_tn(qa, sa, qb, sb)
    mag = oracle.gemm_tn_abs(qa, sa, qb, sb)
    for panel in (64, 199, 1000):
        got = oracle.gemm_tn(qa, sa, qb, sb, panel=panel)
        assert got.shape == whole.shape
        assert np.all(np.abs(got - whole) <= mag * 2 * 384 * 2.0 ** -53)
    rng = np.random.default_rng(18)
    A = rng.integers(-14, 15, size=(130, 256))
    B = rng.integers(-14, 15, size=(40, 256))
    qa, sa = oracle.quantize_rowwise(bf16_bits(A.astype(np.float64)))
    qb, sb = oracle.quantize_rowwise(bf16_bits(B.astype(np.float64)))
    assert np.array_equal(oracle.gemm_tn(qa, sa, qb, sb, panel=32), (A @ B.T).astype(np.float64))


def test_gemm_scale_byte_doubles_one_row_block():
    rng = np.random.default_rng(12)
    qa = oracle.quantize_rowwise(workloads.normal_bf16((64, 256), 3))
    qb = oracle.quantize_rowwise(workloads.normal_bf16((32, 256), 4))
    base = oracle.gemm_tn(*qa, *qb)
    sa2 = qa[1].copy()
    sa2[5, :] += 1            # every block of row 5 scaled by 2
    c2 = oracle.gemm_tn(qa[0], sa2, *qb)
    assert np.array_equal(c2[5], 2 * base[5])
    assert np.array_equal(np.delete(c2, 5, 0), np.delete(base, 5, 0))
    _ = rng



def test_gemm_abs_equals_gemm_on_nonnegative_operands():
    """With every code's sign bit clear the terms are non-negative, so the
    size of the terms is the product itself (same dequantized operands)."""
    rng = np.random.default_rng(14)
    qa = rng.integers(0, 0x7F, size=(48, 256)).astype(np.uint8)      # 0x00..0x7E: non-negative, finite
    qb = rng.integers(0, 0x7F, size=(40, 256)).astype(np.uint8)
    sa = rng.integers(100, 150, size=(48, 8)).astype(np.uint8)
    sb = rng.integers(100, 150, size=(40, 8)).astype(np.uint8)
    assert np.array_equal(oracle.gemm_tn_abs(qa, sa, qb, sb), oracle.gemm_tn(qa, sa, qb, sb))
    rows, cols = np.array([3, 0, 47]), np.array([39, 5])
    sub = oracle.gemm_tn_abs(qa, sa, qb, sb, rows=rows, cols=cols)
    full = oracle.gemm_tn(qa, sa, qb, sb)[np.ix_(rows, cols)]
    # the sub-grid is summed by BLAS in another order: equal within fp64 summation error
    assert np.all(np.abs(sub - full) <= full * 256 * 2.0 ** -52)


def test_gemm_abs_tiny_mixed_signs_rationals():
    """sum_k |dq(a) dq(b)| on mixed-sign codes against exact rationals built
    from torch's E4M3 decode and the scale bytes (2^(byte - 127)), with a
    row / column selection.  A dropped abs on either operand, a scale applied
    twice or a transposed selection fails here."""
    rng = np.random.default_rng(15)
    M, N, K = 5, 4, 128
    qa = rng.integers(0, 256, size=(M, K)).astype(np.uint8)
    qb = rng.integers(0, 256, size=(N, K)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0xB3
    qb[(qb & 0x7F) == 0x7F] = 0x35
    sa = rng.integers(90, 160, size=(M, K // 32)).astype(np.uint8)
    sb = rng.integers(90, 160, size=(N, K // 32)).astype(np.uint8)
    vals = {c: Fraction(float(v)) for c, v in enumerate(torch_e4m3_values()) if not math.isnan(v)}
    rows, cols = np.array([4, 1, 2]), np.array([3, 0])
    got = oracle.gemm_tn_abs(qa, sa, qb, sb, rows=rows, cols=cols)
    assert got.shape == (3, 2)
    for i, m in enumerate(rows):
        for j, n in enumerate(cols):
            exact = sum(abs(vals[int(qa[m, k])]) * Fraction(2) ** (int(sa[m, k // 32]) - 127) *
                        abs(vals[int(qb[n, k])]) * Fraction(2) ** (int(sb[n, k // 32]) - 127)
                        for k in range(K))
            assert abs(Fraction(got[i, j]) - exact) <= exact * Fraction(K, 2 ** 52), (m, n)

# ------------------------------------------------------------ scale packing

def test_pack_scales_hand_example():
    s = np.arange(16, dtype=np.uint8).reshape(2, 8)     # dim 2, K = 256
    p = oracle.pack_scales(s)
    assert p.shape == (2, 2)
    assert [hex(int(w)) for w in p.reshape(-1)] == ["0x3020100", "0xb0a0908", "0x7060504", "0xf0e0d0c"]


def test_pack_scales_is_a_permutation():
    rng = np.random.default_rng(13)
    s = rng.integers(0, 256, size=(96, 64)).astype(np.uint8)
    p = oracle.pack_scales(s)
    back = p.view(np.uint8).reshape(16, 96, 4).transpose(1, 0, 2).reshape(96, 64)
    assert np.array_equal(back, s)


# ---------------------------------------------------------------- grouped

def test_grouped_gemm_single_group_is_dense():
    x = oracle.quantize_rowwise(workloads.normal_bf16((96, 256), 1))
    w = oracle.quantize_rowwise(workloads.normal_bf16((64, 256), 2))
    g = oracle.grouped_gemm_tn(x[0], x[1], w[0][None], w[1][None], [0, 96])
    assert np.array_equal(g, oracle.gemm_tn(*x, *w))


def test_grouped_gemm_ragged_with_empty_groups():
    xq, xs = oracle.quantize_rowwise(workloads.normal_bf16((160, 128), 1))
    ws = [oracle.quantize_rowwise(workloads.normal_bf16((64, 128), 10 + g)) for g in range(4)]
    qw = np.stack([w[0] for w in ws])
    sw = np.stack([w[1] for w in ws])
    off = workloads.offsets_from_counts([0, 64, 0, 96])
    out = oracle.grouped_gemm_tn(xq, xs, qw, sw, off)
    assert np.array_equal(out[:64], oracle.gemm_tn(xq[:64], xs[:64], qw[1], sw[1]))
    assert np.array_equal(out[64:], oracle.gemm_tn(xq[64:], xs[64:], qw[3], sw[3]))
    part = workloads.offsets_from_counts([32, 32, 0, 32])     # rows 96.. in no group
    out2 = oracle.grouped_gemm_tn(xq, xs, qw, sw, part)
    assert np.all(np.isnan(out2[96:])) and not np.any(np.isnan(out2[:96]))


# ------------------------------------------------------------------ amax

def test_amax_matches_torch_and_special_cases():
    """Per-tensor amax against torch's own BF16 reduction (an independent
    implementation), plus cases whose answer is known by construction."""
    import torch
    rng = np.random.default_rng(41)
    for shape in ((64, 96), (3, 32), (257, 64)):
        bits = workloads.wide_range_bf16(shape, int(rng.integers(1 << 30)), n_maxbf16=0, n_subnormal=16,
                                         n_subnormal_blocks=1)
        t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
        assert oracle.amax(bits) == float(t.abs().max().float())
    z = np.zeros((32, 64), dtype=np.uint16)
    assert oracle.amax(z) == 0.0
    z[31, 63] = 0xC2F6                 # -123.0 in the last element: the sign is dropped
    assert oracle.amax(z) == 123.0
    z[0, 0] = workloads.BF16_MAX_BITS  # largest finite BF16
    assert oracle.amax(z) == float(np.float32(3.3895313892515355e38))
    assert oracle.amax(np.zeros((0, 32), dtype=np.uint16)) == 0.0
    sub = np.full((32, 32), 0x8001, dtype=np.uint16)   # -2^-133 everywhere
    assert oracle.amax(sub) == 2.0 ** -133


# ------------------------------------------------ activation-fused quantize

def test_sqrelu_and_its_derivative_match_torch_float32():
    """The activation values against torch's own float32 arithmetic."""
    import torch
    x = workloads.wide_range_bf16((64, 96), 51, u_lo=-20, u_hi=20, n_maxbf16=0, n_subnormal=32,
                                  n_subnormal_blocks=1)
    g = workloads.normal_bf16((64, 96), 52)
    tx = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float()
    tg = torch.from_numpy(g.view(np.int16)).view(torch.bfloat16).float()
    assert np.array_equal(oracle.act_sqrelu(x), (torch.relu(tx) ** 2).numpy())
    assert np.array_equal(oracle.dact_sqrelu(g, x), (tg * (2.0 * torch.relu(tx))).numpy())
    assert oracle.act_sqrelu(np.array([[0xBF80] * 32], dtype=np.uint16)).max() == 0.0   # -1 -> 0


def test_value_quantizer_by_brute_force():
    """fp32 blocks (not BF16-representable: 24-bit mantissas, wide exponents)
    against the exact-rational reference of the block rule."""
    rng = np.random.default_rng(53)
    v = (rng.standard_normal((200, 32)) * np.exp2(rng.integers(-30, 30, size=(200, 1)))).astype(np.float32)
    v[5, :] = 0.0
    v[6, 3] = np.float32(-0.0)
    q, s = oracle.quantize_rowwise_values(v)
    for i in range(v.shape[0]):
        vals = [Fraction(float(t)) for t in v[i]]
        amax = max(abs(t) for t in vals)
        if amax == 0:
            X = -127
        else:
            X = -200
            while not (amax / Fraction(2) ** X < 512):
                X += 1
            X = max(X, -127)
        assert s[i, 0] == (X + 127 if amax != 0 else 0)
        for j, t in enumerate(vals):
            assert q[i, j] == brute_force_encode(t / Fraction(2) ** X, bool(np.signbit(v[i, j]))), (i, j)
    # BF16-representable values give exactly the BF16 path's result
    bits = workloads.normal_bf16((64, 64), 54)
    assert all(np.array_equal(a, b) for a, b in zip(oracle.quantize_rowwise_values(oracle.bf16_value(bits)),
                                                    oracle.quantize_rowwise(bits)))
    qT, sT = oracle.quantize_colwise_values(v[:192])
    qr, sr = oracle.quantize_rowwise_values(np.ascontiguousarray(v[:192].T))
    assert np.array_equal(qT, qr) and np.array_equal(sT, sr)


def test_dbias_values_rounded_once():
    v = np.full((4096, 32), np.float32(1.0) + np.float32(2.0 ** -23), dtype=np.float32)
    want = np.float32(4096 * (1.0 + 2.0 ** -23))
    assert np.all(oracle.dbias_values(v) == want)


def test_dbias_values_match_correctly_rounded_column_sums():
    """fp32 column sums of distinct values (full 24-bit significands, exponents
    over 2^-40 .. 2^40, both signs, a non-square shape) against the correctly
    rounded sum of each column (math.fsum).  A transposed index, a wrong
    leading dimension or an fp32 running sum fails here."""
    rng = np.random.default_rng(56)
    R, C = 300, 96
    v = (rng.standard_normal((R, C)) * np.exp2(rng.integers(-40, 41, size=(R, C)))).astype(np.float32)
    v[7, :] = np.float32(2.0 ** 30)          # large terms that an fp32 running sum would absorb small ones into
    v[8, :] = np.float32(-(2.0 ** 30))
    got = oracle.dbias_values(v)
    assert got.dtype == np.float32 and got.shape == (C,)
    for c in range(C):
        assert got[c] == np.float32(math.fsum(float(t) for t in v[:, c])), c


def test_golden_e8m0_readback():
    """tests/golden/e8m0_readback.txt: the page's byte << 23 readback for a
    few bytes, and its rule that an all-zero block gets scale byte 0."""
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "e8m0_readback.txt")
    rows = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    checked = 0
    for r in rows:
        if r[0] == "zero_block_byte":
            q, s = oracle.quantize_rowwise(np.zeros((2, 64), dtype=np.uint16))
            assert np.all(s == int(r[1])) and not q.any()
            checked += 1
            continue
        b, bits = int(r[0]), int(r[1], 16)
        assert bits == b << 23
        assert oracle.e8m0_decode(b) == float(np.array([bits], dtype=np.uint32).view(np.float32)[0])
        checked += 1
    assert checked == 8


def test_sqrelu_epilogue_matches_the_activation_and_torch():
    """The GEMM epilogue's relu(r)^2 (fp64) against torch's float64 relu and
    power, and against the activation quantizer's fp32 relu(x)^2 on BF16
    values (where both are exact)."""
    import torch
    rng = np.random.default_rng(57)
    r = rng.standard_normal(5000) * np.exp2(rng.integers(-20, 20, size=5000))
    r[:5] = [0.0, -0.0, -1.0, 3.0, -1e300]
    want = (torch.relu(torch.from_numpy(r)) ** 2).numpy()
    assert np.array_equal(oracle.sqrelu_epilogue(r), want)
    bits = workloads.wide_range_bf16((8, 64), 58, u_lo=-20, u_hi=20, n_maxbf16=0, n_subnormal=0, n_subnormal_blocks=0)
    assert np.array_equal(oracle.sqrelu_epilogue(oracle.bf16_value(bits)),
                          oracle.act_sqrelu(bits).astype(np.float64))


# ------------------------------------------------------------------ GELU

def test_gelu_matches_torch_and_closed_forms():
    """GELU(x) = x Phi(x) against torch's float64 gelu (erf form) where that is
    accurate (|x| <= 5: torch adds 1 + erf(x / sqrt 2), which cancels in the
    negative tail), against tabulated normal-CDF values in the tail, and the
    exact identity GELU(x) - GELU(-x) = x (Phi(x) + Phi(-x) = 1)."""
    import torch
    rng = np.random.default_rng(60)
    x = np.concatenate([rng.standard_normal(4000) * 2.0, np.linspace(-5, 5, 1001)])
    got = oracle.gelu_f64(x)
    want = torch.nn.functional.gelu(torch.from_numpy(x)).numpy()
    assert np.all(np.abs(got - want) <= 1e-8 * np.abs(want) + 1e-15)
    # Phi(-3) = 0.00134989803163009, Phi(-8) = 6.22096057427178e-16 (normal CDF tables)
    assert abs(oracle.gelu_f64(-3.0) - (-3.0 * 0.00134989803163009)) <= 1e-15
    assert abs(oracle.gelu_f64(-8.0) / (-8.0 * 6.22096057427178e-16) - 1.0) <= 1e-12
    assert oracle.gelu_f64(0.0) == 0.0 and oracle.gelu_f64(40.0) == 40.0
    y = rng.standard_normal(2000) * 8.0
    assert np.all(np.abs(oracle.gelu_f64(y) - oracle.gelu_f64(-y) - y) <= 4 * np.spacing(np.abs(y)))


def test_gelu_derivative_terms():
    """GELU'(a) = Phi(a) + a phi(a): the sum against torch's float64 autograd of
    gelu (|a| <= 5) and central differences of the oracle's GELU; Phi(0) = 1/2,
    and the sign change of GELU' at GELU's minimum near a = -0.7518."""
    import torch
    a = np.linspace(-5, 5, 2001)
    t1, t2 = oracle.dgelu_terms(a)
    ta = torch.from_numpy(a).requires_grad_(True)
    torch.nn.functional.gelu(ta).sum().backward()
    assert np.all(np.abs((t1 + t2) - ta.grad.numpy()) <= 1e-9)
    h = 1e-5
    fd = (oracle.gelu_f64(a + h) - oracle.gelu_f64(a - h)) / (2 * h)
    assert np.all(np.abs((t1 + t2) - fd) <= 1e-8)
    p0, q0 = oracle.dgelu_terms(0.0)
    assert p0 == 0.5 and q0 == 0.0
    # GELU has its minimum (about -0.16997) at x = -0.75179...: GELU' changes sign there
    lo, hi = oracle.dgelu_terms(-0.75180), oracle.dgelu_terms(-0.75178)
    assert sum(lo) < 0.0 < sum(hi)
    assert abs(oracle.gelu_f64(-0.75179) - (-0.16997)) < 1e-5
    g = workloads.normal_bf16((4, 64), 61)
    ab = workloads.normal_bf16((4, 64), 62)
    want = oracle.bf16_value(g) * np.add(*oracle.dgelu_terms(oracle.bf16_value(ab)))
    assert np.array_equal(oracle.dact_gelu(g, ab), want)
    assert np.array_equal(oracle.act_gelu(ab), oracle.gelu_f64(oracle.bf16_value(ab)))


def test_silu_matches_torch_and_closed_forms():
    """SiLU(z) = z sigma(z) against torch's float64 silu, the tabulated
    logistic value sigma(1) = 0.7310585786300049, the identity
    SiLU(z) - SiLU(-z) = z (sigma(z) + sigma(-z) = 1), the negative tail
    SiLU(z) ~ z e^z, and no NaN at the overflow ends."""
    import torch
    rng = np.random.default_rng(64)
    z = np.concatenate([rng.standard_normal(4000) * 4.0, np.linspace(-30, 30, 601)])
    want = torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    assert np.all(np.abs(oracle.silu_f64(z) - want) <= 1e-15 * np.abs(want) + 1e-300)
    assert abs(oracle.silu_f64(1.0) - 0.7310585786300049) <= 1e-16
    assert oracle.silu_f64(0.0) == 0.0
    y = rng.standard_normal(2000) * 20.0
    assert np.all(np.abs(oracle.silu_f64(y) - oracle.silu_f64(-y) - y) <= 4 * np.spacing(np.abs(y)))
    t = np.array([-40.0, -60.0, -100.0])
    assert np.all(np.abs(oracle.silu_f64(t) / (t * np.exp(t)) - 1.0) <= 1e-15 + np.exp(t))
    big = oracle.silu_f64(np.array([-1e300, -800.0, 800.0, 1e300]))
    assert np.all(np.isfinite(big)) and big[0] == 0.0 and big[1] == 0.0 and big[2] == 800.0 and big[3] == 1e300


def test_swiglu_epilogue_pairs_gate_and_up_columns():
    """C[m][n] = SiLU(R[m][n]) * R[m][N + n]: checked on a hand example
    (SiLU(0) = 0, SiLU(1) = sigma(1), up = 0) and against torch's float64 silu
    on the two halves of a random product, including the grouped shape."""
    import torch
    r = np.array([[0.0, 1.0, 2.0, 5.0, -3.0, 0.0]])
    got = oracle.swiglu_epilogue(r)
    assert got.shape == (1, 3)
    assert got[0, 0] == 0.0 and abs(got[0, 1] - (-3.0 * 0.7310585786300049)) <= 1e-15 and got[0, 2] == 0.0
    rng = np.random.default_rng(65)
    r = rng.standard_normal((3, 7, 64)) * 6.0
    want = (torch.nn.functional.silu(torch.from_numpy(r[..., :32])) * torch.from_numpy(r[..., 32:])).numpy()
    assert np.allclose(oracle.swiglu_epilogue(r), want, rtol=1e-15, atol=0)
    with pytest.raises(ValueError):
        oracle.swiglu_epilogue(np.zeros((2, 5)))


def test_bias_add_broadcasts_one_value_per_column():
    """R + bias[n]: zero bias is the identity; with a zero product the result
    is the bias on every row (exact BF16 values, e.g. 0x3FC0 = 1.5 and
    0xC080 = -4); a transposed bias (per row) is rejected."""
    r = np.arange(12, dtype=np.float64).reshape(3, 4) - 5.0
    assert np.array_equal(oracle.bias_add(r, np.zeros(4, dtype=np.uint16)), r)
    b = np.array([0x3FC0, 0xC080, 0x0000, 0x8000], dtype=np.uint16)
    got = oracle.bias_add(np.zeros((3, 4)), b)
    assert np.array_equal(got, np.tile([1.5, -4.0, 0.0, 0.0], (3, 1)))
    assert np.array_equal(oracle.bias_add(r, b)[:, 1], r[:, 1] - 4.0)
    with pytest.raises(ValueError):
        oracle.bias_add(r, np.zeros(3, dtype=np.uint16))


def test_scale_bytes_array_matches_the_scalar_rule():
    rng = np.random.default_rng(63)
    a = np.abs(rng.standard_normal(3000)) * np.exp2(rng.integers(-140, 130, size=3000))
    a[:4] = [0.0, 2.0 ** -130, 448.0 * 2.0 ** 119, 1.0]
    assert np.array_equal(oracle.scale_bytes(a), np.array([oracle.scale_byte(v) for v in a], dtype=np.uint8))
