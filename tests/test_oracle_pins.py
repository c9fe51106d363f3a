"""Pins of the CPU oracle against things other than itself.

Each group checks one oracle step against an independent route: hand-worked
fixtures (tests/golden), exact rational arithmetic (tests/exact.py), closed
forms, invariants and brute force on tiny inputs. ``test_planted_mistakes``
plants plausible mistakes into copies of oracle steps and shows that these
same checks reject them.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import workloads as W
from tests import exact as E

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def bits_of(values) -> np.ndarray:
    return np.array([E.bf16_bits(Fraction(v)) for v in values], dtype=np.uint16)


def parse_fraction(s: str) -> Fraction:
    return Fraction(s.strip())


def read_cases(name):
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


# ---------------------------------------------------------------------------
# Quantisation
# ---------------------------------------------------------------------------

def quant_golden_rows():
    rows = []
    for line in read_cases("quant_worked_examples.txt"):
        xs, sc, qs = line.split("|")
        rows.append(([Fraction(t) for t in xs.split()], parse_fraction(sc),
                     [int(t) for t in qs.split()]))
    return rows


def check_quant_golden(quant_rows_fn) -> bool:
    for xs, sc, qs in quant_golden_rows():
        q, s = quant_rows_fn(bits_of(xs)[None, :])
        if list(q[0]) != qs or Fraction(float(s.reshape(-1)[0])) != sc:
            return False
    return True


def test_quant_golden_worked_examples():
    assert check_quant_golden(O.quantize_rows)
    # the grouped form (1, cols) takes the same decisions
    assert check_quant_golden(lambda b: O.quantize_groups(b, 1, b.shape[1]))


def exact_quant_row(bits_row):
    xs = [E.bf16_value(b) for b in bits_row]
    amax = max(abs(x) for x in xs)
    s = E.quant_scale(amax)
    return [E.quant_code(x, s) for x in xs], s


def near_tie_rows(n_amax=48, per_row=64, seed=7):
    """Rows [amax, x1, x2, ...] whose quotients x/scale fall within ~1e-4 of a
    half-integer: the cases where rounding direction, tie handling and the
    exact form of the division decide the code."""
    rng = np.random.default_rng(seed)
    pos = np.arange(0x0080, 0x7F00, dtype=np.uint32)             # normal positives
    amax_bits = rng.choice(pos, n_amax, replace=False)
    rows = []
    for ab in amax_bits:
        a = float((np.uint32(ab) << 16).view(np.float32))
        xs = (pos[pos <= ab] << 16).view(np.float32).astype(np.float64)
        t = xs * 127.0 / a
        frac = np.abs(t - np.floor(t) - 0.5)
        cand = pos[pos <= ab][np.argsort(frac)[:per_row - 1]]
        sign = rng.choice([0, 0x8000], cand.size).astype(np.uint32)
        rows.append(np.concatenate([[ab], cand | sign]).astype(np.uint16))
    return np.stack(rows)


def check_quant_exact(quant_rows_fn, x_bits) -> bool:
    q, s = quant_rows_fn(x_bits)
    for i in range(x_bits.shape[0]):
        qe, se = exact_quant_row(x_bits[i])
        if list(q[i]) != qe or Fraction(float(s[i])) != se:
            return False
    return True


def test_quant_near_ties_exact():
    rows = near_tie_rows()
    assert check_quant_exact(O.quantize_rows, rows)


def test_quant_random_rows_exact():
    x = W.random_bits((24, 96), seed=11, std=3.0)
    x[3] = 0                                   # all-zero row
    x[5, :] = 0
    x[5, 17] = E.bf16_bits(Fraction(-5, 8))    # single nonzero
    x[7] = W.random_bits((96,), seed=12, std=1e-30)   # tiny (subnormal-range) scale
    x[8] = W.random_bits((96,), seed=13, std=1e30)    # huge values
    assert check_quant_exact(O.quantize_rows, x)


def test_quant_invariants():
    x = W.random_bits((64, 256), seed=21, std=2.0)
    q, s = O.quantize_rows(x)
    # symmetry: q(-x) = -q(x), same scale
    qn, sn = O.quantize_rows(x ^ np.uint16(0x8000))
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    # the absmax element maps to +-127
    xf = O.bf16_to_f32(x)
    i = np.argmax(np.abs(xf), axis=1)
    assert np.all(np.abs(q[np.arange(64), i]) == 127)
    # power-of-two equivariance in the normal range: q(2^j x) = q(x), s scales
    for j in (-20, -3, 5, 40):
        x2 = O.f32_to_bf16(xf * np.float32(2.0 ** j))
        q2, s2 = O.quantize_rows(x2)
        assert np.array_equal(q2, q)
        assert np.array_equal(s2, (s * np.float32(2.0 ** j)).astype(np.float32))
    # error bound |x - q s| <= s/2 + 2^-24 |x|, exact in fp64
    err = np.abs(xf.astype(np.float64) - q.astype(np.float64) * s[:, None].astype(np.float64))
    bound = s[:, None].astype(np.float64) / 2 + 2.0 ** -24 * np.abs(xf.astype(np.float64))
    assert np.all(err <= bound)
    # codes never reach -128
    assert q.min() >= -127


def test_quant_groups_blockwise():
    x = W.random_bits((200, 384), seed=31, std=1.0)
    x[:, 128:256] = W.random_bits((200, 128), seed=32, std=50.0)   # a loud K block
    q, s = O.quantize_groups(x, 1, 128)
    assert s.shape == (200, 3)
    for kb in range(3):
        qe, se = O.quantize_rows(x[:, kb * 128:(kb + 1) * 128])
        assert np.array_equal(q[:, kb * 128:(kb + 1) * 128], qe)
        assert np.array_equal(s[:, kb], se)
    # 128 x 128 weight groups, ragged last row group (200 = 128 + 72)
    qw, sw = O.quantize_groups(x, 128, 128)
    assert sw.shape == (2, 3)
    xf = O.bf16_to_f32(x)
    for gr, (r0, r1) in enumerate(((0, 128), (128, 200))):
        for kb in range(3):
            blk = xf[r0:r1, kb * 128:(kb + 1) * 128]
            amax = Fraction(float(np.max(np.abs(blk))))
            assert Fraction(float(sw[gr, kb])) == E.quant_scale(amax)
            codes = [[E.quant_code(Fraction(float(v)), E.quant_scale(amax)) for v in row]
                     for row in blk[:4]]
            assert np.array_equal(qw[r0:r0 + 4, kb * 128:(kb + 1) * 128], np.array(codes))


@pytest.mark.slow
def test_quant_exhaustive_against_integer_division():
    """Every (absmax, x) pair of positive finite BF16 values with x <= absmax
    (sign symmetry covers negative x), about 5.3e8 pairs: the oracle's codes
    equal those formed by integer long division. Takes a few minutes."""
    pos = np.arange(1, 0x7F80, dtype=np.int64)
    for ai in range(pos.size):
        ab = int(pos[ai])
        xs_bits = pos[: ai + 1]
        q, s = O.quantize_rows(xs_bits.astype(np.uint16)[None, :])
        s_exact = E.quant_scale(E.bf16_value(ab))
        assert Fraction(float(s[0])) == s_exact
        qe = int_quant_codes(s_exact, xs_bits)
        assert np.array_equal(q[0].astype(np.int64), qe), hex(ab)


def int_quant_codes(s: Fraction, xs_bits: np.ndarray) -> np.ndarray:
    """Codes round-half-even(RN32(x / s)) for positive BF16 x, by integer
    long division on significands (no floating-point division involved).

    x = mx * 2^e2 and s = num * 2^s_exp (num odd), so x/s = mx * 2^sh / num. For
    t = x/s >= 1/4 the fp32 quantum is 2^(e-23) with e = floor(log2 t);
    below 1/4 the code is 0 whatever the rounding.
    """
    num, den = s.numerator, s.denominator          # one of them is a power of two
    s_exp = -(den.bit_length() - 1)
    while num % 2 == 0:                             # s = num * 2^s_exp, num odd
        num //= 2
        s_exp += 1
    assert num < 2**24
    xs = xs_bits.astype(np.int64)
    ex = (xs >> 7) & 0xFF
    mx = np.where(ex == 0, xs & 0x7F, (xs & 0x7F) | 0x80)
    e2 = np.where(ex == 0, -133, ex - 134)          # x = mx * 2^e2
    sh = e2 - s_exp                                  # x/s = mx * 2^sh / num
    codes = np.zeros(xs.size, dtype=np.int64)
    with np.errstate(all="ignore"):
        t_est = mx.astype(np.float64) * np.exp2(sh.astype(np.float64)) / float(num)
    big = t_est >= 0.2
    if not np.any(big):
        return codes
    mx, sh, t_est = mx[big], sh[big], t_est[big]
    e = np.floor(np.log2(t_est)).astype(np.int64)
    for _ in range(3):                               # settle e exactly
        P = 23 - e
        numer = mx << (sh + P)
        n = numer // num
        lo = n < (1 << 23)
        hi = n >= (1 << 24)
        if not (np.any(lo) or np.any(hi)):
            break
        e = e - lo.astype(np.int64) + hi.astype(np.int64)
    rem = numer - n * num
    up = (2 * rem > num) | ((2 * rem == num) & ((n & 1) == 1))
    n = n + up
    ip = n >> P
    frac = n & ((np.int64(1) << P) - 1)
    half = np.int64(1) << (P - 1)
    q = ip + ((frac > half) | ((frac == half) & ((ip & 1) == 1)))
    codes[big] = np.minimum(q, 127)
    return codes


def test_int_quant_codes_sample():
    """The integer route itself agrees with Fraction arithmetic on a sample."""
    rng = np.random.default_rng(3)
    for ab in rng.integers(0x0100, 0x7F00, 12):
        xs = rng.integers(1, int(ab) + 1, 200)
        s = E.quant_scale(E.bf16_value(int(ab)))
        want = [E.quant_code(E.bf16_value(int(x)), s) for x in xs]
        assert int_quant_codes(s, xs).tolist() == want


# ---------------------------------------------------------------------------
# RMSNorm prologue
# ---------------------------------------------------------------------------

def test_rmsnorm_golden_worked_examples():
    for line in read_cases("rmsnorm_worked_examples.txt"):
        eps_s, xs, gs, rs, qs = [t.strip() for t in line.split("|")]
        x = bits_of([Fraction(t) for t in xs.split()])[None, :]
        g = bits_of([Fraction(t) for t in gs.split()])
        q, s, r = O.rmsnorm_quant(x, g, float(eps_s))
        if rs != "-":
            assert Fraction(float(r[0])) == Fraction(rs)
        assert list(q[0]) == [int(t) for t in qs.split()]
        if all(Fraction(t) == 0 for t in gs.split()):
            assert s[0] == 0


def exact_inv_rms(x_bits_row, eps):
    xs = [E.bf16_value(b) for b in x_bits_row]
    ss = sum(x * x for x in xs)
    return E.inv_sqrt_f32(ss / len(xs) + Fraction(float(np.float32(eps))))


def test_rmsnorm_inv_rms_exact():
    x = W.random_bits((16, 256), seed=41, std=1.0)
    x[2] = W.random_bits((256,), seed=42, std=1e-3)   # eps comparable to mean x^2
    x[3] = 0                                           # r = 1/sqrt(eps)
    r = O.rmsnorm_inv_rms(x, 1e-6)
    for i in range(16):
        assert Fraction(float(r[i])) == exact_inv_rms(x[i], 1e-6), i


def test_rmsnorm_closed_forms():
    K = 512
    for c, eps in ((3.0, 1e-6), (0.0009765625, 1e-6), (-7.5, 0.25)):
        x = np.full((1, K), E.bf16_bits(Fraction(c)), dtype=np.uint16)
        r = O.rmsnorm_inv_rms(x, eps)
        want = E.inv_sqrt_f32(Fraction(c) ** 2 + Fraction(float(np.float32(eps))))
        assert Fraction(float(r[0])) == want
    # gamma = 1, |c| >> sqrt(eps): y = bf16(c r) ~ sign(c), all codes +-127
    x = np.full((2, K), E.bf16_bits(Fraction(5)), dtype=np.uint16)
    x[1] = E.bf16_bits(Fraction(-5))
    g = np.full(K, E.bf16_bits(Fraction(1)), dtype=np.uint16)
    q, s, _ = O.rmsnorm_quant(x, g, 1e-6)
    assert np.all(q[0] == 127) and np.all(q[1] == -127)
    # gamma = 0: everything quantises to zero with scale zero
    q, s, _ = O.rmsnorm_quant(W.random_bits((3, K), seed=5), np.zeros(K, np.uint16), 1e-6)
    assert np.all(q == 0) and np.all(s == 0)


def test_rmsnorm_apply_exact():
    x = W.random_bits((6, 128), seed=51)
    g = W.random_bits((128,), seed=52, std=0.1, mean=1.0)
    r = O.rmsnorm_inv_rms(x, 1e-6)
    y = O.rmsnorm_bf16(x, g, r)
    for i in range(6):
        ri = Fraction(float(r[i]))
        for k in range(128):
            t = E.f32(E.bf16_value(x[i, k]) * ri)
            want = E.bf16(E.f32(t * E.bf16_value(g[k])))
            assert E.bf16_value(y[i, k]) == want
    # the fused prologue equals a BF16 RMSNorm followed by the quantisation
    q, s, _ = O.rmsnorm_quant(x, g, 1e-6, r=r)
    q2, s2 = O.quantize_rows(y)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


# ---------------------------------------------------------------------------
# INT32 GEMM
# ---------------------------------------------------------------------------

def brute_gemm(qa, qw):
    M, K = qa.shape
    N = qw.shape[0]
    return [[sum(int(qa[m, k]) * int(qw[n, k]) for k in range(K)) for n in range(N)]
            for m in range(M)]


def check_gemm_pins(gemm_fn) -> bool:
    for (M, N, K), seed in (((4, 4, 4), 4), ((1, 128, 128), 1), ((3, 5, 7), 2),
                            ((17, 9, 256), 3)):
        qa = W.random_int8((M, K), seed)
        qw = W.random_int8((N, K), seed + 100)
        try:
            got = gemm_fn(qa, qw).tolist()
        except ValueError:
            return False
        if got != brute_gemm(qa, qw):
            return False
    return True


def test_gemm_golden_worked_examples():
    text = "\n".join(read_cases("gemm_worked_examples.txt"))
    cases = []
    cur = {}
    for line in text.splitlines():
        key, val = line.split(":", 1)
        cur[key.strip()] = [[float(t) for t in row.split()] for row in val.split(";")]
        if key.strip() == "out":
            cases.append(cur)
            cur = {}
    assert len(cases) == 2
    for c in cases:
        qa = np.array(c["qa"], dtype=np.int8)
        qw = np.array(c["qw"], dtype=np.int8)
        acc = O.gemm_i32(qa, qw)
        assert acc.tolist() == np.array(c["acc"], dtype=np.int64).tolist()
        out = O.postscale_bf16(acc, np.array(c["sa"][0], np.float32), np.array(c["sw"][0], np.float32))
        assert O.bf16_to_f32(out).tolist() == np.array(c["out"], np.float32).tolist()


def test_gemm_brute_force():
    assert check_gemm_pins(O.gemm_i32)


def test_gemm_identities():
    qa = W.random_int8((33, 256), 61)
    qw = W.random_int8((40, 256), 62)
    acc = O.gemm_i32(qa, qw)
    assert np.array_equal(O.gemm_i32(qw, qa), acc.T)               # transposition
    onehot = np.zeros((3, 256), np.int8)
    onehot[0, 5] = 1
    onehot[1, 255] = -1
    onehot[2, 0] = 127
    acc1 = O.gemm_i32(onehot, qw)
    assert np.array_equal(acc1[0], qw[:, 5].astype(np.int32))
    assert np.array_equal(acc1[1], -qw[:, 255].astype(np.int32))
    assert np.array_equal(acc1[2], 127 * qw[:, 0].astype(np.int32))
    # the largest accumulator of the down-projection shape (K = 13824)
    K = 13824
    a = np.full((1, K), 127, np.int8)
    w = np.full((2, K), -127, np.int8)
    w[1] = 127
    assert O.gemm_i32(a, w).tolist() == [[-16129 * K, 16129 * K]]


# ---------------------------------------------------------------------------
# Post-scale epilogue
# ---------------------------------------------------------------------------

def check_postscale_pins(post_fn) -> bool:
    acc = W.random_int8((16, 16), 71).astype(np.int32) * 1_000_003
    acc[0, 0] = 0
    acc[0, 1] = 2**24 + 1             # int32 -> fp32 conversion rounds here
    acc[0, 2] = -(2**27) - 3
    sa = W.random_scales((16,), 72)
    sw = W.random_scales((16,), 73, lo=1e-5, hi=10.0)
    out = post_fn(acc, sa, sw)
    for m in range(16):
        for n in range(16):
            a = Fraction(int(acc[m, n]))
            s1, s2 = Fraction(float(sa[m])), Fraction(float(sw[n]))
            # fp32 steps, in the stated order
            step = E.bf16(E.f32(E.f32(E.f32(a) * s1) * s2))
            if E.bf16_value(out[m, n]) != step:
                return False
            # and within one BF16 ulp of the exact product
            if O.bf16_ulp_distance(out[m, n], E.bf16_bits(E.bf16(a * s1 * s2))) > 1:
                return False
    return True


def test_postscale_exact():
    assert check_postscale_pins(O.postscale_bf16)


def check_postscale_bias_pins(post_fn) -> bool:
    acc = W.random_int8((16, 16), 74).astype(np.int32) * 1_000_003
    acc[0, 1] = 2**24 + 1
    sa = W.random_scales((16,), 75)
    sw = W.random_scales((16,), 76, lo=1e-5, hi=10.0)
    bias = W.random_bits((16,), seed=77, std=0.5)
    bias[3] = 0
    out = post_fn(acc, sa, sw, bias)
    for m in range(16):
        for n in range(16):
            a = Fraction(int(acc[m, n]))
            s1, s2 = Fraction(float(sa[m])), Fraction(float(sw[n]))
            want = E.bf16(E.f32(E.f32(E.f32(E.f32(a) * s1) * s2) + E.bf16_value(bias[n])))
            if E.bf16_value(out[m, n]) != want:
                return False
    # a zero activation scale leaves exactly the bias; a zero bias the post-scale value
    sa0 = sa.copy()
    sa0[5] = 0
    if not np.array_equal(O.bf16_to_f32(post_fn(acc, sa0, sw, bias)[5]), O.bf16_to_f32(bias)):
        return False
    zero = np.zeros(16, np.uint16)
    return np.array_equal(O.bf16_to_f32(post_fn(acc, sa, sw, zero)),
                          O.bf16_to_f32(O.postscale_bf16(acc, sa, sw)))


def test_postscale_bias_exact():
    assert check_postscale_bias_pins(O.postscale_bias_bf16)


def test_w8a8_linear_bias_close_to_bf16_product():
    """Informational bound: the W8A8 Linear with bias stays within quantisation
    noise of torch's float64 Linear on the unquantised inputs."""
    x = W.random_bits((32, 256), seed=78)
    w = W.random_bits((128, 256), seed=79, std=0.02)
    b = W.random_bits((128,), seed=80, std=0.1)
    out, *_ = O.w8a8_linear(x, w, b)
    ref = (O.bf16_to_f32(x).astype(np.float64) @ O.bf16_to_f32(w).astype(np.float64).T
           + O.bf16_to_f32(b).astype(np.float64))
    rel = np.linalg.norm(O.bf16_to_f32(out) - ref) / np.linalg.norm(ref)
    assert rel < 0.02


def test_postscale_special_cases():
    acc = np.arange(-256, 256, dtype=np.int32).reshape(2, 256)
    out = O.postscale_bf16(acc, np.ones(2, np.float32), np.ones(256, np.float32))
    # |acc| <= 256 is exact in BF16 and unit scales leave it unchanged
    assert np.array_equal(O.bf16_to_f32(out), acc.astype(np.float32))
    out = O.postscale_bf16(acc, np.zeros(2, np.float32), np.ones(256, np.float32))
    assert np.all(O.bf16_to_f32(out) == 0)


# ---------------------------------------------------------------------------
# fp32 FMA and the blockwise variant
# ---------------------------------------------------------------------------

def test_fma_f32_exact():
    # the midpoint case: the fp64 sum lands exactly between two fp32 values
    a = np.float32(8 * (1 + 2**-23))
    b = np.float32(8 * (1 - 2**-23))
    c = np.float32(2**30 + 2**7)
    got = O.fma_f32(np.array([a]), np.array([b]), np.array([c]))[0]
    assert Fraction(float(got)) == E.f32(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))
    assert float(got) == 2**30 + 2**7
    rng = np.random.default_rng(81)
    av = rng.standard_normal(2000).astype(np.float32)
    bv = (rng.standard_normal(2000) * 1e-3).astype(np.float32)
    cv = (rng.standard_normal(2000) * 10.0 ** rng.integers(-6, 6, 2000)).astype(np.float32)
    got = O.fma_f32(av, bv, cv)
    for i in range(2000):
        want = E.f32(Fraction(float(av[i])) * Fraction(float(bv[i])) + Fraction(float(cv[i])))
        assert Fraction(float(got[i])) == want


def blockwise_inputs(M, N, K, seed):
    qa = W.random_int8((M, K), seed)
    qw = W.random_int8((N, K), seed + 1)
    sa = W.random_scales((M, K // 128), seed + 2)
    sw = W.random_scales((N // 128, K // 128), seed + 3)
    return qa, sa, qw, sw


def cancelling_blockwise_inputs():
    """One row whose K-block sums are +2064512, -2064512 and 1 (with a weight
    scale of 1 + 2^-20 on the first block): the fp32 result depends on the
    accumulation order (ascending gives 3, descending 2.96875)."""
    qa = np.zeros((2, 384), np.int8)
    qw = np.zeros((128, 384), np.int8)
    qa[:, :256] = 127
    qw[0, :128] = 127
    qw[0, 128:256] = -127
    qa[:, 256] = 1
    qw[0, 256] = 1
    qw[1:, :] = W.random_int8((127, 384), 95)
    sa = np.ones((2, 3), np.float32)
    sw = np.ones((1, 3), np.float32)
    sw[0, 0] = np.float32(1 + 2**-20)
    return qa, sa, qw, sw


def check_blockwise_pins(bw_fn) -> bool:
    for qa, sa, qw, sw in (blockwise_inputs(3, 256, 384, 91), cancelling_blockwise_inputs()):
        if not _check_blockwise_case(bw_fn, qa, sa, qw, sw):
            return False
    return True


def _check_blockwise_case(bw_fn, qa, sa, qw, sw) -> bool:
    out = bw_fn(qa, sa, qw, sw)
    M, N = out.shape
    for m in range(M):
        for n in list(range(0, N, 7)) + [0]:
            c = Fraction(0)
            for kb in range(qa.shape[1] // 128):
                blk = sum(int(qa[m, k]) * int(qw[n, k]) for k in range(kb * 128, kb * 128 + 128))
                s = E.f32(Fraction(float(sa[m, kb])) * Fraction(float(sw[n // 128, kb])))
                c = E.f32(Fraction(blk) * s + c)
            if E.bf16_value(out[m, n]) != E.bf16(c):
                return False
    return True


def test_blockwise_exact_steps():
    assert check_blockwise_pins(O.gemm_blockwise_bf16)
    out = O.gemm_blockwise_bf16(*cancelling_blockwise_inputs())
    assert O.bf16_to_f32(out)[0, 0] == 3.0


def test_blockwise_reductions():
    # one K block: blockwise = fl32(fl32(acc) * fl32(sa*sw)), within 1 ulp of post-scale
    qa, sa, qw, sw = blockwise_inputs(16, 256, 128, 101)
    out = O.gemm_blockwise_bf16(qa, sa, qw, sw)
    acc = O.gemm_i32(qa, qw)
    sw_n = np.repeat(sw[:, 0], 128)
    ref = O.postscale_bf16(acc, sa[:, 0], sw_n)
    assert np.max(O.bf16_ulp_distance(out, ref)) <= 1
    # block-constant scales: equals the post-scale result within 1 ulp when no
    # cancellation makes fp32 order matter (all codes positive here)
    qa = np.abs(W.random_int8((8, 512), 111)).astype(np.int8)
    qw = np.abs(W.random_int8((128, 512), 112)).astype(np.int8)
    sa = np.repeat(W.random_scales((8, 1), 113), 4, axis=1)
    sw = np.full((1, 4), np.float32(0.01))
    out = O.gemm_blockwise_bf16(qa, sa, qw, sw)
    ref = O.postscale_bf16(O.gemm_i32(qa, qw), sa[:, 0], np.full(128, np.float32(0.01)))
    assert np.max(O.bf16_ulp_distance(out, ref)) <= 1


# ---------------------------------------------------------------------------
# Whole linear (informational accuracy) and shape rules
# ---------------------------------------------------------------------------

def test_w8a8_linear_close_to_bf16_product():
    wl = W.WORKLOADS["tiny"]
    x = W.x_bits(wl)
    w = W.w_bits(wl)
    out, qa, sa, qw, sw, acc = O.w8a8_linear(x, w)
    ref = O.bf16_to_f32(x).astype(np.float64) @ O.bf16_to_f32(w).astype(np.float64).T
    rel = np.linalg.norm(O.bf16_to_f32(out) - ref) / np.linalg.norm(ref)
    assert rel < 0.02, rel


def test_shape_rules():
    O.check_gemm_shape(1, 128, 128)
    O.check_gemm_shape(32760, 5120, 13824)
    for bad in ((0, 128, 128), (4, 100, 128), (4, 128, 100), (4, 128, 133248)):
        with pytest.raises(O.ShapeError):
            O.check_gemm_shape(*bad)


# ---------------------------------------------------------------------------
# Planted mistakes: the pins above must reject each of these
# ---------------------------------------------------------------------------

def _quant_mul_reciprocal(x_bits):
    x = O.bf16_to_f32(x_bits)
    amax = np.max(np.abs(x), axis=1).astype(np.float32)
    s = (amax / np.float32(127)).astype(np.float32)
    with np.errstate(over="ignore"):
        r = np.where(s == 0, 0, np.float32(1) / np.where(s == 0, 1, s)).astype(np.float32)
    q = np.clip(np.rint(x * r[:, None]), -127, 127).astype(np.int8)
    return q, s


def _quant_half_away(x_bits):
    x = O.bf16_to_f32(x_bits)
    amax = np.max(np.abs(x), axis=1).astype(np.float32)
    s = (amax / np.float32(127)).astype(np.float32)
    t = x / np.where(s == 0, 1, s)[:, None]
    q = np.clip(np.sign(t) * np.floor(np.abs(t) + 0.5), -127, 127).astype(np.int8)
    q[s == 0] = 0
    return q, s


def _quant_scale_128(x_bits):
    x = O.bf16_to_f32(x_bits)
    amax = np.max(np.abs(x), axis=1).astype(np.float32)
    s = (amax / np.float32(127.5)).astype(np.float32)
    t = x / np.where(s == 0, 1, s)[:, None]
    q = np.clip(np.rint(t), -128, 127).astype(np.int8)
    q[s == 0] = 0
    return q, s


def _gemm_dropped_term(qa, qw):
    return O.gemm_i32(qa[:, :-1], qw[:, :-1])


def _gemm_transposed(qa, qw):
    # W taken as [K, N] instead of [N, K] (only shape-valid when N == K)
    return (qa.astype(np.int64) @ qw.astype(np.int64)).astype(np.int32)


def _post_dropped_weight_scale(acc, sa, sw):
    return O.postscale_bf16(acc, sa, np.ones_like(sw))


def _post_swapped_scales(acc, sa, sw):
    # activation scale indexed by output channel and vice versa
    return O.postscale_bf16(acc, sw, sa)


def _bias_before_weight_scale(acc, sa, sw, bias):
    a = np.asarray(acc, np.int32).astype(np.float32)
    t = (a * sa[:, None]).astype(np.float32)
    t = (t + O.bf16_to_f32(bias)[None, :]).astype(np.float32)
    return O.f32_to_bf16((t * sw[None, :]).astype(np.float32))


def _bias_after_rounding(acc, sa, sw, bias):
    y = O.bf16_to_f32(O.postscale_bf16(acc, sa, sw))
    return O.f32_to_bf16((y + O.bf16_to_f32(bias)[None, :]).astype(np.float32))


def _bias_by_row(acc, sa, sw, bias):
    return O.postscale_bias_bf16(acc.T.copy(), sw, sa, bias).T.copy()


def _bw_wrong_block_index(qa, sa, qw, sw):
    sw2 = np.roll(sw, 1, axis=0)
    return O.gemm_blockwise_bf16(qa, sa, qw, sw2)


def _bw_descending(qa, sa, qw, sw):
    K = qa.shape[1]
    idx = np.arange(K).reshape(-1, 128)[::-1].reshape(-1)
    return O.gemm_blockwise_bf16(qa[:, idx], sa[:, ::-1].copy(), qw[:, idx], sw[:, ::-1].copy())


def test_planted_mistakes():
    rows = near_tie_rows(n_amax=24, per_row=32)
    assert not check_quant_exact(_quant_mul_reciprocal, rows) or \
        not check_quant_golden(_quant_mul_reciprocal)
    assert not check_quant_golden(_quant_half_away)
    assert not check_quant_golden(_quant_scale_128)
    assert not check_gemm_pins(_gemm_dropped_term)
    assert not check_gemm_pins(_gemm_transposed)
    assert not check_postscale_pins(_post_swapped_scales)
    assert not check_postscale_pins(_post_dropped_weight_scale)
    assert not check_blockwise_pins(_bw_wrong_block_index)
    assert not check_blockwise_pins(_bw_descending)
    assert not check_postscale_bias_pins(_bias_before_weight_scale)
    assert not check_postscale_bias_pins(_bias_after_rounding)
    assert not check_postscale_bias_pins(_bias_by_row)
