"""Plain CPU oracle of the W8A8 INT8 Linear (TEST INFRASTRUCTURE ONLY).

What the method computes, per the pages:

* "TurboDiffusion Integration Notes" (TurboT2AV docs/acceleration.md),
  section "Reused Components", W8A8 Linear bullet: selected weights become
  INT8 once, when the model is initialised; activations are quantised
  dynamically, on every call, right before the transformer Linear.
* Same page, section "Differences From TurboDiffusion", the W8A8-kernel row
  and the paragraph under the table: the post-scale kernel keeps one integer
  accumulation running over the whole K dimension and multiplies the
  activation and weight scales in only in the epilogue; the older TurboDiffusion
  kernel was a blockwise-scaled one.
* Same page, "Reused Components", FastNorm bullet: RMSNorm is replaced by a
  fused implementation; here it is the optional prologue of the activation
  quantisation.

Readings taken where the pages are silent:

R1  scale = absmax / 127, symmetric, no zero point, stored as fp32.
R2  code = round-half-even(fl32(x / scale)), clamped to [-127, 127]. The
    quotient is one IEEE fp32 division by the *stored* scale. This decision
    turns floating point into an integer, so it is taken in fp32, the
    kernel's precision.
R3  an all-zero group has scale 0 and codes 0.
R4  "INT8 accumulation" means exact INT32 sums of INT8 products with no
    rescale inside K.
R5  the post-scale epilogue runs in fp32: bf16(fl32(fl32(fl32(acc)*sa)*sw)).
R6  RMSNorm: r = 1/sqrt(mean_k x^2 + eps), eps an fp32 argument, no bias;
    y = bf16(fl32(fl32(x*r)*gamma)); y is rounded to BF16 before the quant,
    so the fused prologue equals a BF16 RMSNorm followed by the quant.
    r itself is computed in fp64 and rounded once to fp32.
R7  blockwise: 1x128 activation groups and 128x128 weight groups; for each
    128-wide K block, in ascending order, the exact block sum is scaled by
    s = fl32(sa*sw) and accumulated with an fp32 fused multiply-add.
R11 LayerNorm prologue ("Turbodiffusion Video", "Custom Kernel Optimizations":
    mean and variance, normalise, affine; "TurboDiffusion Integration Notes",
    FastNorm bullet: LayerNorm and the LTX modulation helpers are fused):
    mu = mean_k x, var = mean_k (x - mu)^2 (population variance), r =
    1/sqrt(var + eps), both statistics from fp64 sums rounded once to fp32;
    y = bf16(fl32(fl32(fl32(fl32(x - mu) * r) * gamma) + beta)) with an
    optional affine; then an optional adaLN modulation in BF16 tensor
    arithmetic, z = bf16(fl32(bf16(fl32(y * m)) + shift)), m =
    bf16(fl32(1 + scale)), with per-channel scale and shift; then the
    per-token quantisation of z.
R12 bias of an Int8Linear (next row f2: "Reused Components", W8A8 Linear
    bullet, Int8Linear replaces Linear, which may carry a bias): added in fp32
    after both scales, before the one BF16 rounding:
    out = bf16(fl32(fl32(fl32(fl32(acc) * sa) * sw) + bias)).
R13 the FFN activation between the up and down projections (next row f3;
    "Differences From TurboDiffusion", W8A8-kernel row: the kernel is tuned
    for the LTX FFN shapes; the pages do not name the activation): GELU in
    its erf form, GELU(y) = y * Phi(y) = y/2 * erfc(-y/sqrt(2)), applied to
    the BF16 output y of the up projection (post-scale and optional bias as
    R5/R12), evaluated in fp64 and rounded once to BF16. The down
    projection's per-token quantisation (R1-R3) then reads that BF16 tensor.

Floating-point values are BF16 bit patterns (uint16) at the interface.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "QMAX", "BLOCK", "bf16_to_f32", "f32_to_bf16", "quantize_groups",
    "quantize_rows", "rmsnorm_inv_rms", "rmsnorm_bf16", "rmsnorm_quant",
    "layernorm_stats", "layernorm_bf16", "modulate_bf16", "layernorm_quant",
    "gemm_i32", "postscale_bf16", "postscale_bias_bf16", "fma_f32", "gemm_blockwise_bf16",
    "f64_to_bf16", "gelu_f64", "gelu_bf16", "postscale_gelu_bf16",
    "w8a8_linear", "check_gemm_shape", "ShapeError", "bf16_ulp_distance",
]

QMAX = 127          # R1/R2: symmetric INT8 range [-127, 127]
BLOCK = 128         # R7: block edge of the blockwise variant
INT32_MAX = 2**31 - 1


class ShapeError(ValueError):
    """A shape the method (as read here) does not cover."""


# ---------------------------------------------------------------------------
# BF16 <-> fp32
# ---------------------------------------------------------------------------

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns -> float32 values (exact: BF16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bit patterns, round to nearest, ties to even.

    The 16 dropped low bits are compared with one half of the kept last place;
    a tie goes to the even neighbour. NaN stays NaN (quiet).
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    if np.any(nan):
        rounded = np.where(nan, ((u >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint16),
                           rounded)
    return rounded


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> BF16 bit patterns, one rounding (nearest, ties to even).

    Goes through fp32 with round-to-odd: the value is cut toward zero to
    fp32 and, if that was inexact, the last fp32 bit is set. fp32 keeps 16
    more bits than BF16, so the final round-to-nearest-even to BF16 equals a
    direct rounding of the fp64 value (no double-rounding error).
    """
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    over = np.abs(f.astype(np.float64)) > np.abs(x)           # rounded away from zero
    f = np.where(over, np.nextafter(f, np.float32(0)), f).astype(np.float32)
    u = f.view(np.uint32).copy()
    inexact = f.astype(np.float64) != x
    u = np.where(inexact & ~np.isnan(x), u | np.uint32(1), u).astype(np.uint32)
    return f32_to_bf16(u.view(np.float32))


def bf16_ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance in BF16 units in the last place between two BF16 arrays.

    Bit patterns are mapped to a monotone integer line (+0 and -0 coincide),
    so neighbouring BF16 values are 1 apart.
    """
    def key(b):
        b = np.asarray(b, dtype=np.uint16).astype(np.int64)
        mag = b & 0x7FFF
        return np.where(b & 0x8000, -mag, mag)
    return np.abs(key(a_bits) - key(b_bits))


# ---------------------------------------------------------------------------
# Activation / weight quantisation (R1, R2, R3)
# ---------------------------------------------------------------------------

def _quantize_block(x: np.ndarray):
    """Quantise one group of fp32 values that share a single scale."""
    amax = np.max(np.abs(x)) if x.size else np.float32(0)
    amax = np.float32(amax)
    if amax == 0:
        return np.zeros(x.shape, dtype=np.int8), np.float32(0)
    s = np.float32(amax / np.float32(QMAX))          # one fp32 division (R1)
    t = x / s                                        # fp32 division per element (R2)
    q = np.clip(np.rint(t), -QMAX, QMAX).astype(np.int8)
    return q, s


def quantize_groups(x_bits: np.ndarray, group_rows: int, group_cols: int):
    """Symmetric absmax INT8 quantisation over (group_rows x group_cols) groups.

    Per-token activation quant ("Reused Components", W8A8 Linear bullet:
    activations quantised dynamically before each Linear) is group (1, cols);
    per-output-channel weight quant at initialisation is the same with the
    weight's rows; the blockwise variant ("Differences From TurboDiffusion",
    W8A8 kernel row) uses (1, 128) for activations and (128, 128) for weights.

    Returns (q int8 [rows, cols], scale fp32 [ceil(rows/gr), cols/gc]).
    """
    x = bf16_to_f32(x_bits)
    rows, cols = x.shape
    if group_cols <= 0 or cols % group_cols or group_rows <= 0:
        raise ShapeError("group must tile the columns")
    n_gr = -(-rows // group_rows)
    n_gc = cols // group_cols
    q = np.zeros((rows, cols), dtype=np.int8)
    s = np.zeros((n_gr, n_gc), dtype=np.float32)
    for gr in range(n_gr):
        r0, r1 = gr * group_rows, min((gr + 1) * group_rows, rows)
        for gc in range(n_gc):
            c0, c1 = gc * group_cols, (gc + 1) * group_cols
            q[r0:r1, c0:c1], s[gr, gc] = _quantize_block(x[r0:r1, c0:c1])
    return q, s


def quantize_rows(x_bits: np.ndarray):
    """Per-row quantisation, vectorised over rows (same arithmetic as
    ``quantize_groups(x, 1, cols)``): one scale per token / output channel."""
    x = bf16_to_f32(x_bits)
    amax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    amax = amax.astype(np.float32)
    s = (amax / np.float32(QMAX)).astype(np.float32)
    zero = amax == 0
    safe = np.where(zero, np.float32(1), s).astype(np.float32)
    t = x / safe[:, None]
    q = np.clip(np.rint(t), -QMAX, QMAX).astype(np.int8)
    q[zero] = 0
    s[zero] = 0
    return q, s


# ---------------------------------------------------------------------------
# RMSNorm prologue (R6)
# ---------------------------------------------------------------------------

def rmsnorm_inv_rms(x_bits: np.ndarray, eps: float) -> np.ndarray:
    """r[m] = 1 / sqrt(mean_k x[m,k]^2 + eps), in fp64, rounded once to fp32.

    "Reused Components", FastNorm bullet (RMSNorm replaced by a fused
    implementation). Squares of BF16 values are exact in fp64; eps is taken
    as the fp32 value the library receives.
    """
    x = bf16_to_f32(x_bits).astype(np.float64)
    k = x.shape[1]
    ss = np.sum(x * x, axis=1)
    eps64 = float(np.float32(eps))
    return (1.0 / np.sqrt(ss / k + eps64)).astype(np.float32)


def rmsnorm_bf16(x_bits: np.ndarray, gamma_bits: np.ndarray, r: np.ndarray) -> np.ndarray:
    """y = bf16(fl32(fl32(x * r) * gamma)) with the given per-row r (fp32)."""
    x = bf16_to_f32(x_bits)
    g = bf16_to_f32(gamma_bits)
    t = (x * np.asarray(r, dtype=np.float32)[:, None]).astype(np.float32)
    y = (t * g[None, :]).astype(np.float32)
    return f32_to_bf16(y)


def rmsnorm_quant(x_bits: np.ndarray, gamma_bits: np.ndarray, eps: float,
                  r: np.ndarray | None = None):
    """RMSNorm prologue followed by per-token quantisation.

    With ``r`` given (e.g. the inv_rms a device kernel reports), everything
    downstream of r is recomputed from it, so codes and scales can be compared
    bit for bit even though the fp32 reduction order of r is not fixed.
    Returns (q, s, r).
    """
    if r is None:
        r = rmsnorm_inv_rms(x_bits, eps)
    y = rmsnorm_bf16(x_bits, gamma_bits, r)
    q, s = quantize_rows(y)
    return q, s, np.asarray(r, dtype=np.float32)


# ---------------------------------------------------------------------------
# LayerNorm + adaLN modulation prologue (R11)
# ---------------------------------------------------------------------------

def layernorm_stats(x_bits: np.ndarray, eps: float):
    """mu[m] = mean_k x[m,k] and r[m] = 1 / sqrt(mean_k (x - mu)^2 + eps).

    "Turbodiffusion Video", "Custom Kernel Optimizations": a LayerNorm takes
    the mean and the variance of each row, normalises, then applies the
    affine step. The variance is the population one (divided by K). Both are
    computed from fp64 sums and rounded once to fp32; eps is the fp32 value
    the library receives. Returns (mu, r) as fp32 vectors.
    """
    x = bf16_to_f32(x_bits).astype(np.float64)
    k = x.shape[1]
    mu = np.sum(x, axis=1) / k
    d = x - mu[:, None]
    var = np.sum(d * d, axis=1) / k
    eps64 = float(np.float32(eps))
    return mu.astype(np.float32), (1.0 / np.sqrt(var + eps64)).astype(np.float32)


def layernorm_bf16(x_bits: np.ndarray, mu: np.ndarray, r: np.ndarray,
                   gamma_bits: np.ndarray | None = None,
                   beta_bits: np.ndarray | None = None) -> np.ndarray:
    """y = bf16(fl32(fl32(fl32(fl32(x - mu) * r) * gamma) + beta)).

    The given per-row mu and r (fp32) are used as they are; without gamma
    (beta) that step is left out, which is the same as gamma = 1 (beta = 0)
    up to the sign of a zero.
    """
    x = bf16_to_f32(x_bits)
    mu = np.asarray(mu, dtype=np.float32)[:, None]
    r = np.asarray(r, dtype=np.float32)[:, None]
    u = ((x - mu).astype(np.float32) * r).astype(np.float32)
    if gamma_bits is not None:
        u = (u * bf16_to_f32(gamma_bits)[None, :]).astype(np.float32)
    if beta_bits is not None:
        u = (u + bf16_to_f32(beta_bits)[None, :]).astype(np.float32)
    return f32_to_bf16(u)


def modulate_bf16(y_bits: np.ndarray, scale_bits: np.ndarray | None = None,
                  shift_bits: np.ndarray | None = None) -> np.ndarray:
    """adaLN modulation as BF16 tensor arithmetic, each operation rounded to BF16:
    m = bf16(fl32(1 + scale)), z = bf16(fl32(bf16(fl32(y * m)) + shift)).

    "TurboDiffusion Integration Notes", FastNorm bullet (the LTX modulation
    helpers are fused with the norms). scale and shift are per channel; a
    missing one leaves its step out.
    """
    z = bf16_to_f32(y_bits)
    if scale_bits is not None:
        m = bf16_to_f32(f32_to_bf16((np.float32(1) + bf16_to_f32(scale_bits)).astype(np.float32)))
        z = bf16_to_f32(f32_to_bf16((z * m[None, :]).astype(np.float32)))
    if shift_bits is not None:
        z = bf16_to_f32(f32_to_bf16((z + bf16_to_f32(shift_bits)[None, :]).astype(np.float32)))
    return f32_to_bf16(z)


def layernorm_quant(x_bits: np.ndarray, eps: float, gamma_bits=None, beta_bits=None,
                    scale_bits=None, shift_bits=None, mu=None, r=None):
    """LayerNorm, adaLN modulation, then per-token quantisation.

    With ``mu`` and ``r`` given (the statistics a device kernel reports),
    everything downstream of them is recomputed from them, so codes and scales
    can be compared bit for bit although the fp32 reduction order of the
    statistics is not fixed. Returns (q, s, mu, r).
    """
    if mu is None or r is None:
        mu0, r0 = layernorm_stats(x_bits, eps)
        mu = mu0 if mu is None else mu
        r = r0 if r is None else r
    y = layernorm_bf16(x_bits, mu, r, gamma_bits, beta_bits)
    z = modulate_bf16(y, scale_bits, shift_bits)
    q, s = quantize_rows(z)
    return q, s, np.asarray(mu, dtype=np.float32), np.asarray(r, dtype=np.float32)


# ---------------------------------------------------------------------------
# INT8 x INT8 -> INT32 GEMM (R4)
# ---------------------------------------------------------------------------

def gemm_i32(qa: np.ndarray, qw: np.ndarray, row_block: int = 2048) -> np.ndarray:
    """acc[m,n] = sum_k qa[m,k] * qw[n,k], exact.

    "Differences From TurboDiffusion", paragraph under the table: a single
    accumulation over the whole K, scales applied afterwards. The sum is
    formed with an fp64 matrix product: every product is an integer of
    magnitude <= 127^2 and every partial sum an integer below 2^53, so any
    summation order (and any fused multiply-add) is exact.
    """
    qa = np.asarray(qa, dtype=np.int8)
    qw = np.asarray(qw, dtype=np.int8)
    M, K = qa.shape
    N, K2 = qw.shape
    if K != K2:
        raise ShapeError("K mismatch")
    if QMAX * QMAX * K >= 2**53:
        raise ShapeError("K too large for an exact fp64 sum")
    wt = qw.astype(np.float64).T
    out = np.empty((M, N), dtype=np.int64)
    for r0 in range(0, M, row_block):
        r1 = min(r0 + row_block, M)
        out[r0:r1] = (qa[r0:r1].astype(np.float64) @ wt).astype(np.int64)
    if out.size and np.max(np.abs(out)) > INT32_MAX:
        raise OverflowError("INT32 accumulator overflow")
    return out.astype(np.int32)


# ---------------------------------------------------------------------------
# Post-scale epilogue (R5)
# ---------------------------------------------------------------------------

def postscale_bf16(acc: np.ndarray, sa: np.ndarray, sw: np.ndarray) -> np.ndarray:
    """out[m,n] = bf16(fl32(fl32(fl32(acc[m,n]) * sa[m]) * sw[n])).

    "Differences From TurboDiffusion": activation and weight scales are
    applied in the epilogue; output is BF16.
    """
    a = np.asarray(acc, dtype=np.int32).astype(np.float32)      # RN int32 -> fp32
    t = (a * np.asarray(sa, dtype=np.float32)[:, None]).astype(np.float32)
    v = (t * np.asarray(sw, dtype=np.float32)[None, :]).astype(np.float32)
    return f32_to_bf16(v)


def postscale_bias_bf16(acc: np.ndarray, sa: np.ndarray, sw: np.ndarray,
                        bias_bits: np.ndarray) -> np.ndarray:
    """out[m,n] = bf16(fl32(fl32(fl32(fl32(acc[m,n]) * sa[m]) * sw[n]) + bias[n])).

    R12: an Int8Linear's bias joins the post-scale epilogue in fp32, so the
    output is rounded to BF16 once, as a BF16 Linear with bias is.
    """
    a = np.asarray(acc, dtype=np.int32).astype(np.float32)
    t = (a * np.asarray(sa, dtype=np.float32)[:, None]).astype(np.float32)
    v = (t * np.asarray(sw, dtype=np.float32)[None, :]).astype(np.float32)
    v = (v + bf16_to_f32(bias_bits)[None, :]).astype(np.float32)
    return f32_to_bf16(v)


def gelu_f64(y_bits: np.ndarray) -> np.ndarray:
    """GELU(y) = y * Phi(y) = y/2 * erfc(-y / sqrt(2)) in fp64 on BF16 values y
    (R13). erfc rather than 1 + erf, which loses all its digits for large
    negative y."""
    from scipy.special import erfc
    y = bf16_to_f32(y_bits).astype(np.float64)
    return 0.5 * y * erfc(-y / np.sqrt(2.0))


def gelu_bf16(y_bits: np.ndarray) -> np.ndarray:
    """h = bf16(GELU(y)) (R13): the fp64 value rounded once to BF16."""
    return f64_to_bf16(gelu_f64(y_bits))


def postscale_gelu_bf16(acc: np.ndarray, sa: np.ndarray, sw: np.ndarray,
                        bias_bits: np.ndarray | None = None) -> np.ndarray:
    """The up projection with its activation (R13): GELU of the BF16 post-scale
    output (R5, or R12 with a bias)."""
    if bias_bits is None:
        return gelu_bf16(postscale_bf16(acc, sa, sw))
    return gelu_bf16(postscale_bias_bf16(acc, sa, sw, bias_bits))


# ---------------------------------------------------------------------------
# Blockwise-scaled variant (R7)
# ---------------------------------------------------------------------------

def _round_f64_to_f32_exact(hi: np.ndarray, lo: np.ndarray) -> np.ndarray:
    """Round the exact value hi + lo to fp32 (nearest, ties to even).

    hi = fl64(hi + lo) and lo is its exact error (|lo| <= ulp64(hi)/2). Rounding
    hi alone is right unless hi sits exactly half-way between two fp32 values
    and lo != 0; then the exact value lies on lo's side of that midpoint.
    """
    r = hi.astype(np.float32)
    r64 = r.astype(np.float64)
    toward = np.where(r64 > hi, np.float32(-np.inf), np.float32(np.inf)).astype(np.float32)
    other = np.nextafter(r, toward).astype(np.float32)
    other64 = other.astype(np.float64)
    midpoint = (r64 != hi) & (np.abs(r64 - hi) == np.abs(other64 - hi))
    fix = midpoint & (lo != 0)
    # pick the neighbour on the side lo points to
    up = np.where(r64 > other64, r, other)
    dn = np.where(r64 > other64, other, r)
    return np.where(fix, np.where(lo > 0, up, dn), r).astype(np.float32)


def fma_f32(a: np.ndarray, b: np.ndarray, c: np.ndarray) -> np.ndarray:
    """fp32 fused multiply-add, rounded once: RN32(a*b + c).

    a*b of two fp32 values is exact in fp64 (48 significant bits); the sum
    with c is formed in fp64 together with its exact rounding error (Knuth's
    TwoSum), and the exact total is rounded to fp32 once.
    """
    a = np.asarray(a, dtype=np.float32).astype(np.float64)
    b = np.asarray(b, dtype=np.float32).astype(np.float64)
    c = np.asarray(c, dtype=np.float32).astype(np.float64)
    p = a * b
    s = p + c
    bp = s - c
    err = (p - bp) + (c - (s - bp))
    return _round_f64_to_f32_exact(s, err)


def gemm_blockwise_bf16(qa: np.ndarray, sa: np.ndarray, qw: np.ndarray,
                        sw: np.ndarray) -> np.ndarray:
    """Blockwise-scaled W8A8 GEMM (the original TurboDiffusion kernel's scheme,
    "Differences From TurboDiffusion", W8A8 kernel row).

    qa [M,K] int8 with sa [M, K/128] fp32; qw [N,K] int8 with sw [N/128, K/128].
    For kb = 0, 1, ... in order: acc_kb = exact block sum (|acc_kb| <= 127^2*128
    < 2^24, so fl32(acc_kb) is exact); s = fl32(sa[m,kb] * sw[n//128,kb]);
    c = fma_f32(acc_kb, s, c). Output bf16(c).
    """
    qa = np.asarray(qa, dtype=np.int8)
    qw = np.asarray(qw, dtype=np.int8)
    M, K = qa.shape
    N = qw.shape[0]
    if K % BLOCK or N % BLOCK:
        raise ShapeError("blockwise needs K and N multiples of 128")
    nkb = K // BLOCK
    sa = np.asarray(sa, dtype=np.float32).reshape(M, nkb)
    sw = np.asarray(sw, dtype=np.float32).reshape(N // BLOCK, nkb)
    c = np.zeros((M, N), dtype=np.float32)
    nblk = np.arange(N) // BLOCK
    for kb in range(nkb):
        k0, k1 = kb * BLOCK, (kb + 1) * BLOCK
        acc = gemm_i32(qa[:, k0:k1], qw[:, k0:k1]).astype(np.float32)
        s = (sa[:, kb][:, None] * sw[nblk, kb][None, :]).astype(np.float32)
        c = fma_f32(acc, s, c)
    return f32_to_bf16(c)


# ---------------------------------------------------------------------------
# Composition and shape rules
# ---------------------------------------------------------------------------

def check_gemm_shape(M: int, N: int, K: int) -> None:
    """Shapes the INT8 GEMMs cover: K and N multiples of 128 (anything else is
    left to the caller's native BF16 Linear, "Reused Components", W8A8 Linear
    bullet), M >= 1 arbitrary, and K small enough that the INT32 sum cannot
    overflow (127^2 * K <= 2^31 - 1)."""
    if M < 1 or N < 1 or K < 1:
        raise ShapeError("empty GEMM")
    if K % BLOCK or N % BLOCK:
        raise ShapeError("K and N must be multiples of 128")
    if QMAX * QMAX * K > INT32_MAX:
        raise ShapeError("K too large for an INT32 accumulator")


def w8a8_linear(x_bits: np.ndarray, w_bits: np.ndarray, bias_bits: np.ndarray | None = None):
    """Whole W8A8 Linear: per-channel weight quant (init), per-token activation
    quant (per call), exact INT32 GEMM, fp32 post-scale (and bias, R12) to BF16.
    Returns (out_bits, qa, sa, qw, sw, acc)."""
    qw, sw = quantize_rows(w_bits)
    qa, sa = quantize_rows(x_bits)
    acc = gemm_i32(qa, qw)
    if bias_bits is None:
        return postscale_bf16(acc, sa, sw), qa, sa, qw, sw, acc
    return postscale_bias_bf16(acc, sa, sw, bias_bits), qa, sa, qw, sw, acc

