"""Pins of the oracle's BF16 distance ruler (``bf16_ulp_distance``).

Every BF16 output comparison reports its distance in BF16 units in the last
place, and the epilogue's tolerance ("TurboDiffusion Integration Notes",
section "Differences From TurboDiffusion": the scales are applied in the
epilogue, which produces BF16) is stated in those units. The ruler is pinned
by

* hand-worked distances (tests/golden/bf16_ulp_worked_examples.txt), counted
  from the BF16 format's binades;
* brute force: the rank of each value along the sorted list of every
  distinct non-NaN BF16 value (built from the values themselves, not from bit
  tricks), whose rank difference is the distance by definition;
* invariants: symmetry, the triangle equality along one side of zero.

``test_ulp_planted_mistakes`` shows that two plausible wrong rulers fail
these pins: a raw bit-pattern difference (it puts -x about 32768 steps from
+x) and a magnitude-only distance (it drops the sign).
"""
from __future__ import annotations

import os

import numpy as np

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden", "bf16_ulp_worked_examples.txt")


def golden_cases():
    out = []
    with open(GOLD) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b, d, _ = (t.strip() for t in line.split("|"))
            out.append((int(a, 16), int(b, 16), int(d)))
    return out


def _values_of_all_patterns():
    """float64 value of every BF16 pattern (NaN where the pattern is NaN)."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    with np.errstate(invalid="ignore"):       # signalling-NaN patterns
        return (bits << np.uint32(16)).astype(np.uint32).view(np.float32).astype(np.float64)


def brute_rank():
    """rank[bits]: position of the value in the sorted list of distinct
    non-NaN BF16 values (+0 and -0 are equal floats, hence one entry)."""
    v = _values_of_all_patterns()
    finite_or_inf = ~np.isnan(v)
    distinct = np.unique(v[finite_or_inf])      # sorted; 0.0 == -0.0 merged
    rank = np.full(v.shape, -1, dtype=np.int64)
    rank[finite_or_inf] = np.searchsorted(distinct, v[finite_or_inf])
    return rank, finite_or_inf


def check_ulp_pins(dist_fn) -> bool:
    for a, b, d in golden_cases():
        got = int(np.asarray(dist_fn(np.array([a], np.uint16), np.array([b], np.uint16)))[0])
        if got != d:
            return False
    rank, ok = brute_rank()
    valid = np.flatnonzero(ok).astype(np.uint16)
    rng = np.random.default_rng(20240601)
    a = rng.choice(valid, size=200_000)
    b = rng.choice(valid, size=200_000)
    # plus every value against its neighbours in bit order and against its negation
    a = np.concatenate([a, valid[:-1], valid])
    b = np.concatenate([b, valid[1:], valid ^ np.uint16(0x8000)])
    want = np.abs(rank[a] - rank[b])
    got = np.asarray(dist_fn(a, b)).astype(np.int64)
    return bool(np.array_equal(got, want))


def test_ulp_golden_and_brute_force():
    assert check_ulp_pins(O.bf16_ulp_distance)


def test_ulp_invariants():
    rank, ok = brute_rank()
    valid = np.flatnonzero(ok).astype(np.uint16)
    rng = np.random.default_rng(7)
    a, b = rng.choice(valid, 50_000), rng.choice(valid, 50_000)
    d_ab = O.bf16_ulp_distance(a, b)
    assert np.array_equal(d_ab, O.bf16_ulp_distance(b, a))
    # negating both values keeps their distance
    assert np.array_equal(d_ab, O.bf16_ulp_distance(a ^ np.uint16(0x8000), b ^ np.uint16(0x8000)))
    # along one side of zero the steps add up: d(a, c) = d(a, b) + d(b, c) for a <= b <= c
    pos = valid[(valid < 0x7F81)]
    s = np.sort(rng.choice(pos, size=(20_000, 3)), axis=1)
    lhs = O.bf16_ulp_distance(s[:, 0], s[:, 2])
    rhs = O.bf16_ulp_distance(s[:, 0], s[:, 1]) + O.bf16_ulp_distance(s[:, 1], s[:, 2])
    assert np.array_equal(lhs, rhs)


# ---------------------------------------------------------------------------
# Planted mistakes
# ---------------------------------------------------------------------------

def _ulp_raw_bits(a, b):
    return np.abs(np.asarray(a, np.int64) - np.asarray(b, np.int64))


def _ulp_magnitude_only(a, b):
    return np.abs((np.asarray(a, np.int64) & 0x7FFF) - (np.asarray(b, np.int64) & 0x7FFF))


def _ulp_two_zeros(a, b):
    # sign-magnitude folded to a line on which -0 and +0 are distinct points
    def key(x):
        x = np.asarray(x, np.int64)
        return np.where(x & 0x8000, -(x & 0x7FFF) - 1, x)
    return np.abs(key(a) - key(b))


def test_ulp_planted_mistakes():
    assert not check_ulp_pins(_ulp_raw_bits)
    assert not check_ulp_pins(_ulp_magnitude_only)
    assert not check_ulp_pins(_ulp_two_zeros)
