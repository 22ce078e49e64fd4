"""Pins the encoder's fixed fp32 operation order (CPU, no GPU).

The encoding of a new token (DepthWeave-KV paper, §3 Method, second
paragraph: coefficients by projecting the vector onto the current basis,
then the residual of that projection) makes integer decisions, so the
oracle fixes its arithmetic: IEEE binary32, sequential fused multiply-adds
in ascending index order, each rounded once to nearest-even.

This test recomputes steps 1 and 2 with exact integer arithmetic and one
rounding per fused multiply-add written from the IEEE 754 definition of
binary32 (24-bit significand; the smallest quantum is 2^-149), independent
of any floating-point unit.  It runs on general (non-sparse) orthonormal
fp16 bases of the Llama-3-8B workloads at ranks 8 to 64, where a different
order or a wider accumulator changes bits.  The oracle's fp32 sums of
step 1, its fp16 coefficients and its fp32 residual must match bit for bit.

Every product the encoder forms is of two fp16 values (basis entries times
input components, or times fp16 coefficients), and binary32 holds such a
product exactly (at most 22 significant bits, magnitude at least 2^-48), so
a fused multiply-add and a multiply followed by an add round identically;
the last test here checks that exactness.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workload as w
from workload.gen import gen_append_inputs, make_bases

Q = 149                       # binary32's smallest quantum is 2^-149


def to_units(v) -> int:
    """An exactly representable fp16/fp32 value as an integer count of 2^-149."""
    f = Fraction(float(v)) * (1 << Q)
    assert f.denominator == 1
    return int(f.numerator)


def round_binary32(n: int) -> int:
    """Round n * 2^-149 to the nearest binary32 value (ties to the even
    significand), returned in the same units.  Below 2^-126 (n < 2^23) every
    multiple of 2^-149 is representable; above, a value keeps its 24 leading
    significant bits."""
    a = abs(n)
    drop = a.bit_length() - 24
    if drop <= 0:
        return n
    q, rem = divmod(a, 1 << drop)
    half = 1 << (drop - 1)
    if rem > half or (rem == half and q & 1):
        q += 1
    r = q << drop
    return r if n >= 0 else -r


def fma_units(a: int, b: int, c: int) -> int:
    """fmaf(a, b, c): the exact a*b + c, rounded once."""
    p = a * b
    assert p % (1 << Q) == 0          # fp16 x fp16 products are multiples of 2^-48
    return round_binary32(p // (1 << Q) + c)


def units_to_f32(n: int) -> np.float32:
    v = np.float32(Fraction(n, 1 << Q))
    assert to_units(v) == n
    return v


def exact_steps_1_2(basis16: np.ndarray, x16: np.ndarray, r: int):
    """Steps 1-2 of the encoder: step-1 sums (fp32), c (fp16), e (fp32)."""
    R, d = basis16.shape
    B = [[to_units(basis16[i, j]) for j in range(d)] for i in range(r)]
    X = [to_units(x16[j]) for j in range(d)]
    sums, c16, C = [], [], []
    for i in range(r):
        acc = 0
        for j in range(d):                    # ascending j
            acc = fma_units(B[i][j], X[j], acc)
        s32 = units_to_f32(acc)
        sums.append(s32)
        h = s32.astype(np.float16)            # round to nearest even (library conversion)
        c16.append(h)
        C.append(to_units(h))
    e = []
    for j in range(d):
        acc = 0
        for i in range(r):                    # ascending i
            acc = fma_units(B[i][j], C[i], acc)
        e.append(units_to_f32(round_binary32(X[j] - acc)))
    return (np.array(sums, np.float32), np.array(c16, np.float16), np.array(e, np.float32))


def test_binary32_rounding_matches_the_definition_on_known_cases():
    """The integer rounding reproduces a few values fixed by the format:
    1 + 2^-24 is a tie between 1 and 1 + 2^-23 (even: 1); 1 + 3*2^-24 rounds
    to 1 + 2^-22; the smallest subnormal stays; signs are symmetric."""
    one = 1 << Q
    assert round_binary32(one + (1 << (Q - 24))) == one
    assert round_binary32(one + 3 * (1 << (Q - 24))) == one + (1 << (Q - 22))
    assert round_binary32(1) == 1
    assert round_binary32(-(one + (1 << (Q - 24)))) == -one
    # against the hardware conversion from fp64 (a library routine) on random
    # values that sit between binary32 neighbours
    rng = np.random.default_rng(0)
    for _ in range(2000):
        v = float(rng.standard_normal()) * 2.0 ** int(rng.integers(-30, 30))
        n = int(Fraction(v) * (1 << Q))
        if Fraction(v) * (1 << Q) != n:
            continue
        assert units_to_f32(round_binary32(n)) == np.float32(v)


@pytest.mark.parametrize("ci", [1, 2])
@pytest.mark.parametrize("r", [8, 16, 32, 64])
def test_encoder_steps_match_exact_fma_chain(ci, r):
    cfg = w.get_config(ci)
    bases = make_bases(cfg)
    a = gen_append_inputs(cfg, layer=4 * ci + 1, step=r, bases=bases)
    m = (4 * ci + 1) // cfg.layers_per_group
    checked = 0
    for zi, z in enumerate("KV"):
        h = (r // 8 + zi) % cfg.num_kv_heads
        basis = bases[z][m, h]
        x = a[z.lower()][0, h]
        sums, c16, e = exact_steps_1_2(basis, x, r)
        got_sums = oracle.append_projection(basis, x, r)
        assert np.array_equal(got_sums.view(np.uint32), sums.view(np.uint32)), f"{z}: step-1 sums"
        c, *_ = oracle.append_vector(basis, x, r, 0, cfg.qmax)
        assert np.array_equal(c.view(np.uint16), c16.view(np.uint16)), f"{z}: coefficients"
        got_e = oracle.append_residual(basis, x, r)
        assert np.array_equal(got_e.view(np.uint32), e.view(np.uint32)), f"{z}: residual"
        checked += 1
    assert checked == 2


def test_fp16_products_are_exact_in_binary32():
    """Products of two finite fp16 values: at most 11 + 11 significant bits
    and at least 2^-24 * 2^-24, so binary32 represents each one exactly -- a
    fused and an unfused multiply-add give the same bits in steps 1-2.
    Checked on every pair of fp16 significands (exponents only shift) and on
    extreme exponents."""
    sig = np.arange(1024, 2048, dtype=np.int64)            # normal significands
    prod = np.multiply.outer(sig, sig).reshape(-1)
    # significant bits of each product, trailing zeros stripped
    odd = prod // (prod & -prod)
    assert int(odd.max()).bit_length() <= 22
    sub = np.arange(1, 1024, dtype=np.int64)               # subnormal significands
    odd2 = np.multiply.outer(sub, sig).reshape(-1)
    odd2 = odd2 // (odd2 & -odd2)
    assert int(odd2.max()).bit_length() <= 22
    for a, b in [(2.0 ** -24, 2.0 ** -24), (65504.0, 65504.0), (2.0 ** -24, 65504.0),
                 (np.float16(0.1), np.float16(-0.3))]:
        p = to_units(np.float16(a)) * to_units(np.float16(b))
        assert p % (1 << Q) == 0
        n = p // (1 << Q)
        assert round_binary32(n) == n
