"""Pins of oracle.append_vector (CPU): exact bases, brute force, bounds, ties."""
import itertools

import numpy as np
import pytest

import oracle
from workload import make_bases
from tests.helpers import signed_permutation_basis, tiny_config


def _rand_x(rng, d, scale=1.0):
    return (rng.standard_normal(d) * scale).astype(np.float16)


@pytest.mark.parametrize("bits,qmax", [(4, 7), (8, 127)])
@pytest.mark.parametrize("seed", range(6))
def test_identity_basis_by_hand(bits, qmax, seed):
    """B = I: c = x[:r]; the residual is x on channels >= r; the kept channels
    are the s largest |x_j| there (ties to the smaller j); one fp16 scale
    max|x_S|/qmax; codes rint(x_j/scale) -- all checked with NumPy fp32."""
    rng = np.random.default_rng(seed)
    d, r, s = 32, 8, 5
    basis = np.eye(d, dtype=np.float16)
    x = _rand_x(rng, d)
    c, idx, val, scale = oracle.append_vector(basis, x, r, s, qmax)
    assert np.array_equal(c.view(np.uint16), x[:r].view(np.uint16))
    tail = np.abs(x[r:].astype(np.float32))
    order = sorted(range(d - r), key=lambda j: (-tail[j], j))[:s]
    S = np.sort(np.asarray(order) + r)
    assert np.array_equal(idx, S.astype(np.uint8))
    amax = np.float32(np.abs(x[S].astype(np.float32)).max())
    s16 = (amax / np.float32(qmax)).astype(np.float16)
    assert scale.view(np.uint16) == s16.view(np.uint16)
    ref = np.clip(np.rint(x[S].astype(np.float32) / np.float32(s16)), -qmax, qmax).astype(np.int8)
    assert np.array_equal(val, ref)


def test_signed_permutation_basis_projects_exactly():
    rng = np.random.default_rng(3)
    d, R = 64, 32
    basis, perm, sign = signed_permutation_basis(d, R, 9)
    for r in (4, 16, 32):
        x = _rand_x(rng, d)
        c, idx, val, scale = oracle.append_vector(basis, x, r, 0, 7)
        assert np.array_equal(c.astype(np.float32), (sign[:r] * x[perm[:r]].astype(np.float32)))
        e = oracle.append_residual(basis, x, r)
        ref = x.astype(np.float32).copy()
        ref[perm[:r]] = 0
        assert np.array_equal(e, ref)
        assert scale == 0


def test_residual_matches_projection_residual_in_fp64():
    """General orthonormal basis: e = x - B^T fp16(B x) up to fp32 rounding."""
    cfg = tiny_config(head_dim=128, r_max=64)
    bases = make_bases(cfg)
    B = bases["K"][0, 0]
    rng = np.random.default_rng(5)
    Bd = B.astype(np.float64)
    for r in (8, 16, 32, 64):
        x = _rand_x(rng, 128)
        c, *_ = oracle.append_vector(B, x, r, 0, 7)
        cref = (Bd[:r] @ x.astype(np.float64))
        assert np.abs(c.astype(np.float64) - cref).max() <= 2e-3 * max(1.0, np.abs(cref).max())
        e = oracle.append_residual(B, x, r).astype(np.float64)
        eref = x.astype(np.float64) - Bd[:r].T @ c.astype(np.float64)
        assert np.abs(e - eref).max() <= 1e-5


@pytest.mark.parametrize("seed", range(20))
def test_kept_channels_are_best_subset_by_brute_force(seed):
    """d=8, s=2: over all 28 subsets the kept one leaves the least residual
    energy (largest sum of e_j^2 kept) -- the error-minimising choice."""
    rng = np.random.default_rng(100 + seed)
    d, R = 8, 4
    g = np.linalg.qr(rng.standard_normal((d, R)))[0]
    basis = g.T.astype(np.float16)
    x = _rand_x(rng, d)
    for r in (0, 2, 4):
        c, idx, val, scale = oracle.append_vector(basis, x, r, 2, 127)
        e = oracle.append_residual(basis, x, r).astype(np.float64)
        best = max(float(e[list(S)] @ e[list(S)]) for S in itertools.combinations(range(d), 2))
        assert float(e[idx] @ e[idx]) == best


@pytest.mark.parametrize("qmax", [7, 127])
def test_quantisation_error_bound(qmax):
    rng = np.random.default_rng(qmax)
    cfg = tiny_config(head_dim=128, r_max=64)
    B = make_bases(cfg)["V"][0, 1]
    for trial in range(200):
        x = _rand_x(rng, 128, scale=rng.choice([1e-3, 0.1, 1.0, 10.0]))
        r = int(rng.choice([8, 16, 32, 64]))
        c, idx, val, scale = oracle.append_vector(B, x, r, 8, qmax)
        e = oracle.append_residual(B, x, r).astype(np.float64)
        sc = float(scale)
        assert np.abs(val.astype(int)).max() <= qmax
        amax = np.abs(e[idx]).max()
        # half a step, plus the fp16 rounding of the scale on the largest code
        bound = sc / 2 + amax * 2.0 ** -11 * 1.01 + 1e-30
        assert np.abs(sc * val - e[idx]).max() <= bound
        # no unkept channel is larger than a kept one
        rest = np.delete(np.abs(e), idx)
        assert rest.max() <= np.abs(e[idx]).min()


def test_ties_prefer_smaller_channel_and_zero_residual():
    d = 16
    basis = np.eye(d, dtype=np.float16)
    x = np.zeros(d, np.float16)
    x[[3, 5, 9, 12]] = [0.5, -0.5, 0.5, 0.25]
    c, idx, val, scale = oracle.append_vector(basis, x, 2, 2, 7)
    assert list(idx) == [3, 5]
    assert float(scale) == float(np.float16(np.float32(0.5) / np.float32(7)))
    # residual exactly zero: scale 0 and all codes 0; kept channels are 0..s-1
    x2 = np.zeros(d, np.float16)
    x2[:4] = [1, 2, 3, 4]
    c, idx, val, scale = oracle.append_vector(basis, x2, 4, 3, 7)
    assert float(scale) == 0.0 and not val.any() and list(idx) == [0, 1, 2]


def test_gate_is_folded_into_scale():
    rng = np.random.default_rng(17)
    d = 32
    basis = np.eye(d, dtype=np.float16)
    x = _rand_x(rng, d)
    _, idx1, val1, s1 = oracle.append_vector(basis, x, 4, 4, 7)
    for gbits in (np.float16(0.5), np.float16(0.3), np.float16(0.0)):
        _, idx, val, s = oracle.append_vector(basis, x, 4, 4, 7, gate=gbits)
        assert np.array_equal(idx, idx1) and np.array_equal(val, val1)
        assert s.view(np.uint16) == (np.float32(gbits) * np.float32(s1)).astype(np.float16).view(np.uint16)
    _, _, _, s_one = oracle.append_vector(basis, x, 4, 4, 7, gate=np.float16(1.0))
    assert s_one.view(np.uint16) == s1.view(np.uint16)


def test_rejects_invalid_arguments():
    basis = np.eye(8, dtype=np.float16)
    x = np.zeros(8, np.float16)
    with pytest.raises(ValueError):
        oracle.append_vector(basis, x, 9, 1, 7)      # rank above the basis width
    with pytest.raises(ValueError):
        oracle.append_vector(basis, x, 2, 9, 7)      # more channels than d


def test_codes_round_half_to_even():
    """Codes that land exactly on k + 1/2 steps round to the even integer."""
    d = 16
    basis = np.eye(d, dtype=np.float16)
    x = np.zeros(d, np.float16)
    step = 2.0 ** -6
    # kept: 7 steps (sets scale = step exactly), 2.5, -3.5, 0.5 steps
    x[[4, 6, 8, 10]] = np.array([7, 2.5, -3.5, 0.5]) * step
    c, idx, val, scale = oracle.append_vector(basis, x, 2, 4, 7)
    assert float(scale) == step
    assert list(idx) == [4, 6, 8, 10]
    assert list(val) == [7, 2, -4, 0]
