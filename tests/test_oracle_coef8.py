"""Pins of the oracle's 8-bit blockwise coefficient form (the paper's §3,
second paragraph: coefficients stored in 8-bit blockwise quantised form;
one block = one token's r coefficients, one fp16 scale per token and Z).
CPU only."""
import numpy as np
import pytest

import oracle
from workload.gen import gen_layer, gen_query, make_bases, gen_append_inputs
from tests.helpers import dense_from_logical, sdpa_fp64, tiny_config
from tests.test_oracle_encoder_order import (exact_steps_1_2, fma_units, round_binary32, to_units,
                                             units_to_f32)


def _cfg(**kw):
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=32, r_max=16, tier_rank=(4, 8, 16),
                tier_prob=(0.5, 0.3, 0.2), resid_channels=3, resid_bits=4, n_tokens=40, coef_bits=8)
    base.update(kw)
    return tiny_config(**base)


def test_decode_with_8bit_coefficients_equals_sdpa_on_materialised_cache():
    cfg = _cfg()
    bases = make_bases(cfg)
    lay = gen_layer(cfg, 1)
    assert lay["coefK"].dtype == np.int8 and "cscaleK" in lay
    q = gen_query(cfg, 1, peak=4.0)
    K = dense_from_logical(cfg, lay, bases["K"][0], "K")
    V = dense_from_logical(cfg, lay, bases["V"][0], "V")
    ref = sdpa_fp64(q, K, V, lay["n_tokens"], 1.0 / np.sqrt(cfg.head_dim))
    got = oracle.decode(cfg, lay, bases["K"][0], bases["V"][0], q)
    assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())
    Km, Vm = oracle.materialize(cfg, lay, bases["K"][0], bases["V"][0])
    assert np.abs(Km - K).max() <= 1e-12 and np.abs(Vm - V).max() <= 1e-12


def test_identity_basis_encoding_by_hand():
    """B = I: the step-1 sums are x[:r] exactly; scale fp16(max|x[:r]|/127),
    codes rint(x_i / scale) (half to even), the residual x minus the
    dequantised coefficients; the s kept channels by |e| (ties: smaller j)."""
    rng = np.random.default_rng(3)
    d, r, s = 32, 8, 4
    basis = np.eye(d, dtype=np.float16)
    for _ in range(20):
        x = rng.standard_normal(d).astype(np.float16)
        c, idx, val, scale, cs = oracle.append_vector(basis, x, r, s, 7, coef_bits=8)
        xr = x[:r].astype(np.float32)
        cs_ref = (np.abs(xr).max() / np.float32(127)).astype(np.float16)
        assert cs.view(np.uint16) == cs_ref.view(np.uint16)
        codes = np.clip(np.rint(xr / np.float32(cs_ref)), -127, 127).astype(np.int8)
        assert np.array_equal(c, codes)
        e = x.astype(np.float32).copy()
        e[:r] = xr - codes.astype(np.float32) * np.float32(cs_ref)
        assert np.array_equal(oracle.append_residual(basis, x, r, coef_bits=8), e)
        order = sorted(range(d), key=lambda j: (-abs(float(e[j])), j))[:s]
        assert list(idx) == sorted(order)


@pytest.mark.parametrize("r", [8, 16, 32, 64])
def test_step2_against_exact_chain_with_dequantised_coefficients(r):
    """General orthonormal fp16 basis: the residual equals the exact-integer
    fused multiply-add chain over the dequantised coefficients (codes times
    the block scale, exact in fp32)."""
    cfg = tiny_config(head_dim=128, r_max=64, num_kv_heads=2)
    bases = make_bases(cfg)
    basis = bases["K"][0, 1]
    x = (np.random.default_rng(r).standard_normal(128)).astype(np.float16)
    sums, _, _ = exact_steps_1_2(basis, x, r)
    amax = np.float32(np.abs(sums).max())
    cs = (amax / np.float32(127)).astype(np.float16)
    codes = np.clip(np.rint(sums / np.float32(cs)), -127, 127)
    c_deq = (codes * np.float32(cs)).astype(np.float32)
    c, *_ , cs_got = oracle.append_vector(basis, x, r, 0, 7, coef_bits=8)
    assert cs_got.view(np.uint16) == cs.view(np.uint16)
    assert np.array_equal(c.astype(np.float32), codes.astype(np.float32))
    C = [to_units(v) for v in c_deq]
    X = [to_units(v) for v in x]
    e = []
    for j in range(128):
        acc = 0
        for i in range(r):
            acc = fma_units(to_units(basis[i, j]), C[i], acc)
        e.append(units_to_f32(round_binary32(X[j] - acc)))
    assert np.array_equal(oracle.append_residual(basis, x, r, coef_bits=8).view(np.uint32),
                          np.array(e, np.float32).view(np.uint32))


def test_coefficient_quantisation_bound():
    cfg = tiny_config(head_dim=128, r_max=64)
    B = make_bases(cfg)["V"][0, 0]
    rng = np.random.default_rng(11)
    for _ in range(100):
        x = (rng.standard_normal(128) * rng.choice([0.01, 1.0, 30.0])).astype(np.float16)
        r = int(rng.choice([8, 16, 32, 64]))
        c, _, _, _, cs = oracle.append_vector(B, x, r, 0, 7, coef_bits=8)
        sums = oracle.append_projection(B, x, r).astype(np.float64)
        sc = float(cs)
        assert np.abs(c.astype(int)).max() <= 127
        bound = sc / 2 + np.abs(sums).max() * 2.0 ** -11 * 1.01 + 1e-30
        assert np.abs(c.astype(np.float64) * sc - sums).max() <= bound
    # an all-zero projection: scale 0, codes 0
    c, _, _, _, cs = oracle.append_vector(np.eye(16, dtype=np.float16), np.zeros(16, np.float16), 8, 0, 7,
                                          coef_bits=8)
    assert float(cs) == 0.0 and not c.any()


def test_coefficient_codes_round_half_to_even():
    """Planted ties: with B = I and x[:4] = (127, 2.5, -3.5, 0.5) * 2^-6 the
    block scale is 2^-6 exactly and the codes are 127, 2, -4, 0."""
    d = 16
    basis = np.eye(d, dtype=np.float16)
    x = np.zeros(d, np.float16)
    x[:4] = np.array([127, 2.5, -3.5, 0.5]) * 2.0 ** -6
    c, _, _, _, cs = oracle.append_vector(basis, x, 4, 0, 7, coef_bits=8)
    assert float(cs) == 2.0 ** -6
    assert list(c) == [127, 2, -4, 0]
