"""Pins of the prefill oracle (oracle/prefill.py), CPU only.

The range finder is pinned against what the mathematics fixes: NumPy's
Householder QR (orth spans the same columns), LAPACK's symmetric
eigensolver on the full Gram matrix (the converged subspace and Ritz
values), the SVD of exactly low-rank data, a diagonal Gram matrix whose
basis is known by hand, Cauchy interlacing and the Ky Fan bound (no
subspace captures more energy than the top eigenvectors), orthonormality,
the sign and order conventions, and the exclusion of positions beyond a
sequence's length.  The bulk encoder is pinned as the composition it is
(each token one append) and by hand on identity bases.  The last test
plants mistakes in a copy of the module and checks that these pins catch
each one."""
import importlib.util
import inspect
import os
import sys

import numpy as np
import pytest

import oracle
import oracle.prefill as PF
import workload as w
from tests.helpers import tiny_config


def _cfg(**kw):
    base = dict(batch=2, num_layers=4, layers_per_group=2, num_q_heads=4, num_kv_heads=2, head_dim=32,
                r_max=8, tier_rank=(2, 4, 8), tier_prob=(0.5, 0.3, 0.2), resid_channels=3, resid_bits=4,
                n_tokens=300)
    base.update(kw)
    return tiny_config(**base)


def _proj(B):
    """Orthogonal projector onto the row space of B [r][d] (rows orthonormal)."""
    return B.T @ B


def _gram_with_spectrum(rng, d, lam):
    U, _ = np.linalg.qr(rng.standard_normal((d, d)))
    return (U * lam[None, :]) @ U.T, U


# ------------------------------------------------------------------ orth
def pin_orth_spans_like_householder_qr(P=PF):
    rng = np.random.default_rng(1)
    Y = rng.standard_normal((24, 9)) * np.logspace(0, -6, 9)[None, :]
    Q = P.orth(Y)
    Qn, _ = np.linalg.qr(Y)
    assert np.abs(Q.T @ Q - np.eye(9)).max() <= 1e-12
    # column by column the same direction up to sign
    assert np.abs(np.abs(np.sum(Q * Qn, axis=0)) - 1.0).max() <= 1e-9


def pin_orth_completes_a_rank_deficient_sketch(P=PF):
    rng = np.random.default_rng(2)
    a, b = rng.standard_normal(6), rng.standard_normal(6)
    Y = np.stack([a, 2.0 * a, b, np.zeros(6)], axis=1)
    Q = P.orth(Y)
    q0 = a / np.linalg.norm(a)
    v = b - q0 * (q0 @ b)
    q1 = v / np.linalg.norm(v)
    e0 = np.eye(6)[:, 0]
    u = e0 - q0 * (q0 @ e0) - q1 * (q1 @ e0)
    q2 = u / np.linalg.norm(u)
    e1 = np.eye(6)[:, 1]
    u = e1 - q0 * (q0 @ e1) - q1 * (q1 @ e1) - q2 * (q2 @ e1)
    q3 = u / np.linalg.norm(u)
    assert np.abs(Q - np.stack([q0, q1, q2, q3], axis=1)).max() <= 1e-12


def pin_orth_stays_orthonormal_when_ill_conditioned(P=PF):
    """A power-iterated sketch of a Gram matrix with condition number 1e14:
    a single Gram-Schmidt pass loses orthogonality here, two do not."""
    rng = np.random.default_rng(3)
    lam = np.logspace(0, -14, 20)
    C, _ = _gram_with_spectrum(rng, 20, lam)
    Y = C @ C @ rng.standard_normal((20, 12))
    Q = P.orth(Y)
    assert np.abs(Q.T @ Q - np.eye(12)).max() <= 1e-12


# ------------------------------------------------------------------ Gram
def pin_gram_by_brute_force(P=PF):
    rng = np.random.default_rng(4)
    xs = [rng.standard_normal((5, 4)).astype(np.float16), rng.standard_normal((3, 4)).astype(np.float16)]
    C = P.window_gram(xs)
    ref = np.zeros((4, 4))
    for X in xs:
        for t in range(X.shape[0]):
            for i in range(4):
                for j in range(4):
                    ref[i, j] += float(X[t, i]) * float(X[t, j])
    assert np.abs(C - ref).max() <= 1e-12


# ------------------------------------------------------------------ range finder
def pin_diagonal_gram_gives_the_axes_by_hand(P=PF):
    """C = diag with rank 5 <= r: the Ritz vectors are the axes in decreasing
    variance, each +1 exactly; the Ritz values are the variances."""
    d, r, k = 16, 6, 10
    var = np.zeros(d)
    axes = [11, 2, 7, 0, 13]
    for v, a in zip((9.0, 5.0, 4.0, 2.5, 1.0), axes):
        var[a] = v
    C = np.diag(var)
    om = np.random.default_rng(5).standard_normal((d, k))
    B, theta, B16 = P.range_finder(C, om, r, 2)
    for i, a in enumerate(axes):
        ref = np.zeros(d)
        ref[a] = 1.0
        assert np.abs(B[i] - ref).max() <= 1e-12
        assert np.array_equal(B16[i].astype(np.float64), ref)
    assert np.abs(theta[:5] - [9.0, 5.0, 4.0, 2.5, 1.0]).max() <= 1e-12
    assert np.abs(theta[5:]).max() <= 1e-12
    # the sixth vector completes the basis orthogonally to the five axes
    assert np.abs(B[5, axes]).max() <= 1e-12 and abs(np.linalg.norm(B[5]) - 1) <= 1e-12


def pin_exact_low_rank_data_matches_its_svd(P=PF):
    rng = np.random.default_rng(6)
    n, d, rho, r, k = 200, 24, 5, 8, 12
    X = rng.standard_normal((n, rho)) @ (rng.standard_normal((rho, d)) * np.array([5, 3, 2, 1, 0.5])[:, None])
    C = P.window_gram([X])
    B, theta, _ = P.range_finder(C, rng.standard_normal((d, k)), r, 1)
    _, sv, Vt = np.linalg.svd(X, full_matrices=False)
    assert np.abs(_proj(B[:rho]) - _proj(Vt[:rho])).max() <= 1e-9
    assert np.abs(theta[:rho] / sv[:rho] ** 2 - 1).max() <= 1e-10
    assert np.abs(theta[rho:]).max() <= 1e-9 * theta[0]


def pin_converged_subspace_matches_eigh(P=PF):
    """Enough power iterations converge to the top-r eigenvectors of C, in
    order, with the Ritz values equal to the eigenvalues."""
    rng = np.random.default_rng(7)
    d, r, k = 32, 6, 10
    lam = np.concatenate([np.array([10, 8, 6.5, 5, 4, 3.2]), 1.6 * 0.8 ** np.arange(d - 6)])
    C, _ = _gram_with_spectrum(rng, d, lam)
    B, theta, _ = P.range_finder(C, rng.standard_normal((d, k)), r, 40)
    ev, EV = np.linalg.eigh(C)
    ev, EV = ev[::-1], EV[:, ::-1]
    assert np.abs(theta[:r] - ev[:r]).max() <= 1e-9 * ev[0]
    for i in range(r):
        assert abs(abs(B[i] @ EV[:, i]) - 1.0) <= 1e-9


def pin_gapped_spectrum_with_two_power_iterations(P=PF):
    rng = np.random.default_rng(8)
    d, r, k = 48, 8, 16
    lam = np.concatenate([np.linspace(10, 3, r), 1e-4 * np.ones(d - r)])
    C, U = _gram_with_spectrum(rng, d, lam)
    B, theta, _ = P.range_finder(C, rng.standard_normal((d, k)), r, 2)
    ev, EV = np.linalg.eigh(C)
    assert np.abs(_proj(B) - _proj(EV[:, ::-1][:, :r].T)).max() <= 1e-10
    assert np.abs(theta[:r] - np.sort(ev)[::-1][:r]).max() <= 1e-9 * lam[0]


def pin_interlacing_and_ky_fan(P=PF):
    """For any Q the Ritz values sit below the eigenvalues in order, and the
    energy tr(B C B^T) of the first r never exceeds the top-r sum."""
    rng = np.random.default_rng(9)
    d, r, k = 40, 10, 14
    for q in (0, 1, 2):
        C, _ = _gram_with_spectrum(rng, d, 0.9 ** np.arange(d))
        B, theta, _ = P.range_finder(C, rng.standard_normal((d, k)), r, q)
        ev = np.sort(np.linalg.eigvalsh(C))[::-1]
        assert np.all(theta <= ev[:k] + 1e-12)
        energy = np.trace(B @ C @ B.T)
        assert energy <= ev[:r].sum() + 1e-10
        assert abs(energy - theta[:r].sum()) <= 1e-10
        assert np.all(np.diff(theta) <= 1e-15)


def pin_conventions(P=PF):
    """Rows orthonormal, each row's first largest-magnitude entry positive,
    the fp16 basis the rounding of the fp64 one."""
    rng = np.random.default_rng(10)
    d, r, k = 32, 8, 12
    C, _ = _gram_with_spectrum(rng, d, 0.85 ** np.arange(d))
    B, _, B16 = P.range_finder(C, rng.standard_normal((d, k)), r, 2)
    assert np.abs(B @ B.T - np.eye(r)).max() <= 1e-12
    for i in range(r):
        assert B[i, np.argmax(np.abs(B[i]))] > 0
    assert np.array_equal(B16, B.astype(np.float16))


def pin_prefill_bases_ignore_tail_positions(P=PF):
    """Positions at or beyond a sequence's length carry no weight: the bases
    of padded inputs equal those of the trimmed ones, and the Gram matrix
    sums the window's layers and sequences."""
    cfg = _cfg()
    lengths = [300, 170]
    Ks, Vs, Kt, Vt = [], [], [], []
    for layer in range(2):
        K, V = w.gen_prefill(cfg, layer, lengths=lengths, tail=1000.0)
        Ks.append(K)
        Vs.append(V)
    om = w.gen_sketch(cfg, 12)[0]
    got = P.prefill_bases(cfg, Ks, Vs, lengths, om)
    for h in range(cfg.num_kv_heads):
        for z, L in (("K", Ks), ("V", Vs)):
            xs = [L[layer][b, h, :lengths[b]] for layer in range(2) for b in range(2)]
            C = sum(x.astype(np.float64).T @ x.astype(np.float64) for x in xs)
            assert np.abs(got["gram" + z][h] - C).max() <= 1e-9 * np.abs(C).max()
            B, th, B16 = P.range_finder(C, om[0 if z == "K" else 1, h], cfg.r_max, 2)
            assert np.array_equal(got[z][h], B16)
            assert np.abs(got["theta" + z][h] - th).max() <= 1e-9 * th[0]


# ------------------------------------------------------------------ bulk encode
def pin_bulk_encode_is_one_append_per_token(P=PF):
    cfg = _cfg(coef_bits=16)
    for cb in (16, 8):
        c = cfg.with_(coef_bits=cb)
        lengths = [57, 33]
        K, V = w.gen_prefill(c, 1, lengths=lengths)
        bases = w.make_bases(c)
        tier = w.gen_tiers(c, 1, 57)
        gK, gV = w.gen_gates(c, 1, 57)
        lay = P.prefill_encode(c, bases["K"][0], bases["V"][0], K, V, lengths, tier, gK, gV)
        res = c.resid_per_tier
        for b in range(2):
            for h in range(c.num_kv_heads):
                for t in range(lengths[b]):
                    k = int(tier[b, h, t])
                    r, s = c.tier_rank[k], res[k]
                    assert lay["tier"][b, h, t] == k
                    for z, X, g in (("K", K, gK), ("V", V, gV)):
                        enc = oracle.append_vector(bases[z][0][h], X[b, h, t], r, s, c.qmax, g[b, h, t],
                                                   coef_bits=cb)
                        assert np.array_equal(lay["coef" + z][b, h, t, :r], enc[0])
                        assert not lay["coef" + z][b, h, t, r:].astype(np.float32).any()
                        assert np.array_equal(lay["idx" + z][b, h, t, :s], enc[1])
                        assert np.array_equal(lay["val" + z][b, h, t, :s], enc[2])
                        assert lay["scale" + z][b, h, t].view(np.uint16) == enc[3].view(np.uint16)
                        if cb == 8:
                            assert lay["cscale" + z][b, h, t].view(np.uint16) == enc[4].view(np.uint16)
        assert list(lay["n_tokens"]) == lengths


def pin_bulk_encode_identity_basis_by_hand(P=PF):
    """B = I: the coefficients are the vector's first r channels and the
    residual keeps the largest |x_j| among the rest (gate 1)."""
    cfg = _cfg(batch=1, num_kv_heads=1, head_dim=16, r_max=16, tier_rank=(4, 16), tier_prob=(0.5, 0.5),
               resid_channels=2, resid_bits=8)
    bases = w.make_bases(cfg, identity=True)
    K, V = w.gen_prefill(cfg, 0, lengths=[20])
    tier = w.gen_tiers(cfg, 0, 20)
    lay = P.prefill_encode(cfg, bases["K"][0], bases["V"][0], K, V, [20], tier)
    for t in range(20):
        r = cfg.tier_rank[int(tier[0, 0, t])]
        x = K[0, 0, t].astype(np.float64)
        assert np.array_equal(lay["coefK"][0, 0, t, :r].astype(np.float64), x[:r])
        rest = np.abs(x.copy())
        rest[:r] = -1
        top = sorted(np.argsort(-rest, kind="stable")[:2])
        if r < 16:
            assert list(lay["idxK"][0, 0, t]) == top


PINS = [
    pin_orth_spans_like_householder_qr,
    pin_orth_completes_a_rank_deficient_sketch,
    pin_orth_stays_orthonormal_when_ill_conditioned,
    pin_gram_by_brute_force,
    pin_diagonal_gram_gives_the_axes_by_hand,
    pin_exact_low_rank_data_matches_its_svd,
    pin_converged_subspace_matches_eigh,
    pin_gapped_spectrum_with_two_power_iterations,
    pin_interlacing_and_ky_fan,
    pin_conventions,
    pin_prefill_bases_ignore_tail_positions,
    pin_bulk_encode_is_one_append_per_token,
    pin_bulk_encode_identity_basis_by_hand,
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_prefill_oracle_pin(pin):
    pin()


# ------------------------------------------------------------------ planted mistakes
MUTANTS = {
    "ascending_ritz_order": ("order = np.argsort(-theta, kind=\"stable\")",
                             "order = np.argsort(theta, kind=\"stable\")"),
    "no_rayleigh_ritz": ("V = sign_fix(Q @ U[:, order])", "V = sign_fix(Q)"),
    "no_power_iterations": ("for _ in range(q):", "for _ in range(0):"),
    "no_sign_fix": ("        if V[p, j] < 0:\n            V[:, j] = -V[:, j]", "        pass"),
    "single_gram_schmidt_pass": ("        for _ in range(2):\n            if kept:",
                                 "        for _ in range(1):\n            if kept:"),
    "no_completion": ("cand = np.concatenate([Y, np.eye(d)], axis=1)", "cand = np.concatenate([Y, Y], axis=1)"),
    "tail_positions_included": ("return [K[b, h, : int(n_tokens[b])] for b in range(K.shape[0])]",
                                "return [K[b, h] for b in range(K.shape[0])]"),
    "one_layer_only": ("xs = [x for L in layers for x in window_vectors(L, n_tokens, h)]",
                       "xs = [x for L in layers[:1] for x in window_vectors(L, n_tokens, h)]"),
    "rows_not_columns": ("B = V[:, :r].T.copy()", "B = V[:r, :].copy()"),
    "tier_off_by_one": ("_p(np.ascontiguousarray(ranks[t])), _p(np.ascontiguousarray(res[t])),",
                        "_p(np.ascontiguousarray(ranks[np.minimum(t + 1, len(ranks) - 1)])), "
                        "_p(np.ascontiguousarray(res[t])),"),
    "gates_swapped": ("for z, X, bas, gate in ((\"K\", K, basisK, gateK), (\"V\", V, basisV, gateV)):",
                      "for z, X, bas, gate in ((\"K\", K, basisK, gateV), (\"V\", V, basisV, gateK)):"),
}


def _mutant(src, name):
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    spec = importlib.util.spec_from_loader(f"oracle._prefill_mutant_{name}", loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    sys.modules[spec.name] = mod
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    src = inspect.getsource(PF)
    mod = _mutant(src, name)
    caught = []
    for pin in PINS:
        try:
            pin(mod)
        except Exception:          # an assertion, or a mistake that breaks the computation
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
