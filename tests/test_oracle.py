"""Pins for the fp64 CPU oracle (CPU only, no GPU).

The oracle computes the recurrent / state form of kernelized linear attention
(page "Efficient Transformers Survey", section "Linear Attention", Proposition
"Linear Attention via Kernel Decomposition").  None of these checks re-types the
oracle's own formula: each compares it with something the pages or plain
mathematics fix independently --

  * the quadratic form of the proof sketch, written here in numpy as explicit
    n x n weights (a different algorithm from the oracle's S/z recurrence);
  * a hand-worked example with exact rational answers (tests/golden);
  * closed-form special cases (constant V, constant K, N = 1, first row);
  * invariants (convex combination, causality, Euler homogeneity, sum of dV);
  * central finite differences of the numpy quadratic form for the backward.

A dropped term, a swapped operand, an off-by-one in the causal mask, a wrong
sign in the backward or an exclusive instead of inclusive prefix each fails at
least one of these.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import la_inputs as inp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---- independent reference: the proof-sketch quadratic form in numpy --------
def np_phi(x):
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def np_quadratic(q, k, v, causal):
    """Attn_i = sum_j k(q_i,k_j) v_j / sum_j k(q_i,k_j), k(q,k) = phi(q).phi(k)."""
    A = np_phi(q) @ np.swapaxes(np_phi(k), -1, -2)
    if causal:
        n = q.shape[-2]
        A = A * np.tril(np.ones((n, n)))
    den = A.sum(-1)
    return (A @ v) / den[..., None], den


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def rel(x, y):
    return float(np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-300))


# ---- feature map ---------------------------------------------------------------
def test_phi_values(oracle):
    assert oracle.phi(0.0) == 1.0
    assert oracle.phi(1.0) == 2.0
    assert oracle.phi(2.5) == 3.5
    assert oracle.phi(-1.0) == pytest.approx(math.exp(-1.0), rel=1e-15)
    assert oracle.phi(-700.0) > 0.0
    assert oracle.dphi(3.0) == 1.0
    assert oracle.dphi(0.0) == 1.0
    assert oracle.dphi(-2.0) == pytest.approx(math.exp(-2.0), rel=1e-15)
    # continuity at 0 from both sides
    assert oracle.phi(1e-12) == pytest.approx(oracle.phi(-1e-12), abs=1e-11)


# ---- hand-worked example -----------------------------------------------------------
def _val(x):
    if isinstance(x, str):
        if x.startswith("-ln"):
            return -math.log(float(x[3:]))
        return float(Fraction(x))
    return float(x)


def _arr(rows):
    return np.array([[_val(e) for e in r] if isinstance(r, list) else _val(r) for r in rows], dtype=np.float64)


def test_hand_example(oracle):
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    q, k, v, do = (_arr(g[n]) for n in ("q", "k", "v", "dout"))
    o, den, S, z = oracle.forward_causal(q, k, v, return_den=True, return_state=True)
    np.testing.assert_allclose(o, _arr(g["causal_o"]), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(den, _arr(g["causal_den"]), rtol=1e-13)
    np.testing.assert_allclose(S, _arr(g["final_S"]), rtol=1e-13)
    np.testing.assert_allclose(z, _arr(g["final_z"]), rtol=1e-13)
    o2, den2, S2, z2 = oracle.forward_noncausal(q, k, v, return_den=True, return_state=True)
    np.testing.assert_allclose(o2, _arr(g["noncausal_o"]), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(den2, _arr(g["noncausal_den"]), rtol=1e-13)
    np.testing.assert_allclose(S2, _arr(g["final_S"]), rtol=1e-13)
    np.testing.assert_allclose(z2, _arr(g["final_z"]), rtol=1e-13)
    dq, dk, dv = oracle.backward_causal(q, k, v, do)
    np.testing.assert_allclose(dv, _arr(g["causal_dv"]), rtol=1e-13, atol=1e-14)


# ---- forward vs the quadratic form -------------------------------------------------
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape,scale", [((2, 3, 17, 5), 1.0), ((1, 2, 40, 8), 0.35), ((1, 1, 1, 4), 1.0)])
def test_forward_matches_quadratic(oracle, causal, shape, scale):
    q, k, v = rand(shape, 1, scale), rand(shape, 2, scale), rand(shape, 3)
    ref, ref_den = np_quadratic(q, k, v, causal)
    fn = oracle.forward_causal if causal else oracle.forward_noncausal
    o, den = fn(q, k, v, return_den=True)
    assert rel(o, ref) < 1e-13
    assert rel(den, ref_den) < 1e-13
    # the oracle's own brute force agrees as well
    o_q, den_q = oracle.quadratic_forward(q, k, v, causal=causal, return_den=True)
    assert rel(o_q, ref) < 1e-13 and rel(den_q, ref_den) < 1e-13


def test_reassociation_identity():
    """(phi(Q) phi(K)^T) V == phi(Q) (phi(K)^T V): the associativity the method rests on."""
    q, k, v = rand((30, 6), 4), rand((30, 6), 5), rand((30, 6), 6)
    lhs = (np_phi(q) @ np_phi(k).T) @ v
    rhs = np_phi(q) @ (np_phi(k).T @ v)
    assert rel(lhs, rhs) < 1e-13


def test_state_matches_definition(oracle):
    q, k, v = rand((2, 9, 4), 7), rand((2, 9, 4), 8), rand((2, 9, 4), 9)
    _, S, z = oracle.forward_causal(q, k, v, return_state=True)
    S_ref = np.einsum("hja,hjb->hab", np_phi(k), v)
    z_ref = np_phi(k).sum(1)
    assert rel(S, S_ref) < 1e-14 and rel(z, z_ref) < 1e-14
    _, S2, z2 = oracle.forward_noncausal(q, k, v, return_state=True)
    assert rel(S2, S_ref) < 1e-14 and rel(z2, z_ref) < 1e-14


# ---- closed-form special cases ----------------------------------------------------
@pytest.mark.parametrize("causal", [True, False])
def test_constant_v_returns_constant(oracle, causal):
    n, d = 23, 6
    q, k = rand((n, d), 10), rand((n, d), 11)
    c = rand((d,), 12)
    v = np.tile(c, (n, 1))
    fn = oracle.forward_causal if causal else oracle.forward_noncausal
    o = fn(q, k, v)
    np.testing.assert_allclose(o, v, rtol=1e-13, atol=1e-14)


def test_constant_k_gives_prefix_mean(oracle):
    n, d = 19, 5
    q, v = rand((n, d), 13), rand((n, d), 14)
    k = np.tile(rand((d,), 15), (n, 1))
    o = oracle.forward_causal(q, k, v)
    pm = np.cumsum(v, 0) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(o, pm, rtol=1e-12, atol=1e-13)
    o2 = oracle.forward_noncausal(q, k, v)
    np.testing.assert_allclose(o2, np.tile(v.mean(0), (n, 1)), rtol=1e-12, atol=1e-13)


def test_first_row_last_row_and_n1(oracle):
    q, k, v = rand((3, 31, 7), 16), rand((3, 31, 7), 17), rand((3, 31, 7), 18)
    oc = oracle.forward_causal(q, k, v)
    on = oracle.forward_noncausal(q, k, v)
    np.testing.assert_allclose(oc[:, 0], v[:, 0], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(oc[:, -1], on[:, -1], rtol=1e-12, atol=1e-13)
    o1 = oracle.forward_causal(q[:, :1], k[:, :1], v[:, :1])
    np.testing.assert_allclose(o1, v[:, :1], rtol=1e-13, atol=1e-14)


def test_convex_combination(oracle):
    """phi > 0, so every output row is a convex combination of the value rows it sees."""
    n, d = 40, 4
    q, k, v = rand((n, d), 19, 2.0), rand((n, d), 20, 2.0), rand((n, d), 21)
    o = oracle.forward_causal(q, k, v)
    for i in range(n):
        lo, hi = v[: i + 1].min(0), v[: i + 1].max(0)
        assert np.all(o[i] >= lo - 1e-12) and np.all(o[i] <= hi + 1e-12)


def test_causality_nan_in_future(oracle):
    n, d, cut = 20, 4, 11
    q, k, v = rand((n, d), 22), rand((n, d), 23), rand((n, d), 24)
    o = oracle.forward_causal(q, k, v)
    k2, v2 = k.copy(), v.copy()
    k2[cut + 1:] = np.nan
    v2[cut + 1:] = np.inf
    o2 = oracle.forward_causal(q, k2, v2)
    np.testing.assert_array_equal(o2[: cut + 1], o[: cut + 1])
    assert not np.isfinite(o2[cut + 1:]).any()


# ---- backward ----------------------------------------------------------------------------
def _fd_grads(q, k, v, do, causal, h=1e-6):
    def loss(q_, k_, v_):
        return float((np_quadratic(q_, k_, v_, causal)[0] * do).sum())

    grads = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(args[which])
        it = np.nditer(g, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[which][idx] += h
            minus[which][idx] -= h
            g[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        grads.append(g)
    return grads


@pytest.mark.parametrize("causal", [True, False])
def test_backward_finite_differences(oracle, causal):
    n, d = 12, 5
    q, k, v, do = rand((n, d), 25), rand((n, d), 26), rand((n, d), 27), rand((n, d), 28)
    fd = _fd_grads(q, k, v, do, causal)
    fn = oracle.backward_causal if causal else oracle.backward_noncausal
    got = fn(q, k, v, do)
    for name, g, f in zip(("dq", "dk", "dv"), got, fd):
        assert rel(g, f) < 1e-7, name


@pytest.mark.parametrize("causal", [True, False])
def test_backward_matches_quadratic_backward(oracle, causal):
    shape = (2, 2, 21, 6)
    q, k, v, do = rand(shape, 29, 0.5), rand(shape, 30, 0.5), rand(shape, 31), rand(shape, 32)
    fn = oracle.backward_causal if causal else oracle.backward_noncausal
    got = fn(q, k, v, do)
    ref = oracle.quadratic_backward(q, k, v, do, causal=causal)
    for g, r in zip(got, ref):
        assert rel(g, r) < 1e-12


@pytest.mark.parametrize("causal", [True, False])
def test_backward_invariants(oracle, causal):
    n, d = 33, 6
    q, k, v, do = rand((n, d), 33), rand((n, d), 34), rand((n, d), 35), rand((n, d), 36)
    fn = oracle.backward_causal if causal else oracle.backward_noncausal
    dq, dk, dv = fn(q, k, v, do)
    # shifting every value row by c shifts every output row by c
    np.testing.assert_allclose(dv.sum(0), do.sum(0), rtol=1e-11, atol=1e-12)
    # each O_i is homogeneous of degree 0 in phi(Q_i): sum_a dphi(Q)_ia phi(Q_ia) = 0
    dqf = dq / np.where(q > 0, 1.0, np.exp(np.minimum(q, 0)))
    euler_q = (dqf * np_phi(q)).sum(1)
    assert np.abs(euler_q).max() < 1e-11 * max(1.0, np.abs(dqf).max())
    # ... and of degree 0 in all phi(K_j) jointly
    dkf = dk / np.where(k > 0, 1.0, np.exp(np.minimum(k, 0)))
    assert abs((dkf * np_phi(k)).sum()) < 1e-10 * max(1.0, np.abs(dkf).max())


def test_constant_v_zero_grads(oracle):
    n, d = 17, 4
    q, k, do = rand((n, d), 37), rand((n, d), 38), rand((n, d), 39)
    v = np.tile(rand((d,), 40), (n, 1))
    dq, dk, dv = oracle.backward_causal(q, k, v, do)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12


# ---- decode --------------------------------------------------------------------------------
def test_decode_reproduces_causal_rows(oracle):
    bh, n, d = 3, 14, 5
    q, k, v = rand((bh, n, d), 41), rand((bh, n, d), 42), rand((bh, n, d), 43)
    o_ref, S_ref, z_ref = oracle.forward_causal(q, k, v, return_state=True)
    S, z = np.zeros((bh, d, d)), np.zeros((bh, d))
    for t in range(n):
        o, S, z = oracle.decode_step(S, z, q[:, t], k[:, t], v[:, t])
        np.testing.assert_allclose(o, o_ref[:, t], rtol=1e-12, atol=1e-13)
    _, S_nc, z_nc = oracle.forward_noncausal(q, k, v, return_state=True)
    assert rel(S, S_ref) < 1e-13 and rel(S, S_nc) < 1e-13 and rel(z, z_nc) < 1e-13


def test_decode_from_prefix_state(oracle):
    bh, n, d = 2, 10, 4
    q, k, v = rand((bh, n + 1, d), 44), rand((bh, n + 1, d), 45), rand((bh, n + 1, d), 46)
    _, S0, z0 = oracle.forward_causal(q[:, :n], k[:, :n], v[:, :n], return_state=True)
    o, _, _ = oracle.decode_step(S0, z0, q[:, n], k[:, n], v[:, n])
    full = oracle.forward_causal(q, k, v)
    np.testing.assert_allclose(o, full[:, n], rtol=1e-12, atol=1e-13)


# ---- a recurrence started from a given state ---------------------------------------------
def test_start_state_equals_prepended_tokens(oracle):
    """(S0, z0) left by virtual tokens (k*, v*) act exactly as those tokens placed before the
    sequence: checked against the numpy quadratic form over the longer sequence."""
    bh, m, n, d = 3, 4, 9, 5
    kx, vx = rand((bh, m, d), 60), rand((bh, m, d), 61)
    q, k, v = rand((bh, n, d), 62), rand((bh, n, d), 63), rand((bh, n, d), 64)
    S0 = np.einsum("hja,hjb->hab", np_phi(kx), vx)
    z0 = np_phi(kx).sum(1)
    o, den, S, z = oracle.forward_causal(q, k, v, return_den=True, return_state=True, S0=S0, z0=z0)
    qx = rand((bh, m, d), 65)
    full_q, full_k, full_v = (np.concatenate(t, axis=1) for t in ((qx, q), (kx, k), (vx, v)))
    ref, ref_den = np_quadratic(full_q, full_k, full_v, causal=True)
    assert rel(o, ref[:, m:]) < 1e-12
    assert rel(den, ref_den[:, m:]) < 1e-12
    assert rel(S, np.einsum("hja,hjb->hab", np_phi(full_k), full_v)) < 1e-12
    assert rel(z, np_phi(full_k).sum(1)) < 1e-12


def test_start_state_continues_a_sequence(oracle):
    """Processing [0, p) and then [p, n) from the state the first part left equals one pass."""
    shape, p = (2, 2, 23, 6), 10
    q, k, v = rand(shape, 66), rand(shape, 67), rand(shape, 68)
    full, S_f, z_f = oracle.forward_causal(q, k, v, return_state=True)
    _, S_p, z_p = oracle.forward_causal(q[..., :p, :], k[..., :p, :], v[..., :p, :], return_state=True)
    rest, S_r, z_r = oracle.forward_causal(q[..., p:, :], k[..., p:, :], v[..., p:, :], return_state=True,
                                           S0=S_p, z0=z_p)
    assert rel(rest, full[..., p:, :]) < 1e-12
    assert rel(S_r, S_f) < 1e-12 and rel(z_r, z_f) < 1e-12
    # a zero start state is the plain forward
    zero = oracle.forward_causal(q, k, v, S0=np.zeros(shape[:2] + (6, 6)), z0=np.zeros(shape[:2] + (6,)))
    np.testing.assert_array_equal(zero, full)


def test_start_state_matches_decode_steps(oracle):
    """T decode steps from a state give the rows of the recurrence started from that state."""
    bh, t, d = 3, 6, 4
    S0 = np.abs(rand((bh, d, d), 69)) + 0.5
    z0 = np.abs(rand((bh, d), 70)) + 2.0
    q, k, v = rand((bh, t, d), 71), rand((bh, t, d), 72), rand((bh, t, d), 73)
    o, S, z = oracle.forward_causal(q, k, v, return_state=True, S0=S0, z0=z0)
    Sd, zd = S0.copy(), z0.copy()
    for i in range(t):
        od, Sd, zd = oracle.decode_step(Sd, zd, q[:, i], k[:, i], v[:, i])
        np.testing.assert_allclose(od, o[:, i], rtol=1e-12, atol=1e-13)
    assert rel(Sd, S) < 1e-13 and rel(zd, z) < 1e-13


# ---- backward of the recurrence from a start state ------------------------------------------------
def _np_forward_from(q, k, v, S0, z0):
    """Recurrence from (S0, z0) by cumulative sums (numpy): outputs and final state."""
    kf, qf = np_phi(k), np_phi(q)
    S = S0[None] + np.cumsum(kf[:, :, None] * v[:, None, :], axis=0)
    z = z0[None] + np.cumsum(kf, axis=0)
    o = np.einsum("ia,iab->ib", qf, S) / np.einsum("ia,ia->i", qf, z)[:, None]
    return o, S[-1], z[-1]


def test_backward_from_state_finite_differences(oracle):
    """Gradients of sum(dO O) + sum(dSN S_N) + sum(dzN z_N) for the recurrence from (S0, z0),
    against central differences of a numpy cumulative-sum forward (q, k, v, S0 and z0)."""
    rng = np.random.default_rng(100)
    n, d, h = 9, 4, 1e-6
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    S0, z0 = rng.uniform(0.5, 2.0, (d, d)), rng.uniform(2.0, 4.0, d)
    dSN, dzN = rng.standard_normal((d, d)), rng.standard_normal(d)

    def loss(q, k, v, S0, z0):
        o, S, z = _np_forward_from(q, k, v, S0, z0)
        return (do * o).sum() + (dSN * S).sum() + (dzN * z).sum()

    args = [q, k, v, S0, z0]
    got = oracle.backward_causal_state(q, k, v, do, S0=S0, z0=z0, dSN=dSN, dzN=dzN)
    for which, g in enumerate(got):
        fd = np.zeros_like(args[which])
        for idx in np.ndindex(*fd.shape):
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        assert rel(g, fd) < 1e-7, which


def test_backward_from_state_chains_pieces(oracle):
    """A sequence's backward in two pieces: the second piece from the state the first left,
    then the first with the second's start-state gradient as its final-state gradient,
    equals the backward of the whole sequence."""
    shape, p = (2, 2, 19, 5), 8
    q, k, v, do = rand(shape, 101), rand(shape, 102), rand(shape, 103), rand(shape, 104)
    full = oracle.backward_causal(q, k, v, do)
    cut = lambda x, a, b: x[..., a:b, :]
    _, S_p, z_p = oracle.forward_causal(cut(q, 0, p), cut(k, 0, p), cut(v, 0, p), return_state=True)
    dq2, dk2, dv2, dS0, dz0 = oracle.backward_causal_state(cut(q, p, None), cut(k, p, None), cut(v, p, None),
                                                           cut(do, p, None), S0=S_p, z0=z_p)
    dq1, dk1, dv1, _, _ = oracle.backward_causal_state(cut(q, 0, p), cut(k, 0, p), cut(v, 0, p), cut(do, 0, p),
                                                       dSN=dS0, dzN=dz0)
    for f, a, b in zip(full, (dq1, dk1, dv1), (dq2, dk2, dv2)):
        assert rel(np.concatenate([a, b], axis=-2), f) < 1e-12
    # no state and no upstream gradient: the plain backward, bit for bit
    plain = oracle.backward_causal_state(q, k, v, do)
    for a, b in zip(plain[:3], full):
        np.testing.assert_array_equal(a, b)


# ---- FAVOR+ features and attention on given features ------------------------------------------
def test_favor_features_special_directions(oracle):
    """omega = 0 leaves only the norm factor; omega = a unit vector picks one coordinate."""
    x = np.array([[0.3, -1.2, 0.5], [2.0, 0.1, -0.4]])
    omega = np.array([[0.0, 0.0, 0.0], [1.0, 0.0, 0.0], [0.0, 0.0, 1.0], [0.0, -1.0, 0.0]])
    f = oracle.favor_features(x, omega)
    nrm = (x * x).sum(1)
    for r in range(2):
        base = math.exp(-nrm[r] / 2) / 2.0  # m = 4
        assert f[r, 0] == pytest.approx(base, rel=1e-14)
        assert f[r, 1] == pytest.approx(base * math.exp(x[r, 0]), rel=1e-14)
        assert f[r, 2] == pytest.approx(base * math.exp(x[r, 2]), rel=1e-14)
        assert f[r, 3] == pytest.approx(base * math.exp(-x[r, 1]), rel=1e-14)


def test_favor_estimator_is_unbiased(oracle):
    """E_omega[phi(q).phi(k)] = exp(q.k) (Performer Approximation Quality): the Monte Carlo
    mean over many directions lands within 5 standard errors of the exact kernel."""
    rng = np.random.default_rng(80)
    d, m = 6, 200_000
    omega = rng.standard_normal((m, d))
    for _ in range(4):
        q, k = rng.standard_normal(d) * 0.4, rng.standard_normal(d) * 0.4
        fq, fk = oracle.favor_features(q[None], omega)[0], oracle.favor_features(k[None], omega)[0]
        terms = m * fq * fk                      # one unbiased sample per direction
        est, se = terms.mean(), terms.std() / math.sqrt(m)
        assert abs(est - fq @ fk) < 1e-12 * abs(est)
        assert abs(est - math.exp(q @ k)) < 5 * se, (est, math.exp(q @ k), se)


def test_favor_variance_falls_like_one_over_m(oracle):
    """Var[phi(q).phi(k)] over independent draws of omega scales as 1/m: quadrupling m
    divides it by about four."""
    rng = np.random.default_rng(81)
    d, reps = 5, 600
    q, k = rng.standard_normal(d) * 0.3, rng.standard_normal(d) * 0.3
    var = {}
    for m in (16, 64):
        est = []
        for _ in range(reps):
            omega = rng.standard_normal((m, d))
            est.append(oracle.favor_features(q[None], omega)[0] @ oracle.favor_features(k[None], omega)[0])
        var[m] = np.var(est)
    assert 2.8 < var[16] / var[64] < 5.7, var


def test_orthogonal_favor_directions(oracle):
    """Orthogonal random features (Performer Approximation Quality: orthogonal draws lower the
    variance below i.i.d. Gaussian ones): every block of d directions is orthogonal, the estimate
    stays unbiased, and its variance over draws falls below that of i.i.d. directions."""
    import torch
    d = 32
    om = inp.favor_omega(d, seed=3, m=3 * d, orthogonal=True).double().numpy()
    for b in range(3):
        blk = om[b * d:(b + 1) * d]
        gram = blk @ blk.T
        off = gram - np.diag(np.diag(gram))
        assert np.abs(off).max() < 1e-4 * np.diag(gram).max()
    rng = np.random.default_rng(83)
    q, k = rng.standard_normal(d) * 0.15, rng.standard_normal(d) * 0.15
    reps = 4000
    est = {}
    for orth in (False, True):
        e = []
        for r in range(reps):
            w = inp.favor_omega(d, seed=1000 + r, orthogonal=orth).double().numpy()
            e.append(oracle.favor_features(q[None], w)[0] @ oracle.favor_features(k[None], w)[0])
        est[orth] = np.array(e)
    exact = math.exp(q @ k)
    for e in est.values():
        assert abs(e.mean() - exact) < 5 * e.std() / math.sqrt(reps)
    assert np.var(est[True]) < 0.85 * np.var(est[False]), (np.var(est[True]), np.var(est[False]))


def test_features_form_matches_quadratic_and_elu_path(oracle):
    """Given features: the explicit n x n weights (numpy), and with elu+1 features the
    oracle's own elementwise-map recurrence."""
    rng = np.random.default_rng(82)
    bh, n, m, dv = 2, 13, 7, 5
    fq, fk = rng.uniform(0.1, 2.0, (bh, n, m)), rng.uniform(0.1, 2.0, (bh, n, m))
    v = rng.standard_normal((bh, n, dv))
    for causal in (True, False):
        A = fq @ np.swapaxes(fk, -1, -2)
        if causal:
            A = A * np.tril(np.ones((n, n)))
        ref = (A @ v) / A.sum(-1, keepdims=True)
        o, den, S, z = oracle.forward_features(fq, fk, v, causal, return_den=True, return_state=True)
        assert rel(o, ref) < 1e-13 and rel(den, A.sum(-1)) < 1e-13
        assert rel(S, np.einsum("hja,hjb->hab", fk, v)) < 1e-13 and rel(z, fk.sum(1)) < 1e-13
    q, k, v = rand((2, 11, 4), 83), rand((2, 11, 4), 84), rand((2, 11, 4), 85)
    for causal in (True, False):
        ref = (oracle.forward_causal if causal else oracle.forward_noncausal)(q, k, v)
        assert rel(oracle.forward_features(np_phi(q), np_phi(k), v, causal), ref) < 1e-13


def test_favor_attention_approximates_softmax(oracle):
    """With many features, linear attention on FAVOR+ features approaches softmax attention
    (the kernel the estimator targets), causal and not."""
    rng = np.random.default_rng(86)
    n, d, m = 12, 4, 100_000
    q, k, v = rng.standard_normal((n, d)) * 0.5, rng.standard_normal((n, d)) * 0.5, rng.standard_normal((n, d))
    omega = rng.standard_normal((m, d))
    fq, fk = oracle.favor_features(q, omega), oracle.favor_features(k, omega)
    for causal in (True, False):
        w = np.exp(q @ k.T)
        if causal:
            w = w * np.tril(np.ones((n, n)))
        ref = (w @ v) / w.sum(1, keepdims=True)
        assert rel(oracle.forward_features(fq, fk, v, causal), ref) < 0.02


def test_thread_count_does_not_change_results(oracle):
    shape = (4, 3, 25, 6)
    q, k, v, do = rand(shape, 47), rand(shape, 48), rand(shape, 49), rand(shape, 50)
    oracle.set_threads(1)
    a = oracle.backward_causal(q, k, v, do)
    oracle.set_threads(4)
    b = oracle.backward_causal(q, k, v, do)
    oracle.set_threads(0)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


# ---- backward on given features, and through the FAVOR+ feature map --------------------
def _np_features_forward(fq, fk, v, causal):
    """The explicit n x n weights form on given features (numpy)."""
    A = fq @ fk.T
    if causal:
        A = A * np.tril(np.ones(A.shape))
    return (A @ v) / A.sum(-1, keepdims=True)


@pytest.mark.parametrize("causal", [True, False])
def test_backward_features_finite_differences(oracle, causal):
    """m != dv: central differences of sum(dout * O) of the explicit-weights form."""
    rng = np.random.default_rng(120 + causal)
    n, m, dv, h = 9, 6, 4, 1e-6
    fq, fk = rng.uniform(0.2, 2.0, (n, m)), rng.uniform(0.2, 2.0, (n, m))
    v, do = rng.standard_normal((n, dv)), rng.standard_normal((n, dv))
    args = [fq, fk, v]
    got = oracle.backward_features(fq, fk, v, do, causal)
    for which, g in enumerate(got):
        fd = np.zeros_like(args[which])
        for idx in np.ndindex(*fd.shape):
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd[idx] = ((_np_features_forward(*plus, causal) - _np_features_forward(*minus, causal)) * do).sum() / (2 * h)
        assert rel(g, fd) < 1e-7, which


@pytest.mark.parametrize("causal", [True, False])
def test_backward_features_chain_to_elu_backward(oracle, causal):
    """With elu+1 features, dfq phi'(q), dfk phi'(k) and dv are the oracle's elementwise-map
    backward (itself pinned by finite differences above)."""
    q, k, v, do = rand((2, 15, 5), 130), rand((2, 15, 5), 131), rand((2, 15, 5), 132), rand((2, 15, 5), 133)
    dfq, dfk, dv = oracle.backward_features(np_phi(q), np_phi(k), v, do, causal)
    dphi = lambda x: np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))
    ref = (oracle.backward_causal if causal else oracle.backward_noncausal)(q, k, v, do)
    for got, r in zip((dfq * dphi(q), dfk * dphi(k), dv), ref):
        assert rel(got, r) < 1e-12


def test_favor_features_backward_finite_differences(oracle):
    rng = np.random.default_rng(140)
    rows, d, m, h = 5, 4, 7, 1e-6
    x = rng.standard_normal((rows, d)) * 0.7
    om = rng.standard_normal((m, d))
    dF = rng.standard_normal((rows, m))
    got = oracle.favor_features_backward(x, om, dF)
    fd = np.zeros_like(x)
    for idx in np.ndindex(*x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        fd[idx] = ((oracle.favor_features(xp, om) - oracle.favor_features(xm, om)) * dF).sum() / (2 * h)
    assert rel(got, fd) < 1e-7
