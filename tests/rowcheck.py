"""Per-row parity bars for the sequence outputs O, dQ, dK, dV.

Every output row is defined on its own (page "Efficient Transformers Survey",
Linear Attention proposition, Statement: one Attn_i per query i; the backward
rows follow by the chain rule), so every row is checked on its own:

    ||x_i - y_i|| <= tol ||y_i|| + floor_i

with x the GPU row, y the fp64 oracle row and tol the bar of the workload
(2e-2 for bf16 inputs, 1e-4 for fp32 inputs).  floor_i covers rows whose exact
value is zero or much smaller than the terms summed into it (dQ_0 = 0 exactly;
a tail row of dK whose G . (V - O) nearly cancels).  It is a first-order,
probabilistic rounding bound (independent rounding errors add in quadrature):

    floor_i = LAMBDA (u T_i + 2^-24 sqrt(n_i + d) Tf_i)

  * u = 2^-8 for bf16 inputs (the unit roundoff of the bf16 operands the
    products take), 0 for fp32 inputs (fp32 operands);
  * T_i: root-sum-square, over every summand of row i, of the first-order
    change a relative perturbation of each rounded operand causes;
  * Tf_i: the same for the fp32 sums, before their cancellation (the constant
    parts of phi(K) = 1 + E(K) that the kernels carry in fp32); n_i the number
    of summands;
  * LAMBDA = 4 standard deviations.

Per head, with Qf = phi(Q), Kf = phi(K), E = Kf - 1 the part of the key
features that enters bf16 products (E = Kf for features given as they are),
G = dO / den, g = -G . O, and sums over j <= i (causal) or all j:

  O_i  : the weights w_ij = A_ij / den_i of O_i = sum_j w_ij V_j perturbed:
         T^2 = sum_j w_ij^2 |V_j - O_i|^2 with A_ij <= |Qf_i| |Kf_j|
         (Cauchy-Schwarz; tight where phi sits near 1);
  dV_j : sum_{i>=j} A_ij G_i, A and G perturbed: T^2 = |Kf_j|^2 sum_i |Qf_i|^2 |G_i|^2;
  dK_j : sum_{i>=j} (G_i . (V_j - O_i)) Qf_i with every component of G perturbed:
         T^2 = sum_i |Qf_i|^2 sum_b G_ib^2 (V_jb - O_ib)^2;
  dQ_i : sum_{j<=i} (G_i . (V_j - O_i)) Kf_j, likewise, split as the kernels
         split it: T^2 = sum_b G_ib^2 [sum_j |E_j|^2 (V_jb - O_ib)^2
         + d (P_ib - n_i O_ib)^2] with P_i = sum_j V_j (the second part is the
         constant 1 of Kf, summed in fp32); Tf^2 adds d sum_b G_ib^2 (P_ib^2 + n_i^2 O_ib^2),
         the fp32 terms before they cancel.

A start state (S0, z0) enters as one more summand (taken apart around its mean
as the kernels take it), and upstream gradients of the final state (dS_N, dz_N)
likewise.  Each bound needs only running sums over the sequence: O(N d) per head.

Where a backward takes g from outside its own products (the feature-block
backward over m = KF d features: the head's den from the forward, or g = -G . O
from the forward's rounded output), the identity sum_j A_ij dA_ij = 0 no longer
holds exactly and g carries that rounding: |dg_i| <= u (|g_i| + sum_b |G_ib O_ib|)
(gerr).  It adds dg_i z_i to dQ_i (z_i = sum_{j<=i} Kf_j) and sum_{i>=j} dg_i Qf_i
to dK_j, each in quadrature.
"""
from __future__ import annotations

import numpy as np

LAMBDA = 4.0
U_BF16 = 2.0 ** -8
U_F32 = 2.0 ** -24


def _f64(x):
    import la_inputs as inp
    return inp.to_f64(x) if not isinstance(x, np.ndarray) else x.astype(np.float64, copy=False)


def phi(x):
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def _heads3(x):
    x = np.asarray(x, dtype=np.float64)
    return x.reshape(-1, x.shape[-2], x.shape[-1])


def _cum(x, causal):
    """sum over j <= i along axis 1 (causal) or the total over all j, broadcast."""
    if causal:
        return np.cumsum(x, axis=1)
    return np.broadcast_to(x.sum(axis=1, keepdims=True), x.shape)


def _rcum(x, causal):
    """sum over i >= j along axis 1 (causal) or the total, broadcast."""
    if causal:
        return np.cumsum(x[:, ::-1], axis=1)[:, ::-1]
    return np.broadcast_to(x.sum(axis=1, keepdims=True), x.shape)


def _count(N, causal, n0=None):
    n = np.arange(1, N + 1, dtype=np.float64) if causal else np.full(N, float(N))
    n = n[None, :]
    return n if n0 is None else n + np.asarray(n0, dtype=np.float64).reshape(-1, 1)


class Features:
    """Per-head features: qf, kf [BH, N, d]; e = the part of kf in bf16 products;
    split: the kernels carry kf = 1 + e with the 1 in fp32."""

    def __init__(self, qf, kf, split):
        self.qf, self.kf, self.split = _heads3(qf), _heads3(kf), split
        self.e = self.kf - 1.0 if split else self.kf

    @classmethod
    def elu(cls, q, k):
        return cls(phi(_heads3(_f64(q))), phi(_heads3(_f64(k))), True)

    @classmethod
    def given(cls, fq, fk):
        return cls(_f64(fq), _f64(fk), False)


def _split_state(S0, z0, split):
    """(S0_E, z0_E, P0, n0) as the kernels carry a start state: around the means over the
    feature index when split, as it is otherwise.  S0 [BH, d, d], z0 [BH, d]."""
    S0 = np.asarray(S0, dtype=np.float64).reshape(-1, S0.shape[-2], S0.shape[-1])
    z0 = np.asarray(z0, dtype=np.float64).reshape(-1, z0.shape[-1])
    if not split:
        return S0, z0, np.zeros(S0.shape[::2]), np.zeros(z0.shape[0])
    P0 = S0.mean(axis=1)                 # [BH, d(b)]
    n0 = z0.mean(axis=1)                 # [BH]
    return S0 - P0[:, None, :], z0 - n0[:, None], P0, n0


def floor_o(F, v, o, den, causal, u, S0=None, z0=None):
    v, o = _heads3(v), _heads3(o)
    den = np.asarray(den, dtype=np.float64).reshape(o.shape[:2])
    N, d = o.shape[1], o.shape[2]
    kf2 = (F.kf ** 2).sum(-1)
    a = _cum(kf2 * (v ** 2).sum(-1), causal)
    b = _cum(kf2[..., None] * v, causal)
    c = _cum(kf2, causal)
    s = a - 2.0 * (o * b).sum(-1) + (o ** 2).sum(-1) * c
    T2 = (F.qf ** 2).sum(-1) * np.maximum(s, 0.0)
    if S0 is not None:
        S0h = np.asarray(S0, dtype=np.float64).reshape(-1, d, d)
        z0h = np.asarray(z0, dtype=np.float64).reshape(-1, d)
        m = np.einsum("hna,hab->hnb", F.qf, S0h) - np.einsum("hna,ha->hn", F.qf, z0h)[..., None] * o
        T2 = T2 + (m ** 2).sum(-1)
    T = np.sqrt(T2) / den
    n = _count(N, causal)
    return LAMBDA * (u + U_F32 * np.sqrt(n + d)) * T


def floor_dv(F, g, causal, u, dSN=None):
    g = _heads3(g)
    N, d = g.shape[1], g.shape[2]
    s = _rcum((F.qf ** 2).sum(-1) * (g ** 2).sum(-1), causal)
    T2 = (F.kf ** 2).sum(-1) * s
    if dSN is not None:
        r = (np.asarray(dSN, dtype=np.float64).reshape(-1, d, d) ** 2).sum(-1)  # [BH, a]
        T2 = T2 + np.einsum("hna,ha->hn", F.kf ** 2, r)
    # summands: tokens i >= j (causal) or all tokens
    n = (N - np.arange(N, dtype=np.float64))[None, :] if causal else np.full((1, N), float(N))
    return LAMBDA * (u + U_F32 * np.sqrt(n + d)) * np.sqrt(T2)


def g_error(o, g, u):
    """Bound on the error of g = -G . O where g is not formed from the sweep's own products."""
    o, g = _heads3(o), _heads3(g)
    return u * (np.abs((g * o).sum(-1)) + np.abs(g * o).sum(-1))


def floor_dk(F, v, o, g, causal, u, dSN=None, gerr=None):
    v, o, g = _heads3(v), _heads3(o), _heads3(g)
    N, d = v.shape[1], v.shape[2]
    w = (F.qf ** 2).sum(-1)
    g2 = g ** 2
    C1 = _rcum(w[..., None] * g2, causal)
    C2 = _rcum(w[..., None] * g2 * o, causal)
    C3 = _rcum(w * (g2 * o * o).sum(-1), causal)
    T2 = np.maximum((v * v * C1).sum(-1) - 2.0 * (v * C2).sum(-1) + C3, 0.0)
    if dSN is not None:
        cs = (np.asarray(dSN, dtype=np.float64).reshape(-1, d, d) ** 2).sum(1)  # [BH, b]
        T2 = T2 + np.einsum("hnb,hb->hn", v * v, cs)
    # summands: tokens i >= j (causal) or all tokens
    n = (N - np.arange(N, dtype=np.float64))[None, :] if causal else np.full((1, N), float(N))
    fl = LAMBDA * (u + U_F32 * np.sqrt(n + d)) * np.sqrt(T2)
    if gerr is not None:
        fl = fl + LAMBDA * np.sqrt(_rcum(gerr ** 2 * w, causal))
    return fl


def floor_dq(F, v, o, g, causal, u, S0=None, z0=None, gerr=None):
    v, o, g = _heads3(v), _heads3(o), _heads3(g)
    N, d = v.shape[1], v.shape[2]
    e2 = (F.e ** 2).sum(-1)
    D1 = _cum(e2[..., None] * v * v, causal)
    D2 = _cum(e2[..., None] * v, causal)
    D3 = _cum(e2, causal)
    g2 = g ** 2
    T2 = np.maximum((g2 * (D1 - 2.0 * o * D2 + o * o * D3[..., None])).sum(-1), 0.0)
    Tf2 = (g2 * (D1 + o * o * D3[..., None])).sum(-1)
    n0 = None
    P = _cum(v, causal)
    if S0 is not None:
        SE, zE, P0, n0 = _split_state(S0, z0, F.split)
        cn = (SE ** 2).sum(1)                          # |S0_E[:, b]|^2, [BH, b]
        cz = np.einsum("hab,ha->hb", SE, zE)           # S0_E[:, b] . z0_E
        z2 = (zE ** 2).sum(-1)                         # |z0_E|^2
        T2 = T2 + (g2 * (cn[:, None, :] - 2.0 * o * cz[:, None, :] + o * o * z2[:, None, None])).sum(-1)
        Tf2 = Tf2 + (g2 * (cn[:, None, :] + o * o * z2[:, None, None])).sum(-1)
        P = P + P0[:, None, :]
    n = _count(N, causal, n0)
    extra = 0.0
    if gerr is not None:
        z = _cum(F.kf, causal)
        if S0 is not None:
            z = z + np.asarray(z0, dtype=np.float64).reshape(-1, 1, d)
        extra = LAMBDA * gerr * np.sqrt((z ** 2).sum(-1))
    if F.split:
        T2 = T2 + d * (g2 * (P - n[..., None] * o) ** 2).sum(-1)
        Tf2 = Tf2 + d * (g2 * (P * P + (n[..., None] * o) ** 2)).sum(-1)
    return LAMBDA * (u * np.sqrt(T2) + U_F32 * np.sqrt(n + d) * np.sqrt(T2 + Tf2)) + extra


def u_of(dtype_is_bf16):
    return U_BF16 if dtype_is_bf16 else 0.0


def row_check(gpu, ref, tol, floor):
    """max over rows of ||x_i - y_i|| / (tol ||y_i|| + floor_i) (pass: <= 1), and the fraction
    of rows whose floor exceeds tol ||y_i|| (how often the floor, not the relative bar, decides)."""
    x = _heads3(_f64(gpu))
    y = _heads3(ref)
    assert np.isfinite(x).all(), "non-finite GPU output"
    fl = np.asarray(floor, dtype=np.float64)
    fl = fl.reshape(x.shape[:2]) if fl.size == x.shape[0] * x.shape[1] else np.broadcast_to(fl, x.shape[:2])
    err = np.sqrt(((x - y) ** 2).sum(-1))
    rel = tol * np.sqrt((y ** 2).sum(-1))
    bar = rel + fl
    ratio = np.where(bar > 0, err / np.where(bar > 0, bar, 1.0), np.where(err > 0, np.inf, 0.0))
    return float(ratio.max()) if ratio.size else 0.0, float((fl > rel).mean()) if fl.size else 0.0


def grads_g(dout, o, den):
    """G = dO / den per row, from the oracle's exact den."""
    dout, o = _heads3(_f64(dout)), _heads3(o)
    den = np.asarray(den, dtype=np.float64).reshape(o.shape[:2])
    return dout / den[..., None]
