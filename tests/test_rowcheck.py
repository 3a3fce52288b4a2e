"""The per-row parity bars of rowcheck.py, checked on the CPU with the oracle alone.

* The floors are rounding bounds: the oracle run on operands rounded the way the
  kernels round them (phi(Q), E(K) and G = dO / den to bf16, or to fp32 for fp32
  inputs) moves every row of O, dQ, dK and dV by less than its floor alone.
* The bars see errors confined to late rows: scaling the last 512 rows (or just the
  ragged tail) of an exact output by 1.1 fails the check, where the per-head
  Frobenius error of the same change stays far below the tolerance.
"""
import numpy as np
import pytest
import torch

import la_inputs as inp
import rowcheck as rc

TOL_BF16 = 2e-2


def _round(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).double().numpy()


def _problem(oracle, N, d, causal, seed):
    q, k, v, do = (inp.to_f64(t) for t in inp.qkv(1, 2, N, d, torch.bfloat16, seed=seed, with_dout=True))
    fwd = oracle.forward_causal if causal else oracle.forward_noncausal
    o, den = fwd(q, k, v, return_den=True)
    bwd = oracle.backward_causal if causal else oracle.backward_noncausal
    dq, dk, dv = bwd(q, k, v, do)
    return q, k, v, do, o, den, (dq, dk, dv)


def _floors(q, k, v, do, o, den, causal, u):
    F = rc.Features.elu(q, k)
    g = rc.grads_g(do, o, den)
    return {"o": rc.floor_o(F, v, o, den, causal, u), "dq": rc.floor_dq(F, v, o, g, causal, u),
            "dk": rc.floor_dk(F, v, o, g, causal, u), "dv": rc.floor_dv(F, g, causal, u)}


def _rounded_run(oracle, q, k, v, do, den, causal, dtype):
    """The oracle on the operands the kernels round: phi(Q), E(K) and G to `dtype`."""
    fq = _round(rc.phi(q), dtype)
    fk = 1.0 + _round(rc.phi(k) - 1.0, dtype)
    G = _round(do / den[..., None], dtype)
    o = oracle.forward_features(fq, fk, v, causal)
    dfq, dfk, dv = oracle.backward_features(fq, fk, v, G * den[..., None], causal)
    dphi_q = np.minimum(rc.phi(q), 1.0)
    dphi_k = np.minimum(rc.phi(k), 1.0)
    return o, dfq * dphi_q, dfk * dphi_k, dv


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_floors_cover_operand_rounding(oracle, causal, dtype):
    N, d = 777, 64
    q, k, v, do, o, den, grads = _problem(oracle, N, d, causal, seed=3)
    u = rc.u_of(dtype == torch.bfloat16)
    fl = _floors(q, k, v, do, o, den, causal, u if dtype == torch.bfloat16 else rc.U_F32)
    got = _rounded_run(oracle, q, k, v, do, den, causal, dtype)
    for name, x, y in zip(("o", "dq", "dk", "dv"), got, (o,) + grads):
        ratio, _ = rc.row_check(x, y, 2.0 ** -40, fl[name])  # 2^-40: the oracle's own fp64 rounding
        assert ratio <= 1.0, (name, ratio)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
@pytest.mark.parametrize("rows", [512, 17], ids=["last512", "tail17"])
def test_late_row_errors_fail(oracle, causal, rows):
    N, d = 64 * 40 + 17, 64
    q, k, v, do, o, den, grads = _problem(oracle, N, d, causal, seed=4)
    fl = _floors(q, k, v, do, o, den, causal, rc.U_BF16)
    for name, y in zip(("o", "dq", "dk", "dv"), (o,) + grads):
        assert rc.row_check(y, y, TOL_BF16, fl[name])[0] == 0.0
        x = y.copy()
        x[..., N - rows:, :] *= 1.1
        ratio, _ = rc.row_check(x, y, TOL_BF16, fl[name])
        assert ratio > 1.0, (name, rows, ratio)
        fro = np.linalg.norm((x - y).reshape(2, -1), axis=1) / np.linalg.norm(y.reshape(2, -1), axis=1)
        if causal and name == "o" and rows == 512:
            assert fro.max() < TOL_BF16  # what a per-head norm would have let through


def test_dq_row0_floor_covers_fp32_noise(oracle):
    """dQ_0 = 0 exactly (O_0 = V_0 whatever q and k are); its floor is the fp32 rounding
    of the terms that cancel there, so a residual of a few fp32 ulps of them passes."""
    N, d = 70, 32
    q, k, v, do, o, den, (dq, dk, dv) = _problem(oracle, N, d, True, seed=5)
    assert np.abs(dq[..., 0, :]).max() < 1e-12
    fl = _floors(q, k, v, do, o, den, True, 0.0)["dq"]
    assert (fl[:, 0] > 0).all()
    G0 = do[..., 0, :] / den[..., 0, None]
    noise = 2.0 ** -23 * np.abs((G0 * v[..., 0, :]).sum(-1)) * np.linalg.norm(rc.phi(k[..., 0, :]), axis=-1)
    assert (noise.reshape(-1) < fl[:, 0]).all()
