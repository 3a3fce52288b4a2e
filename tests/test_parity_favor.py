"""GPU parity of the FAVOR+ path (Performer section of the page "Efficient
Transformers Survey") against the fp64 oracle: the random-feature kernel, the
forward calls and multi-token decode on given features.  Queries and keys are
pre-normalized by d^(-1/4) as the page prescribes (la_inputs.favor_qkv); without
it the features of d = 128 rows fall below fp32's range.

The library's features leave out the page's constant 1/sqrt(m) (m = d): it
cancels in every output O, so outputs compare directly, while features, states
and denominators compare after scaling the oracle's by sqrt(m) (states, z) or m
(den).  Directions omega come from la_inputs.favor_omega (rows ~ N(0, I_d)).
Sequence outputs (O, dfq, dfk, dv, and dq, dk through the feature map) are checked
row by row against the bars of rowcheck.py, on the features as given.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import la_inputs as inp  # noqa: E402
import rowcheck as rc  # noqa: E402
from test_parity import TOL, bwd_rows, draw, f64, fwd_rows, record, row_ratios, rows, slice_err  # noqa: E402


def given_o_rows(o, ro, rden, fq, fk, v, dtype, causal, first=0):
    """The worst row ratio of an output on given features (oracle features fq, fk of the
    whole sequence, natural order); only rows from `first` on are compared."""
    F = rc.Features.given(fq, fk)
    fl = rc.floor_o(F, f64(v), ro, rden, causal, rc.u_of(dtype == torch.bfloat16))
    ratio, _ = rc.row_check(o, ro[..., first:, :], TOL[dtype], fl.reshape(ro.shape[:-1])[..., first:])
    return ratio


@pytest.fixture(scope="module")
def la():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_02_amd as m
    m.load_library()
    return m


def feat_bound(ref, x, om, dtype):
    """First-order bound on the error of every feature (the tests hold each error to it).  exp turns the
    exponent's absolute error into a relative one: the exponent omega_i.x - |x|^2/2 is an
    fp32 dot product of d terms (error <= (d + 2) 2^-24 (sum_k |omega_ik x_k| + |x|^2/2)),
    bf16 rows take omega as bf16 hi + lo parts (a further 2^-16 sum_k |omega_ik x_k|) and
    round the feature to bf16 (u = 2^-8); fp32 rows add a few ulp of exp2.  ref: the
    oracle's features without the constant, [..., m] in the natural feature order."""
    xx, oo = f64(x), f64(om)
    d = xx.shape[-1]
    s = np.abs(xx) @ np.abs(oo).T + 0.5 * (xx * xx).sum(-1, keepdims=True)
    c = (d + 2) * 2.0 ** -24 + (2.0 ** -16 if dtype == torch.bfloat16 else 0.0)
    u = 2.0 ** -8 if dtype == torch.bfloat16 else 4 * 2.0 ** -24
    return ref * (u + c * s)


# States and denominators on bf16 features: sums of features each rounded once (<= u);
# FAVOR+ features are heavy-tailed (lognormal), so a few large terms carry the sums and the
# rounding does not average out: the bar is 1.25 u (fp32: 1e-4).
SUM_TOL = {torch.float32: 1e-4, torch.bfloat16: 1.25 * 2.0 ** -8}


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_favor_features(la, oracle, d, dtype):
    rows = 777  # several workgroups of 256 rows and a ragged tail
    x = inp.normal((rows, d), inp.generator(d), dtype, d ** -0.25).cuda()
    om = inp.favor_omega(d, seed=d + 1).cuda()
    f = la.favor_features(x, om)
    torch.cuda.synchronize()
    ref = oracle.favor_features(f64(x), f64(om)) * math.sqrt(d)
    err = slice_err(f[None], ref[None])
    ratio = float((np.abs(f64(f) - ref) / feat_bound(ref, x, om, dtype)).max())
    assert (f64(f) > 0).all()
    record(f"favor_features d={d} {dtype}", f=err, ratio=ratio)
    assert ratio <= 1.0, (ratio, err)


SHAPES = [(1, 1, 1, 32), (1, 2, 63, 64), (2, 3, 200, 64), (1, 2, 300, 128), (2, 2, 1000, 64), (1, 8, 64 * 130 + 17, 64)]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_favor_forward(la, oracle, shape, dtype, causal):
    B, H, N, d = shape
    if dtype == torch.float32 and d == 128 and causal:
        pytest.skip("fp32 causal path is built for d <= 64")
    q, k, v = (t.cuda() for t in inp.favor_qkv(B, H, N, d, dtype, seed=N + 40))
    om = inp.favor_omega(d, seed=N + 41).cuda()
    fq, fk = la.favor_features(q, om), la.favor_features(k, om)
    if causal:
        o, den, S, z = la.la_forward_causal_features(fq, fk, v, return_den=True, return_state=True)
    else:
        o = la.la_forward_noncausal_features(fq, fk, v)
    torch.cuda.synchronize()
    rfq, rfk = oracle.favor_features(f64(q), f64(om)), oracle.favor_features(f64(k), f64(om))
    errs = {}
    if causal:
        ro, rden, rS, rz = oracle.forward_features(rfq, rfk, f64(v), True, return_den=True, return_state=True)
        m = float(d)
        errs.update(den=slice_err(den, rden * m), S=slice_err(S, rS * math.sqrt(m)),
                    z=slice_err(z[..., None], rz[..., None] * math.sqrt(m)))
    else:
        ro, rden = oracle.forward_features(rfq, rfk, f64(v), False, return_den=True)
    errs["o"] = given_o_rows(o, ro, rden, rfq, rfk, v, dtype, causal)
    errs["o_fro"] = slice_err(o, ro)
    record(f"favor_fwd {'causal' if causal else 'noncausal'} {B}x{H}x{N}x{d} {dtype}", **errs)
    assert errs["o"] <= 1.0, errs
    if causal:
        assert max(errs["den"], errs["S"], errs["z"]) < SUM_TOL[dtype], errs


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_favor_prefill_then_decode(la, oracle, dtype):
    """Prefill on FAVOR+ features, then multi-token decode with grouped heads from the
    state it left: the oracle runs each query head over its key/value head's whole
    sequence of features."""
    B, Hkv, G, N0, T, d = 2, 2, 3, 150, 9, 64
    H = Hkv * G
    om = inp.favor_omega(d, seed=5).cuda()
    pq, pk, pv = (t.cuda() for t in inp.favor_qkv(B, Hkv, N0, d, dtype, seed=6))
    _, S, z = la.la_forward_causal_features(la.favor_features(pq, om), la.favor_features(pk, om), pv,
                                            return_state=True)
    q = inp.favor_qkv(B, H, T, d, dtype, seed=7)[0].cuda()
    _, k, v = (t.cuda() for t in inp.favor_qkv(B, Hkv, T, d, dtype, seed=8))
    o = la.la_decode_steps_features(S, z, la.favor_features(q, om), la.favor_features(k, om), v)
    torch.cuda.synchronize()
    worst = 0.0
    for h in range(H):
        j = h // G
        kk, vv = np.concatenate([f64(pk[:, j]), f64(k[:, j])], 1), np.concatenate([f64(pv[:, j]), f64(v[:, j])], 1)
        qq = np.concatenate([f64(pq[:, j]), f64(q[:, h])], 1)  # prefix rows are not compared
        ffq, ffk = oracle.favor_features(qq, f64(om)), oracle.favor_features(kk, f64(om))
        ro, rden = oracle.forward_features(ffq, ffk, vv, True, return_den=True)
        worst = max(worst, given_o_rows(o[:, h], ro, rden, ffq, ffk, vv, dtype, True, first=N0))
    record(f"favor prefill+decode {dtype}", o=worst)
    assert worst <= 1.0, worst


def test_given_elu_features_match_builtin_map(la):
    """Features elu(x) + 1 applied by the caller give the built-in map's outputs (fp32)."""
    q, k, v, _ = draw(2, 3, 333, 64, torch.float32, seed=50)
    phi = lambda x: torch.nn.functional.elu(x) + 1.0
    a = la.la_forward_causal_features(phi(q), phi(k), v)
    b = la.la_forward_causal(q, k, v)
    c = la.la_forward_noncausal_features(phi(q), phi(k), v)
    e = la.la_forward_noncausal(q, k, v)
    torch.cuda.synchronize()
    assert torch.allclose(a, b, rtol=1e-4, atol=1e-5) and torch.allclose(c, e, rtol=1e-4, atol=1e-5)


# ---- more random features than d: m = KF d in KF blocks ---------------------------------------
def to_blocks(f, KF):
    """[..., N, m] features (natural order) -> [..., KF, N, d] block layout."""
    *lead, N, m = f.shape
    d = m // KF
    return np.moveaxis(f.reshape(*lead, N, KF, d), -2, -3)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("d,KF", [(32, 2), (64, 2), (64, 4), (128, 2)], ids=lambda x: str(x))
def test_favor_features_blocks(la, oracle, d, KF, dtype):
    B, H, N, m = 2, 3, 130, KF * d
    x = inp.normal((B, H, N, d), inp.generator(d + KF), dtype, d ** -0.25).cuda()
    om = inp.favor_omega(d, seed=d + KF, m=m).cuda()
    f = la.favor_features_blocks(x, om)
    torch.cuda.synchronize()
    assert f.shape == (B, H, KF, N, d)
    refn = oracle.favor_features(f64(x), f64(om)) * math.sqrt(m)
    ref = to_blocks(refn, KF)
    err = slice_err(f, ref)
    ratio = float((np.abs(f64(f) - ref) / to_blocks(feat_bound(refn, x, om, dtype), KF)).max())
    assert (f64(f) > 0).all()
    record(f"favor_features_blocks d={d} m={m} {dtype}", f=err, ratio=ratio)
    assert ratio <= 1.0, (ratio, err)


BLOCK_SHAPES = [(1, 1, 1, 32, 2), (2, 3, 200, 64, 2), (1, 2, 300, 128, 2), (2, 2, 1000, 64, 4),
                (1, 4, 64 * 130 + 17, 64, 2)]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("shape", BLOCK_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_favor_forward_blocks(la, oracle, shape, dtype, causal):
    """Attention on m = KF d features against the oracle's explicit m-feature form."""
    B, H, N, d, KF = shape
    m = KF * d
    if dtype == torch.float32 and d == 128 and causal:
        pytest.skip("fp32 causal path is built for d <= 64")
    q, k, v = (t.cuda() for t in inp.favor_qkv(B, H, N, d, dtype, seed=N + 60))
    om = inp.favor_omega(d, seed=N + 61, m=m).cuda()
    fq, fk = la.favor_features_blocks(q, om), la.favor_features_blocks(k, om)
    if causal:
        o, den, S, z = la.la_forward_causal_features_blocks(fq, fk, v, return_den=True, return_state=True)
    else:
        o, den = la.la_forward_noncausal_features_blocks(fq, fk, v, return_den=True)
    torch.cuda.synchronize()
    rfq, rfk = oracle.favor_features(f64(q), f64(om)), oracle.favor_features(f64(k), f64(om))
    ro, rden, rS, rz = oracle.forward_features(rfq, rfk, f64(v), causal, return_den=True, return_state=True)
    errs = {"den": slice_err(den, rden * m)}
    if causal:
        errs.update(S=slice_err(S, rS * math.sqrt(m)), z=slice_err(z[..., None], rz[..., None] * math.sqrt(m)))
    errs["o"] = given_o_rows(o, ro, rden, rfq, rfk, v, dtype, causal)
    record(f"favor_fwd_blocks {'causal' if causal else 'noncausal'} {B}x{H}x{N}x{d} m={m} {dtype}", **errs)
    assert errs["o"] <= 1.0, errs
    assert max(v for n, v in errs.items() if n != "o") < SUM_TOL[dtype], errs


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_favor_blocks_in_pieces(la, oracle, dtype):
    """m = 2 d features fed in two pieces, the second continuing in place from the
    [B, H, m, d] state the first left: the oracle's recurrence over the whole sequence."""
    B, H, N, p, d, KF = 2, 2, 500, 210, 64, 2
    m = KF * d
    q, k, v = (t.cuda() for t in inp.favor_qkv(B, H, N, d, dtype, seed=70))
    om = inp.favor_omega(d, seed=71, m=m).cuda()
    cut = lambda t, a, b: t[:, :, a:b].contiguous()
    fq, fk = la.favor_features_blocks(q, om), la.favor_features_blocks(k, om)
    fcut = lambda f, a, b: f[:, :, :, a:b].contiguous()
    o1, S, z = la.la_forward_causal_features_blocks(fcut(fq, 0, p), fcut(fk, 0, p), cut(v, 0, p), return_state=True)
    o2 = la.la_forward_causal_features_blocks(fcut(fq, p, N), fcut(fk, p, N), cut(v, p, N), S0=S, z0=z, S_out=S,
                                              z_out=z)
    torch.cuda.synchronize()
    rfq, rfk = oracle.favor_features(f64(q), f64(om)), oracle.favor_features(f64(k), f64(om))
    ro, rden, rS, rz = oracle.forward_features(rfq, rfk, f64(v), True, return_den=True, return_state=True)
    errs = {"o": given_o_rows(torch.cat([o1, o2], dim=2), ro, rden, rfq, rfk, v, dtype, True),
            "S": slice_err(S, rS * math.sqrt(m)), "z": slice_err(z[..., None], rz[..., None] * math.sqrt(m))}
    record(f"favor blocks in pieces {dtype}", **errs)
    assert errs["o"] <= 1.0, errs
    assert max(errs["S"], errs["z"]) < SUM_TOL[dtype], errs


def test_favor_blocks_of_one_match_plain_calls(la):
    """m = d through the block calls is the plain feature calls."""
    q, k, v = (t.cuda() for t in inp.favor_qkv(2, 3, 333, 64, torch.bfloat16, seed=80))
    om = inp.favor_omega(64, seed=81).cuda()
    fq, fk = la.favor_features(q, om), la.favor_features(k, om)
    bq, bk = la.favor_features_blocks(q, om), la.favor_features_blocks(k, om)
    a = la.la_forward_causal_features(fq, fk, v)
    b = la.la_forward_causal_features_blocks(bq, bk, v)
    c = la.la_forward_noncausal_features(fq, fk, v)
    e = la.la_forward_noncausal_features_blocks(bq, bk, v)
    torch.cuda.synchronize()
    assert torch.equal(fq, bq[:, :, 0]) and torch.equal(a, b) and torch.equal(c, e)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("KF", [2, 3])
@pytest.mark.parametrize("d", [64, 128])
def test_favor_blocks_prefill_then_decode(la, oracle, d, KF, dtype):
    """m = KF d features: prefill per key/value head, then multi-token decode with 3 query
    heads per key/value head from the [B, Hkv, m, d] state it left, against the oracle's
    m-feature recurrence over each query head's whole sequence."""
    if dtype == torch.float32 and d == 128:
        pytest.skip("fp32 causal path is built for d <= 64")
    B, Hkv, G, N0, T = 2, 2, 3, 150, 11
    H, m = Hkv * G, KF * d
    om = inp.favor_omega(d, seed=15 + KF, m=m).cuda()
    pq, pk, pv = (t.cuda() for t in inp.favor_qkv(B, Hkv, N0, d, dtype, seed=16))
    _, S, z = la.la_forward_causal_features_blocks(la.favor_features_blocks(pq, om), la.favor_features_blocks(pk, om),
                                                   pv, return_state=True)
    q = inp.favor_qkv(B, H, T, d, dtype, seed=17)[0].cuda()
    _, k, v = (t.cuda() for t in inp.favor_qkv(B, Hkv, T, d, dtype, seed=18))
    o = la.la_decode_steps_features_blocks(S, z, la.favor_features_blocks(q, om), la.favor_features_blocks(k, om), v)
    torch.cuda.synchronize()
    worst, rS, rz = 0.0, [None] * Hkv, [None] * Hkv
    for h in range(H):
        j = h // G
        kk, vv = np.concatenate([f64(pk[:, j]), f64(k[:, j])], 1), np.concatenate([f64(pv[:, j]), f64(v[:, j])], 1)
        qq = np.concatenate([f64(pq[:, j]), f64(q[:, h])], 1)  # prefix rows are not compared
        ffq, ffk = oracle.favor_features(qq, f64(om)), oracle.favor_features(kk, f64(om))
        ro, rden, rS[j], rz[j] = oracle.forward_features(ffq, ffk, vv, True, return_den=True, return_state=True)
        worst = max(worst, given_o_rows(o[:, h], ro, rden, ffq, ffk, vv, dtype, True, first=N0))
    rS, rz = np.stack(rS, 1), np.stack(rz, 1)
    errs = {"o": worst, "S": slice_err(S, rS * math.sqrt(m)), "z": slice_err(z[..., None], rz[..., None] * math.sqrt(m))}
    record(f"favor blocks prefill+decode d={d} m={m} {dtype}", **errs)
    assert errs["o"] <= 1.0, errs
    assert max(errs["S"], errs["z"]) < SUM_TOL[dtype], errs


# ---- backward: on given features, through the feature map, and end to end ----------------------
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_favor_backward_given_features(la, oracle, shape, dtype, causal):
    """dfq, dfk, dv on the library's FAVOR+ features against the oracle on the same features."""
    B, H, N, d = shape
    if dtype == torch.float32 and d == 128:
        pytest.skip("fp32 backward is built for d <= 64")
    q, k, v, do = (t.cuda() for t in inp.favor_qkv(B, H, N, d, dtype, seed=N + 90, with_dout=True))
    om = inp.favor_omega(d, seed=N + 91).cuda()
    fq, fk = la.favor_features(q, om), la.favor_features(k, om)
    dfq, dfk, dv = la.la_backward_causal_features(fq, fk, v, do, causal=causal)
    torch.cuda.synchronize()
    ref = oracle.backward_features(f64(fq), f64(fk), f64(v), f64(do), causal)
    if N == 1:
        # A single token: O_0 = V_0 whatever the features, so dfq and dfk vanish exactly and
        # only rounding is left.  Causal: g is formed from the very products of dA, so dA_00 is
        # a few fp32 roundings of M = sum_b |G_b V_b| (G = dO / den).  Non-causal: the state
        # S = fk V^T and R = fq G^T enter their MFMAs rounded to bf16 against fp32 terms that
        # cancel them, which leaves at most 2 u M fk_a in dfq_a and 2 u M fq_a in dfk_a (u = 2^-8).
        ffq, ffk, vv = f64(fq), f64(fk), f64(v)
        den = (ffq * ffk).sum(-1, keepdims=True)
        M = (np.abs(f64(do) / den) * np.abs(vv)).sum(-1, keepdims=True)
        c = 2.0 ** -7 if (dtype == torch.bfloat16 and not causal) else 1e-5
        assert (np.abs(f64(dfq)) <= c * M * ffk + 1e-30).all()
        assert (np.abs(f64(dfk)) <= c * M * ffq + 1e-30).all()
        assert slice_err(dv, ref[2]) < TOL[dtype]
        return
    errs = bwd_rows({}, (dfq, dfk, dv), ref, fq, fk, v, do, dtype, causal, F=rc.Features.given(f64(fq), f64(fk)),
                    names=("dfq", "dfk", "dv"))
    record(f"favor_bwd {'causal' if causal else 'noncausal'} {B}x{H}x{N}x{d} {dtype}", **errs)
    assert max(row_ratios(errs).values()) <= 1.0, errs


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_favor_features_backward(la, oracle, d, dtype):
    """dx of the feature map, each element held to its first-order bound: the features the
    kernel is handed carry their own error (feat_bound), the bf16 Omega split 2^-16, and the
    fp32 sums (d + 2) 2^-24, each times sum_i |dF_i F_i| (|omega_ia| + |x_a|); then dx is
    rounded to the output dtype (u |dx|)."""
    rows = 777
    x = inp.normal((rows, d), inp.generator(d + 7), dtype, d ** -0.25).cuda()
    om = inp.favor_omega(d, seed=d + 8).cuda()
    F = la.favor_features(x, om)
    dF = inp.normal((rows, d), inp.generator(d + 9), dtype, 1.0).cuda()
    dx = la.favor_features_backward(x, om, F, dF)
    torch.cuda.synchronize()
    ref = oracle.favor_features_backward(f64(x), f64(om), f64(dF)) * math.sqrt(d)
    refF = oracle.favor_features(f64(x), f64(om)) * math.sqrt(d)
    xx, oo, g = f64(x), f64(om), np.abs(f64(dF))
    fb = feat_bound(refF, x, om, dtype)
    c = (2.0 ** -16 if dtype == torch.bfloat16 else 0.0) + (d + 2) * 2.0 ** -24
    bound = (g * fb) @ np.abs(oo) + np.abs(xx) * (g * fb).sum(-1, keepdims=True)
    bound += c * ((g * refF) @ np.abs(oo) + np.abs(xx) * (g * refF).sum(-1, keepdims=True))
    bound += (2.0 ** -8 if dtype == torch.bfloat16 else 2.0 ** -24) * np.abs(ref)
    ratio = float((np.abs(f64(dx) - ref) / bound).max())
    record(f"favor_features_bwd d={d} {dtype}", ratio=ratio, dx=slice_err(dx[None], ref[None]))
    assert ratio <= 1.0, ratio


@pytest.mark.parametrize("KF", [1, 2, 3])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_favor_features_blocks_backward(la, oracle, d, dtype, KF):
    """dx through m = KF d features in block layout, against the oracle's feature-map gradient
    over all m features, each element held to the bound of the m = d test with sums of m terms."""
    B, H, N = 2, 3, 129
    m = KF * d
    x = inp.normal((B, H, N, d), inp.generator(d + 17), dtype, d ** -0.25).cuda()
    om = inp.favor_omega(d, seed=d + 18, m=m).cuda()
    F = la.favor_features_blocks(x, om)
    dF = inp.normal((B, H, KF, N, d), inp.generator(d + 19), dtype, 1.0).cuda()
    dx = la.favor_features_blocks_backward(x, om, F, dF)
    torch.cuda.synchronize()
    dFn = from_blocks(f64(dF))
    ref = oracle.favor_features_backward(f64(x), f64(om), dFn) * math.sqrt(m)
    refF = oracle.favor_features(f64(x), f64(om)) * math.sqrt(m)
    xx, oo, g = f64(x), f64(om), np.abs(dFn)
    fb = feat_bound(refF, x, om, dtype)
    c = (2.0 ** -16 if dtype == torch.bfloat16 else 0.0) + (m + 2) * 2.0 ** -24
    bound = (g * fb) @ np.abs(oo) + np.abs(xx) * (g * fb).sum(-1, keepdims=True)
    bound += c * ((g * refF) @ np.abs(oo) + np.abs(xx) * (g * refF).sum(-1, keepdims=True))
    bound += (2.0 ** -8 if dtype == torch.bfloat16 else 2.0 ** -24) * np.abs(ref)
    ratio = float((np.abs(f64(dx) - ref) / bound).max())
    record(f"favor_features_blocks_bwd d={d} m={m} {dtype}", ratio=ratio)
    assert ratio <= 1.0, ratio


@pytest.mark.parametrize("KF", [1, 2])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_favor_attention_autograd(la, oracle, dtype, causal, KF):
    """Performer attention trained end to end: O and dq, dk, dv of the autograd op against the
    oracle's chain (features, attention on features, its backward, the feature map's backward);
    the constant 1/sqrt(m) the library leaves out changes none of them.  KF = 2: m = 2d
    features, run in feature blocks."""
    B, H, N, d = 2, 3, 333, 64
    q, k, v, do = (t.cuda() for t in inp.favor_qkv(B, H, N, d, dtype, seed=100, with_dout=True))
    om = inp.favor_omega(d, seed=101, m=KF * d).cuda()
    q.requires_grad_(True)
    k.requires_grad_(True)
    v.requires_grad_(True)
    o = la.favor_attention(q, k, v, om, causal)
    o.backward(do)
    torch.cuda.synchronize()
    rfq, rfk = oracle.favor_features(f64(q), f64(om)), oracle.favor_features(f64(k), f64(om))
    ro = oracle.forward_features(rfq, rfk, f64(v), causal)
    dfq, dfk, rdv = oracle.backward_features(rfq, rfk, f64(v), f64(do), causal)
    rdq = oracle.favor_features_backward(f64(q), f64(om), dfq)
    rdk = oracle.favor_features_backward(f64(k), f64(om), dfk)
    # Row floors: those of dfq, dfk, dv on the oracle's features, carried through the feature
    # map's chain dx_i = sum_c dF_ic F_ic (omega_c - x_i) (Cauchy-Schwarz over c), plus the
    # features' own rounding (u F) in that chain.
    F = rc.Features.given(rfq, rfk)
    u = rc.u_of(dtype == torch.bfloat16)
    _, rden = oracle.forward_features(rfq, rfk, f64(v), causal, return_den=True)
    g = rc.grads_g(f64(do), ro, rden)
    ww = f64(om)

    def chain(fl_df, df, ff, x):
        x = rc._heads3(x)
        ff, df = rc._heads3(ff), rc._heads3(df)
        w2 = (ww * ww).sum(-1)
        f2 = ff * ff
        c = f2 @ w2 - 2.0 * ((f2 @ ww) * x).sum(-1) + (x * x).sum(-1) * f2.sum(-1)
        c2 = (df * df * f2) @ w2 - 2.0 * (((df * df * f2) @ ww) * x).sum(-1) + (x * x).sum(-1) * (df * df * f2).sum(-1)
        return fl_df * np.sqrt(np.maximum(c, 0.0)) + rc.LAMBDA * max(u, rc.U_F32) * np.sqrt(np.maximum(c2, 0.0))

    # m > d runs in feature blocks, whose backward takes g from the forward's output
    ge = rc.g_error(ro, g, u if u > 0 else 16 * rc.U_F32) if KF > 1 else None
    errs = {}
    rows("o", o, ro, rc.floor_o(F, f64(v), ro, rden, causal, u), dtype, errs)
    rows("dq", q.grad, rdq, chain(rc.floor_dq(F, f64(v), ro, g, causal, u, gerr=ge), dfq, rfq, f64(q)), dtype, errs)
    rows("dk", k.grad, rdk, chain(rc.floor_dk(F, f64(v), ro, g, causal, u, gerr=ge), dfk, rfk, f64(k)), dtype, errs)
    rows("dv", v.grad, rdv, rc.floor_dv(F, g, causal, u), dtype, errs)
    record(f"favor_attention autograd {'causal' if causal else 'noncausal'} m={KF * d} {dtype}", **errs)
    assert max(row_ratios(errs).values()) <= 1.0, errs


def from_blocks(f):
    """[..., KF, N, d] block layout -> [..., N, KF d] features in the natural order."""
    *lead, KF, N, d = f.shape
    return np.moveaxis(f, -3, -2).reshape(*lead, N, KF * d)


@pytest.mark.parametrize("with_o", [False, True], ids=["stats_sweep", "from_output"])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("shape", [(2, 3, 200, 64, 2), (1, 2, 300, 128, 2), (2, 2, 1000, 64, 4),
                                   (1, 2, 257, 32, 3), (1, 4, 64 * 130 + 17, 64, 2)],
                         ids=lambda s: "x".join(map(str, s)))
def test_favor_backward_blocks(la, oracle, shape, dtype, causal, with_o):
    """The causal and non-causal backward on m = KF d features (every block with the head's G and g) against
    the oracle's backward on all m features at once, on the library's own features."""
    B, H, N, d, KF = shape
    m = KF * d
    if dtype == torch.float32 and d == 128:
        pytest.skip("fp32 backward is built for d <= 64")
    q, k, v, do = (t.cuda() for t in inp.favor_qkv(B, H, N, d, dtype, seed=N + 110, with_dout=True))
    om = inp.favor_omega(d, seed=N + 111, m=m).cuda()
    fq, fk = la.favor_features_blocks(q, om), la.favor_features_blocks(k, om)
    # with_o: the head's g from the forward's output instead of a statistics sweep per block.
    if causal:
        o, den = la.la_forward_causal_features_blocks(fq, fk, v, return_den=True)
        dfq, dfk, dv = la.la_backward_causal_features_blocks(fq, fk, v, do, den, o=o if with_o else None)
    else:
        o, den = la.la_forward_noncausal_features_blocks(fq, fk, v, return_den=True)
        dfq, dfk, dv = la.la_backward_noncausal_features_blocks(fq, fk, v, do, den, o=o if with_o else None)
    torch.cuda.synchronize()
    nfq, nfk = from_blocks(f64(fq)), from_blocks(f64(fk))
    rdfq, rdfk, rdv = oracle.backward_features(nfq, nfk, f64(v), f64(do), causal)
    errs = bwd_rows({}, (from_blocks(f64(dfq)), from_blocks(f64(dfk)), dv), (rdfq, rdfk, rdv), nfq, nfk, v, do, dtype,
                    causal, F=rc.Features.given(nfq, nfk), names=("dfq", "dfk", "dv"), outside_g=KF > 1)
    record(f"favor_bwd_blocks {'causal' if causal else 'noncausal'}{' from o' if with_o else ''} {B}x{H}x{N}x{d} "
           f"m={m} {dtype}", **errs)
    assert max(row_ratios(errs).values()) <= 1.0, errs
