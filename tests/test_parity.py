"""GPU parity: the HIP library (through its C ABI) against the fp64 CPU oracle.

Metric: every row of every sequence output (O, dQ, dK, dV) on its own,
||x_i - y_i|| <= tol ||y_i|| + floor_i (rowcheck.py: floor_i is a first-order
rounding bound of the terms summed into row i), and every output finite.
Tolerances: 1e-4 for fp32 inputs and 2e-2 for bf16 inputs with fp32
accumulation.  The per-head Frobenius error is recorded beside it.  Inputs are
seeded synthetic tensors (la_inputs); the oracle sees the exact values the GPU
saw, widened to fp64.  Sizes span several 64-token chunks, several segments and
ragged tails.
"""
import json
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import la_inputs as inp  # noqa: E402
import rowcheck as rc  # noqa: E402

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
# Tighter bars for the fp32 by-products of the forward.  The state (S, z) is
# accumulated in fp32: 1e-3.  The fp32 denominator: 1e-4 like the output.  The
# bf16 denominator is held to a per-element bound instead (den_check).
STATE_TOL = 1e-3
DEN_TOL = {torch.float32: 1e-4}
BF16_U = 2.0 ** -8  # unit roundoff of bf16 (8 significand bits)


@pytest.fixture(scope="module")
def la():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_02_amd as m
    m.load_library()
    return m


def f64(x):
    return x.astype(np.float64, copy=False) if isinstance(x, np.ndarray) else inp.to_f64(x)


def np_phi(x):
    """elu(x) + 1 in fp64 (for error bounds computed in the tests)."""
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def record(name, **errs):
    """Append measured errors to $LA_PARITY_LOG (JSON lines) when it is set."""
    path = os.environ.get("LA_PARITY_LOG")
    if path:
        with open(path, "a") as fh:
            fh.write(json.dumps({"case": name, **errs}) + "\n")


def slice_err(gpu, ref):
    """max over leading slices of the Frobenius relative error (last two dims form a slice)."""
    g = f64(gpu) if isinstance(gpu, torch.Tensor) else gpu
    assert np.isfinite(g).all(), "non-finite GPU output"
    g = g.reshape(-1, *g.shape[-2:]) if g.ndim >= 2 else g.reshape(1, 1, -1)
    r = ref.reshape(g.shape)
    num = np.linalg.norm((g - r).reshape(g.shape[0], -1), axis=1)
    den = np.maximum(np.linalg.norm(r.reshape(g.shape[0], -1), axis=1), 1e-300)
    return float((num / den).max())


def rows(name, gpu, ref, floor, dtype, errs):
    """Per-row check of one output: errs[name] = the worst row's error over its bar
    (pass: <= 1); errs[name + "_fro"] = the per-head Frobenius relative error."""
    ratio, frac = rc.row_check(gpu, ref, TOL[dtype], floor)
    errs[name] = ratio
    errs[name + "_fro"] = slice_err(gpu, ref)
    errs[name + "_floor_rows"] = frac
    return ratio


def row_ratios(errs):
    return {k_: v_ for k_, v_ in errs.items() if not k_.endswith(("_fro", "_floor_rows")) and k_ in ROW_KEYS}


ROW_KEYS = ("o", "dq", "dk", "dv", "dfq", "dfk")


def fwd_rows(errs, o, ro, rden, q, k, v, dtype, causal, S0=None, z0=None, F=None):
    F = F if F is not None else rc.Features.elu(f64(q), f64(k))
    u = rc.u_of(dtype == torch.bfloat16)
    fl = rc.floor_o(F, f64(v), ro, rden, causal, u, S0=S0, z0=z0)
    return rows("o", o, ro, fl, dtype, errs)


def bwd_rows(errs, grads, refs, q, k, v, do, dtype, causal, S0=None, z0=None, dSN=None, F=None,
             names=("dq", "dk", "dv"), outside_g=False):
    """Per-row checks of (dq, dk, dv) against the oracle's; the floors take the oracle's
    own forward (O and den) of the same inputs (from the start state S0, z0 if given).
    outside_g: the backward takes g from outside its own products (feature blocks)."""
    hq, hk, hv, hdo = f64(q), f64(k), f64(v), f64(do)
    F = F if F is not None else rc.Features.elu(hq, hk)
    u = rc.u_of(dtype == torch.bfloat16)
    if F.split:
        fwd = oracle_mod().forward_causal if causal else oracle_mod().forward_noncausal
        ro, rden = (fwd(hq, hk, hv, return_den=True, S0=S0, z0=z0) if S0 is not None
                    else fwd(hq, hk, hv, return_den=True))
    else:
        ro, rden = oracle_mod().forward_features(F.qf.reshape(hq.shape[:-1] + (-1,)),
                                                 F.kf.reshape(hk.shape[:-1] + (-1,)), hv, causal, return_den=True)
    g = rc.grads_g(hdo, ro, rden)
    ge = rc.g_error(ro, g, u if u > 0 else 16 * rc.U_F32) if outside_g else None
    fls = (rc.floor_dq(F, hv, ro, g, causal, u, S0=S0, z0=z0, gerr=ge),
           rc.floor_dk(F, hv, ro, g, causal, u, dSN=dSN, gerr=ge), rc.floor_dv(F, g, causal, u, dSN=dSN))
    for name, x, y, fl in zip(names, grads, refs, fls):
        rows(name, x, y, fl, dtype, errs)
    return errs


def oracle_mod():
    import oracle
    return oracle


def den_check(den, rden, q, k, dtype, z0=None):
    """Error of the fp32 denominator phi(Q_t)^T z_t against the oracle's: for fp32 inputs the
    per-slice Frobenius relative error (bar DEN_TOL); for bf16 inputs the largest ratio of the
    per-element error to its first-order bound (bar 1).  With bf16 inputs phi(Q) is rounded to
    bf16 (relative error <= u = 2^-8 on every positive term of the sum: u den), the in-chunk
    weights A_ts are rounded to bf16 before they are summed (<= u den), and the key features
    enter as 1 + E(K) with E rounded to bf16 (<= u sum_a phi(Q_ta) sum_{s<=t} |E(K_sa)|, and the
    same for a start state's z0 taken apart around its mean); fp32 sums add (N + d) 2^-24 den."""
    if dtype == torch.float32:
        return slice_err(den, rden)
    g, qq, kk = f64(den), f64(q), f64(k)
    fq = np_phi(qq)
    ek = np.cumsum(np.abs(np_phi(kk) - 1.0), axis=-2)  # sum_{s<=t} |E(K_s)|, [.., N, d]
    if z0 is not None:
        zz = f64(z0)
        ek = ek + (np.abs(zz) + np.abs(zz).mean(-1, keepdims=True))[..., None, :]
    N, d = qq.shape[-2], qq.shape[-1]
    bound = BF16_U * (2.0 * np.abs(rden) + (fq * ek).sum(-1)) + (N + d) * 2.0 ** -24 * np.abs(rden)
    assert np.isfinite(g).all(), "non-finite GPU output"
    return float((np.abs(g - rden) / bound).max()) if g.size else 0.0


DEN_BAR = {torch.float32: DEN_TOL[torch.float32], torch.bfloat16: 1.0}


def workspace(la, op, q):
    B, H, N, d = q.shape
    n = la.workspace_size(op, B, H, N, d, q.dtype)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)


def draw(B, H, N, d, dtype, seed=0, scale=None):
    sc = (dtype == torch.bfloat16) if scale is None else scale
    q, k, v, do = inp.qkv(B, H, N, d, dtype, seed=seed, scale=sc, with_dout=True)
    return [t.cuda() for t in (q, k, v, do)]


def run_fwd_causal(la, oracle, B, H, N, d, dtype, seed=0, scale=None):
    q, k, v, _ = draw(B, H, N, d, dtype, seed, scale)
    ws = workspace(la, la.LA_OP_FWD_CAUSAL, q)
    o, den, S, z = la.la_forward_causal(q, k, v, return_den=True, return_state=True, workspace=ws)
    assert la.wait_failures(la.LA_OP_FWD_CAUSAL, ws, q) == 0
    torch.cuda.synchronize()
    ro, rden, rS, rz = oracle.forward_causal(f64(q), f64(k), f64(v), return_den=True, return_state=True)
    tol = TOL[dtype]
    errs = {"den": den_check(den, rden, q, k, dtype), "S": slice_err(S, rS),
            "z": slice_err(z[..., None], rz[..., None])}
    fwd_rows(errs, o, ro, rden, q, k, v, dtype, True)
    record(f"fwd_causal {B}x{H}x{N}x{d} {dtype}", **errs)
    assert errs["o"] <= 1.0, errs
    assert errs["den"] < DEN_BAR[dtype], errs
    assert max(errs["S"], errs["z"]) < min(tol, STATE_TOL), errs


def run_fwd_noncausal(la, oracle, B, H, N, d, dtype, seed=0, scale=None):
    q, k, v, _ = draw(B, H, N, d, dtype, seed, scale)
    o = la.la_forward_noncausal(q, k, v)
    torch.cuda.synchronize()
    ro, rden = oracle.forward_noncausal(f64(q), f64(k), f64(v), return_den=True)
    errs = {}
    fwd_rows(errs, o, ro, rden, q, k, v, dtype, False)
    record(f"fwd_noncausal {B}x{H}x{N}x{d} {dtype}", **errs)
    assert errs["o"] <= 1.0, errs


def run_bwd_causal(la, oracle, B, H, N, d, dtype, seed=0, scale=None, causal=True):
    q, k, v, do = draw(B, H, N, d, dtype, seed, scale)
    if causal:
        ws = workspace(la, la.LA_OP_BWD_CAUSAL, q)
        dq, dk, dv = la.la_backward_causal(q, k, v, do, workspace=ws)
        assert la.backward_wait_failures(ws, q) == 0
    else:
        dq, dk, dv = la.la_backward_noncausal(q, k, v, do)
    torch.cuda.synchronize()
    ref = oracle.backward_causal if causal else oracle.backward_noncausal
    rdq, rdk, rdv = ref(f64(q), f64(k), f64(v), f64(do))
    tol = TOL[dtype]
    if N == 1:
        # A single token: O_0 = V_0 whatever q and k are, so dq and dk vanish exactly and
        # no relative error exists; they must be negligible next to dv = dout.
        scale = float(np.abs(f64(do)).max())
        if causal or dtype == torch.float32:
            assert float(np.abs(f64(dq)).max()) < 1e-3 * tol * scale
            assert float(np.abs(f64(dk)).max()) < 1e-3 * tol * scale
        else:
            # The non-causal path takes S_E = E(K_0) V_0^T and R = phi(Q_0) G_0^T into
            # its MFMAs rounded to bf16 (relative error <= u = 2^-8 per element) against
            # fp32 rank-1 terms that cancel them in exact arithmetic.  With
            # G = dO / den, M = sum_b |G_b V_b| and w = sum_c phi(Q_c) |E(K_c)| / den,
            # the residuals are at most u M (|E(K_a)| + phi(K_a) w) in dphi(Q)_a
            # and u M phi(Q_a) (1 + w) in dphi(K)_a (phi' <= 1): the bar is that bound.
            fq, fk = np_phi(f64(q)), np_phi(f64(k))
            ek = np.abs(fk - 1.0)
            den = (fq * fk).sum(-1, keepdims=True)
            m = (np.abs(f64(do) / den) * np.abs(f64(v))).sum(-1, keepdims=True)
            w = (fq * ek).sum(-1, keepdims=True) / den
            assert (np.abs(f64(dk)) <= 2.0 ** -8 * m * fq * (1 + w) + 1e-7 * scale).all()
            assert (np.abs(f64(dq)) <= 2.0 ** -8 * m * (ek + fk * w) + 1e-7 * scale).all()
        errs = {}
        bwd_rows(errs, (dv,), (rdv,), q, k, v, do, dtype, causal, names=("dv",))
        assert errs["dv"] <= 1.0, errs
        return
    errs = {}
    bwd_rows(errs, (dq, dk, dv), (rdq, rdk, rdv), q, k, v, do, dtype, causal)
    record(f"bwd_{'causal' if causal else 'noncausal'} {B}x{H}x{N}x{d} {dtype}", **errs)
    assert max(row_ratios(errs).values()) <= 1.0, errs


def run_bwd_noncausal(la, oracle, B, H, N, d, dtype, seed=0, scale=None):
    run_bwd_causal(la, oracle, B, H, N, d, dtype, seed, scale, causal=False)


# ---- the small fp32 workload: B1 H2 N256 d32, N(0,1) unscaled ---------------------------
def test_tiny_fp32_all_calls(la, oracle):
    w = inp.TINY
    run_fwd_noncausal(la, oracle, w.B, w.H, w.N, w.d, w.dtype, scale=False)
    run_fwd_causal(la, oracle, w.B, w.H, w.N, w.d, w.dtype, scale=False)
    run_bwd_causal(la, oracle, w.B, w.H, w.N, w.d, w.dtype, scale=False)
    run_bwd_noncausal(la, oracle, w.B, w.H, w.N, w.d, w.dtype, scale=False)


# ---- shapes spanning chunks, segments and ragged tails ----------------------------------------
SHAPES = [
    (1, 1, 1, 32), (1, 2, 63, 64), (2, 1, 64, 64), (1, 1, 65, 128), (2, 3, 200, 64),
    (1, 2, 257, 32), (1, 2, 300, 128), (2, 2, 1000, 64), (1, 1, 4096 + 17, 64),
    # enough chunks per head that segments hold several chunks (about 512
    # workgroups per launch), with ragged last segments and token tails
    (1, 8, 64 * 130 + 17, 64), (2, 4, 64 * 80, 32), (1, 4, 64 * 200 + 5, 128),
]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_forward_causal(la, oracle, shape, dtype):
    """fp32 at d = 128 runs on two blocks of 64 features, one value half at a time."""
    B, H, N, d = shape
    run_fwd_causal(la, oracle, B, H, N, d, dtype, seed=N)


# Many heads whose segments hold several chunks each and number at most 12, so
# that each segment sums the earlier segments' records directly (ragged last
# segments and token tails included).
# (the last: 256 heads of 41 chunks, two segments of 21 and 20 chunks)
DIRECT_SHAPES = [(3, 16, 4096 + 17, 64), (4, 16, 64 * 40, 64), (2, 32, 64 * 50 + 3, 32), (4, 64, 64 * 40 + 7, 32)]


@pytest.mark.parametrize("shape", DIRECT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_forward_causal_direct_records(la, oracle, shape):
    B, H, N, d = shape
    run_fwd_causal(la, oracle, B, H, N, d, torch.bfloat16, seed=N + 9)


# d = 128 heads whose default plan (about 512 workgroups) would need more than 12 segments
# take one round of at most 12 segments per head (16 heads of 65 chunks: ten segments of 6
# chunks, one of 5 with a ragged tail): the forward in one launch, the backward's direct record sums.
# At d = 64 the same holds with two workgroups per CU (32 heads of 65 chunks: 11 segments).
ONE_ROUND_SHAPES = [(1, 16, 64 * 64 + 17, 128), (1, 32, 64 * 64 + 17, 64)]


@pytest.mark.parametrize("shape", ONE_ROUND_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_causal_one_round(la, oracle, shape):
    B, H, N, d = shape
    run_fwd_causal(la, oracle, B, H, N, d, torch.bfloat16, seed=N + 11)
    run_bwd_causal(la, oracle, B, H, N, d, torch.bfloat16, seed=N + 12)


@pytest.mark.parametrize("shape", ONE_ROUND_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_saved_state_one_round(la, shape):
    """Where the causal plan takes fewer segments than the non-causal one, one saved-state
    buffer serves both: each backward reading its forward's saved state is bitwise the
    backward that rebuilds the state itself."""
    B, H, N, d = shape
    q, k, v, do = draw(B, H, N, d, torch.bfloat16, seed=N + 13)
    saved = la.new_saved_state(q)
    la.la_forward_causal(q, k, v, saved_state=saved)
    g1 = la.la_backward_causal(q, k, v, do, saved_state=saved)
    g2 = la.la_backward_causal(q, k, v, do)
    saved2 = la.new_saved_state(q)
    la.la_forward_noncausal(q, k, v, saved_state=saved2)
    h1 = la.la_backward_noncausal(q, k, v, do, saved_state=saved2)
    h2 = la.la_backward_noncausal(q, k, v, do)
    torch.cuda.synchronize()
    for a, b in zip(g1 + h1, g2 + h2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("shape", [(4, 64, 64 * 40 + 7, 32)], ids=lambda s: "x".join(map(str, s)))
def test_backward_causal_long_segments(la, oracle, shape):
    """Segments of more than 16 chunks in the fused backward."""
    B, H, N, d = shape
    run_bwd_causal(la, oracle, B, H, N, d, torch.bfloat16, seed=N + 10)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_forward_noncausal(la, oracle, shape, dtype):
    B, H, N, d = shape
    run_fwd_noncausal(la, oracle, B, H, N, d, dtype, seed=N + 1)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_backward_causal(la, oracle, shape, dtype):
    B, H, N, d = shape
    run_bwd_causal(la, oracle, B, H, N, d, dtype, seed=N + 2)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_backward_noncausal(la, oracle, shape, dtype):
    B, H, N, d = shape
    run_bwd_noncausal(la, oracle, B, H, N, d, dtype, seed=N + 4)


# ---- decode --------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_decode_from_causal_prefix(la, oracle, d, dtype):
    B, H, N0, steps = 2, 3, 130, 5
    q, k, v, _ = draw(B, H, N0, d, dtype, seed=d)
    if dtype == torch.float32 and d == 128:
        # fp32 prefix state through the oracle-independent recurrence: start from zero
        S = torch.zeros(B, H, d, d, device="cuda")
        z = torch.zeros(B, H, d, device="cuda")
        rS, rz = np.zeros((B, H, d, d)), np.zeros((B, H, d))
    else:
        _, S, z = la.la_forward_causal(q, k, v, return_state=True)
        _, rS, rz = oracle.forward_causal(f64(q), f64(k), f64(v), return_state=True)
    sq, sk, sv = inp.decode_tokens(B, H, d, steps, dtype, seed=d + 7)
    for t in range(steps):
        qt, kt, vt = sq[t].cuda(), sk[t].cuda(), sv[t].cuda()
        o = la.la_decode_step(S, z, qt, kt, vt)
        torch.cuda.synchronize()
        ro, rS, rz = oracle.decode_step(rS, rz, f64(qt), f64(kt), f64(vt))
        assert slice_err(o[..., None], ro[..., None]) < TOL[dtype]
    assert slice_err(S, rS) < 1e-3
    assert slice_err(z[..., None], rz[..., None]) < 1e-3


def test_decode_random_state(la, oracle):
    """State with both signs in S and a positive z, as any prefix would give."""
    B, H, d = 3, 2, 64
    gen = inp.generator(11)
    S = torch.randn(B, H, d, d, generator=gen)
    z = torch.rand(B, H, d, generator=gen) * 100 + 1
    q, k, v = (t[0] for t in inp.decode_tokens(B, H, d, 1, torch.bfloat16, seed=12))
    Sg, zg = S.clone().cuda(), z.clone().cuda()
    o = la.la_decode_step(Sg, zg, q.cuda(), k.cuda(), v.cuda())
    torch.cuda.synchronize()
    ro, rS, rz = oracle.decode_step(f64(S), f64(z), f64(q), f64(k), f64(v))
    assert slice_err(o[..., None], ro[..., None]) < 2e-2
    assert slice_err(Sg, rS) < 1e-6
    assert slice_err(zg[..., None], rz[..., None]) < 1e-6


# ---- properties -------------------------------------------------------------------------------------
def test_deterministic(la):
    q, k, v, do = draw(2, 4, 1000, 64, torch.bfloat16, seed=5)
    a = [la.la_forward_causal(q, k, v), la.la_forward_noncausal(q, k, v), *la.la_backward_causal(q, k, v, do),
         *la.la_backward_noncausal(q, k, v, do)]
    b = [la.la_forward_causal(q, k, v), la.la_forward_noncausal(q, k, v), *la.la_backward_causal(q, k, v, do),
         *la.la_backward_noncausal(q, k, v, do)]
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_deterministic_multichunk_segments(la):
    """Repeated calls at a size with several chunks per segment are bitwise equal
    (catches ordering races in the chunk pipelines, which vary run to run)."""
    q, k, v, do = draw(2, 8, 64 * 96 + 9, 64, torch.bfloat16, seed=6)
    ref_o = la.la_forward_causal(q, k, v)
    ref_n = la.la_forward_noncausal(q, k, v)
    ref_g = la.la_backward_causal(q, k, v, do)
    ref_gn = la.la_backward_noncausal(q, k, v, do)
    for _ in range(4):
        o = la.la_forward_causal(q, k, v)
        n = la.la_forward_noncausal(q, k, v)
        g = la.la_backward_causal(q, k, v, do)
        gn = la.la_backward_noncausal(q, k, v, do)
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(n, ref_n)
        assert all(torch.equal(x, y) for x, y in zip(g, ref_g))
        assert all(torch.equal(x, y) for x, y in zip(gn, ref_gn))


def test_constant_v(la):
    B, H, N, d = 1, 2, 333, 64
    q, k, _, _ = draw(B, H, N, d, torch.float32, seed=9)
    c = torch.randn(B, H, 1, d, device="cuda")
    v = c.expand(B, H, N, d).contiguous()
    o = la.la_forward_causal(q, k, v)
    o2 = la.la_forward_noncausal(q, k, v)
    torch.cuda.synchronize()
    assert torch.allclose(o, v, rtol=1e-5, atol=1e-6)
    assert torch.allclose(o2, v, rtol=1e-5, atol=1e-6)


def test_constant_v_noncausal_backward(la):
    """O = V whatever q and k are when every value row is the same: dq and dk vanish,
    dv = dout spread by the attention weights (its column sums equal those of dout)."""
    B, H, N, d = 1, 2, 333, 64
    q, k, _, do = draw(B, H, N, d, torch.float32, seed=19)
    c = torch.randn(B, H, 1, d, device="cuda")
    v = c.expand(B, H, N, d).contiguous()
    dq, dk, dv = la.la_backward_noncausal(q, k, v, do)
    torch.cuda.synchronize()
    scale = float(do.abs().max())
    assert float(dq.abs().max()) < 1e-5 * scale and float(dk.abs().max()) < 1e-5 * scale
    assert torch.allclose(dv.sum(2), do.sum(2), rtol=1e-4, atol=1e-4 * scale)


def test_causality_across_chunks(la):
    """Poisoning keys/values from token 128 on leaves rows 0..127 (two whole chunks) untouched."""
    B, H, N, d = 1, 2, 256, 64
    q, k, v, _ = draw(B, H, N, d, torch.bfloat16, seed=10)
    o = la.la_forward_causal(q, k, v)
    k2, v2 = k.clone(), v.clone()
    k2[:, :, 128:] = float("nan")
    v2[:, :, 128:] = float("inf")
    o2 = la.la_forward_causal(q, k2, v2)
    torch.cuda.synchronize()
    assert torch.equal(o[:, :, :128], o2[:, :, :128])


def test_autograd_function(la, oracle):
    q, k, v, do = draw(1, 2, 150, 32, torch.float32, seed=13)
    q.requires_grad_(True)
    k.requires_grad_(True)
    v.requires_grad_(True)
    o = la.causal_linear_attention(q, k, v)
    o.backward(do)
    torch.cuda.synchronize()
    rdq, rdk, rdv = oracle.backward_causal(f64(q), f64(k), f64(v), f64(do))
    errs = bwd_rows({}, (q.grad, k.grad, v.grad), (rdq, rdk, rdv), q, k, v, do, torch.float32, True)
    assert max(row_ratios(errs).values()) <= 1.0, errs


def test_autograd_function_noncausal(la, oracle):
    q, k, v, do = draw(1, 2, 150, 32, torch.float32, seed=14)
    q.requires_grad_(True)
    k.requires_grad_(True)
    v.requires_grad_(True)
    o = la.linear_attention(q, k, v)
    o.backward(do)
    torch.cuda.synchronize()
    ro, rden = oracle.forward_noncausal(f64(q), f64(k), f64(v), return_den=True)
    rdq, rdk, rdv = oracle.backward_noncausal(f64(q), f64(k), f64(v), f64(do))
    errs = {}
    fwd_rows(errs, o, ro, rden, q, k, v, torch.float32, False)
    bwd_rows(errs, (q.grad, k.grad, v.grad), (rdq, rdk, rdv), q, k, v, do, torch.float32, False)
    assert max(row_ratios(errs).values()) <= 1.0, errs


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("shape", [(2, 3, 1000, 64), (1, 2, 4096 + 17, 32), (1, 1, 300, 128), (1, 8, 64 * 130 + 17, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_saved_state_roundtrip_noncausal(la, shape, dtype):
    """The non-causal backward fed the non-causal forward's saved state gives bitwise
    the results of the one that rebuilds the key aggregates."""
    B, H, N, d = shape
    q, k, v, do = draw(B, H, N, d, dtype, seed=N + 5)
    st = la.new_saved_state(q)
    o1 = la.la_forward_noncausal(q, k, v, saved_state=st)
    o2 = la.la_forward_noncausal(q, k, v)
    g1 = la.la_backward_noncausal(q, k, v, do, saved_state=st)
    g2 = la.la_backward_noncausal(q, k, v, do)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("shape", [(2, 3, 1000, 64), (1, 2, 4096 + 17, 32), (1, 1, 300, 128), (3, 16, 4096 + 17, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_saved_state_roundtrip(la, shape, dtype):
    """The backward fed the forward's saved state gives bitwise the results of the one that rebuilds it."""
    B, H, N, d = shape
    q, k, v, do = draw(B, H, N, d, dtype, seed=N + 3)
    st = la.new_saved_state(q)
    o1 = la.la_forward_causal(q, k, v, saved_state=st)
    o2 = la.la_forward_causal(q, k, v)
    g1 = la.la_backward_causal(q, k, v, do, saved_state=st)
    g2 = la.la_backward_causal(q, k, v, do)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
