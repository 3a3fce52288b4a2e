"""GPU parity of the stateful calls against the fp64 oracle: the causal forward
started from a given state (a long prefill in pieces) and multi-token decode.

Start states are what real prefixes leave behind: the oracle's state after a
seeded prefix of tokens (la_inputs), rounded to fp32 and handed to both sides.
Metric (every output row against its bar; states by their Frobenius error) and
tolerances as in test_parity.py.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import la_inputs as inp  # noqa: E402
from test_parity import (DEN_BAR, STATE_TOL, TOL, bwd_rows, den_check, draw, f64, fwd_rows, record,  # noqa: E402
                         row_ratios, slice_err)


def o_rows(o, ro, rden, q, k, v, dtype, S0=None, z0=None):
    """The worst row ratio of a causal output (from the start state S0, z0 if given)."""
    e = {}
    fwd_rows(e, o, ro, rden, q, k, v, dtype, True, S0=None if S0 is None else f64(S0),
             z0=None if z0 is None else f64(z0))
    return e["o"]


@pytest.fixture(scope="module")
def la():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_02_amd as m
    m.load_library()
    return m


def start_state(oracle, B, H, d, dtype, seed, npre=130):
    """The oracle's state after npre seeded prefix tokens, as fp32 host tensors."""
    pq, pk, pv = inp.qkv(B, H, npre, d, dtype, seed=seed, scale=dtype == torch.bfloat16)
    _, S, z = oracle.forward_causal(f64(pq), f64(pk), f64(pv), return_state=True)
    return torch.from_numpy(S).float(), torch.from_numpy(z).float()


SHAPES = [(1, 1, 1, 32), (1, 2, 63, 64), (2, 3, 200, 64), (1, 2, 300, 128), (2, 2, 1000, 64),
          (1, 2, 257, 32), (1, 8, 64 * 130 + 17, 64)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_forward_causal_from_state(la, oracle, shape, dtype):
    B, H, N, d = shape
    S0, z0 = start_state(oracle, B, H, d, dtype, seed=N + 11)
    q, k, v, _ = draw(B, H, N, d, dtype, seed=N + 12)
    o, den, S, z = la.la_forward_causal(q, k, v, return_den=True, return_state=True, S0=S0.cuda(), z0=z0.cuda())
    torch.cuda.synchronize()
    ro, rden, rS, rz = oracle.forward_causal(f64(q), f64(k), f64(v), return_den=True, return_state=True,
                                             S0=f64(S0), z0=f64(z0))
    errs = {"o": o_rows(o, ro, rden, q, k, v, dtype, S0, z0), "den": den_check(den, rden, q, k, dtype, z0=z0),
            "S": slice_err(S, rS), "z": slice_err(z[..., None], rz[..., None])}
    record(f"fwd_causal_from_state {B}x{H}x{N}x{d} {dtype}", **errs)
    assert errs["o"] <= 1.0, errs
    assert errs["den"] < DEN_BAR[dtype], errs
    assert max(errs["S"], errs["z"]) < min(TOL[dtype], STATE_TOL), errs


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_prefill_in_pieces_in_place(la, oracle, dtype):
    """A sequence fed in three pieces, each continuing in place from the state the last
    one left (S_out = S0), matches the oracle's single pass over the whole sequence."""
    B, H, N, d = 2, 2, 900, 64
    q, k, v, _ = draw(B, H, N, d, dtype, seed=21)
    cuts = [0, 130, 513, N]
    S = torch.empty(B, H, d, d, device="cuda")
    z = torch.empty(B, H, d, device="cuda")
    outs = []
    for i in range(3):
        a, b = cuts[i], cuts[i + 1]
        qs, ks, vs = (t[:, :, a:b].contiguous() for t in (q, k, v))
        if i == 0:
            outs.append(la.la_forward_causal(qs, ks, vs, return_state=True, S_out=S, z_out=z)[0])
        else:
            outs.append(la.la_forward_causal(qs, ks, vs, return_state=True, S0=S, z0=z, S_out=S, z_out=z)[0])
    torch.cuda.synchronize()
    ro, rden, rS, rz = oracle.forward_causal(f64(q), f64(k), f64(v), return_den=True, return_state=True)
    errs = {"o": o_rows(torch.cat(outs, dim=2), ro, rden, q, k, v, dtype), "S": slice_err(S, rS),
            "z": slice_err(z[..., None], rz[..., None])}
    record(f"prefill in pieces {dtype}", **errs)
    assert errs["o"] <= 1.0 and max(errs["S"], errs["z"]) < min(TOL[dtype], STATE_TOL), errs


def test_forward_from_state_without_tokens(la, oracle):
    """N = 0: the final state is the start state; z0 alone (S0 = NULL) leaves S = 0."""
    B, H, d = 2, 3, 64
    S0, z0 = start_state(oracle, B, H, d, torch.bfloat16, seed=5)
    S0, z0 = S0.cuda(), z0.cuda()
    q = torch.empty(B, H, 0, d, dtype=torch.bfloat16, device="cuda")
    _, S, z = la.la_forward_causal(q, q, q, return_state=True, S0=S0, z0=z0)
    _, S2, z2 = la.la_forward_causal(q, q, q, return_state=True, z0=z0)
    torch.cuda.synchronize()
    assert torch.equal(S, S0) and torch.equal(z, z0)
    assert torch.equal(S2, torch.zeros_like(S0)) and torch.equal(z2, z0)


def test_start_state_rejected_with_saved_state(la):
    q, k, v, _ = draw(1, 1, 64, 64, torch.bfloat16, seed=3)
    S0 = torch.zeros(1, 1, 64, 64, device="cuda")
    with pytest.raises(la.LinAttnError):
        la.la_forward_causal(q, k, v, S0=S0, saved_state=la.new_saved_state(q))


# ---- multi-token decode ----------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("T", [1, 7, 16, 37])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_decode_steps(la, oracle, d, T, dtype):
    B, H = 2, 3
    S0, z0 = start_state(oracle, B, H, d, dtype, seed=d + T)
    q, k, v = inp.qkv(B, H, T, d, dtype, seed=d * T + 1, scale=True)
    S, z = S0.cuda(), z0.cuda()
    o = la.la_decode_steps(S, z, q.cuda(), k.cuda(), v.cuda())
    torch.cuda.synchronize()
    rS, rz = f64(S0), f64(z0)
    worst = 0.0
    for t in range(T):
        ro, rS, rz = oracle.decode_step(rS, rz, f64(q[:, :, t]), f64(k[:, :, t]), f64(v[:, :, t]))
        worst = max(worst, slice_err(o[:, :, t][..., None], ro[..., None]))
    errs = {"o": worst, "S": slice_err(S, rS), "z": slice_err(z[..., None], rz[..., None])}
    record(f"decode_steps d={d} T={T} {dtype}", **errs)
    assert errs["o"] < TOL[dtype], errs
    assert max(errs["S"], errs["z"]) < 1e-5, errs


@pytest.mark.parametrize("d", [64, 128])
def test_decode_steps_match_single_steps(la, oracle, d):
    """One call of T steps and T calls of one step update the fp32 state identically up
    to rounding, and give the same outputs to within the reduction order."""
    B, H, T = 3, 4, 19
    S0, z0 = start_state(oracle, B, H, d, torch.bfloat16, seed=d)
    q, k, v = (t.cuda() for t in inp.qkv(B, H, T, d, torch.bfloat16, seed=d + 2, scale=True))
    S1, z1 = S0.cuda(), z0.cuda()
    S2, z2 = S0.cuda(), z0.cuda()
    o1 = la.la_decode_steps(S1, z1, q, k, v)
    o2 = torch.stack([la.la_decode_step(S2, z2, q[:, :, t].contiguous(), k[:, :, t].contiguous(),
                                        v[:, :, t].contiguous()) for t in range(T)], dim=2)
    torch.cuda.synchronize()
    assert torch.allclose(S1, S2, rtol=1e-6, atol=1e-6) and torch.allclose(z1, z2, rtol=1e-6, atol=1e-6)
    assert slice_err(o1.float(), f64(o2.float())) < 2.0 ** -8


# ---- shared key/value heads (GQA / MQA) ------------------------------------------------------
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("heads", [(8, 2), (6, 1), (3, 3), (32, 1), (4, 2), (9, 3)], ids=lambda h: f"H{h[0]}kv{h[1]}")
@pytest.mark.parametrize("T", [1, 5, 19, 40])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_steps_shared_state(la, oracle, d, T, heads, dtype):
    """Each query head continues the causal recurrence of its key/value head from the
    shared start state: the oracle runs that recurrence per query head.  With several
    query heads per state the rows (t, h) go in blocks of 64 (32 for 2 or 3 heads per
    state) whose last token may continue into the next block: T = 19 and 40 cover that."""
    H, Hkv = heads
    B, G = 2, H // Hkv
    S0, z0 = start_state(oracle, B, Hkv, d, dtype, seed=7 * d + T)
    q = inp.qkv(B, H, T, d, dtype, seed=d + 31 * T, scale=True)[0]
    _, k, v = inp.qkv(B, Hkv, T, d, dtype, seed=d + 37 * T, scale=True)
    S, z = S0.cuda(), z0.cuda()
    o = la.la_decode_steps(S, z, q.cuda(), k.cuda(), v.cuda())
    torch.cuda.synchronize()
    worst, rS, rz = 0.0, [None] * Hkv, [None] * Hkv
    for h in range(H):
        j = h // G
        ro, rden, rS[j], rz[j] = oracle.forward_causal(f64(q[:, h]), f64(k[:, j]), f64(v[:, j]), return_den=True,
                                                       return_state=True, S0=f64(S0[:, j]), z0=f64(z0[:, j]))
        worst = max(worst, o_rows(o[:, h], ro, rden, q[:, h], k[:, j], v[:, j], dtype, S0[:, j], z0[:, j]))
    rS, rz = np.stack(rS, axis=1), np.stack(rz, axis=1)
    errs = {"o": worst, "S": slice_err(S, rS), "z": slice_err(z[..., None], rz[..., None])}
    record(f"decode_steps H={H} Hkv={Hkv} d={d} T={T} {dtype}", **errs)
    assert errs["o"] <= 1.0, errs
    assert max(errs["S"], errs["z"]) < 1e-5, errs


# ---- backward from a start state (a sequence trained in pieces) ------------------------------------
BWD_SHAPES = [(1, 1, 1, 32), (2, 3, 200, 64), (1, 2, 300, 128), (2, 2, 1000, 64), (1, 8, 64 * 130 + 17, 64)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("shape", BWD_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_backward_causal_from_state(la, oracle, shape, dtype):
    B, H, N, d = shape
    if dtype == torch.float32 and d == 128:
        pytest.skip("fp32 causal path is built for d <= 64")
    S0, z0 = start_state(oracle, B, H, d, dtype, seed=N + 61)
    q, k, v, do = draw(B, H, N, d, dtype, seed=N + 62)
    rng = np.random.default_rng(N + 63)
    dSN = torch.from_numpy(rng.standard_normal((B, H, d, d)) * 0.01).float()
    dzN = torch.from_numpy(rng.standard_normal((B, H, d)) * 0.01).float()
    dq, dk, dv, dS0, dz0 = la.la_backward_causal_state(q, k, v, do, S0=S0.cuda(), z0=z0.cuda(), dS_out=dSN.cuda(),
                                                       dz_out=dzN.cuda())
    torch.cuda.synchronize()
    r = oracle.backward_causal_state(f64(q), f64(k), f64(v), f64(do), S0=f64(S0), z0=f64(z0), dSN=f64(dSN),
                                     dzN=f64(dzN))
    errs = {"dS0": slice_err(dS0, r[3]), "dz0": slice_err(dz0[..., None], r[4][..., None])}
    bwd_rows(errs, (dq, dk, dv), r[:3], q, k, v, do, dtype, True, S0=f64(S0), z0=f64(z0), dSN=f64(dSN))
    record(f"bwd_causal_from_state {B}x{H}x{N}x{d} {dtype}", **errs)
    assert max(row_ratios(errs).values()) <= 1.0, errs
    assert max(errs["dS0"], errs["dz0"]) < TOL[dtype], errs


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_training_in_pieces(la, oracle, dtype):
    """Forward in two pieces (the second from the first's final state), backward of the
    second piece from that state, then of the first with the second's start-state
    gradients: together the oracle's one-pass backward of the whole sequence."""
    B, H, N, d, p = 2, 2, 700, 64, 300
    q, k, v, do = draw(B, H, N, d, dtype, seed=71)
    cut = lambda t, a, b: t[:, :, a:b].contiguous()
    _, S1, z1 = la.la_forward_causal(cut(q, 0, p), cut(k, 0, p), cut(v, 0, p), return_state=True)
    dq2, dk2, dv2, dS1, dz1 = la.la_backward_causal_state(cut(q, p, N), cut(k, p, N), cut(v, p, N), cut(do, p, N),
                                                          S0=S1, z0=z1)
    dq1, dk1, dv1, _, _ = la.la_backward_causal_state(cut(q, 0, p), cut(k, 0, p), cut(v, 0, p), cut(do, 0, p),
                                                      dS_out=dS1, dz_out=dz1, want_state_grad=False)
    torch.cuda.synchronize()
    ref = oracle.backward_causal(f64(q), f64(k), f64(v), f64(do))
    got = [torch.cat([a, b], dim=2) for a, b in ((dq1, dq2), (dk1, dk2), (dv1, dv2))]
    errs = bwd_rows({}, got, ref, q, k, v, do, dtype, True)
    record(f"training in pieces {dtype}", **errs)
    assert max(row_ratios(errs).values()) <= 1.0, errs


def test_backward_from_state_without_tokens(la):
    B, H, d = 2, 3, 64
    dSN = torch.randn(B, H, d, d, device="cuda")
    dzN = torch.randn(B, H, d, device="cuda")
    q = torch.empty(B, H, 0, d, dtype=torch.bfloat16, device="cuda")
    _, _, _, dS0, dz0 = la.la_backward_causal_state(q, q, q, q, dS_out=dSN, dz_out=dzN)
    torch.cuda.synchronize()
    assert torch.equal(dS0, dSN) and torch.equal(dz0, dzN)


# ---- grouped key/value heads in the causal forward (prefill for shared-state decode) ---------------
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("heads", [(8, 2), (6, 1), (3, 3), (32, 4)], ids=lambda h: f"H{h[0]}kv{h[1]}")
@pytest.mark.parametrize("N", [1, 200, 64 * 130 + 17])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("from_state", [False, True], ids=["zero", "state"])
def test_forward_causal_grouped(la, oracle, d, N, heads, dtype, from_state):
    H, Hkv = heads
    if dtype == torch.float32 and d == 128:
        pytest.skip("fp32 causal path is built for d <= 64")
    if N > 1000 and (H > 8 or d != 64):
        pytest.skip("long rows once per shape family")
    B, G = 2, H // Hkv
    q = inp.qkv(B, H, N, d, dtype, seed=d + 41 * N + H, scale=dtype == torch.bfloat16)[0]
    _, k, v = inp.qkv(B, Hkv, N, d, dtype, seed=d + 43 * N + Hkv, scale=dtype == torch.bfloat16)
    S0 = z0 = None
    if from_state:
        S0, z0 = start_state(oracle, B, Hkv, d, dtype, seed=N + 5 * H)
    o, den, S, z = la.la_forward_causal_grouped(q.cuda(), k.cuda(), v.cuda(), return_den=True, return_state=True,
                                                S0=None if S0 is None else S0.cuda(),
                                                z0=None if z0 is None else z0.cuda())
    torch.cuda.synchronize()
    kw = {}
    errs = {"o": 0.0, "den": 0.0}
    rS, rz = [None] * Hkv, [None] * Hkv
    for h in range(H):
        j = h // G
        if S0 is not None:
            kw = {"S0": f64(S0[:, j]), "z0": f64(z0[:, j])}
        ro, rden, rS[j], rz[j] = oracle.forward_causal(f64(q[:, h]), f64(k[:, j]), f64(v[:, j]), return_den=True,
                                                       return_state=True, **kw)
        errs["o"] = max(errs["o"], o_rows(o[:, h], ro, rden, q[:, h], k[:, j], v[:, j], dtype,
                                          None if S0 is None else S0[:, j], None if z0 is None else z0[:, j]))
        errs["den"] = max(errs["den"], den_check(den[:, h], rden, q[:, h], k[:, j], dtype,
                                                 z0=None if z0 is None else z0[:, j]))
    rS, rz = np.stack(rS, axis=1), np.stack(rz, axis=1)
    errs["S"], errs["z"] = slice_err(S, rS), slice_err(z[..., None], rz[..., None])
    record(f"fwd_causal_grouped H={H} Hkv={Hkv} N={N} d={d} {dtype} {'state' if from_state else 'zero'}", **errs)
    assert errs["o"] <= 1.0, errs
    assert errs["den"] < DEN_BAR[dtype], errs
    assert max(errs["S"], errs["z"]) < min(TOL[dtype], STATE_TOL), errs


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_grouped_prefill_then_decode(la, oracle, dtype):
    """Prefill of 300 tokens with 8 query heads on 2 key/value heads, then 9 decode steps
    from the per-key/value-head state it left: the oracle's recurrence over all 309."""
    B, H, Hkv, N, T, d = 2, 8, 2, 300, 9, 64
    G = H // Hkv
    q = inp.qkv(B, H, N + T, d, dtype, seed=91, scale=dtype == torch.bfloat16)[0]
    _, k, v = inp.qkv(B, Hkv, N + T, d, dtype, seed=92, scale=dtype == torch.bfloat16)
    cut = lambda t, a, b: t[:, :, a:b].contiguous().cuda()
    o1, S, z = la.la_forward_causal_grouped(cut(q, 0, N), cut(k, 0, N), cut(v, 0, N), return_state=True)
    o2 = la.la_decode_steps(S, z, cut(q, N, N + T), cut(k, N, N + T), cut(v, N, N + T))
    torch.cuda.synchronize()
    o = torch.cat([o1, o2], dim=2)
    worst = 0.0
    for h in range(H):
        ro, rden = oracle.forward_causal(f64(q[:, h]), f64(k[:, h // G]), f64(v[:, h // G]), return_den=True)
        worst = max(worst, o_rows(o[:, h], ro, rden, q[:, h], k[:, h // G], v[:, h // G], dtype))
    record(f"grouped prefill then decode {dtype}", o=worst)
    assert worst <= 1.0, worst


def test_forward_causal_grouped_rejects_bad_heads(la):
    q = torch.zeros(1, 6, 16, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 4, 16, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        la.la_forward_causal_grouped(q, k, k)
