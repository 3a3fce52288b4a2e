"""GPU parity at the full measured sizes, in the launch configuration the
benchmark times (default chunk, library-chosen segments, one call per op).

Inputs are drawn on the device with the seeded device generator (la_inputs);
the exact values of the checked heads are copied to the host and the fp64
oracle recomputes those heads from scratch.  Mid is checked on every head;
the larger workloads on a seeded sample of heads (heads are independent).
Metric (every row of O, dQ, dK, dV against its bar) and tolerances as in test_parity.py.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import la_inputs as inp  # noqa: E402
from test_parity import (DEN_BAR, TOL, bwd_rows, den_check, fwd_rows, f64, record, row_ratios, slice_err,  # noqa: E402
                         workspace)


@pytest.fixture(scope="module")
def la():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_02_amd as m
    m.load_library()
    return m


def heads(x, idx):
    """[B, H, ...] -> selected flat heads [len(idx), ...] on the host in fp64."""
    flat = x.reshape(-1, *x.shape[2:])
    return f64(flat[idx])


def pick(BH, n, seed):
    if n >= BH:
        return np.arange(BH)
    return np.sort(np.random.default_rng(seed).choice(BH, size=n, replace=False))


def check_workload(la, oracle, w, nheads, with_bwd, seed=0):
    q, k, v, do = inp.workload_inputs(w, seed=seed, device="cuda", with_dout=True)
    wsf = workspace(la, la.LA_OP_FWD_CAUSAL, q)
    o, den = la.la_forward_causal(q, k, v, return_den=True, workspace=wsf)
    assert la.wait_failures(la.LA_OP_FWD_CAUSAL, wsf, q) == 0
    dq = dk = dv = None
    if with_bwd:
        ws = workspace(la, la.LA_OP_BWD_CAUSAL, q)
        dq, dk, dv = la.la_backward_causal(q, k, v, do, workspace=ws)
        assert la.backward_wait_failures(ws, q) == 0
    torch.cuda.synchronize()
    idx = pick(w.B * w.H, nheads, seed + 1)
    hq, hk, hv = heads(q, idx), heads(k, idx), heads(v, idx)
    ro, rden = oracle.forward_causal(hq, hk, hv, return_den=True)
    errs = {"den": den_check(heads(den, idx), rden, hq, hk, w.dtype)}
    fwd_rows(errs, heads(o, idx), ro, rden, hq, hk, hv, w.dtype, True)
    if with_bwd:
        hdo = heads(do, idx)
        rdq, rdk, rdv = oracle.backward_causal(hq, hk, hv, hdo)
        bwd_rows(errs, (heads(dq, idx), heads(dk, idx), heads(dv, idx)), (rdq, rdk, rdv), hq, hk, hv, hdo, w.dtype,
                 True)
    record(f"full {w.name} heads={len(idx)}", **errs)
    print(w.name, errs, flush=True)
    assert errs["den"] < DEN_BAR[w.dtype], errs
    assert max(row_ratios(errs).values()) <= 1.0, errs


def test_mid_all_heads(la, oracle):
    check_workload(la, oracle, inp.MID, nheads=10**9, with_bwd=True)


def test_grid_beyond_residency(la, oracle):
    """B4 H512 N8192 d32 bf16: 2048 heads of two segments each, 4096 workgroups per fused
    launch, more than the chip holds at once.  A workgroup that waits on another segment's
    record only waits on workgroups dispatched before it (first segments first in the forward,
    last segments first in the backward), so both launches finish with no wait given up and
    sampled heads match the oracle."""
    w = inp.Workload("wide grid", 4, 512, 8192, 32, torch.bfloat16, True)
    la.profile_enable(True)
    try:
        check_workload(la, oracle, w, nheads=8, with_bwd=True, seed=3)
        names = {n for n, _ in la.profile_entries()}
    finally:
        la.profile_enable(False)
    assert {"causal_fwd_fused", "bwd_fused"} <= names, names


def test_mid_noncausal_all_heads(la, oracle):
    """Non-causal forward and backward at the full Mid size, every head, in the
    launch sequence a training step uses (the backward reads the forward's saved state)."""
    w = inp.MID
    q, k, v, do = inp.workload_inputs(w, seed=0, device="cuda", with_dout=True)
    st = la.new_saved_state(q)
    o = la.la_forward_noncausal(q, k, v, saved_state=st)
    dq, dk, dv = la.la_backward_noncausal(q, k, v, do, saved_state=st)
    torch.cuda.synchronize()
    hq, hk, hv, hdo = f64(q), f64(k), f64(v), f64(do)
    ro, rden = oracle.forward_noncausal(hq, hk, hv, return_den=True)
    rdq, rdk, rdv = oracle.backward_noncausal(hq, hk, hv, hdo)
    errs = {}
    fwd_rows(errs, o, ro, rden, hq, hk, hv, w.dtype, False)
    bwd_rows(errs, (dq, dk, dv), (rdq, rdk, rdv), hq, hk, hv, hdo, w.dtype, False)
    record("full mid noncausal", **errs)
    print("mid noncausal", errs, flush=True)
    assert max(row_ratios(errs).values()) <= 1.0, errs


def test_long_sampled_heads(la, oracle):
    check_workload(la, oracle, inp.LONG, nheads=12, with_bwd=True)


def test_verylong_sampled_heads_and_footprint(la, oracle):
    w = inp.VERYLONG
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    check_workload(la, oracle, w, nheads=3, with_bwd=False)
    peak = torch.cuda.max_memory_allocated() - base
    unit = w.B * w.H * w.N * w.d * 2
    # q, k, v, dout, o (bf16) + den (fp32) + workspace (segment states): O(N d) + O(d^2) per segment
    assert peak < 5 * unit + w.B * w.H * w.N * 4 + 64 * 2**20 * w.H, peak


def test_decode_sampled_sequences(la, oracle):
    w = inp.DECODE
    B, H, d, N0, steps = w.batch, w.H, w.d, w.prefix, w.steps
    S = torch.empty(B, H, d, d, device="cuda")
    z = torch.empty(B, H, d, device="cuda")
    idx = pick(B * H, 24, 5)
    pk, pv, pq = [], [], []
    nb = 32  # prefix drawn and reduced 32 sequences at a time
    for b0 in range(0, B, nb):
        q, k, v = inp.qkv(nb, H, N0, d, w.dtype, seed=1000 + b0, device="cuda")
        _, Sb, zb = la.la_forward_causal(q, k, v, return_state=True)
        S[b0:b0 + nb].copy_(Sb)
        z[b0:b0 + nb].copy_(zb)
        sel = [i - b0 * H for i in idx if b0 * H <= i < (b0 + nb) * H]
        if sel:
            pk.append(heads(k, sel))
            pv.append(heads(v, sel))
            pq.append(heads(q, sel))
        del q, k, v
    _, rS, rz = oracle.forward_causal(np.concatenate(pq), np.concatenate(pk), np.concatenate(pv),
                                      return_state=True)
    sq, sk, sv = inp.decode_tokens(B, H, d, steps, w.dtype, seed=2, device="cuda")
    outs = torch.empty(steps, B, H, d, dtype=w.dtype, device="cuda")
    for t in range(steps):
        outs[t] = la.la_decode_step(S, z, sq[t], sk[t], sv[t])
    torch.cuda.synchronize()
    worst = 0.0
    for t in range(steps):
        ro, rS, rz = oracle.decode_step(rS, rz, heads(sq[t], idx), heads(sk[t], idx), heads(sv[t], idx))
        worst = max(worst, slice_err(heads(outs[t], idx)[:, None, :], ro[:, None, :]))
    rS_gpu = heads(S, idx)
    errs = {"o_worst_step": worst, "S_final": slice_err(rS_gpu, rS)}
    record("full decode 512 steps sampled", **errs)
    assert worst < TOL[w.dtype] and errs["S_final"] < 1e-3, errs


# ---- the longest head the ABI takes ------------------------------------------------------------
@pytest.mark.parametrize("d", [64, 128])
def test_longest_head(la, oracle, d):
    """One head of the longest sequence a call accepts (its bytes just under 2^31), causal.
    Keys and values are drawn only for the first and last P tokens and are zero in between, so
    the oracle can follow the whole sequence: a zero key adds phi(0) = 1 to every feature of z
    and nothing to S.  The last P rows are the oracle's recurrence from the state
    (S_1, z_1 + gap) the first block and the gap leave; a row i sampled in the gap reads
    (S_1, z_1 + i - P + 1): the oracle's decode step from (S_1, z_1 + i - P) with the row's
    own zero key and value."""
    P = 1024
    N = ((1 << 31) - 1) // (d * 2) - 64  # the largest N with N d 2 + 64 d 2 < 2^31 bytes per head
    N -= N % 7                            # a ragged last chunk, N not a multiple of 64
    gap = N - 2 * P
    gen = inp.generator(d + 5, "cuda")
    q = torch.zeros((1, 1, N, d), dtype=torch.bfloat16, device="cuda")
    k, v = torch.zeros_like(q), torch.zeros_like(q)
    s = 1.0 / d ** 0.5
    for t in (q, k, v):
        t[:, :, :P] = inp.normal((1, 1, P, d), gen, torch.bfloat16, s, "cuda")
        t[:, :, N - P:] = inp.normal((1, 1, P, d), gen, torch.bfloat16, s, "cuda")
    rows = np.array([P, P + 1, P + 63, N // 2, N // 2 + 1, N - P - 1])
    q[0, 0, torch.from_numpy(rows).cuda()] = inp.normal((len(rows), d), gen, torch.bfloat16, s, "cuda")
    o, S, z = la.la_forward_causal(q, k, v, return_state=True)
    torch.cuda.synchronize()
    hq, hk, hv = (f64(t[:, :, :P]) for t in (q, k, v))
    ro1, rden1, S1, z1 = oracle.forward_causal(hq, hk, hv, return_den=True, return_state=True)
    tq, tk, tv = (f64(t[:, :, N - P:]) for t in (q, k, v))
    ro3, rden3, S3, z3 = oracle.forward_causal(tq, tk, tv, return_den=True, return_state=True, S0=S1, z0=z1 + gap)
    eh, et = {}, {}
    fwd_rows(eh, o[:, :, :P], ro1, rden1, hq, hk, hv, torch.bfloat16, True)
    fwd_rows(et, o[:, :, N - P:], ro3, rden3, tq, tk, tv, torch.bfloat16, True, S0=S1, z0=z1 + gap)
    errs = {"head": eh["o"], "tail": et["o"], "S": slice_err(S, S3), "z": slice_err(z[..., None], z3[..., None])}
    zero = np.zeros((1, d))
    worst = 0.0
    for i in rows:
        ro, _, _ = oracle.decode_step(S1[0], z1[0] + (i - P), f64(q[0, :, i]), zero, zero)
        worst = max(worst, slice_err(o[0, :, i][None], ro[None]))
    errs["gap rows"] = worst
    record(f"longest head N={N} d={d}", **errs)
    print(N, errs, flush=True)
    assert max(errs["head"], errs["tail"]) <= 1.0 and errs["gap rows"] < TOL[torch.bfloat16], errs
    assert max(errs["S"], errs["z"]) < 1e-3, errs
