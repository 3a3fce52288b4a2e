"""Bounded waits between workgroups (GPU): the fused causal backward and forward.

Where a head has at most 12 segments (and d <= 64) both backward sweeps run in
one launch: every workgroup publishes its segment's suffix aggregates and waits
for the later segments' before its suffix sweep.  The fused causal forward
likewise publishes each segment's record and waits for the earlier segments'.
A wait gives up after a bound on its polls; the rows of that segment then become
NaN, and the workgroup counts the give-up where la_wait_failures reads it.  The
tests force every wait to give up at once from the host (bound 0): no kernel
faults or hangs, the rows that needed another segment's record are NaN, the
count names every such workgroup, and everything else is bitwise the result of
an ordinary call.
"""
import os
import sys

import pytest

torch = pytest.importorskip("torch")
sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import la_inputs as inp  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def la():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_02_amd as m
    m.load_library()
    return m


def test_wait_bound_zero_poisons_only_waiting_segments(la):
    # 64 heads x 16 chunks: 8 segments of 2 chunks per head (fused path)
    B, H, N, d = 4, 16, 1024, 64
    q, k, v, do = [t.cuda() for t in inp.qkv(B, H, N, d, torch.bfloat16, seed=11, scale=True, with_dout=True)]
    ref = la.la_backward_causal(q, k, v, do)
    torch.cuda.synchronize()
    assert all(torch.isfinite(t).all() for t in ref)
    default = la.wait_limit()
    assert default > 0
    ws = torch.empty(la.workspace_size(la.LA_OP_BWD_CAUSAL, B, H, N, d, q.dtype), dtype=torch.uint8, device="cuda")
    la.la_backward_causal(q, k, v, do, workspace=ws)
    assert la.backward_wait_failures(ws, q) == 0
    try:
        la.set_wait_limit(0)
        dq, dk, dv = la.la_backward_causal(q, k, v, do, workspace=ws)
        torch.cuda.synchronize()
    finally:
        la.set_wait_limit(default)
    # every segment but the last of each head waited for a later one and gave up
    assert la.backward_wait_failures(ws, q) == B * H * 7
    # dq comes from the prefix sweep, before any wait
    assert torch.equal(dq, ref[0])
    # the first segment of every head waits for the records of the 7 after it
    assert torch.isnan(dk[:, :, :64].float()).all() and torch.isnan(dv[:, :, :64].float()).all()
    # the last segment waits for nothing: its rows are the ordinary result
    assert torch.equal(dk[:, :, -64:], ref[1][:, :, -64:]) and torch.equal(dv[:, :, -64:], ref[2][:, :, -64:])
    # and with the bound restored the call is ordinary again, with no give-ups reported
    again = la.la_backward_causal(q, k, v, do, workspace=ws)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(again, ref))
    assert la.backward_wait_failures(ws, q) == 0


def test_wait_bound_zero_forward(la):
    # 64 heads x 16 chunks: 8 segments of 2 chunks per head (fused forward)
    B, H, N, d = 4, 16, 1024, 64
    q, k, v = [t.cuda() for t in inp.qkv(B, H, N, d, torch.bfloat16, seed=12, scale=True)]
    ref = la.la_forward_causal(q, k, v)
    torch.cuda.synchronize()
    assert torch.isfinite(ref).all()
    default = la.wait_limit()
    ws = torch.empty(la.workspace_size(la.LA_OP_FWD_CAUSAL, B, H, N, d, q.dtype), dtype=torch.uint8, device="cuda")
    la.la_forward_causal(q, k, v, workspace=ws)
    assert la.wait_failures(la.LA_OP_FWD_CAUSAL, ws, q) == 0
    try:
        la.set_wait_limit(0)
        o = la.la_forward_causal(q, k, v, workspace=ws)
        torch.cuda.synchronize()
    finally:
        la.set_wait_limit(default)
    # every segment but the first of each head waited for an earlier one and gave up
    assert la.wait_failures(la.LA_OP_FWD_CAUSAL, ws, q) == B * H * 7
    assert torch.equal(o[:, :, :128], ref[:, :, :128])
    assert torch.isnan(o[:, :, 128:].float()).all()
    again = la.la_forward_causal(q, k, v, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(again, ref)
    assert la.wait_failures(la.LA_OP_FWD_CAUSAL, ws, q) == 0
    # a forward with shared key/value heads runs as two launches that wait for nothing:
    # after the give-ups of a forced bound it leaves the counts at zero
    try:
        la.set_wait_limit(0)
        la.la_forward_causal(q, k, v, workspace=ws)
    finally:
        la.set_wait_limit(default)
    assert la.wait_failures(la.LA_OP_FWD_CAUSAL, ws, q) == B * H * 7
    la.la_forward_causal_grouped(q, k[:, :4].contiguous(), v[:, :4].contiguous(), workspace=ws)
    assert la.wait_failures(la.LA_OP_FWD_CAUSAL, ws, q) == 0


def test_wait_failures_rejects_ops_without_waits(la):
    q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(la.LinAttnError):
        la.wait_failures(la.LA_OP_FWD_NONCAUSAL, None, q)


def test_wait_bound_rejects_negative(la):
    with pytest.raises(la.LinAttnError):
        la.set_wait_limit(-1)
    assert la.wait_limit() > 0
