"""The fused causal backward's bounded waits between workgroups (GPU).

Where a head has at most 12 segments (and d <= 64) both backward sweeps run in
one launch: every workgroup publishes its segment's suffix aggregates and waits
for the later segments' before its suffix sweep.  A wait gives up after a bound
on its polls; the segment's dk, dv rows then become NaN.  The test forces every
wait to give up at once from the host (bound 0): no kernel faults or hangs, the
rows that needed a later segment's record are NaN, and everything else is
bitwise the result of an ordinary call.
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
    try:
        la.set_wait_limit(0)
        dq, dk, dv = la.la_backward_causal(q, k, v, do)
        torch.cuda.synchronize()
    finally:
        la.set_wait_limit(default)
    # dq comes from the prefix sweep, before any wait
    assert torch.equal(dq, ref[0])
    # the first segment of every head waits for the records of the 7 after it
    assert torch.isnan(dk[:, :, :64].float()).all() and torch.isnan(dv[:, :, :64].float()).all()
    # the last segment waits for nothing: its rows are the ordinary result
    assert torch.equal(dk[:, :, -64:], ref[1][:, :, -64:]) and torch.equal(dv[:, :, -64:], ref[2][:, :, -64:])
    # and with the bound restored the call is ordinary again
    again = la.la_backward_causal(q, k, v, do)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(again, ref))


def test_wait_bound_rejects_negative(la):
    with pytest.raises(la.LinAttnError):
        la.set_wait_limit(-1)
    assert la.wait_limit() > 0
