"""The allocation-free causal forward against the causal forward with a workspace (GPU).

la_forward_causal_noalloc keeps its workspace in a static device array of the
library (64 MiB per GPU) instead of taking one from the caller.  Called through the
C ABI twice in a row, the second time on a smaller input and from a start state,
it must give bitwise the outputs of la_forward_causal on the same inputs (the same
kernels and plan, only the workspace's address differs), and those outputs pass
the per-row parity bar against the oracle.  A shape whose workspace exceeds the
array is rejected before anything is launched.
"""
import ctypes

import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import la_inputs as inp  # noqa: E402
from test_parity import draw, f64, fwd_rows  # noqa: E402


@pytest.fixture(scope="module")
def la():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_02_amd as m
    m.load_library()
    return m


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def call_noalloc(la, q, k, v, S0=None, z0=None):
    """la_forward_causal_noalloc through the C ABI into outputs allocated here."""
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    den = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=q.device)
    z = torch.empty((B, H, d), dtype=torch.float32, device=q.device)
    code = la.LA_BF16 if q.dtype == torch.bfloat16 else la.LA_F32
    st = la.load_library().la_forward_causal_noalloc(_p(q), _p(k), _p(v), _p(o), _p(S0), _p(z0), _p(den), _p(S),
                                                     _p(z), B, H, N, d, 0, code,
                                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, la.load_library().la_last_error_message()
    return o, den, S, z


def test_noalloc_matches_workspace_call_twice(la, oracle):
    big = draw(2, 8, 64 * 40 + 17, 64, torch.bfloat16, seed=31)[:3]   # several segments of several chunks
    small = draw(1, 3, 200, 64, torch.bfloat16, seed=32)[:3]
    pq, pk, pv = draw(1, 3, 130, 64, torch.bfloat16, seed=33)[:3]
    _, S0, z0 = la.la_forward_causal(pq, pk, pv, return_state=True)
    for (q, k, v), st in ((big, None), (small, (S0, z0))):
        S0_, z0_ = st if st is not None else (None, None)
        got = call_noalloc(la, q, k, v, S0_, z0_)
        ref = la.la_forward_causal(q, k, v, return_den=True, return_state=True, S0=S0_, z0=z0_)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b)
        ro, rden = oracle.forward_causal(f64(q), f64(k), f64(v), return_den=True,
                                         **({} if st is None else {"S0": f64(S0_), "z0": f64(z0_)}))
        errs = {}
        fwd_rows(errs, got[0], ro, rden, q, k, v, torch.bfloat16, True,
                 S0=None if st is None else f64(S0_), z0=None if st is None else f64(z0_))
        assert errs["o"] <= 1.0, errs


def test_noalloc_rejects_shapes_beyond_the_array(la):
    """B1 H4 N1048576 d128 needs about 130 MiB of workspace (a running-sum plan of 512
    segments per head): LA_ERR_WORKSPACE, nothing launched (the small tensors' addresses
    are never read)."""
    q = torch.zeros((1, 1, 64, 128), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    lib = la.load_library()
    st = lib.la_forward_causal_noalloc(_p(q), _p(q), _p(q), _p(o), None, None, None, None, None, 1, 4, 1 << 20, 128, 0,
                                       la.LA_BF16, None)
    assert st == 3
    assert b"64 MiB" in lib.la_last_error_message()
