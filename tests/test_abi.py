"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/linattn.h declares, size
workspaces on the host, and reject bad arguments with the documented status
before any HIP call.  Pointers passed here are fake addresses: every case fails
validation, so nothing is ever dereferenced or launched.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "linattn.h")

la = pytest.importorskip("linear_attention_02_amd")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(la.LIB_PATH):
        import linear_attention_02_amd._build as b
        b.build()
    return la.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("la_forward_noncausal", "la_forward_causal", "la_backward_causal", "la_backward_noncausal",
              "la_decode_step"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(la.EXPORTS) <= set(declared_functions())


def test_status_strings(lib):
    assert lib.la_status_string(0) == b"LA_OK"
    assert lib.la_status_string(3) == b"LA_ERR_WORKSPACE"
    assert b"gfx950" in lib.la_version()


def ws(lib, op, B, H, N, d, chunk=0, dt=la.LA_BF16):
    out = ctypes.c_size_t(0)
    st = lib.la_workspace_size(op, B, H, N, d, chunk, dt, ctypes.byref(out))
    return st, out.value


def test_saved_state_size(lib):
    out = ctypes.c_size_t(0)
    assert lib.la_saved_state_size(4, 16, 4096, 64, 0, la.LA_BF16, ctypes.byref(out)) == 0
    n = out.value
    assert n > 0 and n % 16 == 0
    # one carried state (d*d + 2d floats) per head and segment, at least one segment per head
    assert n >= 4 * 16 * (64 * 64 + 128) * 4
    assert lib.la_saved_state_size(4, 16, 0, 64, 0, la.LA_BF16, ctypes.byref(out)) == 0 and out.value == 0
    assert lib.la_saved_state_size(4, 16, 64, 40, 0, la.LA_BF16, ctypes.byref(out)) == 2


def test_workspace_sizes(lib):
    for op in (la.LA_OP_FWD_NONCAUSAL, la.LA_OP_FWD_CAUSAL, la.LA_OP_BWD_CAUSAL, la.LA_OP_BWD_NONCAUSAL):
        st, n = ws(lib, op, 4, 16, 4096, 64)
        assert st == 0 and n > 0 and n % 256 == 0
        st, n0 = ws(lib, op, 4, 16, 0, 64)
        assert st == 0 and n0 == 0
    # the backward also keeps two floats per token-head
    _, nb = ws(lib, la.LA_OP_BWD_CAUSAL, 4, 16, 4096, 64)
    assert nb >= 4 * 16 * 4096 * 8
    assert ws(lib, la.LA_OP_FWD_CAUSAL, 1, 1, 64, 48)[0] == 2          # d unsupported
    assert ws(lib, la.LA_OP_FWD_CAUSAL, 1, 1, 64, 64, chunk=32)[0] == 2  # chunk unsupported
    assert ws(lib, la.LA_OP_FWD_CAUSAL, 1, 1, 64, 64, dt=7)[0] == 2    # dtype unknown
    assert ws(lib, la.LA_OP_FWD_CAUSAL, -1, 1, 64, 64)[0] == 1         # negative size
    assert ws(lib, 9, 1, 1, 64, 64)[0] == 1                            # unknown op
    assert lib.la_workspace_size(0, 1, 1, 1, 64, 0, 1, None) == 1      # NULL out


A = 0x10000000  # fake, 256-byte aligned device addresses; never dereferenced


def fwd_causal(lib, q=A, k=A + 0x1000000, v=A + 0x2000000, o=A + 0x3000000, den=None, S=None, z=None,
               saved=None, saved_bytes=0, B=1, H=1, N=64, d=64, chunk=0, dt=la.LA_BF16, wsp=A + 0x4000000, wsb=0,
               S0=None, z0=None):
    return lib.la_forward_causal(q, k, v, o, S0, z0, den, S, z, saved, saved_bytes, B, H, N, d, chunk, dt, wsp, wsb,
                                 None)


def test_forward_causal_validation(lib):
    assert fwd_causal(lib, q=None) == 1
    assert fwd_causal(lib, q=None, k=None, v=None, o=None, N=0) == 0  # no tokens: empty tensors may be NULL
    assert fwd_causal(lib, o=A + 1) == 1                     # misaligned
    assert fwd_causal(lib, o=A) == 1                         # o overlaps q
    assert fwd_causal(lib, d=96) == 2
    assert fwd_causal(lib, chunk=16) == 2
    assert fwd_causal(lib, dt=la.LA_F32, d=128) == 3         # fp32 d=128 (on feature blocks): workspace too small
    # fp32 d=128 takes a saved state (and leaves it unused: its backward recomputes), checked for size like any other
    assert fwd_causal(lib, dt=la.LA_F32, d=128, saved=A + 0x5000000, saved_bytes=1 << 30) == 3
    assert fwd_causal(lib, dt=la.LA_F32, d=128, saved=A + 0x5000000, saved_bytes=4, wsb=1 << 30) == 1
    assert fwd_causal(lib, wsb=16) == 3                      # workspace too small
    assert fwd_causal(lib, wsp=None, wsb=1 << 30) == 3       # NULL workspace
    assert fwd_causal(lib, wsp=A + 0x4000010, wsb=1 << 30) == 1   # workspace misaligned
    assert fwd_causal(lib, wsp=A + 0x2000000, wsb=1 << 30) == 1  # workspace overlaps v
    assert fwd_causal(lib, B=0) == 0                         # nothing to do, no launch
    assert fwd_causal(lib, saved=A + 0x5000000, saved_bytes=8, wsb=1 << 30) == 1       # saved state too small
    assert fwd_causal(lib, saved=A + 0x3000000, saved_bytes=1 << 20, wsb=1 << 30) == 1  # saved state overlaps o
    # start state: may be the final-state buffer itself, nothing else; not with a saved state
    S, z = A + 0x6000000, A + 0x6100000
    assert fwd_causal(lib, S0=S, z0=z, saved=A + 0x5000000, saved_bytes=1 << 30, wsb=1 << 30) == 1
    assert fwd_causal(lib, S0=A + 0x3000000, wsb=1 << 30) == 1                  # S0 overlaps o
    assert fwd_causal(lib, S0=S, S=S + 64, z=z, wsb=1 << 30) == 1               # S0 overlaps S_out partially
    assert fwd_causal(lib, S0=S + 4, wsb=1 << 30) == 1                          # S0 misaligned
    assert fwd_causal(lib, S0=S, z0=S + 256, wsb=1 << 30) == 1                  # S0 and z0 overlap
    # in place passes the pointer checks (and then stops at the too-small workspace, before any launch)
    assert fwd_causal(lib, S0=S, z0=z, S=S, z=z, wsb=16) == 3
    msg = lib.la_last_error_message()
    assert isinstance(msg, bytes)


def test_forward_noncausal_and_backward_validation(lib):
    f = lib.la_forward_noncausal
    qkv = (A, A + 0x1000000, A + 0x2000000)
    assert f(*qkv, None, None, 0, 1, 1, 64, 64, 1, A + 0x4000000, 1 << 30, None) == 1
    assert f(*qkv, A + 0x3000000, None, 0, 1, 1, 64, 64, 1, A + 0x4000000, 8, None) == 3
    assert f(*qkv, A + 0x3000000, None, 0, 1, 1, 0, 64, 1, None, 0, None) == 0
    assert f(*qkv, A + 0x3000000, A + 0x5000000, 8, 1, 1, 64, 64, 1, A + 0x4000000, 1 << 30, None) == 1  # short
    assert f(*qkv, A + 0x3000000, A + 0x1000000, 1 << 20, 1, 1, 64, 64, 1, A + 0x4000000, 1 << 30, None) == 1  # overlaps k
    assert f(*qkv, A + 0x3000000, A + 0x4000000, 1 << 20, 1, 1, 64, 64, 1, A + 0x4000000, 1 << 30, None) == 1  # overlaps ws
    b = lib.la_backward_causal
    args = [A, A + 0x1000000, A + 0x2000000, A + 0x3000000, A + 0x4000000, A + 0x5000000, A + 0x6000000]
    assert b(*args, None, 0, 1, 1, 64, 64, 0, 1, A + 0x7000000, 8, None) == 3
    bad = list(args)
    bad[5] = args[4]                                          # dk aliases dq
    assert b(*bad, None, 0, 1, 1, 64, 64, 0, 1, A + 0x7000000, 1 << 30, None) == 1
    bad = list(args)
    bad[6] = args[3]                                          # dv aliases dout
    assert b(*bad, None, 0, 1, 1, 64, 64, 0, 1, A + 0x7000000, 1 << 30, None) == 1
    assert b(*args, A + 0x8000000, 4, 1, 1, 64, 64, 0, 1, A + 0x7000000, 1 << 30, None) == 1  # saved state short
    assert b(*args, A + 0x4000000, 1 << 20, 1, 1, 64, 64, 0, 1, A + 0x7000000, 1 << 30, None) == 1  # overlaps dq
    assert b(*args, None, 0, 1, 1, 64, 128, 0, 0, A + 0x7000000, 8, None) == 3     # fp32 d=128: workspace too small
    st = lib.la_backward_causal_state
    sargs = [A, A + 0x1000000, A + 0x2000000, A + 0x3000000, A + 0x8000000, None, None, None,
             A + 0x4000000, A + 0x5000000, A + 0x6000000, None, None]
    assert st(*sargs, 1, 1, 64, 128, 0, 0, A + 0x7000000, 1 << 30, None) == 2  # fp32 d=128 from a start state


def test_decode_steps_validation(lib):
    f = lib.la_decode_steps
    S, z, q, k, v, o = A, A + 0x1000000, A + 0x2000000, A + 0x2100000, A + 0x2200000, A + 0x2300000
    assert f(None, z, q, k, v, o, 1, 1, 1, 8, 64, 1, None) == 1
    assert f(S, z, q, k, v, q, 1, 1, 1, 8, 64, 1, None) == 1     # o aliases q
    assert f(S, z, q, k, v, o, 1, 1, 1, 8, 96, 1, None) == 2     # d unsupported
    assert f(S, z, q, k, v, o, 1, 1, 1, -1, 64, 1, None) == 1    # negative T
    assert f(S, z, q, k, v, o, 1, 6, 4, 8, 64, 1, None) == 1     # H not a multiple of Hkv
    assert f(S, z, q, k, v, o, 1, 6, 0, 8, 64, 1, None) == 1     # no key/value heads for 6 query heads
    assert f(S, z, q, k, v, o, 1, 1, 1, 0, 64, 1, None) == 0     # no tokens: nothing to do
    assert f(S, z, None, None, None, None, 1, 1, 1, 0, 64, 1, None) == 0  # ... and the empty tensors may be NULL
    assert f(S, None, None, None, None, None, 1, 1, 1, 0, 64, 1, None) == 1  # the state may not
    assert f(S, z, q, k, v, o, 0, 3, 3, 8, 64, 1, None) == 0     # no heads
    # the state is sized by the key/value heads: 8 query heads on 2 states of 64 x 64 fp32
    assert f(S, S + 2 * 64 * 64 * 4 - 16, q, k, v, o, 1, 8, 2, 8, 64, 1, None) == 1  # z overlaps S
    assert f(S, S + 2 * 64 * 64 * 4, q, k, v, o, 1, 8, 2, 0, 64, 1, None) == 0


def test_decode_validation(lib):
    f = lib.la_decode_step
    S, z, q, k, v, o = A, A + 0x1000000, A + 0x2000000, A + 0x2001000, A + 0x2002000, A + 0x2003000
    assert f(None, z, q, k, v, o, 1, 1, 64, 1, None) == 1
    assert f(S, z, q, k, v, q, 1, 1, 64, 1, None) == 1       # o aliases q
    assert f(S, S, q, k, v, o, 1, 1, 64, 1, None) == 1       # z aliases S
    assert f(S, z, q, k, v, o, 1, 1, 80, 1, None) == 2
    assert f(S, z, q, k, v, o, 1, 1, 64, 5, None) == 2
    assert f(S, z, q + 2, k, v, o, 1, 1, 64, 1, None) == 1   # misaligned
    assert f(S, z, q, k, v, o, 0, 7, 64, 1, None) == 0       # empty


def test_backward_noncausal_validation(lib):
    b = lib.la_backward_noncausal
    args = [A, A + 0x1000000, A + 0x2000000, A + 0x3000000, A + 0x4000000, A + 0x5000000, A + 0x6000000]
    wsp = A + 0x7000000
    assert b(*args, None, 0, 1, 1, 64, 64, 1, wsp, 8, None) == 3                   # workspace too small
    assert b(*args, None, 0, 1, 1, 64, 96, 1, wsp, 1 << 30, None) == 2             # d unsupported
    assert b(*args, None, 0, 1, 1, 64, 128, 0, wsp, 8, None) == 3                  # fp32 d=128: workspace too small
    assert b(*args, None, 0, 1, 1, 0, 64, 1, None, 0, None) == 0                   # empty
    bad = list(args)
    bad[6] = args[0]                                                                # dv aliases q
    assert b(*bad, None, 0, 1, 1, 64, 64, 1, wsp, 1 << 30, None) == 1
    bad = list(args)
    bad[0] = None
    assert b(*bad, None, 0, 1, 1, 64, 64, 1, wsp, 1 << 30, None) == 1
    assert b(*args, A + 0x8000000, 4, 1, 1, 64, 64, 1, wsp, 1 << 30, None) == 1     # saved state short
    assert b(*args, A + 0x5000000, 1 << 20, 1, 1, 64, 64, 1, wsp, 1 << 30, None) == 1  # saved state overlaps dk
    assert b(*args, None, 0, 1, 1, 64, 64, 1, A + 0x6000000, 1 << 30, None) == 1    # workspace overlaps dv


def test_noncausal_backward_workspace_holds_both_record_sets(lib):
    _, nf = ws(lib, la.LA_OP_FWD_NONCAUSAL, 4, 16, 4096, 64)
    _, nb = ws(lib, la.LA_OP_BWD_NONCAUSAL, 4, 16, 4096, 64)
    out = ctypes.c_size_t(0)
    lib.la_saved_state_size(4, 16, 4096, 64, 0, la.LA_BF16, ctypes.byref(out))
    assert nb >= nf + out.value


def test_forward_causal_grouped_validation(lib):
    f = lib.la_forward_causal_grouped
    q, k, v, o, wsp = A, A + 0x1000000, A + 0x1100000, A + 0x2000000, A + 0x4000000
    none4 = (None, None, None, None, None)
    assert f(q, k, v, o, *none4, 1, 6, 4, 64, 64, 0, 1, wsp, 1 << 30, None) == 1   # H not a multiple of Hkv
    assert f(q, k, v, o, *none4, 1, 6, 0, 64, 64, 0, 1, wsp, 1 << 30, None) == 1   # no key/value heads
    assert f(q, k, v, o, *none4, 1, 8, 2, 64, 96, 0, 1, wsp, 1 << 30, None) == 2   # d unsupported
    assert f(q, k, v, o, *none4, 1, 8, 2, 64, 64, 0, 1, wsp, 16, None) == 3        # workspace too small
    # k and v are sized by the key/value heads: 8 query heads on 2 heads of 64 x 64 bf16 rows
    kb = 2 * 64 * 64 * 2
    assert f(q, k, v, k + kb - 16, *none4, 1, 8, 2, 64, 64, 0, 1, wsp, 1 << 30, None) == 1  # o overlaps k
    assert f(q, k, v + 0x1000000, k + kb, *none4, 1, 8, 2, 64, 64, 0, 1, wsp, 16, None) == 3  # passes, then workspace
    # the states are per key/value head too: S_out of 2 x 64 x 64 fp32, z_out right after it
    S = A + 0x6000000
    assert f(q, k, v, o, None, None, None, S, S + 2 * 64 * 64 * 4 - 16, 1, 8, 2, 64, 64, 0, 1, wsp, 1 << 30,
             None) == 1                                                                   # z_out overlaps S_out
    assert f(q, k, v, o, None, None, None, S, S + 2 * 64 * 64 * 4, 1, 8, 2, 64, 64, 0, 1, wsp, 16, None) == 3


def test_feature_blocks_validation(lib):
    out = ctypes.c_size_t(0)
    wsz = lambda causal, m: lib.la_features_workspace_size(causal, 1, 2, 64, 64, m, 1, ctypes.byref(out))
    assert wsz(1, 96) == 1                                    # m not a multiple of d
    assert wsz(1, 32) == 1                                    # fewer features than d
    assert wsz(1, 64 * 65) == 2                               # more than 64 blocks
    assert wsz(1, 64) == 0
    assert out.value == ws(lib, la.LA_OP_FWD_CAUSAL, 1, 2, 64, 64)[1]  # m = d: the plain call's workspace
    assert wsz(1, 128) == 0
    # two blocks: the plain workspace of 4 heads plus the blocks' outputs (bf16 rows) and denominators
    assert out.value >= ws(lib, la.LA_OP_FWD_CAUSAL, 1, 4, 64, 64)[1] + 4 * 64 * 64 * 2 + 4 * 64 * 4
    assert wsz(0, 128) == 0 and out.value >= ws(lib, la.LA_OP_FWD_NONCAUSAL, 1, 4, 64, 64)[1] + 4 * 64 * 64 * 2
    f = lib.la_forward_causal_features_blocks
    fq, fk, v, o, wsp = A, A + 0x1000000, A + 0x2000000, A + 0x3000000, A + 0x4000000
    fb = 2 * 64 * 64 * 2 * 2                                  # B H N d bf16 x 2 blocks
    n5 = (None,) * 5
    assert f(fq, fk, v, o, *n5, 1, 2, 64, 64, 96, 1, wsp, 1 << 30, None) == 1
    assert f(fq, fk, v, o, *n5, 1, 2, 64, 64, 128, 1, wsp, 16, None) == 3          # workspace too small
    assert f(fq, fk, v, fk + fb - 16, *n5, 1, 2, 64, 64, 128, 1, wsp, 1 << 30, None) == 1  # o overlaps fk's blocks
    assert f(fq, fk, v, fk + fb, *n5, 1, 2, 64, 64, 128, 1, wsp, 16, None) == 3            # ... and past them
    assert f(fq, fk, v, o, *n5, 1, 2, 64, 64, 128, 1, o, 1 << 30, None) == 1       # workspace overlaps o
    S, z = A + 0x6000000, A + 0x6100000
    assert f(fq, fk, v, o, None, None, None, S, o + 64, 1, 2, 64, 64, 128, 1, wsp, 1 << 30, None) == 1  # z_out on o
    assert f(fq, fk, v, o, *n5, 1, 2, 0, 64, 128, 1, None, 0, None) == 0            # no tokens
    assert f(fq, fk, v, o, *n5, 1, 2, 64, 128, 256, 0, wsp, 1 << 30, None) == 2     # fp32 causal d = 128
    g = lib.la_forward_noncausal_features_blocks
    assert g(fq, fk, v, o, None, 1, 2, 64, 64, 128, 1, wsp, 16, None) == 3
    assert g(fq, fk, v, o, o + 64, 1, 2, 64, 64, 128, 1, wsp, 1 << 30, None) == 1  # den_out overlaps o
    h = lib.la_favor_features_blocks
    om = A + 0x5000000
    assert h(A, om, A + 0x1000000, 2, 64, 64, 96, 1, None) == 1                    # m not a multiple of d
    assert h(A, om, A + 2 * 64 * 64 * 2 - 16, 2, 64, 64, 128, 1, None) == 1        # out overlaps x
    assert h(A, None, A + 0x1000000, 2, 64, 64, 128, 1, None) == 1                 # no directions
    assert h(A, om, A + 0x1000000, 0, 64, 64, 128, 1, None) == 0                   # no rows


def test_decode_blocks_validation(lib):
    f = lib.la_decode_steps_features_blocks
    S, z, q, k, v, o = A, A + 0x1000000, A + 0x2000000, A + 0x2100000, A + 0x2200000, A + 0x2300000
    wsp = A + 0x4000000
    out = ctypes.c_size_t(0)
    assert lib.la_features_workspace_size(2, 1, 8, 16, 64, 64, 1, ctypes.byref(out)) == 0 and out.value == 0
    assert lib.la_features_workspace_size(2, 1, 8, 16, 64, 128, 1, ctypes.byref(out)) == 0
    assert out.value >= 8 * 2 * 16 * 64 * 2 + 8 * 2 * 16 * 4
    assert f(S, z, q, k, v, o, 1, 8, 2, 16, 64, 96, 1, wsp, 1 << 30, None) == 1    # m not a multiple of d
    assert f(S, z, q, k, v, o, 1, 8, 2, 16, 64, 128, 1, None, 0, None) == 3        # KF = 2 needs a workspace
    assert f(S, z, q, k, v, o, 1, 8, 2, 16, 64, 128, 1, wsp, 16, None) == 3
    assert f(S, z, q, k, v, o, 1, 8, 2, 16, 64, 128, 1, o, 1 << 30, None) == 1     # workspace overlaps o
    # the states are m x d per key/value head: z right after S of 2 x 128 x 64 fp32
    assert f(S, S + 2 * 128 * 64 * 4 - 16, q, k, v, o, 1, 8, 2, 16, 64, 128, 1, wsp, 1 << 30, None) == 1
    assert f(S, z, q, k, v, o, 1, 8, 2, 0, 64, 128, 1, None, 0, None) == 0         # no tokens


def test_features_backward_validation(lib):
    b = lib.la_backward_causal_features
    args = [A, A + 0x1000000, A + 0x2000000, A + 0x3000000, A + 0x4000000, A + 0x5000000, A + 0x6000000]
    wsp = A + 0x7000000
    assert b(*args, 1, 1, 64, 64, 1, wsp, 8, None) == 3                   # workspace too small
    assert b(*args, 1, 1, 64, 96, 1, wsp, 1 << 30, None) == 2             # d unsupported
    bad = list(args)
    bad[5] = args[4]                                                       # dfk aliases dfq
    assert b(*bad, 1, 1, 64, 64, 1, wsp, 1 << 30, None) == 1
    assert b(*args, 1, 1, 0, 64, 1, None, 0, None) == 0                   # no tokens
    n = lib.la_backward_noncausal_features
    assert n(*args, 1, 1, 64, 64, 1, wsp, 8, None) == 3
    assert n(*args, 1, 1, 64, 128, 0, wsp, 1 << 30, None) == 2            # fp32 d = 128 not built
    f = lib.la_favor_features_backward
    x, om, F, dF, dx = A, A + 0x1000000, A + 0x2000000, A + 0x3000000, A + 0x4000000
    assert f(x, None, F, dF, dx, 64, 64, 1, None) == 1                    # no directions
    assert f(x, om, F, dF, F, 64, 64, 1, None) == 1                       # dx aliases F
    assert f(x, om, F, dF, dx, 64, 96, 1, None) == 2                      # d unsupported
    assert f(x, om, F, dF, dx, 0, 64, 1, None) == 0                       # no rows


def test_backward_blocks_validation(lib):
    f = lib.la_backward_causal_features_blocks
    fq, fk, v, do, den = A, A + 0x1000000, A + 0x2000000, A + 0x2100000, A + 0x2200000
    dfq, dfk, dv, wsp = A + 0x3000000, A + 0x4000000, A + 0x5000000, A + 0x6000000
    out = ctypes.c_size_t(0)
    assert lib.la_features_workspace_size(3, 1, 2, 64, 64, 128, 1, ctypes.byref(out)) == 0
    assert out.value >= ws(lib, la.LA_OP_BWD_CAUSAL, 1, 4, 64, 64)[1] + 4 * 64 * 64 * 2   # block heads + their dv
    args = (fq, fk, v, do, den, None, dfq, dfk, dv)
    assert f(*args, 1, 2, 64, 64, 96, 1, wsp, 1 << 30, None) == 1                  # m not a multiple of d
    assert f(*args, 1, 2, 64, 64, 128, 1, wsp, 16, None) == 3                      # workspace too small
    assert f(*args, 1, 2, 64, 64, 128, 1, None, 0, None) == 3                      # no workspace
    assert f(fq, fk, v, do, None, None, dfq, dfk, dv, 1, 2, 64, 64, 128, 1, wsp, 1 << 30, None) == 1  # no den
    assert f(fq, fk, v, do, den, None, dfq, dfq + 64, dv, 1, 2, 64, 64, 128, 1, wsp, 1 << 30, None) == 1  # dfk on dfq
    assert f(*args, 1, 2, 64, 128, 256, 0, wsp, 1 << 30, None) == 2                # fp32 d = 128 not built
    assert f(*args, 1, 2, 0, 64, 128, 1, None, 0, None) == 0                       # no tokens
    assert f(fq, fk, v, do, den, dfq + 64, dfq, dfk, dv, 1, 2, 64, 64, 128, 1, wsp, 1 << 30, None) == 1  # o on dfq


def test_backward_noncausal_blocks_validation(lib):
    f = lib.la_backward_noncausal_features_blocks
    fq, fk, v, do, den = A, A + 0x1000000, A + 0x2000000, A + 0x2100000, A + 0x2200000
    dfq, dfk, dv, wsp = A + 0x3000000, A + 0x4000000, A + 0x5000000, A + 0x6000000
    out = ctypes.c_size_t(0)
    assert lib.la_features_workspace_size(4, 1, 2, 64, 64, 128, 1, ctypes.byref(out)) == 0
    # block heads' workspace + their dv + a (den, g) pair per block row
    assert out.value >= ws(lib, la.LA_OP_BWD_NONCAUSAL, 1, 4, 64, 64)[1] + 4 * 64 * 64 * 2 + 4 * 64 * 8
    args = (fq, fk, v, do, den, None, dfq, dfk, dv)
    assert f(*args, 1, 2, 64, 64, 96, 1, wsp, 1 << 30, None) == 1                  # m not a multiple of d
    assert f(*args, 1, 2, 64, 64, 128, 1, wsp, out.value - 1, None) == 3           # workspace one byte short
    assert f(*args, 1, 2, 64, 64, 128, 1, None, 0, None) == 3                      # no workspace
    assert f(fq, fk, v, do, None, None, dfq, dfk, dv, 1, 2, 64, 64, 128, 1, wsp, 1 << 30, None) == 1  # no den
    assert f(fq, fk, v, do, den, None, dfq, dfk, dfk + 64, 1, 2, 64, 64, 128, 1, wsp, 1 << 30, None) == 1  # dv on dfk
    assert f(*args, 1, 2, 64, 128, 256, 0, wsp, 1 << 30, None) == 2                # fp32 d = 128 not built
    assert f(*args, 1, 2, 0, 64, 128, 1, None, 0, None) == 0                       # no tokens
    assert f(fq, fk, v, do, den, dfq + 64, dfq, dfk, dv, 1, 2, 64, 64, 128, 1, wsp, 1 << 30, None) == 1  # o on dfq


def test_favor_features_blocks_backward_validation(lib):
    f = lib.la_favor_features_blocks_backward
    x, om, F, dF, dx = A, A + 0x1000000, A + 0x2000000, A + 0x3000000, A + 0x4000000
    assert f(x, om, F, dF, dx, 2, 64, 64, 96, 1, None) == 1                         # m not a multiple of d
    assert f(x, None, F, dF, dx, 2, 64, 64, 128, 1, None) == 1                      # no omega
    assert f(x, om, F, dF, F + 64, 2, 64, 64, 128, 1, None) == 1                    # dx on F
    assert f(x, om, F, dF, dx, -1, 64, 64, 128, 1, None) == 1                       # negative heads
    assert f(x, om, F, dF, dx, 2, 64, 48, 96, 1, None) == 2                         # d = 48 not built
    assert f(x, om, F, dF, dx, 2, 0, 64, 128, 1, None) == 0                         # no rows
