"""ctypes binding of ``liblinattn.so`` (the C ABI in include/linattn.h).

Argument marshalling only: tensors are checked, outputs and the workspace are
allocated with ``torch.empty`` on the inputs' device, and the raw device
pointers plus the current HIP stream are handed to the library.  Every step of
the computation runs in the library's gfx950 kernels; there is no fallback,
and a missing or unloadable library raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblinattn.so")

LA_OK, LA_ERR_INVALID_ARGUMENT, LA_ERR_UNSUPPORTED, LA_ERR_WORKSPACE, LA_ERR_HIP = range(5)
LA_F32, LA_BF16 = 0, 1
LA_OP_FWD_NONCAUSAL, LA_OP_FWD_CAUSAL, LA_OP_BWD_CAUSAL, LA_OP_BWD_NONCAUSAL = 0, 1, 2, 3

EXPORTS = ("la_workspace_size", "la_saved_state_size", "la_forward_noncausal", "la_forward_causal", "la_backward_causal",
           "la_backward_noncausal", "la_decode_step", "la_decode_steps", "la_favor_features",
           "la_forward_causal_features", "la_forward_noncausal_features", "la_decode_steps_features",
           "la_backward_causal_state", "la_forward_causal_grouped", "la_features_workspace_size",
           "la_favor_features_blocks", "la_forward_causal_features_blocks", "la_forward_noncausal_features_blocks",
           "la_decode_steps_features_blocks", "la_backward_causal_features", "la_backward_noncausal_features",
           "la_favor_features_backward", "la_favor_features_blocks_backward", "la_backward_causal_features_blocks",
           "la_backward_noncausal_features_blocks", "la_status_string", "la_last_error_message", "la_version",
           "la_profile_enable", "la_profile_count", "la_profile_entry", "la_debug_set_wait_limit",
           "la_debug_wait_limit", "la_wait_failures", "la_forward_causal_noalloc")

_lib = None


class LinAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(message)


def load_library(path: str | None = None):
    """Load liblinattn.so (raises if it is missing; the library is never replaced by Python code).

    $LINATTN_LIBRARY, when set, names another build of the same library to load."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or os.environ.get("LINATTN_LIBRARY") or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
                          "or `python -m linear_attention_02_amd._build`")
    lib = ctypes.CDLL(p)
    i64, sz, vp, i32 = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int
    lib.la_workspace_size.restype = i32
    lib.la_workspace_size.argtypes = [i32, i64, i64, i64, i64, i32, i32, ctypes.POINTER(sz)]
    lib.la_forward_noncausal.restype = i32
    lib.la_forward_noncausal.argtypes = [vp, vp, vp, vp, vp, sz, i64, i64, i64, i64, i32, vp, sz, vp]
    lib.la_saved_state_size.restype = i32
    lib.la_saved_state_size.argtypes = [i64, i64, i64, i64, i32, i32, ctypes.POINTER(sz)]
    lib.la_forward_causal.restype = i32
    lib.la_forward_causal.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, i64, i64, i32, i32, vp, sz, vp]
    lib.la_backward_causal.restype = i32
    lib.la_backward_causal.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, i64, i64, i32, i32, vp, sz, vp]
    lib.la_features_workspace_size.restype = i32
    lib.la_features_workspace_size.argtypes = [i32, i64, i64, i64, i64, i64, i32, ctypes.POINTER(sz)]
    lib.la_favor_features_blocks.restype = i32
    lib.la_favor_features_blocks.argtypes = [vp, vp, vp, i64, i64, i64, i64, i32, vp]
    lib.la_forward_causal_features_blocks.restype = i32
    lib.la_forward_causal_features_blocks.argtypes = [vp] * 9 + [i64, i64, i64, i64, i64, i32, vp, sz, vp]
    lib.la_forward_noncausal_features_blocks.restype = i32
    lib.la_forward_noncausal_features_blocks.argtypes = [vp] * 5 + [i64, i64, i64, i64, i64, i32, vp, sz, vp]
    lib.la_decode_steps_features_blocks.restype = i32
    lib.la_decode_steps_features_blocks.argtypes = [vp] * 6 + [i64, i64, i64, i64, i64, i64, i32, vp, sz, vp]
    for name in ("la_backward_causal_features", "la_backward_noncausal_features"):
        f = getattr(lib, name)
        f.restype = i32
        f.argtypes = [vp] * 7 + [i64, i64, i64, i64, i32, vp, sz, vp]
    for name in ("la_backward_causal_features_blocks", "la_backward_noncausal_features_blocks"):
        getattr(lib, name).restype = i32
        getattr(lib, name).argtypes = [vp] * 9 + [i64, i64, i64, i64, i64, i32, vp, sz, vp]
    lib.la_favor_features_backward.restype = i32
    lib.la_favor_features_backward.argtypes = [vp] * 5 + [i64, i64, i32, vp]
    lib.la_favor_features_blocks_backward.restype = i32
    lib.la_favor_features_blocks_backward.argtypes = [vp] * 5 + [i64, i64, i64, i64, i32, vp]
    lib.la_forward_causal_grouped.restype = i32
    lib.la_forward_causal_grouped.argtypes = [vp] * 9 + [i64, i64, i64, i64, i64, i32, i32, vp, sz, vp]
    lib.la_backward_causal_state.restype = i32
    lib.la_backward_causal_state.argtypes = [vp] * 13 + [i64, i64, i64, i64, i32, i32, vp, sz, vp]
    lib.la_backward_noncausal.restype = i32
    lib.la_backward_noncausal.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, i64, i64, i32, vp, sz, vp]
    lib.la_decode_step.restype = i32
    lib.la_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp]
    lib.la_decode_steps.restype = i32
    lib.la_decode_steps.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, vp]
    lib.la_decode_steps_features.restype = i32
    lib.la_decode_steps_features.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, vp]
    lib.la_favor_features.restype = i32
    lib.la_favor_features.argtypes = [vp, vp, vp, i64, i64, i32, vp]
    lib.la_forward_causal_features.restype = i32
    lib.la_forward_causal_features.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, vp, sz, vp]
    lib.la_forward_noncausal_features.restype = i32
    lib.la_forward_noncausal_features.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i32, vp, sz, vp]
    lib.la_forward_causal_noalloc.restype = i32
    lib.la_forward_causal_noalloc.argtypes = [vp] * 9 + [i64, i64, i64, i64, i32, i32, vp]
    lib.la_wait_failures.restype = i32
    lib.la_wait_failures.argtypes = [i32, vp, sz, i64, i64, i64, i64, i32, vp, ctypes.POINTER(i64)]
    lib.la_status_string.restype = ctypes.c_char_p
    lib.la_status_string.argtypes = [i32]
    lib.la_last_error_message.restype = ctypes.c_char_p
    lib.la_last_error_message.argtypes = []
    lib.la_version.restype = ctypes.c_char_p
    lib.la_version.argtypes = []
    lib.la_profile_enable.restype = i32
    lib.la_profile_enable.argtypes = [i32]
    lib.la_profile_count.restype = i32
    lib.la_profile_count.argtypes = []
    lib.la_debug_set_wait_limit.restype = i32
    lib.la_debug_set_wait_limit.argtypes = [i32]
    lib.la_debug_wait_limit.restype = i32
    lib.la_debug_wait_limit.argtypes = []
    lib.la_profile_entry.restype = i32
    lib.la_profile_entry.argtypes = [i32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float)]
    if path is None:
        _lib = lib
    return lib


def _check(status: int) -> None:
    if status != LA_OK:
        lib = load_library()
        name = lib.la_status_string(status).decode()
        msg = lib.la_last_error_message().decode()
        raise LinAttnError(status, f"{name}: {msg}")


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return LA_BF16
    if dt == torch.float32:
        return LA_F32
    raise ValueError(f"unsupported dtype {dt}; use torch.bfloat16 or torch.float32")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_seq(*ts):
    ref = ts[0]
    if ref.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    for t in ts:
        if t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device:
            raise ValueError("q, k, v (and dout) must share shape, dtype and device")
        if not t.is_cuda:
            raise ValueError("tensors must be on a HIP device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return ref.shape


def workspace_size(op: int, B: int, H: int, N: int, d: int, dtype: torch.dtype, chunk: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().la_workspace_size(op, B, H, N, d, chunk, _dtype_code(dtype), ctypes.byref(out)))
    return int(out.value)


def saved_state_size(B: int, H: int, N: int, d: int, dtype: torch.dtype, chunk: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().la_saved_state_size(B, H, N, d, chunk, _dtype_code(dtype), ctypes.byref(out)))
    return int(out.value)


def new_saved_state(q, chunk: int = 0):
    """An uninitialised buffer for the forward state that a forward call on tensors shaped
    like q saves for the backward of the same form (causal or non-causal)."""
    B, H, N, d = q.shape
    return torch.empty(max(1, saved_state_size(B, H, N, d, q.dtype, chunk)), dtype=torch.uint8, device=q.device)


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _workspace(op, B, H, N, d, dtype, device, chunk, workspace):
    need = workspace_size(op, B, H, N, d, dtype, chunk)
    if workspace is not None:
        return workspace
    if need == 0:
        return None
    return torch.empty(need, dtype=torch.uint8, device=device)


def la_forward_noncausal(q, k, v, *, out=None, workspace=None, saved_state=None):
    """O_i = phi(Q_i)^T S / phi(Q_i)^T z with S, z over all keys.  q, k, v: [B, H, N, d].

    saved_state (optional, from new_saved_state) receives the key aggregates for la_backward_noncausal."""
    B, H, N, d = _check_seq(q, k, v)
    o = torch.empty_like(q) if out is None else out
    ws = _workspace(LA_OP_FWD_NONCAUSAL, B, H, N, d, q.dtype, q.device, 0, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load_library().la_forward_noncausal(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(saved_state),
                                               _nbytes(saved_state), B, H, N, d, _dtype_code(q.dtype), _ptr(ws),
                                               nbytes, _stream(q.device)))
    return o


def _check_state(S, z, B, H, d, device):
    if S is not None and (S.shape != (B, H, d, d) or S.dtype != torch.float32 or not S.is_contiguous()
                          or S.device != device):
        raise ValueError("S0 must be a contiguous [B, H, d, d] fp32 tensor on the inputs' device")
    if z is not None and (z.shape != (B, H, d) or z.dtype != torch.float32 or not z.is_contiguous()
                          or z.device != device):
        raise ValueError("z0 must be a contiguous [B, H, d] fp32 tensor on the inputs' device")


def la_forward_causal(q, k, v, *, chunk=0, return_den=False, return_state=False, out=None, workspace=None,
                      saved_state=None, S0=None, z0=None, S_out=None, z_out=None):
    """Causal forward; returns o, plus den [B,H,N] and/or the final (S [B,H,d,d], z [B,H,d]) if asked.

    S0, z0 (optional fp32 [B,H,d,d], [B,H,d]): the state the recurrence starts from (a
    previous piece of the same sequences).  S_out, z_out (optional): where the final state
    goes when return_state is set (they may be S0, z0 themselves: continuing in place).
    saved_state (optional, from new_saved_state) receives the carried state for la_backward_causal."""
    B, H, N, d = _check_seq(q, k, v)
    _check_state(S0, z0, B, H, d, q.device)
    _check_state(S_out, z_out, B, H, d, q.device)
    o = torch.empty_like(q) if out is None else out
    den = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if return_den else None
    S, z = S_out, z_out  # a state buffer the caller passes is always written
    if return_state:
        S = torch.empty((B, H, d, d), dtype=torch.float32, device=q.device) if S_out is None else S_out
        z = torch.empty((B, H, d), dtype=torch.float32, device=q.device) if z_out is None else z_out
    ws = _workspace(LA_OP_FWD_CAUSAL, B, H, N, d, q.dtype, q.device, chunk, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load_library().la_forward_causal(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(S0), _ptr(z0), _ptr(den),
                                            _ptr(S), _ptr(z), _ptr(saved_state), _nbytes(saved_state), B, H, N, d,
                                            chunk, _dtype_code(q.dtype), _ptr(ws), nbytes, _stream(q.device)))
    res = [o]
    if return_den:
        res.append(den)
    if return_state:
        res += [S, z]
    return res[0] if len(res) == 1 else tuple(res)


def la_forward_causal_noalloc(q, k, v, o, *, den_out=None, S0=None, z0=None, S_out=None, z_out=None, chunk=0):
    """la_forward_causal into caller-allocated outputs (o; den_out, S_out, z_out optional), with
    the library's static device workspace: nothing is allocated, here or in the library."""
    B, H, N, d = _check_seq(q, k, v, o)
    _check_state(S0, z0, B, H, d, q.device)
    _check_state(S_out, z_out, B, H, d, q.device)
    _check(load_library().la_forward_causal_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(S0), _ptr(z0),
                                                    _ptr(den_out), _ptr(S_out), _ptr(z_out), B, H, N, d, chunk,
                                                    _dtype_code(q.dtype), _stream(q.device)))
    return o


def la_backward_causal(q, k, v, dout, *, chunk=0, out=None, workspace=None, saved_state=None):
    """Gradients (dq, dk, dv) of sum(dout * la_forward_causal(q, k, v)).

    saved_state: the buffer a la_forward_causal call on the same q, k, v filled (optional)."""
    B, H, N, d = _check_seq(q, k, v, dout)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    else:
        dq, dk, dv = out
    ws = _workspace(LA_OP_BWD_CAUSAL, B, H, N, d, q.dtype, q.device, chunk, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load_library().la_backward_causal(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                             _ptr(saved_state), _nbytes(saved_state), B, H, N, d, chunk,
                                             _dtype_code(q.dtype), _ptr(ws), nbytes, _stream(q.device)))
    return dq, dk, dv


def la_backward_noncausal(q, k, v, dout, *, out=None, workspace=None, saved_state=None):
    """Gradients (dq, dk, dv) of sum(dout * la_forward_noncausal(q, k, v)).

    saved_state: the buffer a la_forward_noncausal call on the same q, k, v filled (optional)."""
    B, H, N, d = _check_seq(q, k, v, dout)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    else:
        dq, dk, dv = out
    ws = _workspace(LA_OP_BWD_NONCAUSAL, B, H, N, d, q.dtype, q.device, 0, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load_library().la_backward_noncausal(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk),
                                                _ptr(dv), _ptr(saved_state), _nbytes(saved_state), B, H, N, d,
                                                _dtype_code(q.dtype), _ptr(ws), nbytes, _stream(q.device)))
    return dq, dk, dv


def la_forward_causal_grouped(q, k, v, *, chunk=0, return_den=False, return_state=False, out=None, workspace=None,
                              S0=None, z0=None, S_out=None, z_out=None):
    """Causal forward with grouped key/value heads: q [B, H, N, d]; k, v [B, Hkv, N, d] with H a
    multiple of Hkv; start / final states [B, Hkv, d, d], [B, Hkv, d]."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, H, N, d] and k, v [B, Hkv, N, d]")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, N, d) or v.shape != k.shape or Hkv == 0 or H % Hkv:
        raise ValueError("k, v must be [B, Hkv, N, d] with H a multiple of Hkv")
    for t in (q, k, v):
        if t.dtype != q.dtype or t.device != q.device or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("q, k, v must be contiguous HIP tensors of one dtype")
    _check_state(S0, z0, B, Hkv, d, q.device)
    _check_state(S_out, z_out, B, Hkv, d, q.device)
    o = torch.empty_like(q) if out is None else out
    den = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if return_den else None
    S, z = S_out, z_out  # a state buffer the caller passes is always written
    if return_state:
        S = torch.empty((B, Hkv, d, d), dtype=torch.float32, device=q.device) if S_out is None else S_out
        z = torch.empty((B, Hkv, d), dtype=torch.float32, device=q.device) if z_out is None else z_out
    ws = _workspace(LA_OP_FWD_CAUSAL, B, H, N, d, q.dtype, q.device, chunk, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load_library().la_forward_causal_grouped(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(S0), _ptr(z0), _ptr(den),
                                                    _ptr(S), _ptr(z), B, H, Hkv, N, d, chunk, _dtype_code(q.dtype),
                                                    _ptr(ws), nbytes, _stream(q.device)))
    res = [o]
    if return_den:
        res.append(den)
    if return_state:
        res += [S, z]
    return res[0] if len(res) == 1 else tuple(res)


def la_backward_causal_state(q, k, v, dout, *, S0=None, z0=None, dS_out=None, dz_out=None, chunk=0, out=None,
                             workspace=None, want_state_grad=True):
    """Gradients of sum(dout * o) + sum(dS_out * S_N) + sum(dz_out * z_N) for
    la_forward_causal(q, k, v, S0=S0, z0=z0) with final state (S_N, z_N).

    Returns (dq, dk, dv, dS0, dz0); dS0 [B,H,d,d] and dz0 [B,H,d] (fp32) are the start state's
    gradients (None unless want_state_grad)."""
    B, H, N, d = _check_seq(q, k, v, dout)
    for a, b in ((S0, z0), (dS_out, dz_out)):
        _check_state(a, b, B, H, d, q.device)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    else:
        dq, dk, dv = out
    dS0 = torch.empty((B, H, d, d), dtype=torch.float32, device=q.device) if want_state_grad else None
    dz0 = torch.empty((B, H, d), dtype=torch.float32, device=q.device) if want_state_grad else None
    ws = _workspace(LA_OP_BWD_CAUSAL, B, H, N, d, q.dtype, q.device, chunk, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load_library().la_backward_causal_state(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(S0), _ptr(z0),
                                                   _ptr(dS_out), _ptr(dz_out), _ptr(dq), _ptr(dk), _ptr(dv),
                                                   _ptr(dS0), _ptr(dz0), B, H, N, d, chunk, _dtype_code(q.dtype),
                                                   _ptr(ws), nbytes, _stream(q.device)))
    return dq, dk, dv, dS0, dz0


def la_decode_step(S, z, q, k, v, *, out=None):
    """One in-place recurrent step: S += phi(k) v^T, z += phi(k); returns o = phi(q)^T S / phi(q)^T z.

    S: [B, H, d, d] fp32, z: [B, H, d] fp32, q/k/v: [B, H, d] bf16 or fp32 (contiguous, same device)."""
    if q.dim() != 3:
        raise ValueError("q, k, v must be [B, H, d]")
    B, H, d = q.shape
    for t in (k, v):
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device or not t.is_contiguous():
            raise ValueError("q, k, v must share shape, dtype and device and be contiguous")
    if S.shape != (B, H, d, d) or z.shape != (B, H, d) or S.dtype != torch.float32 or z.dtype != torch.float32:
        raise ValueError("S must be [B, H, d, d] fp32 and z [B, H, d] fp32")
    if not (S.is_contiguous() and z.is_contiguous() and q.is_contiguous()):
        raise ValueError("tensors must be contiguous")
    if not q.is_cuda:
        raise ValueError("tensors must be on a HIP device")
    o = torch.empty_like(q) if out is None else out
    _check(load_library().la_decode_step(_ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, d,
                                         _dtype_code(q.dtype), _stream(q.device)))
    return o


def la_decode_steps(S, z, q, k, v, *, out=None, _features=False):
    """T in-place recurrent steps per key/value head in one call; returns o [B, H, T, d].

    q: [B, H, T, d]; k, v: [B, Hkv, T, d] with H a multiple of Hkv (query head h reads the
    state of key/value head h // (H // Hkv)); S: [B, Hkv, d, d] fp32, z: [B, Hkv, d] fp32;
    bf16 or fp32 tokens (token t at row t)."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, H, T, d] and k, v [B, Hkv, T, d]")
    B, H, T, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, T, d) or v.shape != k.shape or Hkv == 0 or H % Hkv:
        raise ValueError("k, v must be [B, Hkv, T, d] with H a multiple of Hkv")
    for t in (q, k, v):
        if t.dtype != q.dtype or t.device != q.device or not t.is_contiguous():
            raise ValueError("q, k, v must share dtype and device and be contiguous")
    if not q.is_cuda:
        raise ValueError("tensors must be on a HIP device")
    if S.shape != (B, Hkv, d, d) or z.shape != (B, Hkv, d) or S.dtype != torch.float32 or z.dtype != torch.float32:
        raise ValueError("S must be [B, Hkv, d, d] fp32 and z [B, Hkv, d] fp32")
    if not (S.is_contiguous() and z.is_contiguous()):
        raise ValueError("S and z must be contiguous")
    o = torch.empty_like(q) if out is None else out
    fn = load_library().la_decode_steps_features if _features else load_library().la_decode_steps
    _check(fn(_ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, Hkv, T, d, _dtype_code(q.dtype),
              _stream(q.device)))
    return o


def la_decode_steps_features(S, z, fq, fk, v, *, out=None):
    """la_decode_steps on features applied beforehand (fq, fk: positive, e.g. from favor_features)."""
    return la_decode_steps(S, z, fq, fk, v, out=out, _features=True)


def favor_features(x, omega, *, out=None):
    """FAVOR+ features exp(omega x - |x|^2/2) of the rows of x [..., d] (bf16 or fp32); omega: [d, d] fp32.

    The page's constant 1/sqrt(m) (m = d) is left out: it cancels in every attention output."""
    d = x.shape[-1]
    if omega.shape != (d, d) or omega.dtype != torch.float32 or not omega.is_contiguous():
        raise ValueError("omega must be a contiguous [d, d] fp32 tensor")
    if not x.is_contiguous() or not x.is_cuda or omega.device != x.device:
        raise ValueError("x must be a contiguous tensor on the same HIP device as omega")
    o = torch.empty_like(x) if out is None else out
    rows = x.numel() // d if d else 0
    _check(load_library().la_favor_features(_ptr(x), _ptr(omega), _ptr(o), rows, d, _dtype_code(x.dtype),
                                            _stream(x.device)))
    return o


def favor_features_blocks(x, omega, *, out=None):
    """FAVOR+ features of x [B, H, N, d] for omega [m, d] fp32 (m a multiple of d), in block
    layout [B, H, m // d, N, d]: block j holds features j d .. j d + d - 1."""
    if x.dim() != 4:
        raise ValueError("x must be [B, H, N, d]")
    B, H, N, d = x.shape
    m = omega.shape[0]
    if omega.dim() != 2 or omega.shape[1] != d or omega.dtype != torch.float32 or not omega.is_contiguous():
        raise ValueError("omega must be a contiguous [m, d] fp32 tensor")
    if not x.is_contiguous() or not x.is_cuda or omega.device != x.device:
        raise ValueError("x must be a contiguous tensor on the same HIP device as omega")
    if m < d or m % d:
        raise ValueError("m must be a positive multiple of d")
    o = torch.empty((B, H, m // d, N, d), dtype=x.dtype, device=x.device) if out is None else out
    _check(load_library().la_favor_features_blocks(_ptr(x), _ptr(omega), _ptr(o), B * H, N, d, m,
                                                   _dtype_code(x.dtype), _stream(x.device)))
    return o


def features_workspace_size(causal, B, H, N, d, m, dtype):
    out = ctypes.c_size_t(0)
    kind = causal if causal in (2, 3, 4) else (1 if causal else 0)
    _check(load_library().la_features_workspace_size(kind, B, H, N, d, m, _dtype_code(dtype),
                                                     ctypes.byref(out)))
    return out.value


def _check_blocks(fq, fk, v):
    if fq.dim() != 5 or fk.shape != fq.shape or v.dim() != 4:
        raise ValueError("fq, fk must be [B, H, m // d, N, d] and v [B, H, N, d]")
    B, H, KF, N, d = fq.shape
    if v.shape != (B, H, N, d):
        raise ValueError("v must be [B, H, N, d] for features [B, H, m // d, N, d]")
    for t in (fq, fk, v):
        if t.dtype != fq.dtype or t.device != fq.device or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("fq, fk, v must be contiguous HIP tensors of one dtype")
    return B, H, N, d, KF * d


def la_forward_causal_features_blocks(fq, fk, v, *, return_den=False, return_state=False, out=None,
                                      workspace=None, S0=None, z0=None, S_out=None, z_out=None):
    """Causal forward on m = KF d features in block layout fq, fk [B, H, KF, N, d]; states [B, H, m, d], [B, H, m]."""
    B, H, N, d, m = _check_blocks(fq, fk, v)
    for S, z in ((S0, z0), (S_out, z_out)):
        if S is not None and (S.shape != (B, H, m, d) or S.dtype != torch.float32 or not S.is_contiguous()):
            raise ValueError("states must be contiguous [B, H, m, d] fp32")
        if z is not None and (z.shape != (B, H, m) or z.dtype != torch.float32 or not z.is_contiguous()):
            raise ValueError("states must be contiguous [B, H, m] fp32")
    o = torch.empty_like(v) if out is None else out
    den = torch.empty((B, H, N), dtype=torch.float32, device=fq.device) if return_den else None
    S, z = S_out, z_out  # a state buffer the caller passes is always written
    if return_state:
        S = torch.empty((B, H, m, d), dtype=torch.float32, device=fq.device) if S_out is None else S_out
        z = torch.empty((B, H, m), dtype=torch.float32, device=fq.device) if z_out is None else z_out
    need = features_workspace_size(True, B, H, N, d, m, fq.dtype)
    ws = workspace if workspace is not None else (torch.empty(need, dtype=torch.uint8, device=fq.device)
                                                  if need else None)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load_library().la_forward_causal_features_blocks(_ptr(fq), _ptr(fk), _ptr(v), _ptr(o), _ptr(S0), _ptr(z0),
                                                            _ptr(den), _ptr(S), _ptr(z), B, H, N, d, m,
                                                            _dtype_code(fq.dtype), _ptr(ws), nbytes,
                                                            _stream(fq.device)))
    res = [o]
    if return_den:
        res.append(den)
    if return_state:
        res += [S, z]
    return res[0] if len(res) == 1 else tuple(res)


def _backward_features_blocks(causal, fq, fk, v, dout, den, out, workspace, o=None):
    B, H, N, d, m = _check_blocks(fq, fk, v)
    if dout.shape != v.shape or dout.dtype != v.dtype or not dout.is_contiguous():
        raise ValueError("dout must match v")
    if den.shape != (B, H, N) or den.dtype != torch.float32 or not den.is_contiguous():
        raise ValueError("den must be the forward's contiguous [B, H, N] fp32 denominators")
    if o is not None and (o.shape != v.shape or o.dtype != v.dtype or not o.is_contiguous()):
        raise ValueError("o must be the forward's output, shaped like v")
    g = (torch.empty_like(fq), torch.empty_like(fk), torch.empty_like(v)) if out is None else out
    need = features_workspace_size(3 if causal else 4, B, H, N, d, m, fq.dtype)
    ws = workspace if workspace is not None else (torch.empty(need, dtype=torch.uint8, device=fq.device)
                                                  if need else None)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    fn = (load_library().la_backward_causal_features_blocks if causal
          else load_library().la_backward_noncausal_features_blocks)
    _check(fn(_ptr(fq), _ptr(fk), _ptr(v), _ptr(dout), _ptr(den), _ptr(o),
              _ptr(g[0]), _ptr(g[1]), _ptr(g[2]), B, H, N, d, m, _dtype_code(fq.dtype), _ptr(ws), nbytes,
              _stream(fq.device)))
    return g


def la_backward_causal_features_blocks(fq, fk, v, dout, den, *, o=None, out=None, workspace=None):
    """Causal backward on m = KF d features in block layout fq, fk [B, H, KF, N, d]; den [B, H, N] is the
    forward's den (return_den=True), o (optional) its output, which replaces the statistics sweep.
    Returns (dfq, dfk) in block layout and dv [B, H, N, d]."""
    return _backward_features_blocks(True, fq, fk, v, dout, den, out, workspace, o)


def la_backward_noncausal_features_blocks(fq, fk, v, dout, den, *, o=None, out=None, workspace=None):
    """Non-causal backward on m = KF d features in block layout (la_forward_noncausal_features_blocks);
    den [B, H, N] is that forward's den, o (optional) its output.  Returns (dfq, dfk) in block layout
    and dv [B, H, N, d]."""
    return _backward_features_blocks(False, fq, fk, v, dout, den, out, workspace, o)


def la_forward_noncausal_features_blocks(fq, fk, v, *, return_den=False, out=None, workspace=None, den_out=None):
    """Non-causal forward on m = KF d features in block layout fq, fk [B, H, KF, N, d]; den_out
    (optional, [B, H, N] fp32) receives the denominators."""
    B, H, N, d, m = _check_blocks(fq, fk, v)
    o = torch.empty_like(v) if out is None else out
    if den_out is not None and (den_out.shape != (B, H, N) or den_out.dtype != torch.float32
                                or not den_out.is_contiguous()):
        raise ValueError("den_out must be a contiguous [B, H, N] fp32 tensor")
    den = den_out if den_out is not None else (
        torch.empty((B, H, N), dtype=torch.float32, device=fq.device) if return_den else None)
    need = features_workspace_size(False, B, H, N, d, m, fq.dtype)
    ws = workspace if workspace is not None else (torch.empty(need, dtype=torch.uint8, device=fq.device)
                                                  if need else None)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load_library().la_forward_noncausal_features_blocks(_ptr(fq), _ptr(fk), _ptr(v), _ptr(o), _ptr(den), B, H,
                                                               N, d, m, _dtype_code(fq.dtype), _ptr(ws), nbytes,
                                                               _stream(fq.device)))
    return (o, den) if return_den else o


def la_decode_steps_features_blocks(S, z, fq, fk, v, *, out=None, workspace=None):
    """Multi-token decode on m = KF d features in block layout: fq [B, H, KF, T, d], fk [B, Hkv, KF, T, d],
    v [B, Hkv, T, d]; S [B, Hkv, m, d] and z [B, Hkv, m] fp32, updated in place.  Returns o [B, H, T, d]."""
    if fq.dim() != 5 or fk.dim() != 5 or v.dim() != 4:
        raise ValueError("fq, fk must be [B, H(kv), KF, T, d] and v [B, Hkv, T, d]")
    B, H, KF, T, d = fq.shape
    Hkv = fk.shape[1]
    m = KF * d
    if fk.shape != (B, Hkv, KF, T, d) or v.shape != (B, Hkv, T, d) or Hkv == 0 or H % Hkv:
        raise ValueError("fk must be [B, Hkv, KF, T, d], v [B, Hkv, T, d], with H a multiple of Hkv")
    if S.shape != (B, Hkv, m, d) or z.shape != (B, Hkv, m) or S.dtype != torch.float32 or z.dtype != torch.float32:
        raise ValueError("S must be [B, Hkv, m, d] and z [B, Hkv, m] fp32")
    for t in (fq, fk, v, S, z):
        if t.device != fq.device or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("all tensors must be contiguous on one HIP device")
    o = torch.empty((B, H, T, d), dtype=fq.dtype, device=fq.device) if out is None else out
    need = features_workspace_size(2, B, H, T, d, m, fq.dtype)
    ws = workspace if workspace is not None else (torch.empty(need, dtype=torch.uint8, device=fq.device)
                                                  if need else None)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load_library().la_decode_steps_features_blocks(_ptr(S), _ptr(z), _ptr(fq), _ptr(fk), _ptr(v), _ptr(o), B, H,
                                                          Hkv, T, d, m, _dtype_code(fq.dtype), _ptr(ws), nbytes,
                                                          _stream(fq.device)))
    return o


def la_backward_causal_features(fq, fk, v, dout, *, out=None, workspace=None, causal=True):
    """Gradients (dfq, dfk, dv) of sum(dout * O) for the forward on given features fq, fk [B, H, N, d]."""
    B, H, N, d = _check_seq(fq, fk, v)
    if dout.shape != v.shape or dout.dtype != v.dtype or not dout.is_contiguous():
        raise ValueError("dout must match v")
    g = tuple(torch.empty_like(t) for t in (fq, fk, v)) if out is None else out
    op = LA_OP_BWD_CAUSAL if causal else LA_OP_BWD_NONCAUSAL
    ws = _workspace(op, B, H, N, d, fq.dtype, fq.device, 0, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    fn = load_library().la_backward_causal_features if causal else load_library().la_backward_noncausal_features
    _check(fn(_ptr(fq), _ptr(fk), _ptr(v), _ptr(dout), _ptr(g[0]), _ptr(g[1]), _ptr(g[2]), B, H, N, d,
              _dtype_code(fq.dtype), _ptr(ws), nbytes, _stream(fq.device)))
    return g


def la_backward_noncausal_features(fq, fk, v, dout, *, out=None, workspace=None):
    return la_backward_causal_features(fq, fk, v, dout, out=out, workspace=workspace, causal=False)


def favor_features_backward(x, omega, F, dF, *, out=None):
    """dx = omega^T (dF * F) - x sum(dF * F) per row: the gradient through favor_features(x, omega) = F."""
    d = x.shape[-1]
    if omega.shape != (d, d) or omega.dtype != torch.float32 or not omega.is_contiguous():
        raise ValueError("omega must be a contiguous [d, d] fp32 tensor")
    for t in (x, F, dF):
        if t.shape != x.shape or t.dtype != x.dtype or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("x, F and dF must be contiguous HIP tensors of one shape and dtype")
    dx = torch.empty_like(x) if out is None else out
    rows = x.numel() // d if d else 0
    _check(load_library().la_favor_features_backward(_ptr(x), _ptr(omega), _ptr(F), _ptr(dF), _ptr(dx), rows, d,
                                                     _dtype_code(x.dtype), _stream(x.device)))
    return dx


def favor_features_blocks_backward(x, omega, F, dF, *, out=None):
    """The gradient through favor_features_blocks(x, omega) = F [B, H, KF, N, d]: x [B, H, N, d], omega [m, d]."""
    if x.dim() != 4 or F.dim() != 5:
        raise ValueError("x must be [B, H, N, d] and F [B, H, KF, N, d]")
    B, H, N, d = x.shape
    m = omega.shape[0]
    if omega.dim() != 2 or omega.shape[1] != d or omega.dtype != torch.float32 or not omega.is_contiguous():
        raise ValueError("omega must be a contiguous [m, d] fp32 tensor")
    if m < d or m % d or F.shape != (B, H, m // d, N, d) or dF.shape != F.shape:
        raise ValueError("F and dF must be [B, H, m // d, N, d]")
    for t in (x, F, dF):
        if t.dtype != x.dtype or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("x, F and dF must be contiguous HIP tensors of one dtype")
    dx = torch.empty_like(x) if out is None else out
    _check(load_library().la_favor_features_blocks_backward(_ptr(x), _ptr(omega), _ptr(F), _ptr(dF), _ptr(dx),
                                                            B * H, N, d, m, _dtype_code(x.dtype),
                                                            _stream(x.device)))
    return dx


class _FavorAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, omega, causal):
        if omega.shape[0] == q.shape[-1]:
            fq, fk = favor_features(q, omega), favor_features(k, omega)
            o = la_forward_causal_features(fq, fk, v) if causal else la_forward_noncausal_features(fq, fk, v)
            den = None
        else:  # m = KF d features in block layout
            fq, fk = favor_features_blocks(q, omega), favor_features_blocks(k, omega)
            fwd = la_forward_causal_features_blocks if causal else la_forward_noncausal_features_blocks
            o, den = fwd(fq, fk, v, return_den=True)
        ctx.save_for_backward(q, k, v, omega, fq, fk, den, o if den is not None else None)
        ctx.causal = causal
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, omega, fq, fk, den, o = ctx.saved_tensors
        if den is None:
            dfq, dfk, dv = la_backward_causal_features(fq, fk, v, do.contiguous(), causal=ctx.causal)
            return favor_features_backward(q, omega, fq, dfq), favor_features_backward(k, omega, fk, dfk), dv, None, None
        bwd = la_backward_causal_features_blocks if ctx.causal else la_backward_noncausal_features_blocks
        dfq, dfk, dv = bwd(fq, fk, v, do.contiguous(), den, o=o)
        return (favor_features_blocks_backward(q, omega, fq, dfq), favor_features_blocks_backward(k, omega, fk, dfk),
                dv, None, None)


def favor_attention(q, k, v, omega, causal=True):
    """Performer attention with FAVOR+ features as an autograd op: O of linear attention on the
    features of q and k for omega [m, d] (m a multiple of d; m > d runs in feature blocks);
    q, k pre-normalized by the caller.  Gradients flow to q, k and v through the library's kernels."""
    return _FavorAttention.apply(q, k, v, omega, causal)


def la_forward_causal_features(fq, fk, v, *, return_den=False, return_state=False, out=None, workspace=None,
                               S0=None, z0=None, S_out=None, z_out=None):
    """Causal forward on given positive features fq = phi(Q), fk = phi(K) [B, H, N, d]."""
    B, H, N, d = _check_seq(fq, fk, v)
    _check_state(S0, z0, B, H, d, fq.device)
    _check_state(S_out, z_out, B, H, d, fq.device)
    o = torch.empty_like(v) if out is None else out
    den = torch.empty((B, H, N), dtype=torch.float32, device=fq.device) if return_den else None
    S, z = S_out, z_out  # a state buffer the caller passes is always written
    if return_state:
        S = torch.empty((B, H, d, d), dtype=torch.float32, device=fq.device) if S_out is None else S_out
        z = torch.empty((B, H, d), dtype=torch.float32, device=fq.device) if z_out is None else z_out
    ws = _workspace(LA_OP_FWD_CAUSAL, B, H, N, d, fq.dtype, fq.device, 0, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load_library().la_forward_causal_features(_ptr(fq), _ptr(fk), _ptr(v), _ptr(o), _ptr(S0), _ptr(z0),
                                                     _ptr(den), _ptr(S), _ptr(z), B, H, N, d,
                                                     _dtype_code(fq.dtype), _ptr(ws), nbytes, _stream(fq.device)))
    res = [o]
    if return_den:
        res.append(den)
    if return_state:
        res += [S, z]
    return res[0] if len(res) == 1 else tuple(res)


def la_forward_noncausal_features(fq, fk, v, *, out=None, workspace=None):
    """Non-causal forward on given positive features fq = phi(Q), fk = phi(K) [B, H, N, d]."""
    B, H, N, d = _check_seq(fq, fk, v)
    o = torch.empty_like(v) if out is None else out
    ws = _workspace(LA_OP_FWD_NONCAUSAL, B, H, N, d, fq.dtype, fq.device, 0, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load_library().la_forward_noncausal_features(_ptr(fq), _ptr(fk), _ptr(v), _ptr(o), B, H, N, d,
                                                        _dtype_code(fq.dtype), _ptr(ws), nbytes,
                                                        _stream(fq.device)))
    return o


def wait_failures(op, workspace, q) -> int:
    """Workgroups whose wait gave up in the last launch of op (LA_OP_FWD_CAUSAL or LA_OP_BWD_CAUSAL) run
    on `workspace` for inputs shaped like q [B, H, N, d] (their rows are NaN); synchronises q's stream."""
    B, H, N, d = q.shape
    out = ctypes.c_int64(0)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().la_wait_failures(op, _ptr(workspace), nbytes, B, H, N, d, _dtype_code(q.dtype),
                                           _stream(q.device), ctypes.byref(out)))
    return int(out.value)


def backward_wait_failures(workspace, q) -> int:
    """wait_failures of the causal backward."""
    return wait_failures(LA_OP_BWD_CAUSAL, workspace, q)


def set_wait_limit(polls: int) -> None:
    """Bound on the polls of the fused backward's waits between workgroups (test hook; 0 = give up at once)."""
    _check(load_library().la_debug_set_wait_limit(int(polls)))


def wait_limit() -> int:
    return int(load_library().la_debug_wait_limit())


def profile_enable(on: bool = True) -> None:
    """Start (or stop) recording HIP events around every kernel this thread's calls launch."""
    _check(load_library().la_profile_enable(1 if on else 0))


def profile_entries():
    """[(kernel name, milliseconds)] for the launches recorded since profile_enable()."""
    lib = load_library()
    out = []
    name, ms = ctypes.c_char_p(), ctypes.c_float()
    for i in range(lib.la_profile_count()):
        _check(lib.la_profile_entry(i, ctypes.byref(name), ctypes.byref(ms)))
        out.append((name.value.decode(), float(ms.value)))
    return out


class _CausalLinearAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v):
        st = new_saved_state(q)
        o = la_forward_causal(q, k, v, saved_state=st)
        ctx.save_for_backward(q, k, v, st)
        return o

    @staticmethod
    def backward(ctx, dout):
        q, k, v, st = ctx.saved_tensors
        return la_backward_causal(q, k, v, dout.contiguous(), saved_state=st)


def causal_linear_attention(q, k, v):
    """Autograd-aware causal linear attention (forward and backward both run the HIP kernels)."""
    return _CausalLinearAttention.apply(q, k, v)


class _LinearAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v):
        st = new_saved_state(q)
        o = la_forward_noncausal(q, k, v, saved_state=st)
        ctx.save_for_backward(q, k, v, st)
        return o

    @staticmethod
    def backward(ctx, dout):
        q, k, v, st = ctx.saved_tensors
        return la_backward_noncausal(q, k, v, dout.contiguous(), saved_state=st)


def linear_attention(q, k, v):
    """Autograd-aware non-causal linear attention (forward and backward both run the HIP kernels)."""
    return _LinearAttention.apply(q, k, v)
