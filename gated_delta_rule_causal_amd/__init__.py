"""Python binding of liblinattn.so (causal linear attention and the gated
delta rule on MI355X / gfx950).

Argument marshalling only: tensors are allocated by PyTorch (device memory
and streams are all torch is used for) and passed to the C ABI as raw device
pointers together with the current HIP stream.  Every step of the computation
runs in the HIP kernels of liblinattn.so; there is no fallback of any kind.
If the library has not been built, importing the binding functions raises.

Layouts (row-major, contiguous): q, k [B,H,T,dk]; v, o [B,H,T,dv];
alpha, beta [B,H,T] float32 (KDA: alpha [B,H,T,dk]); S [B,H,dv,dk] float32;
z [B,H,dk] float32.
q, k, v are float32 or bfloat16 (all three the same).
"""

import ctypes
import os

__all__ = [
    "lin_attn_prefill",
    "gdn_prefill",
    "gdn_prefill_noalloc",
    "gla_prefill",
    "kda_prefill",
    "gdn_prefill_varlen",
    "lin_attn_prefill_varlen",
    "gdn_prefill_prep",
    "gdn_prefill_scan",
    "gdn_preprocess",
    "gdn_preprocess_varlen",
    "lin_attn_decode_step",
    "la_workspace_bytes",
    "la_status_str",
    "la_abi_version",
    "gdn_workspace",
    "library_path",
    "LinAttnError",
    "FORMS",
    "KINDS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liblinattn.so")

LA_F32, LA_BF16 = 0, 1
FORMS = {"chunked": 0, "recurrent": 1, "parallel": 2}
KINDS = {"normalized": 0, "gated_delta": 1, "gated": 2, "kda": 3}
FNS = {"lin_attn_prefill": 0, "gdn_prefill": 1, "decode_step": 2, "gla_prefill": 3, "kda_prefill": 4,
       "gdn_prefill_varlen": 5, "prefill_varlen": 6}

_lib = None


class LinAttnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {la_status_str(status)} (status {status})")


def library_path():
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build the HIP library first "
            "(python -m gated_delta_rule_causal_amd.build)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.lin_attn_prefill.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, I, I, P, Z, P]
    lib.lin_attn_prefill.restype = I
    lib.gdn_prefill.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, I, I, P, Z, P]
    lib.gdn_prefill.restype = I
    lib.gdn_prefill_noalloc.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, I, I, P]
    lib.gdn_prefill_noalloc.restype = I
    lib.gla_prefill.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, I, I, P, Z, P]
    lib.gla_prefill.restype = I
    lib.kda_prefill.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, I, I, P, Z, P]
    lib.kda_prefill.restype = I
    lib.gdn_prefill_varlen.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, I, I, P, I, I, P, Z, P]
    lib.gdn_prefill_varlen.restype = I
    lib.lin_attn_prefill_varlen.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, I, I, P, P, I, I,
                                            P, Z, P]
    lib.lin_attn_prefill_varlen.restype = I
    lib.gdn_preprocess.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, P]
    lib.gdn_preprocess.restype = I
    lib.gdn_preprocess_varlen.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, P, P]
    lib.gdn_preprocess_varlen.restype = I
    lib.gdn_prefill_prep.argtypes = [I, I, I, I, I, I, P, P, P, P, P, I, P, Z, P]
    lib.gdn_prefill_prep.restype = I
    lib.gdn_prefill_scan.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, I, P, Z, P]
    lib.gdn_prefill_scan.restype = I
    lib.lin_attn_decode_step.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P]
    lib.lin_attn_decode_step.restype = I
    lib.la_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I, I]
    lib.la_workspace_bytes.restype = Z
    lib.la_status_str.argtypes = [I]
    lib.la_status_str.restype = ctypes.c_char_p
    lib.la_abi_version.argtypes = []
    lib.la_abi_version.restype = I
    _lib = lib
    return lib


def la_status_str(status):
    return _load().la_status_str(int(status)).decode()


def la_abi_version():
    return int(_load().la_abi_version())


def la_workspace_bytes(fn, dtype, B, H, T, dk, dv, form="chunked", chunk=64):
    fn_i = FNS[fn] if isinstance(fn, str) else int(fn)
    form_i = FORMS[form] if isinstance(form, str) else int(form)
    dt = _dtype_code(dtype) if not isinstance(dtype, int) else dtype
    n = _load().la_workspace_bytes(fn_i, dt, B, H, T, dk, dv, form_i, chunk)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("la_workspace_bytes: invalid or unsupported arguments")
    return int(n)


# ---------------------------------------------------------------- helpers
def _torch():
    import torch
    return torch


def _dtype_code(dt):
    torch = _torch()
    if dt == torch.float32 or dt == "f32":
        return LA_F32
    if dt == torch.bfloat16 or dt == "bf16":
        return LA_BF16
    raise TypeError(f"unsupported activation dtype {dt}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_ptr(stream, device):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _check(t, name, dtype=None, shape=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _workspace(fn, dt, B, H, T, dk, dv, form, chunk, workspace, device):
    torch = _torch()
    need = la_workspace_bytes(fn, dt, B, H, T, dk, dv, form, chunk)
    if need == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


# ------------------------------------------------------------ entry points
def lin_attn_prefill(q, k, v, S0=None, z0=None, form="chunked", chunk=64, out=None,
                     S_out=None, z_out=None, want_state=True, workspace=None, stream=None):
    """Normalised causal linear attention; returns (o, S_out, z_out).

    ``S_out``/``z_out`` may be passed explicitly (``S_out is S0`` updates in
    place); otherwise they are allocated when ``want_state``.
    """
    torch = _torch()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q.dtype)
    _check(q, "q", q.dtype)
    _check(k, "k", q.dtype, (B, H, T, dk))
    _check(v, "v", q.dtype, (B, H, T, dv))
    _check(S0, "S0", torch.float32, (B, H, dv, dk))
    _check(z0, "z0", torch.float32, (B, H, dk))
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    _check(out, "out", q.dtype, (B, H, T, dv))
    if want_state and S_out is None:
        S_out = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    if want_state and z_out is None:
        z_out = torch.empty((B, H, dk), dtype=torch.float32, device=q.device)
    _check(S_out, "S_out", torch.float32, (B, H, dv, dk))
    _check(z_out, "z_out", torch.float32, (B, H, dk))
    ws, ws_bytes = _workspace("lin_attn_prefill", dt, B, H, T, dk, dv, form, chunk, workspace, q.device)
    st = _load().lin_attn_prefill(dt, B, H, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(S0), _ptr(z0),
                                  _ptr(out), _ptr(S_out), _ptr(z_out), FORMS[form], chunk, _ptr(ws),
                                  ws_bytes, _stream_ptr(stream, q.device))
    if st != 0:
        raise LinAttnError(st, "lin_attn_prefill")
    return out, S_out, z_out


def gdn_prefill(q, k, v, alpha, beta, S0=None, form="chunked", chunk=64, out=None, S_out=None,
                want_state=True, workspace=None, stream=None):
    """Gated delta rule over T tokens; returns (o, S_out)."""
    torch = _torch()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q.dtype)
    _check(q, "q", q.dtype)
    _check(k, "k", q.dtype, (B, H, T, dk))
    _check(v, "v", q.dtype, (B, H, T, dv))
    _check(alpha, "alpha", torch.float32, (B, H, T))
    _check(beta, "beta", torch.float32, (B, H, T))
    _check(S0, "S0", torch.float32, (B, H, dv, dk))
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    _check(out, "out", q.dtype, (B, H, T, dv))
    if want_state and S_out is None:
        S_out = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    _check(S_out, "S_out", torch.float32, (B, H, dv, dk))
    ws, ws_bytes = _workspace("gdn_prefill", dt, B, H, T, dk, dv, form, chunk, workspace, q.device)
    st = _load().gdn_prefill(dt, B, H, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                             _ptr(S0), _ptr(out), _ptr(S_out), FORMS[form], chunk, _ptr(ws), ws_bytes,
                             _stream_ptr(stream, q.device))
    if st != 0:
        raise LinAttnError(st, "gdn_prefill")
    return out, S_out


def gdn_prefill_noalloc(q, k, v, alpha, beta, S0=None, form="chunked", chunk=64, out=None, S_out=None,
                        want_state=True, stream=None):
    """gdn_prefill with the library's own workspace (the C entry point takes
    no workspace and allocates nothing; pass `out` and `S_out` to keep this
    call free of allocations too).  Returns (o, S_out)."""
    torch = _torch()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q.dtype)
    _check(q, "q", q.dtype)
    _check(k, "k", q.dtype, (B, H, T, dk))
    _check(v, "v", q.dtype, (B, H, T, dv))
    _check(alpha, "alpha", torch.float32, (B, H, T))
    _check(beta, "beta", torch.float32, (B, H, T))
    _check(S0, "S0", torch.float32, (B, H, dv, dk))
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    _check(out, "out", q.dtype, (B, H, T, dv))
    if want_state and S_out is None:
        S_out = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    _check(S_out, "S_out", torch.float32, (B, H, dv, dk))
    st = _load().gdn_prefill_noalloc(dt, B, H, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                     _ptr(S0), _ptr(out), _ptr(S_out), FORMS[form], chunk,
                                     _stream_ptr(stream, q.device))
    if st != 0:
        raise LinAttnError(st, "gdn_prefill_noalloc")
    return out, S_out


def gla_prefill(q, k, v, alpha, S0=None, form="chunked", chunk=64, out=None, S_out=None, want_state=True,
                workspace=None, stream=None):
    """Scalar-gated unnormalised linear attention over T tokens; returns (o, S_out)."""
    torch = _torch()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q.dtype)
    _check(q, "q", q.dtype)
    _check(k, "k", q.dtype, (B, H, T, dk))
    _check(v, "v", q.dtype, (B, H, T, dv))
    _check(alpha, "alpha", torch.float32, (B, H, T))
    _check(S0, "S0", torch.float32, (B, H, dv, dk))
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    _check(out, "out", q.dtype, (B, H, T, dv))
    if want_state and S_out is None:
        S_out = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    _check(S_out, "S_out", torch.float32, (B, H, dv, dk))
    ws, ws_bytes = _workspace("gla_prefill", dt, B, H, T, dk, dv, form, chunk, workspace, q.device)
    st = _load().gla_prefill(dt, B, H, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(S0), _ptr(out),
                             _ptr(S_out), FORMS[form], chunk, _ptr(ws), ws_bytes, _stream_ptr(stream, q.device))
    if st != 0:
        raise LinAttnError(st, "gla_prefill")
    return out, S_out


def gdn_prefill_varlen(q, k, v, alpha, beta, cu_seqlens, S0=None, form="chunked", chunk=64, snap_interval=0,
                       snap_count=None, out=None, S_out=None, S_snap=None, want_state=True, workspace=None,
                       stream=None):
    """Gated delta rule over a packed batch; returns (o, S_out, S_snap).

    q, k [H,T_total,dk]; v [H,T_total,dv]; alpha, beta [H,T_total] float32;
    cu_seqlens [N+1] int32 on the device; S0 [N,H,dv,dk] or None.  With
    snap_interval > 0 the states after every snap_interval tokens of each
    sequence are returned in S_snap [snap_count,H,dv,dk]; when snap_count is
    None it is counted from a host copy of cu_seqlens (a synchronisation).
    """
    torch = _torch()
    H, T, dk = q.shape
    dv = v.shape[-1]
    N = cu_seqlens.numel() - 1
    dt = _dtype_code(q.dtype)
    _check(q, "q", q.dtype)
    _check(k, "k", q.dtype, (H, T, dk))
    _check(v, "v", q.dtype, (H, T, dv))
    _check(alpha, "alpha", torch.float32, (H, T))
    _check(beta, "beta", torch.float32, (H, T))
    _check(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,))
    _check(S0, "S0", torch.float32, (N, H, dv, dk))
    if out is None:
        out = torch.empty((H, T, dv), dtype=q.dtype, device=q.device)
    _check(out, "out", q.dtype, (H, T, dv))
    if want_state and S_out is None:
        S_out = torch.empty((N, H, dv, dk), dtype=torch.float32, device=q.device)
    _check(S_out, "S_out", torch.float32, (N, H, dv, dk))
    if snap_interval > 0:
        if snap_count is None:
            lens = (cu_seqlens[1:] - cu_seqlens[:-1]).cpu()
            snap_count = int((lens // snap_interval).sum()) if N > 0 else 0
        if S_snap is None:
            S_snap = torch.empty((max(snap_count, 1), H, dv, dk), dtype=torch.float32, device=q.device)
        _check(S_snap, "S_snap", torch.float32)
    else:
        snap_count, S_snap = 0, None
    ws, ws_bytes = _workspace("gdn_prefill_varlen", dt, N, H, T, dk, dv, form, chunk, workspace, q.device)
    st = _load().gdn_prefill_varlen(dt, N, H, T, dk, dv, _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                    _ptr(beta), _ptr(S0), _ptr(out), _ptr(S_out), snap_interval, snap_count,
                                    _ptr(S_snap), FORMS[form], chunk, _ptr(ws), ws_bytes,
                                    _stream_ptr(stream, q.device))
    if st != 0:
        raise LinAttnError(st, "gdn_prefill_varlen")
    return out, S_out, (S_snap[:snap_count] if S_snap is not None else None)


def lin_attn_prefill_varlen(kind, q, k, v, cu_seqlens, alpha=None, beta=None, S0=None, z0=None, form="recurrent",
                            chunk=64, snap_interval=0, snap_count=None, out=None, S_out=None, z_out=None, S_snap=None,
                            z_snap=None, want_state=True, workspace=None, stream=None):
    """Any kind of recurrence over a packed batch; returns (o, S_out, z_out,
    S_snap, z_snap), the z entries None except for the normalised kind.

    kind: "normalized", "gated", "kda" or "gated_delta".  q, k [H,T_total,dk];
    v [H,T_total,dv]; alpha [H,T_total] float32 ("gated", "gated_delta") or
    [H,T_total,dk] ("kda"); beta [H,T_total] float32 ("kda", "gated_delta");
    cu_seqlens [N+1] int32 on the device; S0 [N,H,dv,dk], z0 [N,H,dk]
    ("normalized") or None.  With snap_interval > 0 the states after every
    snap_interval tokens of each sequence are returned in S_snap
    [snap_count,H,dv,dk] (and z_snap [snap_count,H,dk]); when snap_count is
    None it is counted from a host copy of cu_seqlens (a synchronisation).
    """
    torch = _torch()
    kind_i = KINDS[kind]
    has_z = kind == "normalized"
    H, T, dk = q.shape
    dv = v.shape[-1]
    N = cu_seqlens.numel() - 1
    dt = _dtype_code(q.dtype)
    _check(q, "q", q.dtype)
    _check(k, "k", q.dtype, (H, T, dk))
    _check(v, "v", q.dtype, (H, T, dv))
    _check(alpha, "alpha", torch.float32, (H, T, dk) if kind == "kda" else (H, T))
    _check(beta, "beta", torch.float32, (H, T))
    _check(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,))
    _check(S0, "S0", torch.float32, (N, H, dv, dk))
    _check(z0, "z0", torch.float32, (N, H, dk))
    if out is None:
        out = torch.empty((H, T, dv), dtype=q.dtype, device=q.device)
    _check(out, "out", q.dtype, (H, T, dv))
    if want_state and S_out is None:
        S_out = torch.empty((N, H, dv, dk), dtype=torch.float32, device=q.device)
    if want_state and has_z and z_out is None:
        z_out = torch.empty((N, H, dk), dtype=torch.float32, device=q.device)
    _check(S_out, "S_out", torch.float32, (N, H, dv, dk))
    _check(z_out, "z_out", torch.float32, (N, H, dk))
    if snap_interval > 0:
        if snap_count is None:
            lens = (cu_seqlens[1:] - cu_seqlens[:-1]).cpu()
            snap_count = int((lens // snap_interval).sum()) if N > 0 else 0
        if S_snap is None:
            S_snap = torch.empty((max(snap_count, 1), H, dv, dk), dtype=torch.float32, device=q.device)
        if has_z and z_snap is None:
            z_snap = torch.empty((max(snap_count, 1), H, dk), dtype=torch.float32, device=q.device)
        _check(S_snap, "S_snap", torch.float32)
        _check(z_snap, "z_snap", torch.float32)
    else:
        snap_count, S_snap, z_snap = 0, None, None
    ws, ws_bytes = _workspace("prefill_varlen", dt, N, H, T, dk, dv, form, chunk, workspace, q.device)
    st = _load().lin_attn_prefill_varlen(kind_i, dt, N, H, T, dk, dv, _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(alpha), _ptr(beta), _ptr(S0), _ptr(z0), _ptr(out), _ptr(S_out),
                                         _ptr(z_out), snap_interval, snap_count, _ptr(S_snap), _ptr(z_snap),
                                         FORMS[form], chunk, _ptr(ws), ws_bytes, _stream_ptr(stream, q.device))
    if st != 0:
        raise LinAttnError(st, "lin_attn_prefill_varlen")
    cut = (lambda t: t[:snap_count] if t is not None else None)
    return out, S_out, z_out, cut(S_snap), cut(z_snap)


def gdn_preprocess_varlen(x, conv_w, a_logit, b_logit, H, dk, dv, cu_seqlens, conv_state=None, want_state=True,
                          stream=None):
    """Fused pre-operations over a packed batch; returns (q, k, v, alpha, beta,
    conv_state_out).

    x [T_total, H*(2dk+dv)]; a_logit, b_logit [T_total, H] float32;
    cu_seqlens [N+1] int32 on the device; conv_state [N, 3, C] or None.
    Outputs q, k [H, T_total, dk], v [H, T_total, dv], alpha, beta
    [H, T_total] (the layout of gdn_prefill_varlen) and the next states.
    """
    torch = _torch()
    T, C = x.shape
    N = cu_seqlens.numel() - 1
    if C != H * (2 * dk + dv):
        raise ValueError(f"x has {C} channels, expected H*(2dk+dv) = {H * (2 * dk + dv)}")
    dt = _dtype_code(x.dtype)
    _check(x, "x", x.dtype)
    _check(conv_w, "conv_w", torch.float32, (C, 4))
    _check(a_logit, "a_logit", torch.float32, (T, H))
    _check(b_logit, "b_logit", torch.float32, (T, H))
    _check(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,))
    _check(conv_state, "conv_state", x.dtype, (N, 3, C))
    dev = x.device
    q = torch.empty((H, T, dk), dtype=x.dtype, device=dev)
    k = torch.empty((H, T, dk), dtype=x.dtype, device=dev)
    v = torch.empty((H, T, dv), dtype=x.dtype, device=dev)
    alpha = torch.empty((H, T), dtype=torch.float32, device=dev)
    beta = torch.empty((H, T), dtype=torch.float32, device=dev)
    st_out = torch.empty((N, 3, C), dtype=x.dtype, device=dev) if want_state else None
    st = _load().gdn_preprocess_varlen(dt, N, T, H, dk, dv, _ptr(cu_seqlens), _ptr(x), _ptr(conv_w), _ptr(a_logit),
                                       _ptr(b_logit), _ptr(conv_state), _ptr(st_out), _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(alpha), _ptr(beta), _stream_ptr(stream, dev))
    if st != 0:
        raise LinAttnError(st, "gdn_preprocess_varlen")
    return q, k, v, alpha, beta, st_out


def kda_prefill(q, k, v, alpha, beta, S0=None, form="recurrent", chunk=64, out=None, S_out=None, want_state=True,
                workspace=None, stream=None):
    """Kimi Delta Attention (per-channel decay alpha [B,H,T,dk]) over T tokens;
    returns (o, S_out)."""
    torch = _torch()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q.dtype)
    _check(q, "q", q.dtype)
    _check(k, "k", q.dtype, (B, H, T, dk))
    _check(v, "v", q.dtype, (B, H, T, dv))
    _check(alpha, "alpha", torch.float32, (B, H, T, dk))
    _check(beta, "beta", torch.float32, (B, H, T))
    _check(S0, "S0", torch.float32, (B, H, dv, dk))
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    _check(out, "out", q.dtype, (B, H, T, dv))
    if want_state and S_out is None:
        S_out = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    _check(S_out, "S_out", torch.float32, (B, H, dv, dk))
    ws, ws_bytes = _workspace("kda_prefill", dt, B, H, T, dk, dv, form, chunk, workspace, q.device)
    st = _load().kda_prefill(dt, B, H, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S0),
                             _ptr(out), _ptr(S_out), FORMS[form], chunk, _ptr(ws), ws_bytes,
                             _stream_ptr(stream, q.device))
    if st != 0:
        raise LinAttnError(st, "kda_prefill")
    return out, S_out


def gdn_preprocess(x, conv_w, a_logit, b_logit, H, dk, dv, conv_state=None, want_state=True, q=None, k=None, v=None,
                   alpha=None, beta=None, conv_state_out=None, stream=None):
    """Fused pre-operations of a Gated DeltaNet layer; returns
    (q, k, v, alpha, beta, conv_state_out).

    x [B,T,H*(2dk+dv)] (float32 or bfloat16, channels q | k | v); conv_w
    [H*(2dk+dv), 4] float32; a_logit, b_logit [B,T,H] float32; conv_state
    [B,3,H*(2dk+dv)] in x's dtype or None.  Outputs q, k [B,H,T,dk] (convolved,
    L2-normalised), v [B,H,T,dv] (convolved), alpha, beta [B,H,T] float32
    (sigmoids), and the next conv state when ``want_state``.
    """
    torch = _torch()
    B, T, C = x.shape
    if C != H * (2 * dk + dv):
        raise ValueError(f"x has {C} channels, expected H*(2dk+dv) = {H * (2 * dk + dv)}")
    dt = _dtype_code(x.dtype)
    _check(x, "x", x.dtype)
    _check(conv_w, "conv_w", torch.float32, (C, 4))
    _check(a_logit, "a_logit", torch.float32, (B, T, H))
    _check(b_logit, "b_logit", torch.float32, (B, T, H))
    _check(conv_state, "conv_state", x.dtype, (B, 3, C))
    dev = x.device
    q = torch.empty((B, H, T, dk), dtype=x.dtype, device=dev) if q is None else q
    k = torch.empty((B, H, T, dk), dtype=x.dtype, device=dev) if k is None else k
    v = torch.empty((B, H, T, dv), dtype=x.dtype, device=dev) if v is None else v
    alpha = torch.empty((B, H, T), dtype=torch.float32, device=dev) if alpha is None else alpha
    beta = torch.empty((B, H, T), dtype=torch.float32, device=dev) if beta is None else beta
    if want_state and conv_state_out is None:
        conv_state_out = torch.empty((B, 3, C), dtype=x.dtype, device=dev)
    for t, n, d, shp in ((q, "q", x.dtype, (B, H, T, dk)), (k, "k", x.dtype, (B, H, T, dk)),
                         (v, "v", x.dtype, (B, H, T, dv)), (alpha, "alpha", torch.float32, (B, H, T)),
                         (beta, "beta", torch.float32, (B, H, T)),
                         (conv_state_out, "conv_state_out", x.dtype, (B, 3, C))):
        _check(t, n, d, shp)
    st = _load().gdn_preprocess(dt, B, T, H, dk, dv, _ptr(x), _ptr(conv_w), _ptr(a_logit), _ptr(b_logit),
                                _ptr(conv_state), _ptr(conv_state_out), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                _ptr(beta), _stream_ptr(stream, dev))
    if st != 0:
        raise LinAttnError(st, "gdn_preprocess")
    return q, k, v, alpha, beta, conv_state_out


def gdn_workspace(q, v, chunk=64):
    """Allocate the workspace gdn_prefill_prep/gdn_prefill_scan need for q, v."""
    torch = _torch()
    B, H, T, dk = q.shape
    n = la_workspace_bytes("gdn_prefill", _dtype_code(q.dtype), B, H, T, dk, v.shape[-1], "chunked", chunk)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=q.device)


def gdn_prefill_prep(q, k, v, alpha, beta, workspace, chunk=64, stream=None):
    """State-independent half of the chunked gated-delta path (segment maps)."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q.dtype)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (alpha, "alpha"), (beta, "beta"), (workspace, "workspace")):
        _check(t, n)
    st = _load().gdn_prefill_prep(dt, B, H, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), chunk,
                                  _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _stream_ptr(stream, q.device))
    if st != 0:
        raise LinAttnError(st, "gdn_prefill_prep")


def gdn_prefill_scan(q, k, v, alpha, beta, workspace, S0=None, out=None, S_out=None, chunk=64, stream=None):
    """Entering states of the segments, then outputs and final state; returns (o, S_out)."""
    torch = _torch()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q.dtype)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (alpha, "alpha"), (beta, "beta"), (workspace, "workspace")):
        _check(t, n)
    _check(S0, "S0", torch.float32, (B, H, dv, dk))
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    if S_out is None:
        S_out = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    _check(out, "out", q.dtype, (B, H, T, dv))
    _check(S_out, "S_out", torch.float32, (B, H, dv, dk))
    st = _load().gdn_prefill_scan(dt, B, H, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                  _ptr(S0), _ptr(out), _ptr(S_out), chunk, _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream_ptr(stream, q.device))
    if st != 0:
        raise LinAttnError(st, "gdn_prefill_scan")
    return out, S_out


def lin_attn_decode_step(kind, q, k, v, S, z=None, alpha=None, beta=None, out=None, stream=None):
    """One decode step for [N,H] heads, updating S (and z) in place; returns o."""
    torch = _torch()
    N, H, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q.dtype)
    kind_i = KINDS[kind] if isinstance(kind, str) else int(kind)
    _check(q, "q", q.dtype)
    _check(k, "k", q.dtype, (N, H, dk))
    _check(v, "v", q.dtype, (N, H, dv))
    _check(S, "S", torch.float32, (N, H, dv, dk))
    _check(z, "z", torch.float32, (N, H, dk))
    _check(alpha, "alpha", torch.float32, (N, H, dk) if kind_i == KINDS["kda"] else (N, H))
    _check(beta, "beta", torch.float32, (N, H))
    if out is None:
        out = torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    _check(out, "out", q.dtype, (N, H, dv))
    st = _load().lin_attn_decode_step(kind_i, dt, N, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                      _ptr(beta), _ptr(S), _ptr(z), _ptr(out),
                                      _stream_ptr(stream, q.device))
    if st != 0:
        raise LinAttnError(st, "lin_attn_decode_step")
    return out
