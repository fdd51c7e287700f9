"""ctypes binding of libkla.so (C ABI in include/kla.h).

Argument marshalling only: shapes are read from the torch tensors, outputs
are allocated with torch when not given, and every step of the computation
runs in the library's HIP kernels on torch's current stream.  There is no
fallback: a missing library raises ImportError here.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libkla.so")
if not os.path.exists(lib_path):
    raise ImportError(f"{lib_path} is missing: build it with `python -m delta_rule_linear_amd.build`")
_lib = ctypes.CDLL(lib_path)

KLA_OK, KLA_ERR_INVALID_ARG, KLA_ERR_UNSUPPORTED, KLA_ERR_WORKSPACE, KLA_ERR_HIP = 0, -1, -2, -3, -4
KLA_F32, KLA_BF16 = 0, 1
KLA_BETA_KACZMARZ, KLA_BETA_DIRECT = 0, 1
_BETA_MODES = {"kaczmarz": KLA_BETA_KACZMARZ, "direct": KLA_BETA_DIRECT}

_vp, _fp, _i32p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
_lib.kla_fwd_chunked_workspace_size.restype = ctypes.c_size_t
_lib.kla_fwd_chunked_workspace_size.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
_lib.kla_fwd_chunked.restype = ctypes.c_int
_lib.kla_fwd_chunked.argtypes = [_vp, _vp, _vp, _fp, _fp, _i32p, ctypes.c_int32, ctypes.c_int64,
                                 ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.c_float, ctypes.c_int, _fp, _fp, _fp, _vp, ctypes.c_size_t,
                                 _vp]
_lib.kla_fwd_chunked_ex.restype = ctypes.c_int
_lib.kla_fwd_chunked_ex.argtypes = (_lib.kla_fwd_chunked.argtypes[:14] + [ctypes.c_int]
                                    + _lib.kla_fwd_chunked.argtypes[14:])
_lib.kla_fwd_chunked_split_workspace_size.restype = ctypes.c_size_t
_lib.kla_fwd_chunked_split_workspace_size.argtypes = [ctypes.c_int32] * 5
_lib.kla_fwd_chunked_split.restype = ctypes.c_int
_lib.kla_fwd_chunked_split.argtypes = (_lib.kla_fwd_chunked.argtypes[:14] + [ctypes.c_int, ctypes.c_int32]
                                       + _lib.kla_fwd_chunked.argtypes[14:])
_lib.kla_fwd_chunked_split_noalloc.restype = ctypes.c_int
_lib.kla_fwd_chunked_split_noalloc.argtypes = (_lib.kla_fwd_chunked.argtypes[:14]
                                               + [ctypes.c_int, ctypes.c_int32, _fp, _fp, _fp, _vp])
_lib.kla_decode_step.restype = ctypes.c_int
_lib.kla_decode_step.argtypes = [_vp, _vp, _vp, _fp, _fp, _fp, _fp, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_int, _vp]
_lib.kla_decode_step_ex.restype = ctypes.c_int
_lib.kla_decode_step_ex.argtypes = _lib.kla_decode_step.argtypes[:13] + [ctypes.c_int, _vp]
_lib.kla_fwd_chunked_kda.restype = ctypes.c_int
_lib.kla_fwd_chunked_kda.argtypes = _lib.kla_fwd_chunked_ex.argtypes
_lib.kla_decode_step_kda.restype = ctypes.c_int
_lib.kla_decode_step_kda.argtypes = _lib.kla_decode_step_ex.argtypes
_lib.kla_status_string.restype = ctypes.c_char_p
_lib.kla_status_string.argtypes = [ctypes.c_int]
_lib.kla_version.restype = ctypes.c_char_p
_lib.kla_version.argtypes = []


class KLAError(RuntimeError):
    def __init__(self, status):
        self.status = status
        super().__init__(f"libkla: {kla_status_string(status)} ({status})")


def kla_status_string(status: int) -> str:
    return _lib.kla_status_string(int(status)).decode()


def kla_version() -> str:
    return _lib.kla_version().decode()


def kla_fwd_chunked_workspace_size(n_seqs, total_tok, H, dk, dv, chunk=64) -> int:
    return int(_lib.kla_fwd_chunked_workspace_size(n_seqs, total_tok, H, dk, dv, chunk))


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return KLA_BF16
    if t.dtype == torch.float32:
        return KLA_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t, name, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _beta_code(beta_mode):
    try:
        return _BETA_MODES[beta_mode]
    except KeyError:
        raise ValueError(f"beta_mode must be one of {sorted(_BETA_MODES)}, got {beta_mode!r}")


def kla_fwd_chunked(q, k, v, alpha, eta, cu_seqlens=None, initial_state=None, eps=1e-6, chunk=64,
                    output_final_state=False, o=None, final_state=None, workspace=None,
                    stream=None):
    """Chunked KLA prefill (C ABI `kla_fwd_chunked`).

    q, k: [tok, H, dk] (packed, with cu_seqlens int32 [n+1]) or [B, T, H, dk]
    (dense); v likewise with dv.  alpha, eta: [tok, H] or [B, T, H] fp32;
    alpha may be None (no decay).
    Returns (o fp32 shaped like v, final_state [n, H, dk, dv] fp32 or None).
    """
    return _fwd(None, q, k, v, alpha, eta, cu_seqlens, initial_state, eps, chunk,
                output_final_state, o, final_state, workspace, stream)


def kla_fwd_chunked_ex(q, k, v, alpha, eta, cu_seqlens=None, initial_state=None, eps=1e-6,
                       chunk=64, beta_mode="kaczmarz", output_final_state=False, o=None,
                       final_state=None, workspace=None, stream=None):
    """kla_fwd_chunked with the step-size rule chosen by beta_mode (C ABI
    `kla_fwd_chunked_ex`): "kaczmarz" (beta = eta / (|k|^2 + eps)) or
    "direct" (beta = eta, Gated DeltaNet; DeltaNet with alpha None)."""
    return _fwd(_beta_code(beta_mode), q, k, v, alpha, eta, cu_seqlens, initial_state, eps, chunk,
                output_final_state, o, final_state, workspace, stream)


def kla_fwd_chunked_split_workspace_size(n_seqs, H, dk, dv, n_splits) -> int:
    return int(_lib.kla_fwd_chunked_split_workspace_size(n_seqs, H, dk, dv, n_splits))


def kla_fwd_chunked_split(q, k, v, alpha, eta, cu_seqlens=None, initial_state=None, eps=1e-6,
                          chunk=64, beta_mode="kaczmarz", n_splits=2, output_final_state=False,
                          o=None, final_state=None, workspace=None, stream=None):
    """kla_fwd_chunked_ex with every sequence cut into n_splits segments
    (C ABI `kla_fwd_chunked_split`): segment maps, a scan of the maps, then
    all segments at once.  The workspace is allocated with torch when not
    given."""
    return _fwd(_beta_code(beta_mode), q, k, v, alpha, eta, cu_seqlens, initial_state, eps, chunk,
                output_final_state, o, final_state, workspace, stream, n_splits=int(n_splits))


def kla_fwd_chunked_split_noalloc(q, k, v, alpha, eta, cu_seqlens=None, initial_state=None,
                                  eps=1e-6, chunk=64, beta_mode="kaczmarz", n_splits=2, o=None,
                                  final_state=None, stream=None):
    """kla_fwd_chunked_split without a workspace (C ABI
    `kla_fwd_chunked_split_noalloc`): the library keeps the segment maps and
    start states in its static device scratch array (at most
    KLA_NOALLOC_SCRATCH_BYTES = 32 MiB per GPU; calls that overlap in time on
    one GPU race on it).  o and final_state must be given (nothing is
    allocated here either)."""
    if o is None:
        raise ValueError("o must be given: this entry point allocates nothing")
    return _fwd(_beta_code(beta_mode), q, k, v, alpha, eta, cu_seqlens, initial_state, eps, chunk,
                False, o, final_state, None, stream, n_splits=int(n_splits), noalloc=True)


def kla_fwd_chunked_kda(q, k, v, alpha, eta, cu_seqlens=None, initial_state=None, eps=1e-6,
                        chunk=64, beta_mode="kaczmarz", output_final_state=False, o=None,
                        final_state=None, stream=None):
    """Prefill with one decay rate per key channel (C ABI `kla_fwd_chunked_kda`,
    Kimi Delta Attention's gate): alpha is [tok, H, dk] (or [B, T, H, dk])
    fp32 and required.  Other arguments as kla_fwd_chunked_ex."""
    if alpha is None or alpha.shape[:-1] != eta.shape or alpha.shape[-1] != q.shape[-1]:
        raise ValueError("alpha must hold one rate per key channel: shape eta.shape + (dk,)")
    return _fwd(_beta_code(beta_mode), q, k, v, alpha, eta, cu_seqlens, initial_state, eps, chunk,
                output_final_state, o, final_state, None, stream, channel_decay=True)


def _fwd(beta, q, k, v, alpha, eta, cu_seqlens, initial_state, eps, chunk, output_final_state, o,
         final_state, workspace, stream, n_splits=None, channel_decay=False, noalloc=False):
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, q.dtype)
    if alpha is not None:
        _need(alpha, "alpha", torch.float32)
    _need(eta, "eta", torch.float32)
    dk, dv, H = q.shape[-1], v.shape[-1], q.shape[-2]
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32)
        if q.dim() != 3:
            raise ValueError("packed input (cu_seqlens given) must be [tok, H, d]")
        n_seqs = cu_seqlens.numel() - 1
        total = q.shape[0]
    else:
        if q.dim() == 4:
            n_seqs, total = q.shape[0], q.shape[0] * q.shape[1]
        elif q.dim() == 3:
            n_seqs, total = 1, q.shape[0]
        else:
            raise ValueError("q must be [tok, H, d] or [B, T, H, d]")
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32)
    if o is None:
        o = torch.empty(v.shape, dtype=torch.float32, device=v.device)
    else:
        _need(o, "o", torch.float32)
    if final_state is None and output_final_state:
        final_state = torch.empty((n_seqs, H, dk, dv), dtype=torch.float32, device=q.device)
    elif final_state is not None:
        _need(final_state, "final_state", torch.float32)
    if noalloc:
        ws_bytes = 0
    elif n_splits is not None and n_splits > 1:
        ws_bytes = kla_fwd_chunked_split_workspace_size(n_seqs, H, dk, dv, n_splits)
    else:
        ws_bytes = kla_fwd_chunked_workspace_size(n_seqs, total, H, dk, dv, chunk)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_ptr = _ptr(workspace)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(eta), _ptr(cu_seqlens), n_seqs, total, H,
            dk, dv, chunk, float(eps), _dtype_code(q))
    tail = (_ptr(initial_state), _ptr(o), _ptr(final_state), ws_ptr, ws_len, _stream(stream))
    if noalloc:
        st = _lib.kla_fwd_chunked_split_noalloc(*head, beta, n_splits, *tail[:3], tail[5])
    elif channel_decay:
        st = _lib.kla_fwd_chunked_kda(*head, beta, *tail)
    elif n_splits is not None:
        st = _lib.kla_fwd_chunked_split(*head, beta, n_splits, *tail)
    elif beta is None:
        st = _lib.kla_fwd_chunked(*head, *tail)
    else:
        st = _lib.kla_fwd_chunked_ex(*head, beta, *tail)
    if st != KLA_OK:
        raise KLAError(st)
    return o, final_state


def kla_decode_step(q, k, v, alpha, eta, state, eps=1e-6, o=None, stream=None):
    """One KLA decode step (C ABI `kla_decode_step`); `state` is updated in place.

    q, k: [N, H, dk]; v: [N, H, dv]; alpha (or None: no decay), eta: [N, H]
    fp32; state: [N, H, dk, dv] fp32.  Returns o [N, H, dv] fp32.
    """
    return _decode(None, q, k, v, alpha, eta, state, eps, o, stream)


def kla_decode_step_ex(q, k, v, alpha, eta, state, eps=1e-6, beta_mode="kaczmarz", o=None,
                       stream=None):
    """kla_decode_step with the step-size rule chosen by beta_mode (C ABI
    `kla_decode_step_ex`), as in kla_fwd_chunked_ex."""
    return _decode(_beta_code(beta_mode), q, k, v, alpha, eta, state, eps, o, stream)


def kla_decode_step_kda(q, k, v, alpha, eta, state, eps=1e-6, beta_mode="kaczmarz", o=None,
                        stream=None):
    """One decode step with one decay rate per key channel (C ABI
    `kla_decode_step_kda`): alpha [N, H, dk] fp32, required."""
    if alpha is None or tuple(alpha.shape) != tuple(q.shape):
        raise ValueError("alpha must hold one rate per key channel: shape [N, H, dk]")
    return _decode(_beta_code(beta_mode), q, k, v, alpha, eta, state, eps, o, stream,
                   channel_decay=True)


def _decode(beta, q, k, v, alpha, eta, state, eps, o, stream, channel_decay=False):
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, q.dtype)
    if alpha is not None:
        _need(alpha, "alpha", torch.float32)
    _need(eta, "eta", torch.float32)
    _need(state, "state", torch.float32)
    N, H, dk = q.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty((N, H, dv), dtype=torch.float32, device=q.device)
    else:
        _need(o, "o", torch.float32)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(eta), _ptr(state), _ptr(o), N, H, dk, dv,
            float(eps), _dtype_code(q))
    if channel_decay:
        st = _lib.kla_decode_step_kda(*args, beta, _stream(stream))
    elif beta is None:
        st = _lib.kla_decode_step(*args, _stream(stream))
    else:
        st = _lib.kla_decode_step_ex(*args, beta, _stream(stream))
    if st != KLA_OK:
        raise KLAError(st)
    return o


# ---- curvature-conditioned read (C ABI kla_*_ccq) ---------------------------
_lib.kla_ccq_state_floats.restype = ctypes.c_size_t
_lib.kla_ccq_state_floats.argtypes = [ctypes.c_int32]
_lib.kla_fwd_chunked_ccq_workspace_size.restype = ctypes.c_size_t
_lib.kla_fwd_chunked_ccq_workspace_size.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                                    ctypes.c_int32, ctypes.c_int]
_lib.kla_decode_step_ccq_workspace_size.restype = ctypes.c_size_t
_lib.kla_decode_step_ccq_workspace_size.argtypes = [ctypes.c_int32] * 3
_lib.kla_fwd_chunked_ccq.restype = ctypes.c_int
_lib.kla_fwd_chunked_ccq.argtypes = [_vp, _vp, _vp, _fp, _fp, _fp, _i32p, ctypes.c_int32,
                                     ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_int,
                                     ctypes.c_int, _fp, _fp, _fp, _fp, _fp, _vp, ctypes.c_size_t,
                                     _vp]
_lib.kla_decode_step_ccq.restype = ctypes.c_int
_lib.kla_decode_step_ccq.argtypes = [_vp, _vp, _vp, _fp, _fp, _fp, _fp, _fp, _fp, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_float, ctypes.c_int, ctypes.c_int, _vp,
                                     ctypes.c_size_t, _vp]


def kla_ccq_state_floats(dk) -> int:
    """fp32 values per (sequence, head) in the curvature-conditioned read's
    running sums: [sum k k^T | sum k | n | pad]."""
    return int(_lib.kla_ccq_state_floats(dk))


def kla_fwd_chunked_ccq(q, k, v, alpha, eta, lam, cu_seqlens=None, initial_state=None,
                        ccq_state=None, eps=1e-6, chunk=64, beta_mode="kaczmarz",
                        output_final_state=False, output_ccq_state=False, o=None,
                        final_state=None, ccq_out=None, workspace=None, stream=None):
    """Prefill with the curvature-conditioned read (C ABI `kla_fwd_chunked_ccq`):
    o_t = S_t^T (q_t - lam_t Sigma_t q_t), Sigma_t the covariance of the keys
    so far.  lam: [tok, H] (or [B, T, H]) fp32.  ccq_state / ccq_out:
    [n_seqs, H, kla_ccq_state_floats(dk)] fp32 running sums.  Returns
    (o, final_state or None, ccq_out or None)."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, q.dtype)
    if alpha is not None:
        _need(alpha, "alpha", torch.float32)
    _need(eta, "eta", torch.float32)
    _need(lam, "lambda", torch.float32)
    dk, dv, H = q.shape[-1], v.shape[-1], q.shape[-2]
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32)
        n_seqs, total = cu_seqlens.numel() - 1, q.shape[0]
    elif q.dim() == 4:
        n_seqs, total = q.shape[0], q.shape[0] * q.shape[1]
    else:
        n_seqs, total = 1, q.shape[0]
    rec = kla_ccq_state_floats(dk)
    for name, t in (("initial_state", initial_state), ("ccq_state", ccq_state)):
        if t is not None:
            _need(t, name, torch.float32)
    if o is None:
        o = torch.empty(v.shape, dtype=torch.float32, device=v.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((n_seqs, H, dk, dv), dtype=torch.float32, device=q.device)
    if ccq_out is None and output_ccq_state:
        ccq_out = torch.empty((n_seqs, H, rec), dtype=torch.float32, device=q.device)
    ws_bytes = int(_lib.kla_fwd_chunked_ccq_workspace_size(total, H, dk, dv, _dtype_code(q)))
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.kla_fwd_chunked_ccq(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(eta), _ptr(lam),
                                  _ptr(cu_seqlens), n_seqs, total, H, dk, dv, chunk, float(eps),
                                  _dtype_code(q), _beta_code(beta_mode), _ptr(initial_state),
                                  _ptr(ccq_state), _ptr(o), _ptr(final_state), _ptr(ccq_out),
                                  _ptr(workspace), ws_len, _stream(stream))
    if st != KLA_OK:
        raise KLAError(st)
    return o, final_state, ccq_out


def kla_decode_step_ccq(q, k, v, alpha, eta, lam, state, ccq_state, eps=1e-6,
                        beta_mode="kaczmarz", o=None, workspace=None, stream=None):
    """One decode step with the curvature-conditioned read (C ABI
    `kla_decode_step_ccq`); `state` and `ccq_state` are updated in place.
    Returns o [N, H, dv] fp32."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, q.dtype)
    if alpha is not None:
        _need(alpha, "alpha", torch.float32)
    for name, t in (("eta", eta), ("lambda", lam), ("state", state), ("ccq_state", ccq_state)):
        _need(t, name, torch.float32)
    N, H, dk = q.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty((N, H, dv), dtype=torch.float32, device=q.device)
    ws_bytes = int(_lib.kla_decode_step_ccq_workspace_size(N, H, dk))
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_len = workspace.numel() * workspace.element_size()
    st = _lib.kla_decode_step_ccq(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(eta), _ptr(lam),
                                  _ptr(state), _ptr(ccq_state), _ptr(o), N, H, dk, dv, float(eps),
                                  _dtype_code(q), _beta_code(beta_mode), _ptr(workspace), ws_len,
                                  _stream(stream))
    if st != KLA_OK:
        raise KLAError(st)
    return o


_lib.kla_bwd_chunked_workspace_size.restype = ctypes.c_size_t
_lib.kla_bwd_chunked_workspace_size.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
_lib.kla_bwd_chunked.restype = ctypes.c_int
_lib.kla_bwd_chunked.argtypes = ([_vp, _vp, _vp, _fp, _fp, _i32p, ctypes.c_int32, ctypes.c_int64,
                                  ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_float, ctypes.c_int, ctypes.c_int]
                                 + [_fp] * 9 + [_vp, ctypes.c_size_t, _vp])


def kla_bwd_chunked_workspace_size(n_seqs, total_tok, H, dk, dv, chunk=64) -> int:
    return int(_lib.kla_bwd_chunked_workspace_size(n_seqs, total_tok, H, dk, dv, chunk))


def kla_bwd_chunked(q, k, v, alpha, eta, d_o, cu_seqlens=None, initial_state=None, d_final=None,
                    eps=1e-6, chunk=64, beta_mode="kaczmarz", workspace=None, stream=None):
    """Gradients of the prefill (C ABI `kla_bwd_chunked`).

    The forward arguments exactly as given to kla_fwd_chunked_ex, plus d_o
    (fp32, shaped like v) and d_final ([n, H, dk, dv] fp32 or None).
    Returns a dict of fp32 tensors: dq, dk (shaped like q), dv (like v),
    dalpha (like eta, or None without alpha), deta (like eta) and dS0
    ([n, H, dk, dv]).  The workspace is allocated with torch when not given.
    """
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, q.dtype)
    if alpha is not None:
        _need(alpha, "alpha", torch.float32)
    _need(eta, "eta", torch.float32)
    _need(d_o, "d_o", torch.float32)
    dk, dv, H = q.shape[-1], v.shape[-1], q.shape[-2]
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32)
        if q.dim() != 3:
            raise ValueError("packed input (cu_seqlens given) must be [tok, H, d]")
        n_seqs, total = cu_seqlens.numel() - 1, q.shape[0]
    elif q.dim() == 4:
        n_seqs, total = q.shape[0], q.shape[0] * q.shape[1]
    elif q.dim() == 3:
        n_seqs, total = 1, q.shape[0]
    else:
        raise ValueError("q must be [tok, H, d] or [B, T, H, d]")
    if d_o.shape != v.shape:
        raise ValueError("d_o must be shaped like v")
    for name, t in (("initial_state", initial_state), ("d_final", d_final)):
        if t is not None:
            _need(t, name, torch.float32)
    dev = q.device
    out = {"dq": torch.empty(q.shape, dtype=torch.float32, device=dev),
           "dk": torch.empty(k.shape, dtype=torch.float32, device=dev),
           "dv": torch.empty(v.shape, dtype=torch.float32, device=dev),
           "dalpha": None if alpha is None else torch.empty(eta.shape, dtype=torch.float32, device=dev),
           "deta": torch.empty(eta.shape, dtype=torch.float32, device=dev),
           "dS0": torch.empty((n_seqs, H, dk, dv), dtype=torch.float32, device=dev)}
    ws_bytes = kla_bwd_chunked_workspace_size(n_seqs, total, H, dk, dv, chunk)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    ws_len = workspace.numel() * workspace.element_size()
    st = _lib.kla_bwd_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(eta), _ptr(cu_seqlens),
                              n_seqs, total, H, dk, dv, chunk, float(eps), _dtype_code(q),
                              _beta_code(beta_mode), _ptr(initial_state), _ptr(d_o), _ptr(d_final),
                              _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dalpha"]),
                              _ptr(out["deta"]), _ptr(out["dS0"]), _ptr(workspace), ws_len,
                              _stream(stream))
    if st != KLA_OK:
        raise KLAError(st)
    return out
