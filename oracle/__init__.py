"""fp64 CPU reference for the KLA recurrence (test infrastructure only).

Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py
may import this package.  The product library never calls it.

The arithmetic lives in kla_oracle.c (token-by-token definition from the
KLA technical summary, "Resumo Tecnico: Atencao Linear Kaczmarz (KLA)",
sections "Derivacao Teorica" and "A Regra de Atualizacao KLA").  This
module only converts arrays to float64 (exact for bf16/fp32 values) and
calls it.

Parity pins for every function here are in tests/test_oracle_pins.py.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# KLA_ORACLE_LIB: another build of the same source (the sanitizer build of
# the CPU tests); the default is the in-tree build.
_LIB_PATH = os.environ.get("KLA_ORACLE_LIB") or os.path.join(_HERE, "libkla_oracle.so")
_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


_libs = {}


def _load(path=None):
    """Load the compiled reference (the default build, or another build of
    the same source given by path)."""
    path = path or _LIB_PATH
    if path in _libs:
        return _libs[path]
    if path == _LIB_PATH and not os.path.exists(path):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(path)
    lib.kla_oracle_fwd.restype = ctypes.c_int
    lib.kla_oracle_fwd.argtypes = [_dp, _dp, _dp, _dp, _dp, _i64p,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_double, _dp, _dp, _dp]
    lib.kla_oracle_decode_step.restype = ctypes.c_int
    lib.kla_oracle_decode_step.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_double, _dp]
    lib.kla_oracle_fwd_ex.restype = ctypes.c_int
    lib.kla_oracle_fwd_ex.argtypes = [_dp, _dp, _dp, _dp, _dp, _i64p,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_double, ctypes.c_int, _dp, _dp, _dp]
    lib.kla_oracle_decode_step_ex.restype = ctypes.c_int
    lib.kla_oracle_decode_step_ex.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_double, ctypes.c_int, _dp]
    lib.kla_oracle_fwd_ch.restype = ctypes.c_int
    lib.kla_oracle_fwd_ch.argtypes = lib.kla_oracle_fwd_ex.argtypes
    lib.kla_oracle_decode_step_ch.restype = ctypes.c_int
    lib.kla_oracle_decode_step_ch.argtypes = lib.kla_oracle_decode_step_ex.argtypes
    lib.kla_oracle_num_threads.restype = ctypes.c_int
    lib.kla_oracle_num_threads.argtypes = []
    _libs[path] = lib
    return lib


_BETA = {"kaczmarz": 0, "direct": 1}


def _f64(x):
    """Contiguous float64 copy/view of an array-like (torch CPU tensors too)."""
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return a.ctypes.data_as(_dp) if a is not None else None


def num_threads() -> int:
    """OpenMP threads the reference will use (OMP_NUM_THREADS)."""
    return int(_load().kla_oracle_num_threads())


def fwd(q, k, v, alpha, eta, cu_seqlens=None, eps=1e-6, initial_state=None, lib_path=None,
        beta_mode="kaczmarz", channel_decay=False):
    """Sequential fp64 KLA prefill.

    q, k: [tok, H, dk]; v: [tok, H, dv]; alpha, eta: [tok, H].  Packed
    sequences are given by cu_seqlens [n_seqs+1]; without it, q/k/v may
    also be [B, T, H, d] (dense batch, flattened here).  Returns
    (o [tok, H, dv] float64, final_state [n_seqs, H, dk, dv] float64), with
    o shaped like v.  beta_mode "direct" takes beta = eta (Gated DeltaNet);
    alpha None means no decay (alpha = 1).  channel_decay: alpha holds one
    decay per key channel, [tok, H, dk] (Kimi Delta Attention's gate).
    """
    lib = _load(lib_path)
    q, k, v, alpha, eta = (_f64(t) for t in (q, k, v, alpha, eta))
    out_shape = v.shape
    if cu_seqlens is None:
        if q.ndim == 4:
            B, T = q.shape[0], q.shape[1]
            cu = np.arange(B + 1, dtype=np.int64) * T
        else:
            cu = np.array([0, q.shape[0]], dtype=np.int64)
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    dk, dv = q.shape[-1], v.shape[-1]
    H = q.shape[-2]
    q = q.reshape(-1, H, dk)
    k = k.reshape(-1, H, dk)
    v = v.reshape(-1, H, dv)
    if channel_decay:
        if alpha is None:
            raise ValueError("channel_decay needs alpha")
        alpha = alpha.reshape(-1, H, dk)
    else:
        alpha = None if alpha is None else alpha.reshape(-1, H)
    eta = eta.reshape(-1, H)
    n_seqs = cu.shape[0] - 1
    tok = q.shape[0]
    if int(cu[-1]) != tok:
        raise ValueError("cu_seqlens[-1] must equal the token count")
    init = None if initial_state is None else _f64(initial_state).reshape(n_seqs, H, dk, dv)
    o = np.zeros((tok, H, dv), dtype=np.float64)
    fin = np.zeros((n_seqs, H, dk, dv), dtype=np.float64)
    f = lib.kla_oracle_fwd_ch if channel_decay else lib.kla_oracle_fwd_ex
    rc = f(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(eta), cu.ctypes.data_as(_i64p), n_seqs, H,
           dk, dv, float(eps), _BETA[beta_mode], _ptr(init), _ptr(o), _ptr(fin))
    if rc != 0:
        raise RuntimeError("kla_oracle_fwd failed")
    return o.reshape(out_shape), fin


def decode_step(q, k, v, alpha, eta, state, eps=1e-6, lib_path=None, beta_mode="kaczmarz",
                channel_decay=False):
    """One fp64 KLA decode step.

    q, k: [N, H, dk]; v: [N, H, dv]; alpha (or None: no decay), eta: [N, H];
    state [N, H, dk, dv].  Returns (o [N, H, dv], new_state), both float64;
    the input state is not modified.  beta_mode and channel_decay (alpha
    [N, H, dk]) as in fwd.
    """
    lib = _load(lib_path)
    q, k, v, alpha, eta = (_f64(t) for t in (q, k, v, alpha, eta))
    S = _f64(state).copy()
    N, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((N, H, dv), dtype=np.float64)
    if channel_decay and (alpha is None or alpha.shape != (N, H, dk)):
        raise ValueError("channel_decay needs alpha of shape [N, H, dk]")
    f = lib.kla_oracle_decode_step_ch if channel_decay else lib.kla_oracle_decode_step_ex
    rc = f(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(eta), _ptr(S), N, H, dk, dv, float(eps),
           _BETA[beta_mode], _ptr(o))
    if rc != 0:
        raise RuntimeError("kla_oracle_decode_step failed")
    return o, S


def ccq_stride(dk):
    """Doubles (or floats) per (sequence, head) in a curvature-conditioned
    read's state record: P = sum k k^T (dk*dk), m = sum k (dk), n, 3 pad."""
    return dk * dk + dk + 4


def _ccq_lib(lib):
    if not getattr(lib, "_ccq_ready", False):
        lib.kla_oracle_fwd_ccq.restype = ctypes.c_int
        lib.kla_oracle_fwd_ccq.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _i64p, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_double, ctypes.c_int, _dp, _dp, _dp, _dp, _dp]
        lib.kla_oracle_decode_step_ccq.restype = ctypes.c_int
        lib.kla_oracle_decode_step_ccq.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp,
                                                   ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                   ctypes.c_int, ctypes.c_double, ctypes.c_int, _dp]
        lib._ccq_ready = True
    return lib


def fwd_ccq(q, k, v, alpha, eta, lam, cu_seqlens=None, eps=1e-6, initial_state=None,
            ccq_state=None, lib_path=None, beta_mode="kaczmarz"):
    """Sequential fp64 KLA prefill with the curvature-conditioned read
    ("Don't Read Everything: A Curvature-Conditioned Query for Linear
    Attention", section "O Mecanismo"): o_t = S_t^T (q_t - lambda_t Sigma_t q_t),
    Sigma_t the uniformly weighted covariance of the keys so far.

    lam: [tok, H] (like eta).  ccq_state: [n_seqs, H, ccq_stride(dk)] start
    sums or None (zeros).  Returns (o, final_state, final ccq sums).
    """
    lib = _ccq_lib(_load(lib_path))
    q, k, v, alpha, eta, lam = (_f64(t) for t in (q, k, v, alpha, eta, lam))
    out_shape = v.shape
    if cu_seqlens is None:
        if q.ndim == 4:
            B, T = q.shape[0], q.shape[1]
            cu = np.arange(B + 1, dtype=np.int64) * T
        else:
            cu = np.array([0, q.shape[0]], dtype=np.int64)
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    dk, dv, H = q.shape[-1], v.shape[-1], q.shape[-2]
    q, k, v = q.reshape(-1, H, dk), k.reshape(-1, H, dk), v.reshape(-1, H, dv)
    alpha = None if alpha is None else alpha.reshape(-1, H)
    eta, lam = eta.reshape(-1, H), lam.reshape(-1, H)
    n_seqs, tok = cu.shape[0] - 1, q.shape[0]
    if int(cu[-1]) != tok:
        raise ValueError("cu_seqlens[-1] must equal the token count")
    init = None if initial_state is None else _f64(initial_state).reshape(n_seqs, H, dk, dv)
    cin = None if ccq_state is None else _f64(ccq_state).reshape(n_seqs, H, ccq_stride(dk))
    o = np.zeros((tok, H, dv))
    fin = np.zeros((n_seqs, H, dk, dv))
    cout = np.zeros((n_seqs, H, ccq_stride(dk)))
    rc = lib.kla_oracle_fwd_ccq(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(eta), _ptr(lam),
                                cu.ctypes.data_as(_i64p), n_seqs, H, dk, dv, float(eps),
                                _BETA[beta_mode], _ptr(init), _ptr(cin), _ptr(o), _ptr(fin),
                                _ptr(cout))
    if rc != 0:
        raise RuntimeError("kla_oracle_fwd_ccq failed")
    return o.reshape(out_shape), fin, cout


def decode_step_ccq(q, k, v, alpha, eta, lam, state, ccq_state, eps=1e-6, lib_path=None,
                    beta_mode="kaczmarz"):
    """One fp64 decode step with the curvature-conditioned read.  Returns
    (o, new_state, new ccq sums); the inputs are not modified."""
    lib = _ccq_lib(_load(lib_path))
    q, k, v, alpha, eta, lam = (_f64(t) for t in (q, k, v, alpha, eta, lam))
    S = _f64(state).copy()
    N, H, dk = q.shape
    dv = v.shape[-1]
    cs = _f64(ccq_state).reshape(N, H, ccq_stride(dk)).copy()
    o = np.zeros((N, H, dv))
    rc = lib.kla_oracle_decode_step_ccq(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(eta),
                                        _ptr(lam), _ptr(S), _ptr(cs), N, H, dk, dv, float(eps),
                                        _BETA[beta_mode], _ptr(o))
    if rc != 0:
        raise RuntimeError("kla_oracle_decode_step_ccq failed")
    return o, S, cs


def _bwd_lib(lib):
    if not getattr(lib, "_bwd_bound", False):
        lib.kla_oracle_bwd_ex.restype = ctypes.c_int
        lib.kla_oracle_bwd_ex.argtypes = [_dp, _dp, _dp, _dp, _dp, _i64p, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_double, ctypes.c_int, _dp, _dp, _dp, _dp,
                                          _dp, _dp, _dp, _dp, _dp]
        lib._bwd_bound = True
    return lib


def bwd(q, k, v, alpha, eta, d_o, cu_seqlens=None, eps=1e-6, initial_state=None,
        d_final=None, lib_path=None, beta_mode="kaczmarz"):
    """fp64 gradient of the KLA prefill (reverse sweep of the plain
    recurrence, kla_oracle_bwd_ex).

    Inputs as fwd, plus d_o (the loss's gradient with respect to o, shaped
    like v) and d_final ([n_seqs, H, dk, dv] or None: the final state does
    not reach the loss).  Returns a dict with dq, dk, dv, dalpha (None
    when alpha is None), deta and dS0 ([n_seqs, H, dk, dv]), float64,
    shaped like the corresponding inputs.
    """
    lib = _bwd_lib(_load(lib_path))
    q, k, v, alpha, eta, d_o = (_f64(t) for t in (q, k, v, alpha, eta, d_o))
    shapes = {"q": q.shape, "k": k.shape, "v": v.shape, "eta": eta.shape,
              "alpha": None if alpha is None else alpha.shape}
    if cu_seqlens is None:
        if q.ndim == 4:
            B, T = q.shape[0], q.shape[1]
            cu = np.arange(B + 1, dtype=np.int64) * T
        else:
            cu = np.array([0, q.shape[0]], dtype=np.int64)
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    dk, dv = q.shape[-1], v.shape[-1]
    H = q.shape[-2]
    q = q.reshape(-1, H, dk)
    k = k.reshape(-1, H, dk)
    v = v.reshape(-1, H, dv)
    d_o = d_o.reshape(-1, H, dv)
    alpha = None if alpha is None else alpha.reshape(-1, H)
    eta = eta.reshape(-1, H)
    n_seqs = cu.shape[0] - 1
    tok = q.shape[0]
    if int(cu[-1]) != tok:
        raise ValueError("cu_seqlens[-1] must equal the token count")
    init = None if initial_state is None else _f64(initial_state).reshape(n_seqs, H, dk, dv)
    dfin = None if d_final is None else _f64(d_final).reshape(n_seqs, H, dk, dv)
    gq = np.zeros((tok, H, dk))
    gk = np.zeros((tok, H, dk))
    gv = np.zeros((tok, H, dv))
    ga = None if alpha is None else np.zeros((tok, H))
    ge = np.zeros((tok, H))
    g0 = np.zeros((n_seqs, H, dk, dv))
    rc = lib.kla_oracle_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(eta),
                               cu.ctypes.data_as(_i64p), n_seqs, H, dk, dv, float(eps),
                               _BETA[beta_mode], _ptr(init), _ptr(d_o), _ptr(dfin), _ptr(gq),
                               _ptr(gk), _ptr(gv), _ptr(ga), _ptr(ge), _ptr(g0))
    if rc != 0:
        raise RuntimeError("kla_oracle_bwd_ex failed")
    return {"dq": gq.reshape(shapes["q"]), "dk": gk.reshape(shapes["k"]),
            "dv": gv.reshape(shapes["v"]),
            "dalpha": None if ga is None else ga.reshape(shapes["alpha"]),
            "deta": ge.reshape(shapes["eta"]), "dS0": g0}
