"""Seeded synthetic inputs for the KLA prefill and decode workloads.

This module only draws random numbers and casts them; it holds none of the
KLA arithmetic.  Both the GPU library (through the tests and bench.py) and
the fp64 reference consume exactly the tensors produced here.

Recipe.  ss = numpy SeedSequence(seed).  Packed workloads first draw the
sequence lengths (integers uniform in [lo, hi], inclusive) from
PCG64(ss.spawn(1)[0]).  The tokens are then cut into blocks of BLOCK
tokens; block b draws from its own stream PCG64(ss.spawn(n_blocks)[b]),
float32, in this order:
  1. q ~ N(0, 1)                     [tb, H, dk]
  2. z ~ N(0, 1)                     [tb, H, dk]
  3. r ~ N(0, 1)                     [tb, H];  k = z / |z| * exp(r)
     (unnormalised keys with log-normal norms, mu = 0, sigma = 1)
  4. if big_frac > 0: u ~ U[0, 1)    [tb, H];  k *= big_scale where u < big_frac
  5. v ~ N(0, 1)                     [tb, H, dv]
  6. alpha = sigmoid(alpha_mu + N(0, 1))   [tb, H]
  7. eta   = sigmoid(N(0, 1))              [tb, H]
q, k, v are then rounded to bf16 (round-to-nearest-even) or kept fp32;
alpha and eta stay fp32.  eps = 1e-6 and the start state is zero.  Blocks
are independent streams, so they are drawn in parallel and the values do
not depend on the thread count.

Per-channel decay (channel_decay=True, the Kimi Delta Attention gate): a
separate seed sequence SeedSequence([seed, 0x4B4441]) gives, per block of
BLOCK tokens, alpha_ch = sigmoid(alpha_mu + N(0, 1)) fp32 [tb, H, dk], one
decay per key channel (decode step i: SeedSequence([seed, 0x4B4441, i]),
one block of N tokens).  The other tensors are drawn exactly as above.

Curvature-conditioned read gate (ccq_gate): lambda = sigmoid(N(0, 1)) fp32
[tok, H] from SeedSequence([seed, 0x434351]) (one stream, drawn in token order).

Decode: ss.spawn(2) gives a state stream and a step stream.  The state is
0.02 * N(0, 1) fp32 [N, H, dk, dv], drawn per sequence from
PCG64(state_ss.spawn(N)[s]); step i draws one block of N tokens (as above)
from PCG64(step_ss.spawn(steps)[i]).
"""
import os

import numpy as np
import torch

EPS = 1e-6

# The workloads by what they are (sizes and distributions).
PREFILL = {
    # tiny fp32 prefill, d = 64
    "tiny_fp32": dict(n_seqs=1, T=256, H=2, d=64, dtype="f32", alpha_mu=3.0),
    # layer-shaped prefill: 8 x 2048 tokens, 16 heads, d = 128
    "layer": dict(n_seqs=8, T=2048, H=16, d=128, dtype="bf16", alpha_mu=3.0),
    # long-context prefill: 2 x 32768 tokens, slow decay
    "long": dict(n_seqs=2, T=32768, H=16, d=128, dtype="bf16", alpha_mu=5.0),
    # packed variable-length prefill: 64 sequences of 128..8192 tokens,
    # 5% of keys scaled by 10
    "packed": dict(n_seqs=64, lengths=(128, 8192), H=16, d=128, dtype="bf16", alpha_mu=3.0,
                   big_frac=0.05, big_scale=10.0),
}
DECODE = dict(n_seqs=256, H=16, d=128, steps=128, dtype="bf16", alpha_mu=3.0, state_std=0.02)


def _sigmoid(x):
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


BLOCK = 1024
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        from concurrent.futures import ThreadPoolExecutor
        _POOL = ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))
    return _POOL


def _draw_block(seed_seq, tb, H, dk, dv, alpha_mu, big_frac, big_scale):
    rng = np.random.Generator(np.random.PCG64(seed_seq))
    q = rng.standard_normal((tb, H, dk), dtype=np.float32)
    z = rng.standard_normal((tb, H, dk), dtype=np.float32)
    r = rng.standard_normal((tb, H), dtype=np.float32)
    scale = np.exp(r) / np.sqrt(np.einsum("thd,thd->th", z, z))
    if big_frac > 0:
        u = rng.random((tb, H), dtype=np.float32)
        scale = np.where(u < big_frac, scale * np.float32(big_scale), scale)
    z *= scale.astype(np.float32)[..., None]
    v = rng.standard_normal((tb, H, dv), dtype=np.float32)
    alpha = _sigmoid(np.float32(alpha_mu) + rng.standard_normal((tb, H), dtype=np.float32))
    eta = _sigmoid(rng.standard_normal((tb, H), dtype=np.float32))
    return q, z, v, alpha, eta


def _tokens(seed_seqs, tok, H, dk, dv, dtype, alpha_mu, big_frac=0.0, big_scale=10.0):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.empty((tok, H, dk), dtype=tdt)
    k = torch.empty((tok, H, dk), dtype=tdt)
    v = torch.empty((tok, H, dv), dtype=tdt)
    alpha = torch.empty((tok, H), dtype=torch.float32)
    eta = torch.empty((tok, H), dtype=torch.float32)
    bs = BLOCK if len(seed_seqs) > 1 else tok

    def one(b):
        a0 = b * bs
        tb = min(bs, tok - a0)
        qb, kb, vb, ab, eb = _draw_block(seed_seqs[b], tb, H, dk, dv, alpha_mu, big_frac, big_scale)
        q[a0:a0 + tb] = torch.from_numpy(qb)
        k[a0:a0 + tb] = torch.from_numpy(kb)
        v[a0:a0 + tb] = torch.from_numpy(vb)
        alpha[a0:a0 + tb] = torch.from_numpy(ab)
        eta[a0:a0 + tb] = torch.from_numpy(eb)

    list(_pool().map(one, range(len(seed_seqs))))
    return q, k, v, alpha, eta


_CH_TAG = 0x4B4441  # second entropy word of the per-channel gate stream


def _channel_gates(seed, tok, H, dk, alpha_mu, step=None):
    """alpha_ch = sigmoid(alpha_mu + N(0, 1)) fp32 [tok, H, dk], per block."""
    words = [seed, _CH_TAG] if step is None else [seed, _CH_TAG, step]
    nb = max(1, -(-tok // BLOCK))
    seqs = np.random.SeedSequence(words).spawn(nb)
    out = torch.empty((tok, H, dk), dtype=torch.float32)

    def one(b):
        a0 = b * BLOCK
        tb = min(BLOCK, tok - a0)
        rng = np.random.Generator(np.random.PCG64(seqs[b]))
        x = rng.standard_normal((tb, H, dk), dtype=np.float32)
        out[a0:a0 + tb] = torch.from_numpy(_sigmoid(np.float32(alpha_mu) + x))

    list(_pool().map(one, range(nb)))
    return out


def ccq_gate(seed, tok, H):
    """lambda = sigmoid(N(0, 1)) fp32 [tok, H], the contraction gate of the
    curvature-conditioned read."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0x434351])))
    return torch.from_numpy(_sigmoid(rng.standard_normal((tok, H), dtype=np.float32)))


def prefill(name=None, *, seed=0, n_seqs=None, T=None, lengths=None, H=None, d=None, dtype=None,
            alpha_mu=None, big_frac=None, big_scale=None, channel_decay=False):
    """Inputs of a named prefill workload, or of a custom one.

    `lengths` is either a (lo, hi) pair (drawn per sequence) or an explicit
    list of per-sequence lengths.  Returns a dict of CPU tensors:
    q, k, v [tok, H, d] (bf16 or fp32), alpha, eta [tok, H] fp32,
    cu_seqlens int32 [n+1] (None for equal-length batches), n_seqs,
    lengths (list), eps; with channel_decay also alpha_ch [tok, H, d] fp32.
    """
    p = dict(PREFILL[name]) if name else {}
    for key, val in (("n_seqs", n_seqs), ("T", T), ("lengths", lengths), ("H", H), ("d", d),
                     ("dtype", dtype), ("alpha_mu", alpha_mu), ("big_frac", big_frac),
                     ("big_scale", big_scale)):
        if val is not None:
            p[key] = val
    ss = np.random.SeedSequence(seed)
    dense = "lengths" not in p or p["lengths"] is None
    if dense:
        lens = [int(p["T"])] * int(p["n_seqs"])
    elif isinstance(p["lengths"], tuple):
        lo, hi = p["lengths"]
        rng = np.random.Generator(np.random.PCG64(ss.spawn(1)[0]))
        lens = [int(x) for x in rng.integers(lo, hi, endpoint=True, size=int(p["n_seqs"]))]
    else:
        lens = [int(x) for x in p["lengths"]]
    tok = int(sum(lens))
    blocks = ss.spawn(max(1, -(-tok // BLOCK)))
    q, k, v, alpha, eta = _tokens(blocks, tok, p["H"], p["d"], p["d"], p["dtype"],
                                  p.get("alpha_mu", 3.0), p.get("big_frac", 0.0),
                                  p.get("big_scale", 10.0))
    cu = None if dense else torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    out = dict(q=q, k=k, v=v, alpha=alpha, eta=eta, cu_seqlens=cu, n_seqs=len(lens),
               lengths=lens, eps=EPS, H=p["H"], d=p["d"], dtype=p["dtype"])
    if channel_decay:
        out["alpha_ch"] = _channel_gates(seed, tok, p["H"], p["d"], p.get("alpha_mu", 3.0))
    return out


def decode(*, seed=0, n_seqs=None, H=None, d=None, steps=None, dtype=None, alpha_mu=None,
           state_std=None, channel_decay=False):
    """Decode workload: dict(state fp32 [N,H,d,d], steps=[dict(q,k,v,alpha,eta)], eps);
    with channel_decay every step also holds alpha_ch [N, H, d] fp32."""
    p = dict(DECODE)
    for key, val in (("n_seqs", n_seqs), ("H", H), ("d", d), ("steps", steps), ("dtype", dtype),
                     ("alpha_mu", alpha_mu), ("state_std", state_std)):
        if val is not None:
            p[key] = val
    ss = np.random.SeedSequence(seed)
    state_ss, step_ss = ss.spawn(2)
    N, Hh, dd = p["n_seqs"], p["H"], p["d"]
    state = torch.empty((N, Hh, dd, dd), dtype=torch.float32)
    std = np.float32(p["state_std"])

    def one_seq(a):
        i, sq = a
        x = np.random.Generator(np.random.PCG64(sq)).standard_normal((Hh, dd, dd), dtype=np.float32)
        state[i] = torch.from_numpy(x * std)

    list(_pool().map(one_seq, enumerate(state_ss.spawn(N))))
    out = []
    for i, sq in enumerate(step_ss.spawn(p["steps"])):
        q, k, v, alpha, eta = _tokens([sq], N, Hh, dd, dd, p["dtype"], p["alpha_mu"])
        st = dict(q=q, k=k, v=v, alpha=alpha, eta=eta)
        if channel_decay:
            st["alpha_ch"] = _channel_gates(seed, N, Hh, dd, p["alpha_mu"], step=i)
        out.append(st)
    return dict(state=state, steps=out, eps=EPS, n_seqs=N, H=Hh, d=dd,
                dtype=p["dtype"])


def grad_inputs(seed, tok, H, d, n_seqs, state_std=0.02):
    """Seeded upstream gradients and start state for the backward:
    d_o ~ N(0, 1) fp32 [tok, H, d], d_final ~ N(0, 1) fp32 [n_seqs, H, d, d]
    and an initial state ~ N(0, state_std^2) fp32 [n_seqs, H, d, d]."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0x425744])))
    d_o = rng.standard_normal((tok, H, d), dtype=np.float32)
    d_final = rng.standard_normal((n_seqs, H, d, d), dtype=np.float32)
    s0 = rng.standard_normal((n_seqs, H, d, d), dtype=np.float32) * np.float32(state_std)
    return dict(d_o=torch.from_numpy(d_o), d_final=torch.from_numpy(d_final),
                initial_state=torch.from_numpy(s0))
