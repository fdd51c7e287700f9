"""GPU parity of the curvature-conditioned read (kla_fwd_chunked_ccq,
kla_decode_step_ccq; "Don't Read Everything: A Curvature-Conditioned Query
for Linear Attention", section "O Mecanismo") against the fp64 oracle's
fwd_ccq / decode_step_ccq.

Error metric and bars as in test_gpu_parity.py (2e-3 bf16 inputs, 1e-5 fp32
inputs) for o and the KLA state.  The running key sums are fp32
accumulations of the exact inputs and are held to 1e-5 in both cases.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "f32": 1e-5}
SUMS_TOL = 1e-5
LENGTHS = [1, 63, 64, 65, 0, 130, 200, 127]


def rel(x, y):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    den = float(np.max(np.abs(y)))
    return float(np.max(np.abs(x - y)) / (den if den > 0 else 1.0))


def check(name, got, ref, tol):
    err = rel(got, ref)
    print(f"[parity] {name}: max-rel {err:.3e} (bar {tol:.0e})", flush=True)
    assert np.all(np.isfinite(np.asarray(got))), f"{name}: non-finite output"
    assert err <= tol, f"{name}: max-rel {err:.3e} > {tol:.0e}"


@pytest.fixture(scope="module")
def kla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import delta_rule_linear_amd as pkg
    return pkg


def start_sums(n_seqs, H, d, seed):
    """Running sums of a seeded stretch of 37 earlier keys per (sequence, head),
    built by the oracle from keys it is given (fp32 values)."""
    g = torch.Generator().manual_seed(seed)
    kk = torch.randn((37 * n_seqs, H, d), generator=g)
    z = torch.zeros((37 * n_seqs, H, d))
    ones = torch.ones((37 * n_seqs, H))
    cu = np.arange(n_seqs + 1, dtype=np.int64) * 37
    _, _, c = oracle.fwd_ccq(z, kk, z, ones, ones * 0, ones * 0, cu_seqlens=cu)
    return torch.from_numpy(c.astype(np.float32))


@pytest.mark.parametrize("d,dtype,mode", [
    (128, "bf16", "kaczmarz"), (64, "bf16", "kaczmarz"), (128, "f32", "kaczmarz"),
    (64, "f32", "direct"), (128, "bf16", "direct"),
])
def test_ccq_prefill_ragged(kla, d, dtype, mode):
    print(f"[case] CCQ prefill d={d} {dtype} {mode} lengths={LENGTHS} H=3, start state and sums",
          flush=True)
    inp = workloads.prefill(lengths=LENGTHS, H=3, d=d, dtype=dtype, seed=71)
    if mode == "direct":
        kf = inp["k"].float()
        inp["k"] = (kf / kf.norm(dim=-1, keepdim=True).clamp_min(1e-12)).to(inp["k"].dtype)
    tok = inp["q"].shape[0]
    lam = 4.0 * workloads.ccq_gate(72, tok, 3)   # strong contraction: Sigma q is small otherwise
    g = torch.Generator().manual_seed(73)
    s0 = 0.5 * torch.randn((len(LENGTHS), 3, d, d), generator=g)
    c0 = start_sums(len(LENGTHS), 3, d, 74)
    dev = "cuda"
    o, S, c = kla.kla_fwd_chunked_ccq(inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev),
                                      inp["alpha"].to(dev), inp["eta"].to(dev), lam.to(dev),
                                      cu_seqlens=inp["cu_seqlens"].to(dev),
                                      initial_state=s0.to(dev), ccq_state=c0.to(dev),
                                      eps=inp["eps"], beta_mode=mode, output_final_state=True,
                                      output_ccq_state=True)
    torch.cuda.synchronize()
    ro, rS, rc = oracle.fwd_ccq(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["eta"], lam,
                                cu_seqlens=inp["cu_seqlens"].numpy().astype(np.int64),
                                eps=float(np.float32(inp["eps"])), initial_state=s0,
                                ccq_state=c0, beta_mode=mode)
    name = f"ccq d={d} {dtype} {mode}"
    check(f"{name} o", o.cpu(), ro, TOL[dtype])
    check(f"{name} S_T", S.cpu(), rS, TOL[dtype])
    check(f"{name} sums", c.cpu(), rc, SUMS_TOL)
    assert torch.equal(S[4].cpu(), s0[4]) and torch.equal(c[4].cpu(), c0[4])  # empty sequence


def test_ccq_layer_workload(kla):
    print("[case] CCQ prefill, layer shape 8 x 2048 tokens, H=16, d=128 bf16 (full oracle)",
          flush=True)
    inp = workloads.prefill("layer")
    B, H, d = inp["n_seqs"], inp["H"], inp["d"]
    T = inp["lengths"][0]
    lam = workloads.ccq_gate(0, B * T, H)
    dev = "cuda"
    q, k, v = (inp[n].to(dev).view(B, T, H, d) for n in ("q", "k", "v"))
    a, e = (inp[n].to(dev).view(B, T, H) for n in ("alpha", "eta"))
    o, S, c = kla.kla_fwd_chunked_ccq(q, k, v, a, e, lam.to(dev).view(B, T, H), eps=inp["eps"],
                                      output_final_state=True, output_ccq_state=True)
    torch.cuda.synchronize()
    cu = np.arange(B + 1, dtype=np.int64) * T
    ro, rS, rc = oracle.fwd_ccq(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["eta"], lam,
                                cu_seqlens=cu, eps=float(np.float32(inp["eps"])))
    check("ccq layer o", o.reshape(-1, H, d).cpu(), ro, TOL["bf16"])
    check("ccq layer S_T", S.cpu(), rS, TOL["bf16"])
    check("ccq layer sums", c.cpu(), rc, SUMS_TOL)
    # the read changed: the plain prefill's output differs
    o0, _ = kla.kla_fwd_chunked(q, k, v, a, e, eps=inp["eps"])
    assert rel(o0.cpu(), o.cpu()) > 1e-3


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (64, "f32")])
def test_ccq_decode_after_prefill(kla, d, dtype):
    print(f"[case] CCQ prefill 150 tokens x 3 seqs then 4 decode steps, d={d} {dtype}", flush=True)
    L, N, H = 150, 3, 2
    inp = workloads.prefill(lengths=[L + 4] * N, H=H, d=d, dtype=dtype, seed=75)
    tok = inp["q"].shape[0]
    lam = 4.0 * workloads.ccq_gate(76, tok, H)
    dev = "cuda"
    sel = torch.cat([torch.arange(s * (L + 4), s * (L + 4) + L) for s in range(N)])
    pre = {n: inp[n][sel] for n in ("q", "k", "v", "alpha", "eta")}
    cu = torch.tensor([0, L, 2 * L, 3 * L], dtype=torch.int32)
    o, S, c = kla.kla_fwd_chunked_ccq(*(pre[n].to(dev) for n in ("q", "k", "v", "alpha", "eta")),
                                      lam[sel].to(dev), cu_seqlens=cu.to(dev), eps=inp["eps"],
                                      output_final_state=True, output_ccq_state=True)
    for step in range(4):
        idx = torch.tensor([s * (L + 4) + L + step for s in range(N)])
        od = kla.kla_decode_step_ccq(*(inp[n][idx].to(dev) for n in ("q", "k", "v", "alpha", "eta")),
                                     lam[idx].to(dev), S, c, eps=inp["eps"])
    torch.cuda.synchronize()
    ro, rS, rc = oracle.fwd_ccq(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["eta"], lam,
                                cu_seqlens=np.arange(N + 1, dtype=np.int64) * (L + 4),
                                eps=float(np.float32(inp["eps"])))
    last = [s * (L + 4) + L + 3 for s in range(N)]
    check(f"ccq decode d={d} {dtype} o (last step)", od.cpu(), ro[last], TOL[dtype])
    check(f"ccq decode d={d} {dtype} S", S.cpu(), rS, TOL[dtype])
    check(f"ccq decode d={d} {dtype} sums", c.cpu(), rc, SUMS_TOL)


@pytest.mark.parametrize("d,dtype,beta_mode,no_alpha", [
    (128, "f32", "direct", True), (64, "bf16", "kaczmarz", True),
    (128, "bf16", "direct", False), (64, "f32", "kaczmarz", False)])
def test_ccq_decode_modes_from_empty_sums(kla, d, dtype, beta_mode, no_alpha):
    """Decode steps of the fused kernel from zero sums (the first key gives
    n = 1, a zero covariance), against the oracle step by step, for both step
    rules, with and without decay."""
    print(f"[case] CCQ decode from empty sums, d={d} {dtype} {beta_mode} "
          f"{'no alpha' if no_alpha else 'alpha'}", flush=True)
    N, H, steps = 5, 3, 3
    inp = workloads.prefill(lengths=[steps] * N, H=H, d=d, dtype=dtype, seed=77)
    lam = 4.0 * workloads.ccq_gate(78, N * steps, H)
    dev = "cuda"
    rng = np.random.default_rng(79)
    S0 = (0.02 * rng.standard_normal((N, H, d, d))).astype(np.float32)
    S = torch.from_numpy(S0).to(dev)
    c = torch.zeros((N, H, kla.kla_ccq_state_floats(d)), dtype=torch.float32, device=dev)
    rS, rc = S0.astype(np.float64), np.zeros((N, H, kla.kla_ccq_state_floats(d)))
    eta = inp["eta"] * 0.5 if beta_mode == "direct" else inp["eta"]
    for t in range(steps):
        idx = torch.tensor([s * steps + t for s in range(N)])
        a = None if no_alpha else inp["alpha"][idx]
        od = kla.kla_decode_step_ccq(*(inp[n][idx].to(dev) for n in ("q", "k", "v")),
                                     None if a is None else a.to(dev), eta[idx].to(dev),
                                     lam[idx].to(dev), S, c, eps=inp["eps"], beta_mode=beta_mode)
        ro, rS, rc = oracle.decode_step_ccq(inp["q"][idx], inp["k"][idx], inp["v"][idx], a, eta[idx],
                                            lam[idx], rS, rc, eps=float(np.float32(inp["eps"])),
                                            beta_mode=beta_mode)
        torch.cuda.synchronize()
        check(f"ccq decode {d} {dtype} {beta_mode} step {t} o", od.cpu(), ro, TOL[dtype])
    check(f"ccq decode {d} {dtype} {beta_mode} S", S.cpu(), rS, TOL[dtype])
    check(f"ccq decode {d} {dtype} {beta_mode} sums", c.cpu(), rc, SUMS_TOL)
