"""GPU parity of the prefill's backward (kla_bwd_chunked through the C ABI)
against the fp64 oracle's reverse sweep (oracle.bwd).

Every gradient tensor (dq, dk, dv, dalpha, deta, dS0) is compared with
max|gpu - ref| / max|ref|; bars 2e-3 for bf16 q/k/v and 1e-5 for fp32, as
for the forward.  Upstream gradients d_o, d_final and the start state are
seeded (workloads.grad_inputs).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from test_gpu_parity import TOL, check, cu_of, say

pytestmark = pytest.mark.gpu

KEYS = ("dq", "dk", "dv", "dalpha", "deta", "dS0")


@pytest.fixture(scope="module")
def kla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import delta_rule_linear_amd as pkg
    return pkg


def run_case(kla, name, inp, g, beta_mode="kaczmarz", use_alpha=True, with_s0=True, with_dfin=True,
             seqs=None):
    dev = "cuda"
    cu = cu_of(inp)
    alpha = inp["alpha"] if use_alpha else None
    s0 = g["initial_state"] if with_s0 else None
    dfin = g["d_final"] if with_dfin else None
    out = kla.kla_bwd_chunked(inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev),
                              None if alpha is None else alpha.to(dev), inp["eta"].to(dev),
                              g["d_o"].to(dev), cu_seqlens=torch.from_numpy(cu.astype(np.int32)).to(dev),
                              initial_state=None if s0 is None else s0.to(dev),
                              d_final=None if dfin is None else dfin.to(dev), eps=inp["eps"],
                              beta_mode=beta_mode)
    torch.cuda.synchronize()
    got = {k: (None if v is None else v.cpu()) for k, v in out.items()}
    eps = float(np.float32(inp["eps"]))
    if seqs is None:
        ref = oracle.bwd(inp["q"], inp["k"], inp["v"], alpha, inp["eta"], g["d_o"], cu_seqlens=cu,
                         eps=eps, initial_state=s0, d_final=dfin, beta_mode=beta_mode)
        sel, ssel = slice(None), slice(None)
    else:
        idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs]).astype(np.int64)
        sub_cu = np.concatenate([[0], np.cumsum([cu[s + 1] - cu[s] for s in seqs])])
        ti = torch.from_numpy(idx)
        ref = oracle.bwd(inp["q"][ti], inp["k"][ti], inp["v"][ti],
                         None if alpha is None else alpha[ti], inp["eta"][ti], g["d_o"][ti],
                         cu_seqlens=sub_cu, eps=eps,
                         initial_state=None if s0 is None else s0[list(seqs)],
                         d_final=None if dfin is None else dfin[list(seqs)], beta_mode=beta_mode)
        sel, ssel = ti, list(seqs)
    tol = TOL["bf16"] if inp["q"].dtype == torch.bfloat16 else TOL["f32"]
    for key in KEYS:
        if ref[key] is None:
            assert got[key] is None
            continue
        gk = got[key][ssel] if key == "dS0" else got[key][sel]
        check(f"{name} {key}", gk, ref[key], tol)
    return got


def test_bwd_tiny_fp32_workload(kla):
    say("bwd tiny_fp32 workload B=1 H=2 T=256 d=64 fp32, start state and d_final")
    inp = workloads.prefill("tiny_fp32")
    g = workloads.grad_inputs(1, inp["q"].shape[0], inp["H"], inp["d"], inp["n_seqs"])
    run_case(kla, "bwd tiny_fp32", inp, g)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 128), ("bf16", 64), ("f32", 64)])
def test_bwd_ragged(kla, dtype, d):
    lens = [1, 63, 64, 65, 0, 200, 130]
    say(f"bwd ragged lengths {lens} H=3 d={d} {dtype}")
    inp = workloads.prefill(lengths=lens, H=3, d=d, dtype=dtype, seed=11)
    g = workloads.grad_inputs(2, inp["q"].shape[0], 3, d, len(lens))
    got = run_case(kla, f"bwd ragged {dtype} d={d}", inp, g)
    # the empty sequence passes d_final through to its start state
    assert torch.equal(got["dS0"][4], g["d_final"][4])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_direct_and_no_decay(kla, dtype):
    lens = [100, 37, 129]
    say(f"bwd direct step (Gated DeltaNet) and DeltaNet, lengths {lens} H=2 d=64 {dtype}")
    inp = workloads.prefill(lengths=lens, H=2, d=64, dtype=dtype, seed=12)
    # unit-norm keys keep the direct step a contraction (beta = eta <= 1)
    k = inp["k"].float()
    inp["k"] = (k / k.norm(dim=-1, keepdim=True)).to(inp["k"].dtype)
    g = workloads.grad_inputs(3, inp["q"].shape[0], 2, 64, len(lens))
    run_case(kla, f"bwd gdn {dtype}", inp, g, beta_mode="direct")
    run_case(kla, f"bwd deltanet {dtype}", inp, g, beta_mode="direct", use_alpha=False)
    run_case(kla, f"bwd kla no decay {dtype}", inp, g, use_alpha=False)


def test_bwd_no_state_no_final_gradient(kla):
    lens = [70, 190]
    say(f"bwd without start state and without d_final, lengths {lens} H=2 d=128 bf16")
    inp = workloads.prefill(lengths=lens, H=2, d=128, dtype="bf16", seed=13)
    g = workloads.grad_inputs(4, inp["q"].shape[0], 2, 128, len(lens))
    run_case(kla, "bwd bare", inp, g, with_s0=False, with_dfin=False)


def test_bwd_layer_workload_sampled(kla):
    say("bwd layer workload B=8 H=16 T=2048 d=128 bf16 (oracle on 2 sequences, all heads)")
    inp = workloads.prefill("layer")
    g = workloads.grad_inputs(5, inp["q"].shape[0], inp["H"], inp["d"], inp["n_seqs"])
    run_case(kla, "bwd layer", inp, g, seqs=[0, 5])


def test_bwd_deterministic(kla):
    lens = [300, 45]
    say(f"bwd bitwise determinism, lengths {lens} H=2 d=128 bf16")
    inp = workloads.prefill(lengths=lens, H=2, d=128, dtype="bf16", seed=14)
    g = workloads.grad_inputs(6, inp["q"].shape[0], 2, 128, len(lens))
    dev = "cuda"
    args = [inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev), inp["alpha"].to(dev),
            inp["eta"].to(dev), g["d_o"].to(dev)]
    cu = inp["cu_seqlens"].to(dev)
    a = kla.kla_bwd_chunked(*args, cu_seqlens=cu, d_final=g["d_final"].to(dev))
    b = kla.kla_bwd_chunked(*args, cu_seqlens=cu, d_final=g["d_final"].to(dev))
    torch.cuda.synchronize()
    for key in KEYS:
        assert torch.equal(a[key], b[key]), key


def test_bwd_long_workload_sampled_heads(kla):
    say("bwd long workload B=2 H=16 T=32768 d=128 bf16 (oracle on sequence 1, heads 3 and 12)")
    inp = workloads.prefill("long")
    g = workloads.grad_inputs(7, inp["q"].shape[0], inp["H"], inp["d"], inp["n_seqs"])
    dev = "cuda"
    cu = cu_of(inp)
    out = kla.kla_bwd_chunked(inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev),
                              inp["alpha"].to(dev), inp["eta"].to(dev), g["d_o"].to(dev),
                              cu_seqlens=torch.from_numpy(cu.astype(np.int32)).to(dev),
                              d_final=g["d_final"].to(dev), eps=inp["eps"])
    torch.cuda.synchronize()
    heads = [3, 12]
    ti = torch.arange(int(cu[1]), int(cu[2]))
    sub = {n: inp[n][ti][:, heads].contiguous() for n in ("q", "k", "v", "alpha", "eta")}
    ref = oracle.bwd(sub["q"], sub["k"], sub["v"], sub["alpha"], sub["eta"],
                     g["d_o"][ti][:, heads].contiguous(), cu_seqlens=np.array([0, len(ti)]),
                     eps=float(np.float32(inp["eps"])), d_final=g["d_final"][1:2, heads])
    for key in KEYS:
        got = out[key].cpu()
        got = got[1:2, heads] if key == "dS0" else got[ti][:, heads]
        check(f"bwd long {key}", got, ref[key], TOL["bf16"])


def test_bwd_packed_workload_sampled(kla):
    say("bwd packed workload 64 seqs lengths U[128,8192] H=16 d=128 bf16 (oracle on 4 sequences)")
    inp = workloads.prefill("packed")
    g = workloads.grad_inputs(8, inp["q"].shape[0], inp["H"], inp["d"], inp["n_seqs"])
    lens = np.array(inp["lengths"])
    rng = np.random.default_rng(321)
    seqs = sorted(set([int(lens.argmax()), int(lens.argmin())]
                      + [int(x) for x in rng.choice(len(lens), 2, replace=False)]))
    run_case(kla, "bwd packed", inp, g, with_s0=False, seqs=seqs)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_dense_batch(kla, dtype):
    B, T = 3, 200
    say(f"bwd dense batch B={B} T={T} H=2 d=128 {dtype}: dense equals packed, and the oracle")
    inp = workloads.prefill(n_seqs=B, T=T, H=2, d=128, dtype=dtype, seed=15)
    g = workloads.grad_inputs(9, B * T, 2, 128, B)
    dev = "cuda"
    view = lambda x: x.to(dev).view(B, T, *x.shape[1:])
    dense = kla.kla_bwd_chunked(view(inp["q"]), view(inp["k"]), view(inp["v"]), view(inp["alpha"]),
                                view(inp["eta"]), view(g["d_o"]), initial_state=g["initial_state"].to(dev),
                                d_final=g["d_final"].to(dev), eps=inp["eps"])
    torch.cuda.synchronize()
    got = run_case(kla, f"bwd dense-as-packed {dtype}", inp, g)
    for key in KEYS:
        assert torch.equal(dense[key].reshape(got[key].shape).cpu(), got[key]), key
