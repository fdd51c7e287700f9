"""GPU parity of the split-sequence prefill (kla_fwd_chunked_split): every
sequence cut into n_splits segments, segment maps A, B, a scan of the maps,
then all segments at once.  Checked against the fp64 oracle (the plain
token recurrence) and against the one-pass kernel.

Error metric and bars as in test_gpu_parity.py.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "f32": 1e-5}
# a sequence shorter than one chunk, exact chunks, ragged, an empty one, and
# lengths where trailing segments are empty for larger n_splits
LENGTHS = [1, 63, 64, 65, 0, 130, 200, 127, 700]


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


@pytest.mark.parametrize("d,dtype,n_splits", [
    (128, "bf16", 2), (128, "bf16", 3), (128, "bf16", 5), (64, "bf16", 4),
    (128, "f32", 3), (64, "f32", 2),
])
def test_split_ragged(kla, d, dtype, n_splits):
    print(f"[case] split prefill n_splits={n_splits} d={d} {dtype} lengths={LENGTHS} H=3 "
          f"+ initial state", flush=True)
    inp = workloads.prefill(lengths=LENGTHS, H=3, d=d, dtype=dtype, seed=51)
    g = torch.Generator().manual_seed(52)
    s0 = 0.5 * torch.randn((len(LENGTHS), 3, d, d), generator=g)
    dev = "cuda"
    args = (inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev), inp["alpha"].to(dev),
            inp["eta"].to(dev))
    cu = inp["cu_seqlens"].to(dev)
    o, S = kla.kla_fwd_chunked_split(*args, cu_seqlens=cu, initial_state=s0.to(dev),
                                     eps=inp["eps"], n_splits=n_splits, output_final_state=True)
    o1, S1 = kla.kla_fwd_chunked(*args, cu_seqlens=cu, initial_state=s0.to(dev), eps=inp["eps"],
                                 output_final_state=True)
    torch.cuda.synchronize()
    ro, rS = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["eta"],
                        cu_seqlens=inp["cu_seqlens"].numpy().astype(np.int64),
                        eps=float(np.float32(inp["eps"])), initial_state=s0)
    name = f"split P={n_splits} d={d} {dtype}"
    check(f"{name} o", o.cpu(), ro, TOL[dtype])
    check(f"{name} S_T", S.cpu(), rS, TOL[dtype])
    check(f"{name} o vs one pass", o.cpu(), o1.cpu(), TOL[dtype])
    assert torch.equal(S[4].cpu(), s0[4])  # the empty sequence keeps its start state


def test_split_direct_mode_no_decay(kla):
    print("[case] split prefill n_splits=3, direct step, no decay (DeltaNet), d=128 bf16",
          flush=True)
    inp = workloads.prefill(lengths=LENGTHS, H=2, d=128, dtype="bf16", seed=53)
    kf = inp["k"].float()
    inp["k"] = (kf / kf.norm(dim=-1, keepdim=True).clamp_min(1e-12)).to(torch.bfloat16)
    dev = "cuda"
    o, S = kla.kla_fwd_chunked_split(inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev), None,
                                     inp["eta"].to(dev), cu_seqlens=inp["cu_seqlens"].to(dev),
                                     eps=inp["eps"], beta_mode="direct", n_splits=3,
                                     output_final_state=True)
    torch.cuda.synchronize()
    ro, rS = oracle.fwd(inp["q"], inp["k"], inp["v"], None, inp["eta"],
                        cu_seqlens=inp["cu_seqlens"].numpy().astype(np.int64),
                        eps=float(np.float32(inp["eps"])), beta_mode="direct")
    check("split direct/no-decay o", o.cpu(), ro, TOL["bf16"])
    check("split direct/no-decay S_T", S.cpu(), rS, TOL["bf16"])


def test_split_final_state_in_place(kla):
    print("[case] split prefill n_splits=3 with final_state = initial_state (in place)",
          flush=True)
    inp = workloads.prefill(lengths=[300, 513], H=2, d=128, dtype="bf16", seed=54)
    g = torch.Generator().manual_seed(55)
    s0 = 0.3 * torch.randn((2, 2, 128, 128), generator=g)
    st = s0.clone().to("cuda")
    dev = "cuda"
    o, _ = kla.kla_fwd_chunked_split(inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev),
                                     inp["alpha"].to(dev), inp["eta"].to(dev),
                                     cu_seqlens=inp["cu_seqlens"].to(dev), initial_state=st,
                                     final_state=st, eps=inp["eps"], n_splits=3)
    torch.cuda.synchronize()
    ro, rS = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["eta"],
                        cu_seqlens=inp["cu_seqlens"].numpy().astype(np.int64),
                        eps=float(np.float32(inp["eps"])), initial_state=s0)
    check("split in-place o", o.cpu(), ro, TOL["bf16"])
    check("split in-place S_T", st.cpu(), rS, TOL["bf16"])


def test_split_long_workload(kla):
    print("[case] long workload B=2 H=16 T=32768 d=128 bf16, n_splits=3 (full oracle)",
          flush=True)
    inp = workloads.prefill("long")
    B, H, d = inp["n_seqs"], inp["H"], inp["d"]
    T = inp["lengths"][0]
    dev = "cuda"
    q, k, v = (inp[n].to(dev).view(B, T, H, d) for n in ("q", "k", "v"))
    a, e = (inp[n].to(dev).view(B, T, H) for n in ("alpha", "eta"))
    o, S = kla.kla_fwd_chunked_split(q, k, v, a, e, eps=inp["eps"], n_splits=3,
                                     output_final_state=True)
    torch.cuda.synchronize()
    cu = np.arange(B + 1, dtype=np.int64) * T
    ro, rS = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["eta"], cu_seqlens=cu,
                        eps=float(np.float32(inp["eps"])))
    check("long split o", o.reshape(-1, H, d).cpu(), ro, TOL["bf16"])
    check("long split S_T", S.cpu(), rS, TOL["bf16"])
