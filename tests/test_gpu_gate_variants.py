"""GPU parity of the gate variants (kla_fwd_chunked_ex / kla_decode_step_ex)
against the fp64 oracle in the same mode.

- beta_mode "direct": beta = eta, Gated DeltaNet's learned scalar step that
  KLA replaces (KLA summary, introduction).  Gated DeltaNet uses unit-norm
  keys (with beta |k|^2 > 2 the direct step is not a contraction and the
  state grows without bound), so these cases normalise the keys.
- alpha None: no decay gate (alpha = 1); with the direct step this is
  DeltaNet (linear-attention survey page, section "Notacao Unificada").

Error metric and bars as in test_gpu_parity.py.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "f32": 1e-5}
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


def unit_keys(k):
    kf = k.float()
    return (kf / kf.norm(dim=-1, keepdim=True).clamp_min(1e-12)).to(k.dtype)


@pytest.mark.parametrize("mode,no_alpha,d,dtype", [
    ("direct", False, 128, "bf16"),
    ("direct", False, 64, "f32"),
    ("direct", True, 128, "bf16"),
    ("direct", True, 128, "f32"),
    ("direct", True, 64, "bf16"),
    ("kaczmarz", True, 128, "bf16"),
    ("kaczmarz", True, 64, "f32"),
])
def test_prefill_gate_variant(kla, mode, no_alpha, d, dtype):
    name = f"{mode} beta, {'no decay' if no_alpha else 'decay'}, d={d} {dtype}"
    print(f"[case] prefill {name}, ragged lengths {LENGTHS}, H=3, initial state", flush=True)
    inp = workloads.prefill(lengths=LENGTHS, H=3, d=d, dtype=dtype, seed=21)
    if mode == "direct":
        inp["k"] = unit_keys(inp["k"])
    g = torch.Generator().manual_seed(22)
    s0 = 0.5 * torch.randn((len(LENGTHS), 3, d, d), generator=g)
    dev = "cuda"
    alpha = None if no_alpha else inp["alpha"].to(dev)
    o, S = kla.kla_fwd_chunked_ex(inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev), alpha,
                                  inp["eta"].to(dev), cu_seqlens=inp["cu_seqlens"].to(dev),
                                  initial_state=s0.to(dev), eps=inp["eps"], beta_mode=mode,
                                  output_final_state=True)
    torch.cuda.synchronize()
    cu = inp["cu_seqlens"].numpy().astype(np.int64)
    ro, rS = oracle.fwd(inp["q"], inp["k"], inp["v"], None if no_alpha else inp["alpha"],
                        inp["eta"], cu_seqlens=cu, eps=float(np.float32(inp["eps"])),
                        initial_state=s0, beta_mode=mode)
    check(f"{name} o", o.cpu(), ro, TOL[dtype])
    check(f"{name} S_T", S.cpu(), rS, TOL[dtype])
    assert torch.equal(S[4].cpu(), s0[4])  # the empty sequence keeps its start state


@pytest.mark.parametrize("mode,no_alpha,d,dtype", [
    ("direct", False, 128, "bf16"),
    ("direct", True, 128, "bf16"),
    ("direct", True, 64, "f32"),
    ("kaczmarz", True, 128, "f32"),
])
def test_decode_gate_variant(kla, mode, no_alpha, d, dtype):
    name = f"{mode} beta, {'no decay' if no_alpha else 'decay'}, d={d} {dtype}"
    print(f"[case] decode {name}, 7 seqs x 3 heads, 5 steps", flush=True)
    wl = workloads.decode(n_seqs=7, H=3, d=d, steps=5, dtype=dtype, seed=31)
    state = wl["state"].to("cuda")
    ref = wl["state"].double().numpy()
    for st in wl["steps"]:
        k = unit_keys(st["k"]) if mode == "direct" else st["k"]
        alpha = None if no_alpha else st["alpha"]
        o = kla.kla_decode_step_ex(st["q"].to("cuda"), k.to("cuda"), st["v"].to("cuda"),
                                   None if alpha is None else alpha.to("cuda"),
                                   st["eta"].to("cuda"), state, eps=wl["eps"], beta_mode=mode)
        ro, ref = oracle.decode_step(st["q"], k, st["v"], alpha, st["eta"], ref,
                                     eps=float(np.float32(wl["eps"])), beta_mode=mode)
        check(f"decode {name} o", o.cpu(), ro, TOL[dtype])
    check(f"decode {name} S", state.cpu(), ref, TOL[dtype])


def test_plain_entry_points_take_no_alpha(kla):
    """kla_fwd_chunked / kla_decode_step accept alpha=None too (KLA step)."""
    print("[case] plain entry points with alpha=None, d=128 bf16", flush=True)
    inp = workloads.prefill(lengths=[70, 130], H=2, d=128, dtype="bf16", seed=41)
    dev = "cuda"
    cu = inp["cu_seqlens"].to(dev)
    o1, S1 = kla.kla_fwd_chunked(inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev), None,
                                 inp["eta"].to(dev), cu_seqlens=cu, eps=inp["eps"],
                                 output_final_state=True)
    ones = torch.ones_like(inp["alpha"]).to(dev)
    o2, S2 = kla.kla_fwd_chunked(inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev), ones,
                                 inp["eta"].to(dev), cu_seqlens=cu, eps=inp["eps"],
                                 output_final_state=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_unknown_beta_mode_raises(kla):
    print("[case] binding rejects an unknown beta_mode", flush=True)
    q = torch.zeros((64, 2, 64), dtype=torch.bfloat16, device="cuda")
    a = torch.ones((64, 2), device="cuda")
    with pytest.raises(ValueError):
        kla.kla_fwd_chunked_ex(q, q, q, a, a, beta_mode="gdn")
