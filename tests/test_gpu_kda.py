"""GPU parity of the per-channel decay entry points (kla_fwd_chunked_kda,
kla_decode_step_kda; Kimi Delta Attention's gate, one rate per key channel,
linear-attention survey page section "Metodologia e Estrutura") against the
fp64 oracle run with channel_decay=True.

Error metric and bars as in test_gpu_parity.py: normwise max|x-y|/max|y|,
2e-3 for bf16 inputs, 1e-5 for fp32 inputs.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "f32": 1e-5}
# shorter than a chunk, exact chunks, ragged, an empty sequence
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


@pytest.mark.parametrize("d,dtype,mode", [
    (128, "bf16", "kaczmarz"), (64, "bf16", "kaczmarz"), (128, "f32", "kaczmarz"),
    (64, "f32", "kaczmarz"), (128, "bf16", "direct"), (64, "f32", "direct"),
])
def test_kda_prefill_ragged(kla, d, dtype, mode):
    print(f"[case] per-channel prefill d={d} {dtype} {mode} lengths={LENGTHS} H=3 + initial state",
          flush=True)
    inp = workloads.prefill(lengths=LENGTHS, H=3, d=d, dtype=dtype, seed=61, channel_decay=True)
    if mode == "direct":
        inp["k"] = unit_keys(inp["k"])
    g = torch.Generator().manual_seed(62)
    s0 = 0.5 * torch.randn((len(LENGTHS), 3, d, d), generator=g)
    dev = "cuda"
    o, S = kla.kla_fwd_chunked_kda(inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev),
                                   inp["alpha_ch"].to(dev), inp["eta"].to(dev),
                                   cu_seqlens=inp["cu_seqlens"].to(dev), initial_state=s0.to(dev),
                                   eps=inp["eps"], beta_mode=mode, output_final_state=True)
    torch.cuda.synchronize()
    ro, rS = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha_ch"], inp["eta"],
                        cu_seqlens=inp["cu_seqlens"].numpy().astype(np.int64),
                        eps=float(np.float32(inp["eps"])), initial_state=s0, beta_mode=mode,
                        channel_decay=True)
    name = f"kda d={d} {dtype} {mode}"
    check(f"{name} o", o.cpu(), ro, TOL[dtype])
    check(f"{name} S_T", S.cpu(), rS, TOL[dtype])
    assert torch.equal(S[4].cpu(), s0[4])  # the empty sequence keeps its start state


def _tiny(a, case, d):
    if case == "deep_channels":      # a quarter of the channels at 1e-3: 2^-159 per 16 tokens
        a[:, :, : d // 4] = 1e-3
    elif case == "near_zero_run":     # a short run of near-zero rates in some channels
        a[10:14, 0, d // 4: d // 2] = 1e-30
    elif case == "subnormal":         # a single token below the normal fp32 range
        a[70, 1, d // 2:] = 1e-38
    elif case == "past_bound":        # 0.004 per token: just past the fast path's bound
        a[150:160, :, 3 * d // 4:] = 0.004
    elif case == "chunk_deep":        # 0.1 per token: 2^-53 per 16 tokens, 2^-213 per chunk
        a[:, :, : d // 4] = 0.1
    elif case == "near_chunk_bound":  # 0.116 per token: about 2^-199 per chunk
        a[:, :, d // 4: d // 2] = 0.116
    elif case == "all":
        for c in ("deep_channels", "near_zero_run", "subnormal", "past_bound"):
            _tiny(a, c, d)
    return a


@pytest.mark.parametrize("d,dtype,case", [
    (128, "bf16", "deep_channels"), (128, "bf16", "near_zero_run"), (128, "bf16", "subnormal"),
    (128, "bf16", "past_bound"), (128, "bf16", "all"), (64, "bf16", "all"), (64, "f32", "all"),
    (64, "bf16", "deep_channels"), (128, "bf16", "chunk_deep"), (128, "bf16", "near_chunk_bound"),
    (64, "bf16", "chunk_deep"), (64, "bf16", "near_chunk_bound")])
def test_kda_prefill_tiny_rates(kla, d, dtype, case):
    """Per-channel rates whose product inside a 16-token block falls far
    below 2^-126, or whose product over a chunk falls below or just above
    2^-200 (the bf16 kernel's bound for its midpoint-referenced factors),
    mixed with ordinary rates: every output finite and within the bar
    against the oracle."""
    lengths = [200, 64, 1, 130]
    print(f"[case] per-channel prefill with tiny rates ({case}) d={d} {dtype} lengths={lengths} H=2",
          flush=True)
    inp = workloads.prefill(lengths=lengths, H=2, d=d, dtype=dtype, seed=63, channel_decay=True)
    a = _tiny(inp["alpha_ch"].clone(), case, d)
    g = torch.Generator().manual_seed(64)
    s0 = 0.5 * torch.randn((len(lengths), 2, d, d), generator=g)
    dev = "cuda"
    o, S = kla.kla_fwd_chunked_kda(inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev),
                                   a.to(dev), inp["eta"].to(dev),
                                   cu_seqlens=inp["cu_seqlens"].to(dev), initial_state=s0.to(dev),
                                   eps=inp["eps"], output_final_state=True)
    torch.cuda.synchronize()
    ro, rS = oracle.fwd(inp["q"], inp["k"], inp["v"], a, inp["eta"],
                        cu_seqlens=inp["cu_seqlens"].numpy().astype(np.int64),
                        eps=float(np.float32(inp["eps"])), initial_state=s0, channel_decay=True)
    check(f"kda tiny rates {case} d={d} {dtype} o", o.cpu(), ro, TOL[dtype])
    check(f"kda tiny rates {case} d={d} {dtype} S_T", S.cpu(), rS, TOL[dtype])


def test_kda_layer_workload(kla):
    print("[case] per-channel prefill, layer shape 8 x 2048 tokens, H=16, d=128 bf16 (full oracle)",
          flush=True)
    inp = workloads.prefill("layer", channel_decay=True)
    B, H, d = inp["n_seqs"], inp["H"], inp["d"]
    T = inp["lengths"][0]
    dev = "cuda"
    q, k, v = (inp[n].to(dev).view(B, T, H, d) for n in ("q", "k", "v"))
    a = inp["alpha_ch"].to(dev).view(B, T, H, d)
    e = inp["eta"].to(dev).view(B, T, H)
    o, S = kla.kla_fwd_chunked_kda(q, k, v, a, e, eps=inp["eps"], output_final_state=True)
    torch.cuda.synchronize()
    cu = np.arange(B + 1, dtype=np.int64) * T
    ro, rS = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha_ch"], inp["eta"], cu_seqlens=cu,
                        eps=float(np.float32(inp["eps"])), channel_decay=True)
    check("kda layer o", o.reshape(-1, H, d).cpu(), ro, TOL["bf16"])
    check("kda layer S_T", S.cpu(), rS, TOL["bf16"])


def test_kda_uniform_channels_match_scalar_decay(kla):
    """Equal rates in every channel: the per-channel kernel and the scalar
    kernel both meet the oracle's scalar-decay result."""
    print("[case] per-channel prefill with uniform channels vs the scalar kernel, d=128 f32",
          flush=True)
    inp = workloads.prefill(lengths=[70, 130], H=2, d=128, dtype="f32", seed=63)
    ach = inp["alpha"][..., None].expand(-1, -1, 128).contiguous()
    dev = "cuda"
    cu = inp["cu_seqlens"].to(dev)
    args = (inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev))
    o1, S1 = kla.kla_fwd_chunked_kda(*args, ach.to(dev), inp["eta"].to(dev), cu_seqlens=cu,
                                     eps=inp["eps"], output_final_state=True)
    o2, S2 = kla.kla_fwd_chunked(*args, inp["alpha"].to(dev), inp["eta"].to(dev), cu_seqlens=cu,
                                 eps=inp["eps"], output_final_state=True)
    torch.cuda.synchronize()
    ro, rS = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["eta"],
                        cu_seqlens=inp["cu_seqlens"].numpy().astype(np.int64),
                        eps=float(np.float32(inp["eps"])))
    check("kda uniform o", o1.cpu(), ro, TOL["f32"])
    check("kda uniform S_T", S1.cpu(), rS, TOL["f32"])
    check("scalar o", o2.cpu(), ro, TOL["f32"])


def test_kda_in_place_and_deterministic(kla):
    print("[case] per-channel prefill, final_state = initial_state, rerun bitwise", flush=True)
    inp = workloads.prefill(lengths=[300, 513], H=2, d=128, dtype="bf16", seed=64,
                            channel_decay=True)
    g = torch.Generator().manual_seed(65)
    s0 = 0.3 * torch.randn((2, 2, 128, 128), generator=g)
    dev = "cuda"
    args = (inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev), inp["alpha_ch"].to(dev),
            inp["eta"].to(dev))
    cu = inp["cu_seqlens"].to(dev)
    st = s0.clone().to(dev)
    o, _ = kla.kla_fwd_chunked_kda(*args, cu_seqlens=cu, initial_state=st, final_state=st,
                                   eps=inp["eps"])
    o2, S2 = kla.kla_fwd_chunked_kda(*args, cu_seqlens=cu, initial_state=s0.to(dev),
                                     eps=inp["eps"], output_final_state=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(st, S2)
    ro, rS = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha_ch"], inp["eta"],
                        cu_seqlens=inp["cu_seqlens"].numpy().astype(np.int64),
                        eps=float(np.float32(inp["eps"])), initial_state=s0, channel_decay=True)
    check("kda in-place o", o.cpu(), ro, TOL["bf16"])
    check("kda in-place S_T", st.cpu(), rS, TOL["bf16"])


@pytest.mark.parametrize("d,dtype,mode", [
    (128, "bf16", "kaczmarz"), (64, "f32", "kaczmarz"), (128, "f32", "direct"),
])
def test_kda_decode(kla, d, dtype, mode):
    print(f"[case] per-channel decode d={d} {dtype} {mode}, 7 seqs x 3 heads, 5 steps", flush=True)
    wl = workloads.decode(n_seqs=7, H=3, d=d, steps=5, dtype=dtype, seed=66, channel_decay=True)
    state = wl["state"].to("cuda")
    ref = wl["state"].double().numpy()
    for st in wl["steps"]:
        k = unit_keys(st["k"]) if mode == "direct" else st["k"]
        o = kla.kla_decode_step_kda(st["q"].to("cuda"), k.to("cuda"), st["v"].to("cuda"),
                                    st["alpha_ch"].to("cuda"), st["eta"].to("cuda"), state,
                                    eps=wl["eps"], beta_mode=mode)
        ro, ref = oracle.decode_step(st["q"], k, st["v"], st["alpha_ch"], st["eta"], ref,
                                     eps=float(np.float32(wl["eps"])), beta_mode=mode,
                                     channel_decay=True)
        check(f"kda decode d={d} {dtype} {mode} o", o.cpu(), ro, TOL[dtype])
    check(f"kda decode d={d} {dtype} {mode} S", state.cpu(), ref, TOL[dtype])


def test_kda_prefill_then_decode(kla):
    """Prefill of T tokens then one decode step equals the oracle's T+1."""
    print("[case] per-channel prefill 190 tokens then one decode step, d=128 bf16", flush=True)
    inp = workloads.prefill(lengths=[191], H=2, d=128, dtype="bf16", seed=67, channel_decay=True)
    dev = "cuda"
    T = 190
    cu = torch.tensor([0, T], dtype=torch.int32, device=dev)
    _, S = kla.kla_fwd_chunked_kda(inp["q"][:T].to(dev), inp["k"][:T].to(dev),
                                   inp["v"][:T].to(dev), inp["alpha_ch"][:T].to(dev),
                                   inp["eta"][:T].to(dev), cu_seqlens=cu, eps=inp["eps"],
                                   output_final_state=True)
    od = kla.kla_decode_step_kda(inp["q"][T:].to(dev), inp["k"][T:].to(dev), inp["v"][T:].to(dev),
                                 inp["alpha_ch"][T:].to(dev), inp["eta"][T:].to(dev), S,
                                 eps=inp["eps"])
    torch.cuda.synchronize()
    ro, rS = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha_ch"], inp["eta"],
                        cu_seqlens=np.array([0, T + 1]), eps=float(np.float32(inp["eps"])),
                        channel_decay=True)
    check("kda prefill+decode o", od.cpu(), ro[T:], TOL["bf16"])
    check("kda prefill+decode S", S.cpu(), rS, TOL["bf16"])
