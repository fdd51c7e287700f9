"""GPU parity: libkla.so (through the C ABI binding) against the fp64 oracle.

Error metric per output tensor: max|gpu - ref| / max|ref| (normwise max
relative error).  Bars: 2e-3 for bf16 q/k/v, 1e-5 for fp32 q/k/v.  Every
case names itself on stdout before it touches the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "f32": 1e-5}


def rel(x, y):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    den = float(np.max(np.abs(y))) if y.size else 0.0
    return float(np.max(np.abs(x - y)) / (den if den > 0 else 1.0)) if y.size else 0.0


def say(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def kla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import delta_rule_linear_amd as pkg
    return pkg


def cu_of(inp):
    if inp["cu_seqlens"] is not None:
        return inp["cu_seqlens"].numpy().astype(np.int64)
    return np.concatenate([[0], np.cumsum(inp["lengths"])]).astype(np.int64)


def gpu_fwd(kla, inp, initial_state=None, dense=None):
    dev = "cuda"
    q, k, v = inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev)
    a, e = inp["alpha"].to(dev), inp["eta"].to(dev)
    cu = None if inp["cu_seqlens"] is None else inp["cu_seqlens"].to(dev)
    s0 = None if initial_state is None else initial_state.to(dev)
    if cu is None and dense is None:
        B = inp["n_seqs"]
        T = q.shape[0] // B
        q, k, v = (x.view(B, T, *x.shape[1:]) for x in (q, k, v))
        a, e = a.view(B, T, -1), e.view(B, T, -1)
    o, S = kla.kla_fwd_chunked(q, k, v, a, e, cu_seqlens=cu, initial_state=s0, eps=inp["eps"],
                               output_final_state=True)
    torch.cuda.synchronize()
    return o.reshape(inp["v"].shape).cpu(), S.cpu()


def ref_fwd(inp, initial_state=None, seqs=None):
    """Oracle on all sequences, or on the listed subset (packed sub-batch)."""
    cu = cu_of(inp)
    eps = float(np.float32(inp["eps"]))
    if seqs is None:
        return oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["eta"], cu_seqlens=cu,
                          eps=eps, initial_state=initial_state)
    idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs]).astype(np.int64)
    sub_cu = np.concatenate([[0], np.cumsum([cu[s + 1] - cu[s] for s in seqs])])
    ti = torch.from_numpy(idx)
    s0 = None if initial_state is None else initial_state[list(seqs)]
    o, S = oracle.fwd(inp["q"][ti], inp["k"][ti], inp["v"][ti], inp["alpha"][ti], inp["eta"][ti],
                      cu_seqlens=sub_cu, eps=eps, initial_state=s0)
    return o, S, idx


def check(name, got, ref, tol):
    err = rel(got, ref)
    print(f"[parity] {name}: max-rel {err:.3e} (bar {tol:.0e})", flush=True)
    assert np.all(np.isfinite(np.asarray(got))), f"{name}: non-finite output"
    assert err <= tol, f"{name}: max-rel {err:.3e} > {tol:.0e}"
    return err


# ---------------------------------------------------------------- workloads

def test_tiny_fp32_workload(kla):
    say("tiny_fp32 workload B=1 H=2 T=256 d=64 fp32")
    inp = workloads.prefill("tiny_fp32")
    o, S = gpu_fwd(kla, inp)
    ro, rS = ref_fwd(inp)
    check("tiny_fp32 o", o, ro, TOL["f32"])
    check("tiny_fp32 S_T", S, rS, TOL["f32"])


def test_layer_workload_full(kla):
    say("layer workload B=8 H=16 T=2048 d=128 bf16 (full oracle)")
    inp = workloads.prefill("layer")
    o, S = gpu_fwd(kla, inp)
    ro, rS = ref_fwd(inp)
    check("layer o", o, ro, TOL["bf16"])
    check("layer S_T", S, rS, TOL["bf16"])


def test_long_workload_full(kla):
    say("long workload B=2 H=16 T=32768 d=128 bf16 (full oracle)")
    inp = workloads.prefill("long")
    o, S = gpu_fwd(kla, inp)
    ro, rS = ref_fwd(inp)
    check("long o", o, ro, TOL["bf16"])
    check("long S_T", S, rS, TOL["bf16"])


class MaxRel:
    """Normwise max relative error accumulated over parts of one tensor:
    max|x - y| over every part divided by max|y| over every part, the same
    figure as rel() on the whole tensor."""

    def __init__(self):
        self.diff = 0.0
        self.ref = 0.0

    def add(self, got, ref):
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        assert np.all(np.isfinite(got)), "non-finite output"
        if ref.size:
            self.diff = max(self.diff, float(np.max(np.abs(got - ref))))
            self.ref = max(self.ref, float(np.max(np.abs(ref))))

    def value(self):
        return self.diff / (self.ref if self.ref > 0 else 1.0)


def test_packed_workload_full(kla):
    say("packed workload 64 seqs lengths U[128,8192] H=16 d=128 bf16 (full oracle, 8 batches of 8 seqs)")
    inp = workloads.prefill("packed")
    o, S = gpu_fwd(kla, inp)
    n = inp["n_seqs"]
    err_o, err_s = MaxRel(), MaxRel()
    for b0 in range(0, n, 8):
        seqs = list(range(b0, min(n, b0 + 8)))
        ro, rS, idx = ref_fwd(inp, seqs=seqs)
        got_o = o[torch.from_numpy(idx)]
        part_o, part_s = rel(got_o, ro), rel(S[seqs], rS)
        print(f"[parity] packed seqs {seqs[0]}..{seqs[-1]}: o {part_o:.3e}, S_T {part_s:.3e}",
              flush=True)
        assert part_o <= TOL["bf16"] and part_s <= TOL["bf16"]
        err_o.add(got_o, ro)
        err_s.add(S[seqs], rS)
        del ro, rS, got_o
    for name, e in (("packed o (all 64 seqs)", err_o), ("packed S_T (all 64 seqs)", err_s)):
        print(f"[parity] {name}: max-rel {e.value():.3e} (bar {TOL['bf16']:.0e})", flush=True)
        assert e.value() <= TOL["bf16"], f"{name}: max-rel {e.value():.3e}"


def test_decode_workload(kla):
    say("decode workload 256 seqs H=16 d=128, 128 steps (full oracle, every sequence and step)")
    wl = workloads.decode()
    dev = "cuda"
    state = wl["state"].to(dev)
    ref_state = wl["state"].double().numpy()
    worst_o = 0.0
    for i, st in enumerate(wl["steps"]):
        o = kla.kla_decode_step(st["q"].to(dev), st["k"].to(dev), st["v"].to(dev),
                                st["alpha"].to(dev), st["eta"].to(dev), state, eps=wl["eps"])
        ro, ref_state = oracle.decode_step(st["q"], st["k"], st["v"], st["alpha"], st["eta"],
                                           ref_state, eps=float(np.float32(wl["eps"])))
        got = o.cpu()
        assert torch.all(torch.isfinite(got)), f"step {i}: non-finite o"
        err = rel(got, ro)
        worst_o = max(worst_o, err)
        assert err <= TOL["bf16"], f"step {i}: o max-rel {err:.3e}"
        if i % 32 == 31:
            print(f"[parity] decode step {i}: o max-rel {err:.3e}", flush=True)
    torch.cuda.synchronize()
    print(f"[parity] decode o worst step (all 256 x 16 pairs): max-rel {worst_o:.3e}", flush=True)
    check("decode final state (all 256 x 16 pairs)", state.cpu(), ref_state, TOL["bf16"])


# ---------------------------------------------------------------- shapes and edges

@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (64, "bf16"), (128, "f32"), (64, "f32")])
def test_ragged_lengths_with_initial_state(kla, d, dtype):
    lengths = [1, 63, 64, 65, 0, 130, 200, 127]
    say(f"ragged packed d={d} {dtype} lengths={lengths} H=3 + initial state")
    inp = workloads.prefill(lengths=lengths, H=3, d=d, dtype=dtype, seed=3)
    g = torch.Generator().manual_seed(5)
    s0 = 0.5 * torch.randn((len(lengths), 3, d, d), generator=g)
    o, S = gpu_fwd(kla, inp, initial_state=s0)
    ro, rS = ref_fwd(inp, initial_state=s0)
    check(f"ragged d={d} {dtype} o", o, ro, TOL[dtype])
    check(f"ragged d={d} {dtype} S_T", S, rS, TOL[dtype])
    # the empty sequence returns its start state exactly
    assert torch.equal(S[4], s0[4])


def test_packed_longest_first_with_ties(kla):
    """Packed sequences with equal lengths (the longest-first order breaks
    ties by index), an empty one and a single token, in an order the
    schedule permutes; every sequence against the oracle."""
    lengths = [70, 300, 70, 0, 300, 1, 70, 129, 64]
    say(f"packed longest-first with ties lengths={lengths} H=3 + initial state")
    inp = workloads.prefill(lengths=lengths, H=3, d=128, dtype="bf16", seed=31)
    s0 = 0.3 * torch.randn((len(lengths), 3, 128, 128), generator=torch.Generator().manual_seed(4))
    o, S = gpu_fwd(kla, inp, initial_state=s0)
    ro, rS = ref_fwd(inp, initial_state=s0)
    check("ties o", o, ro, TOL["bf16"])
    check("ties S_T", S, rS, TOL["bf16"])
    assert torch.equal(S[3], s0[3])


def test_edge_gates_and_keys(kla):
    say("edges: zero keys, alpha=1, eta=0, 100x keys, length-1 sequence")
    inp = workloads.prefill(lengths=[150, 1, 77], H=4, d=128, dtype="bf16", seed=11)
    k, a, e = inp["k"].clone(), inp["alpha"].clone(), inp["eta"].clone()
    k[5, 0] = 0                     # zero key, eps > 0: no write
    k[40:60, 1] *= 100              # huge key norms
    a[:, 2] = 1.0                   # no decay on head 2
    e[100:140, 3] = 0.0             # no write on head 3 for a stretch
    e[10, 0] = 1.0
    inp.update(k=k, alpha=a, eta=e)
    o, S = gpu_fwd(kla, inp)
    ro, rS = ref_fwd(inp)
    check("edges o", o, ro, TOL["bf16"])
    check("edges S_T", S, rS, TOL["bf16"])


def test_final_state_in_place(kla):
    say("final_state aliasing initial_state (in-place)")
    inp = workloads.prefill(lengths=[100, 260], H=2, d=128, dtype="bf16", seed=12)
    s0 = 0.1 * torch.randn((2, 2, 128, 128), generator=torch.Generator().manual_seed(1))
    dev = "cuda"
    st = s0.to(dev)
    o, S = kla.kla_fwd_chunked(inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev),
                               inp["alpha"].to(dev), inp["eta"].to(dev),
                               cu_seqlens=inp["cu_seqlens"].to(dev), initial_state=st,
                               final_state=st, eps=inp["eps"])
    torch.cuda.synchronize()
    ro, rS = ref_fwd(inp, initial_state=s0)
    check("in-place o", o.cpu(), ro, TOL["bf16"])
    check("in-place S_T", st.cpu(), rS, TOL["bf16"])


def test_resume_and_decode_continuation(kla):
    say("prefill split in two + decode continuation")
    inp = workloads.prefill(lengths=[301], H=2, d=128, dtype="bf16", seed=13)
    dev = "cuda"
    cut = 150
    t = {n: inp[n].to(dev) for n in ("q", "k", "v", "alpha", "eta")}
    cu = lambda n: torch.tensor([0, n], dtype=torch.int32, device=dev)
    o1, S1 = kla.kla_fwd_chunked(*(t[n][:cut] for n in ("q", "k", "v", "alpha", "eta")),
                                 cu_seqlens=cu(cut), eps=inp["eps"], output_final_state=True)
    o2, S2 = kla.kla_fwd_chunked(*(t[n][cut:300].contiguous() for n in ("q", "k", "v", "alpha", "eta")),
                                 cu_seqlens=cu(300 - cut), initial_state=S1, eps=inp["eps"],
                                 output_final_state=True)
    od = kla.kla_decode_step(*(t[n][300:301].contiguous() for n in ("q", "k", "v", "alpha", "eta")),
                             S2, eps=inp["eps"])
    torch.cuda.synchronize()
    ro, rS = ref_fwd(inp)
    check("resume o", torch.cat([o1, o2, od]).cpu(), ro, TOL["bf16"])
    check("resume+decode S", S2.cpu(), rS, TOL["bf16"])


def test_deterministic_and_dense_equals_packed(kla):
    say("bitwise determinism; dense layout equals packed layout")
    inp = workloads.prefill(n_seqs=3, T=190, H=5, d=128, dtype="bf16", seed=14)
    o1, S1 = gpu_fwd(kla, inp)
    o2, S2 = gpu_fwd(kla, inp)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    packed = dict(inp, cu_seqlens=torch.tensor([0, 190, 380, 570], dtype=torch.int32))
    o3, S3 = gpu_fwd(kla, packed)
    assert torch.equal(o1, o3) and torch.equal(S1, S3)


def test_decode_matches_oracle_fp32_and_d64(kla):
    for d, dtype in ((64, "f32"), (128, "f32"), (64, "bf16")):
        say(f"decode d={d} {dtype}, 5 steps")
        wl = workloads.decode(n_seqs=7, H=3, d=d, steps=5, dtype=dtype, seed=d)
        state = wl["state"].to("cuda")
        ref = wl["state"].double().numpy()
        for st in wl["steps"]:
            o = kla.kla_decode_step(*(st[n].to("cuda") for n in ("q", "k", "v", "alpha", "eta")),
                                    state, eps=wl["eps"])
            ro, ref = oracle.decode_step(st["q"], st["k"], st["v"], st["alpha"], st["eta"], ref,
                                         eps=float(np.float32(wl["eps"])))
            check(f"decode d={d} {dtype} o", o.cpu(), ro, TOL[dtype])
        check(f"decode d={d} {dtype} S", state.cpu(), ref, TOL[dtype])


def test_errors_raise(kla):
    say("binding raises on unsupported shapes")
    q = torch.zeros((64, 2, 96), dtype=torch.bfloat16, device="cuda")
    a = torch.ones((64, 2), device="cuda")
    with pytest.raises(kla.KLAError):
        kla.kla_fwd_chunked(q, q, q, a, a)
