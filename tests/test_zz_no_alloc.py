"""The no-allocation split-sequence prefill (C ABI
`kla_fwd_chunked_split_noalloc`, scratch in the library's static device
array) against the workspace entry point `kla_fwd_chunked_split` on the same
inputs: two calls in a row, the second with a smaller input, each equal to
the workspace call bit for bit and within the oracle's bar."""
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
    return float(np.max(np.abs(x - y)) / max(float(np.max(np.abs(y))), 1e-300))


@pytest.fixture(scope="module")
def kla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import delta_rule_linear_amd as pkg
    return pkg


def run_case(kla, lengths, H, d, dtype, n_splits, seed):
    print(f"[case] noalloc split: lengths={lengths} H={H} d={d} {dtype} n_splits={n_splits}",
          flush=True)
    inp = workloads.prefill(lengths=lengths, H=H, d=d, dtype=dtype, seed=seed)
    dev = "cuda"
    t = {n: inp[n].to(dev) for n in ("q", "k", "v", "alpha", "eta", "cu_seqlens")}
    n = len(lengths)
    s0 = 0.1 * torch.randn((n, H, d, d), generator=torch.Generator().manual_seed(seed))
    s0d = s0.to(dev)
    args = (t["q"], t["k"], t["v"], t["alpha"], t["eta"])
    o_ws, S_ws = kla.kla_fwd_chunked_split(*args, cu_seqlens=t["cu_seqlens"], initial_state=s0d,
                                           eps=inp["eps"], n_splits=n_splits,
                                           output_final_state=True)
    o_na = torch.empty_like(o_ws)
    S_na = torch.empty_like(S_ws)
    kla.kla_fwd_chunked_split_noalloc(*args, cu_seqlens=t["cu_seqlens"], initial_state=s0d,
                                      eps=inp["eps"], n_splits=n_splits, o=o_na, final_state=S_na)
    torch.cuda.synchronize()
    assert torch.equal(o_na, o_ws) and torch.equal(S_na, S_ws)
    ro, rS = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["eta"],
                        cu_seqlens=inp["cu_seqlens"].numpy(), eps=float(np.float32(inp["eps"])),
                        initial_state=s0)
    e_o, e_s = rel(o_na.cpu(), ro), rel(S_na.cpu(), rS)
    print(f"[parity] noalloc o {e_o:.3e}, S_T {e_s:.3e} (bar {TOL[dtype]:.0e})", flush=True)
    assert e_o <= TOL[dtype] and e_s <= TOL[dtype]


def test_noalloc_split_two_calls(kla):
    # the larger call first, then a smaller one (fewer sequences, heads and
    # splits, other head size and input type): the second reuses the array
    # the first left filled
    run_case(kla, [3000, 130, 2500, 1], H=8, d=128, dtype="bf16", n_splits=5, seed=21)
    run_case(kla, [700, 65], H=3, d=64, dtype="f32", n_splits=3, seed=22)


def test_noalloc_split_rejects_beyond_the_array(kla):
    print("[case] noalloc split: workspace beyond the 32 MiB array is refused", flush=True)
    # 2 sequences x 16 heads at d = 128 with 7 splits need 38 MiB of maps and states
    q = torch.zeros((2, 64, 16, 128), dtype=torch.bfloat16, device="cuda")
    a = torch.ones((2, 64, 16), device="cuda")
    o = torch.empty((2, 64, 16, 128), device="cuda")
    with pytest.raises(kla.KLAError) as ex:
        kla.kla_fwd_chunked_split_noalloc(q, q, q, a, a, n_splits=7, o=o)
    assert ex.value.status == -3
