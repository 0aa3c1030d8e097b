"""Parity of the packed variable-length prefill (gdn_chunk_fwd_varlen) against the float64 oracle
run on each sequence alone, on every kernel route (fused matrix-core, split matrix-core, float32
vector), with empty, one-token, chunk-sized and ragged sequences; bit equality with the batched
call when all lengths are equal; offsets outside the contract stay in bounds."""
import numpy as np
import pytest

import gdn_inputs as gi
import oracle
from gpu_util import check, dev, f64, host, say

gdn = pytest.importorskip("gated_deltanet_linear_delta_amd")
torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def packed(lengths, Hqk, Hv, dk, dv, dtype, seed):
    """Seeded inputs of sum(lengths) tokens (the recipe of gdn_inputs.generate) and per-sequence
    initial states ~ 0.05 N(0, 1)."""
    total = int(sum(lengths))
    d = gi.generate(B=1, T=max(total, 1), Hqk=Hqk, Hv=Hv, dk=dk, dv=dv, dtype=dtype, mu=3.0, s0_std=0.0, seed=seed)
    for n in ("q", "k", "v", "g", "beta"):
        d[n] = np.ascontiguousarray(d[n][0, :total])
    rng = np.random.Generator(np.random.PCG64(seed + 1))
    d["s0"] = (0.05 * rng.standard_normal((len(lengths), Hv, dk, dv))).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return d, cu


def run_varlen(d, cu, max_len, chunk):
    t = dev(d)
    tcu = torch.from_numpy(cu).to("cuda:0")
    o, sf = gdn.gdn_chunk_fwd_varlen(t["q"], t["k"], t["v"], t["g"], t["beta"], tcu, max_len, t["s0"], chunk=chunk)
    torch.cuda.synchronize()
    return host(o), host(sf)


def oracle_varlen(d, cu):
    os_, ss = [], []
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        sl = {x: f64(d[x][a:b])[None] for x in ("q", "k", "v")}
        o, s = oracle.recurrent(sl["q"], sl["k"], sl["v"], d["g"][a:b][None], d["beta"][a:b][None], d["s0"][n:n + 1])
        os_.append(o[0])
        ss.append(s[0])
    return np.concatenate(os_, axis=0), np.stack(ss)


ROUTES = {"pipe": dict(GDN_MFMA_PATH="pipe"), "fused": dict(GDN_MFMA_PATH="fused"), "split": dict(GDN_MFMA_PATH="split"),
          "f32": dict(GDN_DISABLE_MFMA="1")}


@pytest.mark.parametrize("route", list(ROUTES))
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64)])
def test_varlen_matches_oracle(route, dk, dv, monkeypatch, hooks):
    for k_, v_ in ROUTES[route].items():
        monkeypatch.setenv(k_, v_)
    lengths = [37, 1, 0, 64, 65, 150, 129]
    dtype = "f32" if route == "f32" else "bf16"
    say(f"varlen {route} dk={dk} dv={dv} lengths={lengths}")
    d, cu = packed(lengths, 2, 4, dk, dv, dtype, seed=dk + dv)
    o, s = run_varlen(d, cu, max(lengths), 64 if route != "f32" else 32)
    o_ref, s_ref = oracle_varlen(d, cu)
    check(f"varlen {route}", dtype, o, o_ref, s, s_ref)


@pytest.mark.parametrize("route", ["pipe", "fused", "split"])
def test_varlen_equal_lengths_equal_batched(route, monkeypatch, hooks):
    """Equal lengths L: the same bits as gdn_chunk_fwd over B = N rows of L tokens."""
    monkeypatch.setenv("GDN_MFMA_PATH", route)
    N, L, Hqk, Hv, d_ = 3, 200, 2, 4, 128
    d, cu = packed([L] * N, Hqk, Hv, d_, d_, "bf16", seed=9)
    o, s = run_varlen(d, cu, L, 64)
    t = dev(d)
    rs = lambda x, *shape: x.reshape(*shape).contiguous()
    ob, sb = gdn.gdn_chunk_fwd(rs(t["q"], N, L, Hqk, d_), rs(t["k"], N, L, Hqk, d_), rs(t["v"], N, L, Hv, d_),
                               rs(t["g"], N, L, Hv), rs(t["beta"], N, L, Hv), t["s0"], chunk=64)
    torch.cuda.synchronize()
    assert np.array_equal(o, host(ob).reshape(N * L, Hv, d_)) and np.array_equal(s, host(sb))


def test_varlen_all_empty_and_out_of_contract_offsets():
    d, cu = packed([0, 0], 1, 2, 64, 64, "bf16", seed=3)
    d2, _ = packed([5], 1, 2, 64, 64, "bf16", seed=3)
    t = dev(d2)
    s0 = torch.from_numpy(d["s0"]).to("cuda:0")
    tcu = torch.from_numpy(cu).to("cuda:0")
    o, sf = gdn.gdn_chunk_fwd_varlen(t["q"][:0], t["k"][:0], t["v"][:0], t["g"][:0], t["beta"][:0], tcu, 10, s0)
    torch.cuda.synchronize()
    assert torch.equal(sf, s0)
    # offsets outside the contract (negative, past the end, decreasing, longer than max_seqlen):
    # the kernels clamp them, so the call completes; the results are unspecified
    bad = torch.tensor([-7, 3, 1, 99], dtype=torch.int32, device="cuda:0")
    s3 = torch.zeros((3, 2, 64, 64), device="cuda:0")
    for route in ("pipe", "fused", "split"):
        import os
        os.environ["GDN_MFMA_PATH"] = route
        try:
            with gdn.test_hooks():
                gdn.gdn_chunk_fwd_varlen(t["q"], t["k"], t["v"], t["g"], t["beta"], bad, 2, s3)
                torch.cuda.synchronize()
        finally:
            del os.environ["GDN_MFMA_PATH"]
