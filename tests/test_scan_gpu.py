"""Parity of the affine chunk scan (gdn_chunk_fwd_scan) and of the per-stretch state maps
(gdn_chunk_transport) against the float64 oracle on the same seeded inputs: several segment
counts (one chunk per segment, uneven last segments, more segments asked than chunks), ragged T,
grouped heads, scale, an initial state, in place; maps against oracle.transport, including T = 0;
the scan against the unsegmented call; the 64K-token workloads at full size over whole tensors."""
import numpy as np
import pytest

import gdn_inputs as gi
import oracle
from gpu_util import check, dev, f64, host, rel_l2, say

gdn = pytest.importorskip("gated_deltanet_linear_delta_amd")
torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def run_scan(d, segments, scale=1.0):
    t = dev(d)
    o, sf = gdn.gdn_chunk_fwd_scan(t["q"], t["k"], t["v"], t["g"], t["beta"], t["s0"], segments=segments, scale=scale)
    torch.cuda.synchronize()
    return host(o), host(sf)


def oracle_prefill(d, scale=1.0):
    return oracle.recurrent(f64(d["q"]), f64(d["k"]), f64(d["v"]), d["g"], d["beta"], d["s0"], scale=scale)


@pytest.mark.parametrize("segments", [1, 2, 3, 4, 100])
@pytest.mark.parametrize("dk,dv,T,Hqk,Hv", [(128, 128, 640, 1, 2), (64, 128, 1000, 2, 4), (128, 64, 257, 2, 2),
                                           (64, 64, 450, 1, 3)])
def test_scan_small(segments, dk, dv, T, Hqk, Hv):
    say(f"scan segments={segments} dk={dk} dv={dv} T={T} Hqk={Hqk} Hv={Hv} -> "
        f"{gdn.gdn_chunk_fwd_scan_segments(2, T, Hqk, Hv, dk, dv, 64, gdn.GDN_BF16, segments)} used")
    d = gi.generate(B=2, T=T, Hqk=Hqk, Hv=Hv, dk=dk, dv=dv, dtype="bf16", mu=3.0, s0_std=0.05, seed=T + dk + segments)
    o, s = run_scan(d, segments, scale=0.8)
    o_ref, s_ref = oracle_prefill(d, scale=0.8)
    check(f"scan P={segments}", "bf16", o, o_ref, s, s_ref)


def test_scan_strong_and_weak_decay():
    for mu in (-2.0, 8.0):
        d = gi.generate(B=1, T=700, Hqk=2, Hv=2, dk=128, dv=128, dtype="bf16", mu=mu, s0_std=0.05, seed=11)
        o, s = run_scan(d, 5)
        o_ref, s_ref = oracle_prefill(d)
        check(f"scan mu={mu}", "bf16", o, o_ref, s, s_ref)


def test_scan_equals_unsegmented_and_in_place():
    d = gi.generate(B=1, T=1300, Hqk=2, Hv=4, dk=128, dv=128, dtype="bf16", mu=3.0, s0_std=0.02, seed=12)
    t = dev(d)
    o1, s1 = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["s0"])
    st = t["s0"].clone()
    o2, _ = gdn.gdn_chunk_fwd_scan(t["q"], t["k"], t["v"], t["g"], t["beta"], st, final_state=st, segments=6)
    torch.cuda.synchronize()
    check("scan == unsegmented", "bf16", host(o2), host(o1), host(st), host(s1))
    # one segment is the unsegmented split path itself
    o3, s3 = gdn.gdn_chunk_fwd_scan(t["q"], t["k"], t["v"], t["g"], t["beta"], t["s0"], segments=1)
    torch.cuda.synchronize()
    assert gdn.gdn_chunk_fwd_kernel_name(1, 1300, 2, 4, 128, 128) == "mfma_split"
    assert torch.equal(o3, o1) and torch.equal(s3, s1)


def test_scan_empty_and_no_state():
    d = gi.generate(B=2, T=300, Hqk=1, Hv=2, dk=64, dv=64, dtype="bf16", mu=3.0, s0_std=0.0, seed=13)
    assert d["s0"] is None
    o, s = run_scan(d, 3)
    o_ref, s_ref = oracle_prefill(d)
    check("scan no initial state", "bf16", o, o_ref, s, s_ref)
    t = dev(gi.generate(B=2, T=300, Hqk=1, Hv=2, dk=64, dv=64, dtype="bf16", mu=3.0, s0_std=0.05, seed=14))
    e = {n: (x[:, :0].contiguous() if n != "s0" else x) for n, x in t.items()}
    o0, s0 = gdn.gdn_chunk_fwd_scan(e["q"], e["k"], e["v"], e["g"], e["beta"], e["s0"], segments=4)
    torch.cuda.synchronize()
    assert o0.numel() == 0 and torch.equal(s0, t["s0"])


# ------------------------------------------------------------------- per-stretch state maps

@pytest.mark.parametrize("dk,dv,T,Hqk,Hv,mu", [(128, 128, 200, 1, 2, 3.0), (64, 128, 64, 2, 4, 3.0),
                                              (128, 64, 1, 1, 1, 3.0), (64, 64, 333, 1, 3, 3.0),
                                              (128, 128, 640, 1, 2, 3.0), (128, 128, 1280, 1, 2, 6.0)])
def test_transport_small(dk, dv, T, Hqk, Hv, mu):
    """M to the state tolerance relative to its own size, also after many chunks: after 10 chunks
    at mu = 3 M is near e^-31 (far below float16's range; the kernel rescales its columns by
    powers of two), after 20 chunks at mu = 6 the erases have shrunk it unevenly.  (M is float32:
    stretches that decay it below float32's normal range, about e^-87, are not tested for its
    relative error; the composed state is tested instead.)"""
    say(f"transport dk={dk} dv={dv} T={T} Hqk={Hqk} Hv={Hv} mu={mu}")
    d = gi.generate(B=2, T=T, Hqk=Hqk, Hv=Hv, dk=dk, dv=dv, dtype="bf16", mu=mu, s0_std=0.0, seed=T + dv)
    t = dev(d)
    M, N = gdn.gdn_chunk_transport(t["k"], t["v"], t["g"], t["beta"])
    torch.cuda.synchronize()
    M_ref, N_ref = oracle.transport(f64(d["k"]), f64(d["v"]), d["g"], d["beta"])
    em, en = rel_l2(host(M), M_ref), rel_l2(host(N), N_ref)
    say(f"transport: rel_l2(M)={em:.3e} rel_l2(N)={en:.3e}")
    assert em <= 1e-2 and en <= 1e-2
    # with q given the result is the same (q does not enter the state)
    M2, N2 = gdn.gdn_chunk_transport(t["k"], t["v"], t["g"], t["beta"], q=t["q"])
    torch.cuda.synchronize()
    assert torch.equal(M2, M) and torch.equal(N2, N)


def test_transport_maps_compose_to_the_prefill_state():
    """Two stretches' maps composed from an initial state give the prefill's final state."""
    d = gi.generate(B=1, T=900, Hqk=2, Hv=4, dk=128, dv=128, dtype="bf16", mu=3.0, s0_std=0.05, seed=15)
    t = dev(d)
    h = t["s0"]
    for a, b in ((0, 320), (320, 900)):
        x = {n: y[:, a:b].contiguous() for n, y in t.items() if n != "s0"}
        M, N = gdn.gdn_chunk_transport(x["k"], x["v"], x["g"], x["beta"])
        h = torch.matmul(M, h) + N
    torch.cuda.synchronize()
    _, s_ref = oracle_prefill(d)
    e = rel_l2(host(h), s_ref)
    say(f"composed maps: rel_l2(S)={e:.3e}")
    assert e <= 1e-2


def test_transport_empty():
    d = dev(gi.generate(B=2, T=5, Hqk=1, Hv=2, dk=64, dv=128, dtype="bf16", mu=3.0, s0_std=0.0, seed=16))
    e = {n: (x[:, :0].contiguous() if n != "s0" else x) for n, x in d.items()}
    M = torch.full((2, 2, 64, 64), 7.0, device="cuda:0")
    N = torch.full((2, 2, 64, 128), 7.0, device="cuda:0")
    gdn.gdn_chunk_transport(e["k"], e["v"], e["g"], e["beta"], m_out=M, n_out=N)
    torch.cuda.synchronize()
    assert torch.equal(M, torch.eye(64, device="cuda:0").expand(2, 2, 64, 64)) and not N.any()


# ------------------------------------------------------------------- full-size workloads

@pytest.mark.parametrize("name,segments", [("qwen36_long_prefill_tp8", 6), ("qwen36_long_prefill", 4)])
def test_scan_long_full(name, segments):
    """The scan on one GPU's share of the 64K-token workload under an 8-way head split and on the
    whole workload, against the oracle over whole tensors."""
    cfg = gi.CONFIGS[name]
    say(f"scan {cfg} segments={segments}, whole tensors")
    d = gi.generate(cfg)
    o, s = run_scan(d, segments)
    o_ref, s_ref = oracle_prefill(d)
    check(f"{name} scan", "bf16", o, o_ref, s, s_ref)


def test_chunk_fwd_picks_the_scan_for_scarce_long_chains(monkeypatch, hooks):
    """B1 T17000, 2 value heads of d 64: gdn_chunk_fwd runs the scan by itself (33 segments);
    against the oracle, and against the unsegmented call forced by GDN_SCAN_SEGMENTS=0."""
    assert gdn.gdn_chunk_fwd_kernel_name(1, 17000, 1, 2, 64, 64, 64, gdn.GDN_BF16) == "mfma_scan"
    d = gi.generate(B=1, T=17000, Hqk=1, Hv=2, dk=64, dv=64, dtype="bf16", mu=4.0, s0_std=0.05, seed=17)
    t = dev(d)
    o, s = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["s0"])
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_prefill(d)
    check("gdn_chunk_fwd auto scan", "bf16", host(o), o_ref, host(s), s_ref)
    monkeypatch.setenv("GDN_SCAN_SEGMENTS", "0")
    assert gdn.gdn_chunk_fwd_kernel_name(1, 17000, 1, 2, 64, 64, 64, gdn.GDN_BF16) == "mfma_split"
    o1, s1 = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["s0"])
    torch.cuda.synchronize()
    check("auto scan == unsegmented", "bf16", host(o), host(o1), host(s), host(s1))
