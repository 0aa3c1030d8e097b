"""gdn_chunk_fwd_noalloc (the prefill with its workspace in the library's fixed per-device array)
against gdn_chunk_fwd with a caller workspace, through the C ABI: the same kernels on the same
inputs give the same bits, and both meet the oracle's tolerance.  Two calls in a row on the
split route (the second smaller, so it runs over what the first left in the array), the same on
the split route in pieces, one on the
fused route (no workspace), and sizes beyond the array's limit rejected with nothing written."""
import numpy as np
import pytest

import gdn_inputs as gi
import oracle
from gpu_util import Guarded, check, dev, f64, host, say

gdn = pytest.importorskip("gated_deltanet_linear_delta_amd")
torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def both(d, chunk=64):
    t = dev(d)
    B, T, Hqk, dk = d["q"].shape
    Hv, dv = d["v"].shape[2], d["v"].shape[3]
    tdt = t["q"].dtype
    o_ref, s_ref = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["s0"], chunk=chunk)
    og = Guarded((B, T, Hv, dv), tdt)
    sg = Guarded((B, Hv, dk, dv), torch.float32)
    gdn.gdn_chunk_fwd_noalloc(t["q"], t["k"], t["v"], t["g"], t["beta"], t["s0"], og.t, sg.t, chunk=chunk)
    torch.cuda.synchronize()
    og.check("noalloc o")
    sg.check("noalloc final state")
    return og.t, sg.t, o_ref, s_ref


def test_noalloc_matches_chunk_fwd_twice_split_route():
    shapes = [dict(B=1, T=4096, Hqk=16, Hv=32, seed=11), dict(B=2, T=700, Hqk=2, Hv=6, seed=12)]
    for sh in shapes:
        name = gdn.gdn_chunk_fwd_kernel_name(sh["B"], sh["T"], sh["Hqk"], sh["Hv"], 128, 128, 64, gdn.GDN_BF16)
        ws = gdn.gdn_chunk_fwd_workspace_bytes(sh["B"], sh["T"], sh["Hqk"], sh["Hv"], 128, 128, 64, gdn.GDN_BF16)
        say(f"noalloc {sh} route={name} workspace={ws}")
        assert name == "mfma_split" and 0 < ws <= gdn.GDN_NOALLOC_SCRATCH_BYTES
        d = gi.generate(B=sh["B"], T=sh["T"], Hqk=sh["Hqk"], Hv=sh["Hv"], dk=128, dv=128, dtype="bf16", mu=3.0,
                        s0_std=0.02, seed=sh["seed"])
        o, s, o_ref, s_ref = both(d)
        assert torch.equal(o, o_ref) and torch.equal(s, s_ref)
        oo, so = oracle.recurrent(f64(d["q"]), f64(d["k"]), f64(d["v"]), d["g"], d["beta"], d["s0"])
        check(f"noalloc {sh}", "bf16", host(o), oo, host(s), so)


def test_noalloc_split_route_in_pieces():
    """A shape whose rows are long enough for the pieced split path (256 chunks, 17 chains that
    leave compute units free) and whose workspace, with the state handed between pieces, still
    fits the array; then a smaller call over what it left."""
    sh = dict(B=1, T=16384, Hqk=1, Hv=17)
    args = (sh["B"], sh["T"], sh["Hqk"], sh["Hv"], 128, 128, 64, gdn.GDN_BF16)
    ws = gdn.gdn_chunk_fwd_workspace_bytes(*args)
    say(f"noalloc pieces {sh} workspace={ws}")
    assert gdn.gdn_chunk_fwd_kernel_name(*args) == "mfma_split"
    # operands of 256 chunks plus the handed-on state: the shape takes pieces
    assert ws == 256 * (17 * 13568 + 64 * 128 * 2) + 17 * 128 * 128 * 4 <= gdn.GDN_NOALLOC_SCRATCH_BYTES
    for i, (T, Hv, seed) in enumerate(((16384, 17, 21), (700, 3, 22))):
        d = gi.generate(B=1, T=T, Hqk=1, Hv=Hv, dk=128, dv=128, dtype="bf16", mu=3.0, s0_std=0.02, seed=seed)
        o, s, o_ref, s_ref = both(d)
        assert torch.equal(o, o_ref) and torch.equal(s, s_ref)
        oo, so = oracle.recurrent(f64(d["q"]), f64(d["k"]), f64(d["v"]), d["g"], d["beta"], d["s0"])
        check(f"noalloc pieces call {i}", "bf16", host(o), oo, host(s), so)


def test_noalloc_fused_route_and_in_place_state():
    d = gi.generate(B=8, T=300, Hqk=8, Hv=32, dk=128, dv=128, dtype="bf16", mu=3.0, s0_std=0.02, seed=13)
    assert gdn.gdn_chunk_fwd_kernel_name(8, 300, 8, 32, 128, 128, 64, gdn.GDN_BF16) == "mfma_pipe"
    o, s, o_ref, s_ref = both(d)
    assert torch.equal(o, o_ref) and torch.equal(s, s_ref)
    t = dev(d)
    st = t["s0"].clone()
    o2 = torch.empty_like(o)
    gdn.gdn_chunk_fwd_noalloc(t["q"], t["k"], t["v"], t["g"], t["beta"], st, o2, st)
    torch.cuda.synchronize()
    assert torch.equal(o2, o_ref) and torch.equal(st, s_ref)


def test_noalloc_rejects_sizes_beyond_the_array():
    # the 64K-token workload's split route needs about 0.9 GB of workspace
    B, T, Hqk, Hv = 1, 65536, 16, 48
    need = gdn.gdn_chunk_fwd_workspace_bytes(B, T, Hqk, Hv, 128, 128, 64, gdn.GDN_BF16)
    assert need > gdn.GDN_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, T, Hqk, 128), dtype=torch.bfloat16, device="cuda:0")
    v = torch.zeros((B, T, Hv, 128), dtype=torch.bfloat16, device="cuda:0")
    g = torch.zeros((B, T, Hv), device="cuda:0")
    o = torch.full((B, T, Hv, 128), 3.0, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_chunk_fwd_noalloc(q, q, v, g, g, None, o)
    assert e.value.status == 5   # GDN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((o == 3.0).all())
