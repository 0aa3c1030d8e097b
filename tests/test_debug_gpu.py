"""The debug build of the library (libgdn_debug.so, include/gdn_debug.h): on every prefill route
the kernels' index checks hold (no flag raised), and the results are those of the test-hooks
build on the same route bit for bit (the checks change no arithmetic)."""
import numpy as np
import pytest

import gdn_inputs as gi
from gpu_util import dev, say

gdn = pytest.importorskip("gated_deltanet_linear_delta_amd")
torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

def test_debug_flags_path():
    """A check made to fail on purpose (a one-wave kernel with no other work) comes back as its bit,
    and reading clears it; so an all-clear from the route tests below means the checks held."""
    gdn.gdn_debug_take_flags()
    for bit in (0, 6, 31):
        gdn.gdn_debug_self_test(bit)
        assert gdn.gdn_debug_take_flags() == 1 << bit
        assert gdn.gdn_debug_take_flags() == 0


# (route label, environment of the hooks build, shape)
ROUTES = [
    ("split 16-column", {"GDN_MFMA_PATH": "split", "GDN_SPLIT_BV": "16", "GDN_SCAN_SEGMENTS": "0"},
     dict(B=2, T=1000, Hqk=2, Hv=4)),
    ("split 32-column", {"GDN_MFMA_PATH": "split", "GDN_SPLIT_BV": "32", "GDN_SCAN_SEGMENTS": "0"},
     dict(B=1, T=777, Hqk=1, Hv=3)),
    ("split in pieces", {"GDN_MFMA_PATH": "split", "GDN_SPLIT_BV": "32", "GDN_SPLIT_PIECE": "16",
                         "GDN_SCAN_SEGMENTS": "0"}, dict(B=1, T=2100, Hqk=2, Hv=6)),
    ("split in pieces, 16-column", {"GDN_MFMA_PATH": "split", "GDN_SPLIT_BV": "16", "GDN_SPLIT_PIECE": "16",
                                    "GDN_SCAN_SEGMENTS": "0"}, dict(B=1, T=3000, Hqk=1, Hv=2)),
    ("affine scan", {"GDN_MFMA_PATH": "split", "GDN_SCAN_SEGMENTS": "3"}, dict(B=1, T=2000, Hqk=1, Hv=2)),
    ("pipelined", {"GDN_MFMA_PATH": "pipe", "GDN_PIPE_BV": "64"}, dict(B=2, T=300, Hqk=2, Hv=4)),
    ("fused", {"GDN_MFMA_PATH": "fused"}, dict(B=2, T=200, Hqk=2, Hv=4)),
]


def _run(t, env, monkeypatch):
    for kk, vv in env.items():
        monkeypatch.setenv(kk, vv)
    o, sf = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["s0"], chunk=64)
    torch.cuda.synchronize()
    return o, sf


@pytest.mark.parametrize("label,env,shape", ROUTES, ids=[r[0] for r in ROUTES])
def test_debug_checks_hold_on_every_route(monkeypatch, label, env, shape):
    say(f"debug build: {label} {shape}")
    d = gi.generate(dk=128, dv=128, dtype="bf16", mu=3.0, s0_std=0.02, seed=shape["T"] + shape["Hv"], **shape)
    t = dev(d)
    with gdn.test_hooks():
        o_ref, s_ref = _run(t, env, monkeypatch)
    gdn.gdn_debug_take_flags()   # clear whatever an earlier call left
    with gdn.debug_checks():
        o, s = _run(t, env, monkeypatch)
    flags = gdn.gdn_debug_take_flags()
    assert flags == 0, f"{label}: index checks failed, flags {flags:#x}"
    assert torch.equal(o, o_ref) and torch.equal(s, s_ref), label


def test_debug_checks_hold_on_packed_sequences(monkeypatch):
    """Packed variable-length sequences on the split and pipelined routes, an empty one included."""
    lens = [130, 0, 64, 257, 5]
    total = sum(lens)
    d = gi.generate(B=1, T=total, Hqk=2, Hv=4, dk=128, dv=128, dtype="bf16", mu=3.0, s0_std=0.0, seed=7)
    for n in ("q", "k", "v", "g", "beta"):
        d[n] = np.ascontiguousarray(d[n][0])
    rng = np.random.Generator(np.random.PCG64(8))
    d["s0"] = (0.05 * rng.standard_normal((len(lens), 4, 128, 128))).astype(np.float32)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to("cuda:0")
    t = dev(d)
    for env in ({"GDN_MFMA_PATH": "split", "GDN_SCAN_SEGMENTS": "0"}, {"GDN_MFMA_PATH": "pipe"}):
        for kk, vv in env.items():
            monkeypatch.setenv(kk, vv)
        with gdn.test_hooks():
            o_ref, s_ref = gdn.gdn_chunk_fwd_varlen(t["q"], t["k"], t["v"], t["g"], t["beta"], cu, max(lens), t["s0"])
        torch.cuda.synchronize()
        gdn.gdn_debug_take_flags()
        with gdn.debug_checks():
            o, s = gdn.gdn_chunk_fwd_varlen(t["q"], t["k"], t["v"], t["g"], t["beta"], cu, max(lens), t["s0"])
        flags = gdn.gdn_debug_take_flags()
        say(f"debug build: packed {env} flags {flags:#x}")
        assert flags == 0, f"packed {env}: flags {flags:#x}"
        assert torch.equal(o, o_ref) and torch.equal(s, s_ref), env
