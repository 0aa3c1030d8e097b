"""Parity of the HIP library against the float64 oracle, on the same seeded inputs.

Small shapes span several chunks and a ragged tail and are compared element by element over
whole tensors; the five workload configurations are run in full on the GPU in the launch
configuration the benchmark times, and compared on whole tensors (every chain and token of
every workload, and the 64 decode steps)."""
import numpy as np
import pytest

import gdn_inputs as gi
import oracle
from gpu_util import DEV, TOL, Guarded, check, dev, f64, host, rel_l2, sample_chains, say

gdn = pytest.importorskip("gated_deltanet_linear_delta_amd")
torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def run_prefill(d, chunk, scale=1.0, want_state=True):
    t = dev(d)
    o, sf = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["s0"],
                              output_final_state=want_state, chunk=chunk, scale=scale)
    torch.cuda.synchronize()
    return host(o), (None if sf is None else host(sf))


def oracle_prefill(d, scale=1.0):
    return oracle.recurrent(f64(d["q"]), f64(d["k"]), f64(d["v"]), d["g"], d["beta"], d["s0"], scale=scale)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 128), (128, 64), (128, 128), (32, 128)])
@pytest.mark.parametrize("Hqk,Hv", [(1, 1), (2, 4)])
def test_decode_small(dtype, dk, dv, Hqk, Hv):
    say(f"decode small dtype={dtype} dk={dk} dv={dv} Hqk={Hqk} Hv={Hv}")
    cfg = gi.Config("s", B=3, T=1, Hqk=Hqk, Hv=Hv, dk=dk, dv=dv, chunk=64, dtype=dtype, mu=3.0,
                    s0_std=0.05, seed=dk * 7 + dv + Hv, steps=5)
    d = gi.generate_decode(cfg)
    o_ref, s_ref = oracle.decode(f64(d["q"]), f64(d["k"]), f64(d["v"]), d["g"], d["beta"], d["s0"])
    t = dev(d)
    state = t["s0"].clone()
    outs = []
    for s in range(cfg.steps):
        outs.append(gdn.gdn_recurrent_step(t["q"][s], t["k"][s], t["v"][s], t["g"][s], t["beta"][s], state))
    torch.cuda.synchronize()
    o = np.stack([host(x) for x in outs])
    check(f"decode {dtype} {dk}x{dv}", dtype, o, o_ref, host(state), s_ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv,C,T", [
    (32, 32, 16, 128), (32, 32, 16, 1), (32, 64, 32, 77), (64, 64, 64, 130), (64, 32, 16, 49),
    (128, 128, 64, 200), (128, 128, 32, 96), (128, 64, 64, 65), (32, 128, 64, 63), (128, 128, 16, 40),
])
def test_chunk_small(dtype, dk, dv, C, T):
    say(f"chunk small dtype={dtype} dk={dk} dv={dv} C={C} T={T}")
    d = gi.generate(B=2, T=T, Hqk=2, Hv=4, dk=dk, dv=dv, dtype=dtype, mu=3.0, s0_std=0.05,
                    seed=T * 31 + dk + dv + C)
    o_ref, s_ref = oracle_prefill(d)
    o, s = run_prefill(d, C)
    check(f"chunk {dtype} dk={dk} dv={dv} C={C} T={T}", dtype, o, o_ref, s, s_ref)


def test_tiny_f32_config():
    cfg = gi.CONFIGS["tiny_f32"]
    say(f"config {cfg}")
    d = gi.generate(cfg)
    o_ref, s_ref = oracle_prefill(d)
    o, s = run_prefill(d, cfg.chunk)
    check("tiny_f32", "f32", o, o_ref, s, s_ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_scale_and_no_final_state(dtype):
    say(f"chunk scale dtype={dtype}")
    d = gi.generate(B=1, T=70, Hqk=1, Hv=2, dk=64, dv=64, dtype=dtype, mu=2.0, s0_std=0.1, seed=5)
    o_ref, _ = oracle_prefill(d, scale=0.125)
    o, s = run_prefill(d, 32, scale=0.125, want_state=False)
    assert s is None
    check(f"scale {dtype}", dtype, o, o_ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_in_place_state_and_resume(dtype):
    """final_state == initial_state (in place); two calls over halves equal one call."""
    say(f"chunk in-place/resume dtype={dtype}")
    d = gi.generate(B=2, T=150, Hqk=2, Hv=2, dk=128, dv=128, dtype=dtype, mu=3.0, s0_std=0.05, seed=9)
    o_ref, s_ref = oracle_prefill(d)
    t = dev(d)
    state = t["s0"].clone()
    o1, _ = gdn.gdn_chunk_fwd(t["q"][:, :64].contiguous(), t["k"][:, :64].contiguous(), t["v"][:, :64].contiguous(),
                              t["g"][:, :64].contiguous(), t["beta"][:, :64].contiguous(), state,
                              final_state=state, chunk=64)
    o2, _ = gdn.gdn_chunk_fwd(t["q"][:, 64:].contiguous(), t["k"][:, 64:].contiguous(), t["v"][:, 64:].contiguous(),
                              t["g"][:, 64:].contiguous(), t["beta"][:, 64:].contiguous(), state,
                              final_state=state, chunk=64)
    torch.cuda.synchronize()
    o = np.concatenate([host(o1), host(o2)], axis=1)
    check(f"resume {dtype}", dtype, o, o_ref, host(state), s_ref)


def test_chunk_empty_sequence_and_batch():
    say("chunk T=0 / B=0")
    d = gi.generate(B=2, T=0, Hqk=1, Hv=1, dk=32, dv=32, dtype="f32", mu=3.0, s0_std=0.1, seed=3)
    t = dev(d)
    o, sf = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["s0"], chunk=16)
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 1, 32)
    np.testing.assert_array_equal(host(sf), d["s0"])
    o, sf = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], None, chunk=16)
    torch.cuda.synchronize()
    assert not host(sf).any()
    d = gi.generate(B=0, T=5, Hqk=1, Hv=1, dk=32, dv=32, dtype="bf16", mu=3.0, s0_std=0.0, seed=3)
    t = dev(d)
    o, sf = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], None, chunk=16)
    torch.cuda.synchronize()
    assert o.shape == (0, 5, 1, 32) and sf.shape == (0, 1, 32, 32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_steps_equal_prefill(dtype):
    """T single-token decode steps reach the prefill's outputs and state (both vs the oracle,
    and against each other)."""
    say(f"decode == prefill dtype={dtype}")
    d = gi.generate(B=2, T=40, Hqk=1, Hv=2, dk=128, dv=128, dtype=dtype, mu=3.0, s0_std=0.05, seed=21)
    o_p, s_p = run_prefill(d, 16)
    t = dev(d)
    state = t["s0"].clone()
    outs = []
    for s in range(40):
        outs.append(gdn.gdn_recurrent_step(t["q"][:, s].contiguous(), t["k"][:, s].contiguous(),
                                           t["v"][:, s].contiguous(), t["g"][:, s].contiguous(),
                                           t["beta"][:, s].contiguous(), state))
    torch.cuda.synchronize()
    o_d = np.stack([host(x) for x in outs], axis=1)
    check(f"decode-vs-prefill {dtype}", dtype, o_d, o_p, host(state), s_p)


def test_deterministic():
    say("determinism")
    d = gi.generate(B=1, T=300, Hqk=2, Hv=4, dk=128, dv=128, dtype="bf16", mu=3.0, s0_std=0.02, seed=4)
    t = dev(d)
    r1 = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["s0"], chunk=64)
    r2 = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["s0"], chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1])


def test_qwen3next_prefill_full():
    cfg = gi.CONFIGS["qwen3next_prefill"]
    say(f"config {cfg}")
    d = gi.generate(cfg)
    o, s = run_prefill(d, cfg.chunk)
    o_ref, s_ref = oracle_prefill(d)
    check("qwen3next_prefill", "bf16", o, o_ref, s, s_ref)


@pytest.mark.parametrize("name", ["batched_prefill", "qwen36_long_prefill"])
def test_large_prefill_full(name):
    """The batched (256 chains, S0 != 0) and the 64K-token (48 chains) workloads at full size, in
    the launch configuration the benchmark times, against the oracle over whole tensors (every
    chain, every token), with guard bands after O and the final state."""
    cfg = gi.CONFIGS[name]
    say(f"config {cfg}, whole tensors")
    d = gi.generate(cfg)
    t = dev(d)
    og = Guarded((cfg.B, cfg.T, cfg.Hv, cfg.dv), torch.bfloat16)
    sg = Guarded((cfg.B, cfg.Hv, cfg.dk, cfg.dv), torch.float32)
    gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["s0"], chunk=cfg.chunk, o=og.t,
                      final_state=sg.t)
    torch.cuda.synchronize()
    og.check(name)
    sg.check(name)
    o, s = host(og.t), host(sg.t)
    del t, og, sg
    o_ref, s_ref = oracle_prefill(d)
    check(name, "bf16", o, o_ref, s, s_ref)


def test_decode_config_full():
    """The decode workload (B=256, 32 value heads, 64 steps, state updated in place): every
    output of every step and the whole final state against the oracle."""
    cfg = gi.CONFIGS["decode"]
    say(f"config {cfg}, whole tensors")
    d = gi.generate_decode(cfg)
    t = dev(d)
    state = t["s0"].clone()
    og = Guarded((cfg.steps, cfg.B, cfg.Hv, cfg.dv), torch.bfloat16)
    for s in range(cfg.steps):
        gdn.gdn_recurrent_step(t["q"][s], t["k"][s], t["v"][s], t["g"][s], t["beta"][s], state, o=og.t[s])
    torch.cuda.synchronize()
    og.check("decode")
    oh, sh = host(og.t), host(state)
    del t, state, og
    o_ref, s_ref = oracle.decode(f64(d["q"]), f64(d["k"]), f64(d["v"]), d["g"], d["beta"], d["s0"])
    check("decode config", "bf16", oh, o_ref, sh, s_ref)


def test_kernel_family_dispatch():
    assert gdn.gdn_chunk_fwd_kernel_name(1, 4096, 16, 32, 128, 128, 64, gdn.GDN_BF16) == "mfma_split"
    assert gdn.gdn_chunk_fwd_kernel_name(8, 8192, 16, 32, 128, 128, 64, gdn.GDN_BF16) == "mfma_pipe"
    assert gdn.gdn_chunk_fwd_kernel_name(1, 4096, 16, 32, 128, 128, 32, gdn.GDN_BF16) == "mfma_f32"
    assert gdn.gdn_chunk_fwd_kernel_name(1, 4096, 16, 32, 128, 128, 64, gdn.GDN_F32) == "mfma_f32"


@pytest.mark.parametrize("bv", ["64", "128"])
@pytest.mark.parametrize("dk,dv,T,Hqk,Hv", [(128, 128, 333, 2, 6), (64, 128, 129, 1, 2), (128, 64, 64, 2, 2),
                                            (64, 64, 1, 1, 1), (128, 128, 700, 1, 1)])
def test_mfma_tile_widths(bv, dk, dv, T, Hqk, Hv, monkeypatch, hooks):
    """The fused matrix-core kernel at both column-tile widths, with grouped heads, a ragged last
    chunk and a nonzero initial state."""
    if dv == 64 and bv == "128":
        pytest.skip("a 128-wide tile needs dv = 128")
    monkeypatch.setenv("GDN_MFMA_PATH", "fused")
    monkeypatch.setenv("GDN_MFMA_BV", bv)
    say(f"mfma bv={bv} dk={dk} dv={dv} T={T} Hqk={Hqk} Hv={Hv}")
    assert gdn.gdn_chunk_fwd_kernel_name(2, T, Hqk, Hv, dk, dv, 64, gdn.GDN_BF16) == "mfma"
    d = gi.generate(B=2, T=T, Hqk=Hqk, Hv=Hv, dk=dk, dv=dv, dtype="bf16", mu=3.0, s0_std=0.05, seed=T + dk)
    sc = 0.5 if T == 129 else 1.0
    o_ref, s_ref = oracle_prefill(d, scale=sc)
    o, s = run_prefill(d, 64, scale=sc)
    check(f"mfma bv={bv} dk={dk} dv={dv} T={T}", "bf16", o, o_ref, s, s_ref)


@pytest.mark.parametrize("bv", ["16", "32", "64", "128"])
@pytest.mark.parametrize("dk,dv,T,Hqk,Hv", [(128, 128, 333, 2, 6), (64, 128, 129, 1, 2), (128, 64, 64, 2, 2),
                                            (64, 64, 1, 1, 1), (128, 128, 700, 1, 1), (128, 128, 127, 1, 3)])
def test_pipe_tile_widths(bv, dk, dv, T, Hqk, Hv, monkeypatch, hooks):
    """The pipelined fused kernel (prep waves build chunk n + 1 while the chain waves carry chunk
    n) at every column-tile width, with grouped heads, a ragged last chunk, a nonzero initial
    state and a scale."""
    if int(bv) > dv:
        pytest.skip("tile wider than dv")
    monkeypatch.setenv("GDN_MFMA_PATH", "pipe")
    monkeypatch.setenv("GDN_PIPE_BV", bv)
    say(f"pipe bv={bv} dk={dk} dv={dv} T={T} Hqk={Hqk} Hv={Hv}")
    assert gdn.gdn_chunk_fwd_kernel_name(2, T, Hqk, Hv, dk, dv, 64, gdn.GDN_BF16) == "mfma_pipe"
    d = gi.generate(B=2, T=T, Hqk=Hqk, Hv=Hv, dk=dk, dv=dv, dtype="bf16", mu=3.0, s0_std=0.05, seed=T + dk + 2)
    sc = 0.5 if T == 129 else 1.0
    o_ref, s_ref = oracle_prefill(d, scale=sc)
    o, s = run_prefill(d, 64, scale=sc)
    check(f"pipe bv={bv} dk={dk} dv={dv} T={T}", "bf16", o, o_ref, s, s_ref)


@pytest.mark.parametrize("bv", ["16", "32"])
@pytest.mark.parametrize("dk,dv,T,Hqk,Hv", [(128, 128, 333, 2, 6), (64, 128, 129, 1, 2), (128, 64, 64, 2, 2),
                                            (64, 64, 1, 1, 1), (128, 128, 700, 1, 1), (128, 128, 127, 1, 3)])
def test_split_tile_widths(bv, dk, dv, T, Hqk, Hv, monkeypatch, hooks):
    """The split matrix-core path (per-chunk prep kernel into the workspace, then the state pass)
    at every column-tile width, with grouped heads, a ragged last chunk, a nonzero initial state
    and a scale."""
    if int(bv) > dv:
        pytest.skip("tile wider than dv")
    monkeypatch.setenv("GDN_MFMA_PATH", "split")
    monkeypatch.setenv("GDN_SPLIT_BV", bv)
    say(f"split bv={bv} dk={dk} dv={dv} T={T} Hqk={Hqk} Hv={Hv}")
    assert gdn.gdn_chunk_fwd_kernel_name(2, T, Hqk, Hv, dk, dv, 64, gdn.GDN_BF16) == "mfma_split"
    d = gi.generate(B=2, T=T, Hqk=Hqk, Hv=Hv, dk=dk, dv=dv, dtype="bf16", mu=3.0, s0_std=0.05, seed=T + dk + 1)
    sc = 0.5 if T == 129 else 1.0
    o_ref, s_ref = oracle_prefill(d, scale=sc)
    o, s = run_prefill(d, 64, scale=sc)
    check(f"split bv={bv} dk={dk} dv={dv} T={T}", "bf16", o, o_ref, s, s_ref)


@pytest.mark.parametrize("path", ["fused", "split", "pipe"])
@pytest.mark.parametrize("mu", [3.0, 8.0])
def test_mfma_identical_keys_dense_solve(mu, path, monkeypatch, hooks):
    """All keys of a head equal: the strictly-lower A of every chunk is dense, so every block of
    the (I + A)^{-1} merge carries weight."""
    monkeypatch.setenv("GDN_MFMA_PATH", path)
    say(f"mfma identical keys mu={mu} path={path}")
    d = gi.generate(B=1, T=256, Hqk=2, Hv=4, dk=128, dv=128, dtype="bf16", mu=mu, s0_std=0.05, seed=31)
    d["k"][:] = d["k"][:, :1]
    o_ref, s_ref = oracle_prefill(d)
    o, s = run_prefill(d, 64)
    check(f"identical keys mu={mu}", "bf16", o, o_ref, s, s_ref)


@pytest.mark.parametrize("path", ["fused", "split", "pipe"])
def test_mfma_matches_simt(path, monkeypatch, hooks):
    """Two independent GPU implementations of the chunk algebra agree (and both match the oracle)."""
    say(f"mfma ({path}) vs simt")
    d = gi.generate(B=2, T=500, Hqk=2, Hv=4, dk=128, dv=128, dtype="bf16", mu=3.0, s0_std=0.02, seed=41)
    monkeypatch.setenv("GDN_MFMA_PATH", path)
    assert gdn.gdn_chunk_fwd_kernel_name(2, 500, 2, 4, 128, 128, 64, gdn.GDN_BF16) == \
        {"fused": "mfma", "split": "mfma_split", "pipe": "mfma_pipe"}[path]
    o_m, s_m = run_prefill(d, 64)
    monkeypatch.setenv("GDN_DISABLE_MFMA", "1")
    assert gdn.gdn_chunk_fwd_kernel_name(2, 500, 2, 4, 128, 128, 64, gdn.GDN_BF16) == "mfma_f32"
    o_s, s_s = run_prefill(d, 64)
    check("mfma-vs-simt", "bf16", o_m, o_s, s_m, s_s)


# ---------------------------------------------------------------- layer steps around the recurrence

def _close(name, x, ref, dtype):
    """bf16 outputs: every element within 2^-8 of the oracle relative to its size (one bf16
    rounding is at most 2^-9), plus 1e-5 of the largest; float32: 1e-5 relative plus 1e-6."""
    rel, floor = (2.0 ** -8, 1e-5) if dtype == "bf16" else (1e-5, 1e-6)
    err = np.abs(x - ref)
    bound = rel * np.abs(ref) + floor * max(float(np.abs(ref).max()) if ref.size else 0.0, 1.0)
    worst = float((err / bound).max()) if ref.size else 0.0
    say(f"{name}: max err/bound {worst:.3f}")
    assert worst <= 1.0, f"{name}: error exceeds the bound by {worst:.3f}x"


def run_layer_prologue(d, state_in=True, want_state=True):
    t = dev(d)
    q, k, v, so = gdn.gdn_qkv_prologue(t["q_in"], t["k_in"], t["v_in"], t["conv_q"], t["conv_k"], t["conv_v"],
                                       t["conv_state"] if state_in else None, output_conv_state=want_state)
    torch.cuda.synchronize()
    return host(q), host(k), host(v), (None if so is None else host(so))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,Hqk,Hv,dk,dv,W", [
    (2, 70, 2, 4, 128, 128, 4), (1, 1, 1, 1, 64, 32, 4), (2, 2, 1, 2, 32, 64, 4), (1, 33, 2, 2, 128, 64, 3),
    (3, 64, 1, 3, 64, 128, 2), (1, 96, 2, 4, 32, 32, 1), (2, 31, 4, 8, 128, 128, 4),
])
@pytest.mark.parametrize("state_in", [True, False])
def test_qkv_prologue_small(dtype, B, T, Hqk, Hv, dk, dv, W, state_in):
    say(f"prologue {dtype} B={B} T={T} Hqk={Hqk} Hv={Hv} dk={dk} dv={dv} W={W} state_in={state_in}")
    d = gi.generate_layer(B, T, Hqk, Hv, dk, dv, W=W, dtype=dtype, seed=T * 13 + dk + W, state=True)
    ref = oracle.qkv_prologue(f64(d["q_in"]), f64(d["k_in"]), f64(d["v_in"]), d["conv_q"], d["conv_k"], d["conv_v"],
                              d["conv_state"] if state_in else None)
    q, k, v, so = run_layer_prologue(d, state_in=state_in)
    for nm, x, r in (("q", q, ref[0]), ("k", k, ref[1]), ("v", v, ref[2])):
        _close(f"prologue {nm}", x, r, dtype)
    if W > 1:
        assert np.array_equal(so, ref[3]), "conv state out differs"


def test_qkv_prologue_continuation():
    """Two calls over the halves with the state carried give the one-call result exactly."""
    d = gi.generate_layer(2, 100, 2, 4, 128, 64, W=4, dtype="bf16", seed=77)
    t = dev(d)
    full = gdn.gdn_qkv_prologue(t["q_in"], t["k_in"], t["v_in"], t["conv_q"], t["conv_k"], t["conv_v"],
                                t["conv_state"], output_conv_state=True)
    a = gdn.gdn_qkv_prologue(t["q_in"][:, :37].contiguous(), t["k_in"][:, :37].contiguous(),
                             t["v_in"][:, :37].contiguous(), t["conv_q"], t["conv_k"], t["conv_v"],
                             t["conv_state"], output_conv_state=True)
    b = gdn.gdn_qkv_prologue(t["q_in"][:, 37:].contiguous(), t["k_in"][:, 37:].contiguous(),
                             t["v_in"][:, 37:].contiguous(), t["conv_q"], t["conv_k"], t["conv_v"], a[3],
                             output_conv_state=True)
    torch.cuda.synchronize()
    for i in range(3):
        assert torch.equal(torch.cat([a[i], b[i]], dim=1), full[i])
    assert torch.equal(b[3], full[3])


def test_qkv_prologue_empty_sequence_copies_state():
    d = gi.generate_layer(2, 0, 2, 4, 64, 64, W=4, dtype="bf16", seed=5)
    t = dev(d)
    *_, so = gdn.gdn_qkv_prologue(t["q_in"], t["k_in"], t["v_in"], t["conv_q"], t["conv_k"], t["conv_v"],
                                  t["conv_state"], output_conv_state=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(so), d["conv_state"].astype(np.float64))


def test_qkv_prologue_qwen3next_full():
    """The prologue at the Qwen3-Next shape (T 4096, 16 q/k and 32 value heads of 128), width 4."""
    c = gi.CONFIGS["qwen3next_prefill"]
    say("prologue qwen3next full")
    d = gi.generate_layer(c.B, c.T, c.Hqk, c.Hv, c.dk, c.dv, W=4, dtype="bf16", seed=2002)
    ref = oracle.qkv_prologue(f64(d["q_in"]), f64(d["k_in"]), f64(d["v_in"]), d["conv_q"], d["conv_k"], d["conv_v"],
                              d["conv_state"])
    q, k, v, so = run_layer_prologue(d)
    for nm, x, r in (("q", q, ref[0]), ("k", k, ref[1]), ("v", v, ref[2])):
        _close(f"prologue qwen3next {nm}", x, r, "bf16")
    assert np.array_equal(so, ref[3])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,Hv,dv", [(2, 70, 4, 128), (1, 1, 1, 32), (3, 33, 2, 64), (1, 4096, 32, 128)])
@pytest.mark.parametrize("per_head", [False, True])
def test_gated_rmsnorm(dtype, B, T, Hv, dv, per_head):
    say(f"gated rmsnorm {dtype} B={B} T={T} Hv={Hv} dv={dv} per_head={per_head}")
    d = gi.generate_layer(B, T, 1, Hv, 32, dv, W=1, dtype=dtype, seed=T + dv + Hv, state=False, w_per_head=per_head)
    ref = oracle.gated_rmsnorm(f64(d["o"]), f64(d["z"]), d["weight"])
    t = dev(d)
    y = gdn.gdn_gated_rmsnorm(t["o"], t["z"], t["weight"])
    torch.cuda.synchronize()
    _close("gated rmsnorm", host(y), ref, dtype)
    # in place over o, then over z
    o2, z2 = t["o"].clone(), t["z"].clone()
    gdn.gdn_gated_rmsnorm(o2, t["z"], t["weight"], y=o2)
    gdn.gdn_gated_rmsnorm(t["o"], z2, t["weight"], y=z2)
    torch.cuda.synchronize()
    assert torch.equal(o2, y) and torch.equal(z2, y)


# ------------------------------------------------------- prefill followed by the gated RMSNorm

def _gate_inputs(d, dtype, seed, per_head=False):
    B, T, Hv, dv = d["v"].shape
    return gi.generate_gate(B, T, Hv, dv, dtype=dtype, seed=seed, w_per_head=per_head)


def run_gated(d, gz, chunk=64, y=None):
    t, tz = dev(d), dev(gz)
    y, sf = gdn.gdn_chunk_fwd_gated(t["q"], t["k"], t["v"], t["g"], t["beta"], tz["z"], tz["weight"], t["s0"],
                                    chunk=chunk, y=y)
    torch.cuda.synchronize()
    return y, sf, t, tz


def check_gated(name, dtype, y, y_ref, s, s_ref):
    """y = RMSNorm(O) w silu(z): the norm is scale-invariant per (token, head) row, so the error
    of y relative to its size is that of O's row; the whole-tensor relative L2 bar of O applies.
    Per element the bf16 path rounds O and then y (2 x 2^-9 relative) on top of O's own error,
    so a row's error is bounded by 2^-6 of the row's largest |y| (float32: rel-L2 only)."""
    tol = TOL[dtype]
    r = rel_l2(y, y_ref)
    s_r = rel_l2(s, s_ref)
    msg = f"{name}: rel_l2(y)={r:.3e} rel_l2(S)={s_r:.3e}"
    ok = r <= tol["rel"] and s_r <= tol["rel"]
    if dtype == "bf16":
        rowmax = np.abs(y_ref).max(axis=-1, keepdims=True)
        worst = float((np.abs(y - y_ref) / (2.0 ** -6 * rowmax + 1e-6)).max())
        msg += f" max row-relative err/bound {worst:.3f}"
        ok &= worst <= 1.0
    say(msg)
    assert ok, msg


@pytest.mark.parametrize("route", ["fused", "split", "f32"])
@pytest.mark.parametrize("dk,dv,T,Hqk,Hv", [(128, 128, 333, 2, 6), (64, 128, 129, 1, 2), (128, 64, 64, 2, 2),
                                           (64, 64, 200, 2, 4), (128, 128, 1, 1, 2)])
@pytest.mark.parametrize("per_head", [False, True])
def test_chunk_gated_small(route, dk, dv, T, Hqk, Hv, per_head, monkeypatch, hooks):
    """Every route of gdn_chunk_fwd_gated against the oracle's recurrence followed by the
    oracle's gated RMSNorm, and bit for bit against gdn_chunk_fwd then gdn_gated_rmsnorm."""
    if route == "fused":
        monkeypatch.setenv("GDN_MFMA_PATH", "fused")
        monkeypatch.setenv("GDN_MFMA_BV", str(dv))
    elif route == "split":
        monkeypatch.setenv("GDN_MFMA_PATH", "split")
    else:
        monkeypatch.setenv("GDN_DISABLE_MFMA", "1")
    B = 2
    ws = gdn.gdn_chunk_fwd_gated_workspace_bytes(B, T, Hqk, Hv, dk, dv, 64, gdn.GDN_BF16)
    say(f"gated {route} dk={dk} dv={dv} T={T} Hqk={Hqk} Hv={Hv} per_head={per_head} workspace={ws}")
    assert (ws == 0) == (route == "fused")
    d = gi.generate(B=B, T=T, Hqk=Hqk, Hv=Hv, dk=dk, dv=dv, dtype="bf16", mu=3.0, s0_std=0.02, seed=T + dk + Hv)
    gz = _gate_inputs(d, "bf16", seed=T + 7, per_head=per_head)
    y, sf, t, tz = run_gated(d, gz)
    o_ref, s_ref = oracle_prefill(d)
    y_ref = oracle.gated_rmsnorm(o_ref, f64(gz["z"]), gz["weight"])
    check_gated(f"gated {route}", "bf16", host(y), y_ref, host(sf), s_ref)
    o, sf2 = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["s0"], chunk=64)
    y2 = gdn.gdn_gated_rmsnorm(o, tz["z"], tz["weight"])
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(sf, sf2)


def test_chunk_gated_f32_and_in_place():
    """float32 inputs (vector path; O through the workspace) and y written over z."""
    d = gi.generate(B=2, T=100, Hqk=2, Hv=4, dk=32, dv=64, dtype="f32", mu=3.0, s0_std=0.02, seed=5)
    gz = _gate_inputs(d, "f32", seed=6)
    y, sf, t, tz = run_gated(d, gz, chunk=32)
    o_ref, s_ref = oracle_prefill(d)
    y_ref = oracle.gated_rmsnorm(o_ref, f64(gz["z"]), gz["weight"])
    check_gated("gated f32", "f32", host(y), y_ref, host(sf), s_ref)
    z2 = tz["z"].clone()
    gdn.gdn_chunk_fwd_gated(t["q"], t["k"], t["v"], t["g"], t["beta"], z2, tz["weight"], t["s0"], chunk=32, y=z2)
    torch.cuda.synchronize()
    assert torch.equal(z2, y)


@pytest.mark.parametrize("route", ["fused", "split"])
def test_chunk_gated_bf16_in_place_and_empty(route, monkeypatch, hooks):
    monkeypatch.setenv("GDN_MFMA_PATH", route)
    monkeypatch.setenv("GDN_MFMA_BV", "128")
    d = gi.generate(B=1, T=150, Hqk=1, Hv=2, dk=128, dv=128, dtype="bf16", mu=3.0, s0_std=0.02, seed=8)
    gz = _gate_inputs(d, "bf16", seed=9)
    y, sf, t, tz = run_gated(d, gz)
    z2 = tz["z"].clone()
    gdn.gdn_chunk_fwd_gated(t["q"], t["k"], t["v"], t["g"], t["beta"], z2, tz["weight"], t["s0"], y=z2)
    torch.cuda.synchronize()
    assert torch.equal(z2, y)
    # T == 0: only the final state is written (a copy of the initial state)
    e = {n: (x[:, :0].contiguous() if n not in ("s0",) and x is not None else x) for n, x in t.items()}
    ye, se = gdn.gdn_chunk_fwd_gated(e["q"], e["k"], e["v"], e["g"], e["beta"], tz["z"][:, :0].contiguous(),
                                     tz["weight"], e["s0"])
    torch.cuda.synchronize()
    assert ye.numel() == 0 and torch.equal(se, t["s0"])


def test_chunk_gated_batched_full(monkeypatch, hooks):
    """The many-chain workload at full size with the gated epilogue inside the fused kernel: bit
    for bit equal to that kernel's plain call followed by gdn_gated_rmsnorm, and against the
    oracle over whole tensors."""
    monkeypatch.setenv("GDN_MFMA_PATH", "fused")
    cfg = gi.CONFIGS["batched_prefill"]
    assert gdn.gdn_chunk_fwd_gated_workspace_bytes(cfg.B, cfg.T, cfg.Hqk, cfg.Hv, cfg.dk, cfg.dv, 64, gdn.GDN_BF16) == 0
    say(f"gated batched full {cfg}")
    d = gi.generate(cfg)
    gz = _gate_inputs(d, "bf16", seed=cfg.seed + 5)
    y, sf, t, tz = run_gated(d, gz)
    o, sf2 = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["s0"], chunk=64)
    y2 = gdn.gdn_gated_rmsnorm(o, tz["z"], tz["weight"])
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(sf, sf2)
    del o, y2, sf2
    yh, sh = host(y), host(sf)
    del y, sf, t, tz
    o_ref, s_ref = oracle_prefill(d)
    y_ref = oracle.gated_rmsnorm(o_ref, f64(gz["z"]), gz["weight"])
    del o_ref
    check_gated("gated batched", "bf16", yh, y_ref, sh, s_ref)


def test_chunk_gated_qwen3next_full():
    cfg = gi.CONFIGS["qwen3next_prefill"]
    say(f"gated qwen3next full {cfg}")
    d = gi.generate(cfg)
    gz = _gate_inputs(d, "bf16", seed=cfg.seed + 5, per_head=True)
    y, sf, t, tz = run_gated(d, gz)
    o_ref, s_ref = oracle_prefill(d)
    y_ref = oracle.gated_rmsnorm(o_ref, f64(gz["z"]), gz["weight"])
    check_gated("gated qwen3next", "bf16", host(y), y_ref, host(sf), s_ref)


@pytest.mark.parametrize("T,Hqk,Hv,bv,s0", [
    (2048, 2, 4, 16, True), (4160, 2, 6, 32, True), (3000, 2, 2, 32, False), (2100, 1, 3, 16, True),
])
def test_split_pieces_bitwise(monkeypatch, hooks, T, Hqk, Hv, bv, s0):
    """The split path cut into pieces of 16 chunks (each piece's state pass in one launch with the
    next piece's prep, the state handed on through the workspace; ragged last pieces) gives the
    uncut split path's O and final state bit for bit, and the oracle's to tolerance."""
    monkeypatch.setenv("GDN_MFMA_PATH", "split")
    monkeypatch.setenv("GDN_SPLIT_BV", str(bv))
    monkeypatch.setenv("GDN_SCAN_SEGMENTS", "0")   # not the affine scan, which few chains would take
    say(f"split pieces T={T} Hqk={Hqk} Hv={Hv} bv={bv} s0={s0}")
    d = gi.generate(B=1, T=T, Hqk=Hqk, Hv=Hv, dk=128, dv=128, dtype="bf16", mu=3.0, s0_std=0.05 if s0 else 0.0,
                    seed=T + Hv + bv)
    t = dev(d)
    args = (1, T, Hqk, Hv, 128, 128, 64, gdn.GDN_BF16)
    monkeypatch.setenv("GDN_SPLIT_PIECE", "100000")
    whole_ws = gdn.gdn_chunk_fwd_workspace_bytes(*args)
    o2, s2 = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["s0"], chunk=64)
    monkeypatch.setenv("GDN_SPLIT_PIECE", "16")
    # the pieced route's workspace also holds the state handed from piece to piece
    assert gdn.gdn_chunk_fwd_workspace_bytes(*args) == whole_ws + Hv * 128 * 128 * 4
    o1, s1 = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["s0"], chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    o_ref, s_ref = oracle_prefill(d)
    check(f"split pieces T={T} Hv={Hv}", "bf16", host(o1), o_ref, host(s1), s_ref)


def test_split_pieces_in_place_state_and_gated(monkeypatch, hooks):
    """The pieced split path with the final state written over the initial one (piece 0 reads it,
    the last piece writes it, the pieces between hand the state on through the workspace), and
    under gdn_chunk_fwd_gated (O through the workspace, then the norm): bit for bit the uncut
    split path's results."""
    monkeypatch.setenv("GDN_MFMA_PATH", "split")
    monkeypatch.setenv("GDN_SPLIT_BV", "16")
    monkeypatch.setenv("GDN_SCAN_SEGMENTS", "0")
    d = gi.generate(B=2, T=2200, Hqk=2, Hv=4, dk=128, dv=128, dtype="bf16", mu=3.0, s0_std=0.05, seed=31)
    t = dev(d)
    rng = np.random.Generator(np.random.PCG64(32))
    z = torch.from_numpy(rng.standard_normal((2, 2200, 4, 128)).astype(np.float32)).to("cuda:0").to(torch.bfloat16)
    w = torch.from_numpy((1.0 + 0.1 * rng.standard_normal(128)).astype(np.float32)).to("cuda:0")
    res = {}
    for piece in ("100000", "16"):
        monkeypatch.setenv("GDN_SPLIT_PIECE", piece)
        st = t["s0"].clone()
        o, s = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], st, final_state=st, chunk=64)
        assert s.data_ptr() == st.data_ptr()
        y, sy = gdn.gdn_chunk_fwd_gated(t["q"], t["k"], t["v"], t["g"], t["beta"], z, w, t["s0"], chunk=64)
        torch.cuda.synchronize()
        res[piece] = (o, st, y, sy)
    args = (2, 2200, 2, 4, 128, 128, 64, gdn.GDN_BF16)
    assert gdn.gdn_chunk_fwd_workspace_bytes(*args) == 2 * 35 * (4 * 13568 + 2 * 64 * 128 * 2) + 2 * 4 * 128 * 128 * 4
    a, b = res["100000"], res["16"]
    for x, y_ in zip(a, b):
        assert torch.equal(x, y_)
    o_ref, s_ref = oracle_prefill(d)
    check("split pieces in place", "bf16", host(b[0]), o_ref, host(b[1]), s_ref)
