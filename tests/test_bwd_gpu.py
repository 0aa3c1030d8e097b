"""Parity of the HIP backward pass (gdn_chunk_bwd) against the float64 oracle's adjoint
(oracle.recurrent_bwd), on the same seeded inputs: small shapes over several chunks with a ragged
tail, grouped heads, scale, optional initial state and final-state gradient, float32 and bf16;
the Qwen3-Next-shaped workload at full size on sampled query/key-head groups; determinism."""
import numpy as np
import pytest

import gdn_inputs as gi
import oracle
from gpu_util import dev, f64, host, rel_l2, say

gdn = pytest.importorskip("gated_deltanet_linear_delta_amd")
torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

# float32 inputs: relative L2 <= 1e-4 per gradient tensor.  bf16 inputs: the oracle sees the same
# bf16 values; the sequential passes take float16 matrix-core operands (2^-11 relative), the
# per-chunk gradients are float32 and dq, dk, dv are rounded to bf16 (2^-9 relative), so relative
# L2 <= 1e-2 as for the forward outputs.
TOL = {"f32": 1e-4, "bf16": 1e-2}
KEYS = ("dq", "dk", "dv", "dg", "dbeta", "ds0")


def _grad_inputs(d, dtype, seed, with_dsf=True):
    """dL/dO ~ N(0, 1) in the input dtype, dL/dS_final ~ 0.1 N(0, 1) float32."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B, T, Hv, dv = d["v"].shape
    dk = d["q"].shape[3]
    do = rng.standard_normal((B, T, Hv, dv), dtype=np.float32)
    do = gi.bf16_bits(do) if dtype == "bf16" else do
    dsf = (0.1 * rng.standard_normal((B, Hv, dk, dv))).astype(np.float32) if with_dsf else None
    return do, dsf


def run_bwd(d, do, dsf, scale=1.0):
    t = dev(d)
    gdo = gi.to_torch(do, None, "cuda:0")
    gdsf = None if dsf is None else gi.to_torch(dsf, None, "cuda:0")
    r = gdn.gdn_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], gdo, t["s0"], gdsf, scale=scale)
    torch.cuda.synchronize()
    return {kk: (None if x is None else host(x)) for kk, x in r.items()}


def oracle_bwd(d, do, dsf, scale=1.0):
    return oracle.recurrent_bwd(f64(d["q"]), f64(d["k"]), f64(d["v"]), d["g"], d["beta"], d["s0"], f64(do), dsf,
                                scale=scale)


def check_bwd(name, dtype, got, ref, keys=KEYS):
    msgs, ok = [], True
    for kk in keys:
        e = rel_l2(got[kk], ref[kk])
        msgs.append(f"{kk}={e:.2e}")
        ok &= e <= TOL[dtype]
    say(f"{name}: rel_l2 " + " ".join(msgs))
    assert ok, f"{name}: " + " ".join(msgs) + f" tolerance {TOL[dtype]}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv,T,Hqk,Hv", [
    (32, 32, 100, 1, 1), (64, 128, 65, 1, 2), (128, 64, 32, 2, 2), (128, 128, 97, 2, 4), (32, 128, 1, 2, 6),
    (64, 32, 130, 1, 3),
])
def test_chunk_bwd_small(dtype, dk, dv, T, Hqk, Hv):
    say(f"bwd {dtype} dk={dk} dv={dv} T={T} Hqk={Hqk} Hv={Hv}")
    d = gi.generate(B=2, T=T, Hqk=Hqk, Hv=Hv, dk=dk, dv=dv, dtype=dtype, mu=3.0, s0_std=0.05, seed=T + dk + Hv)
    do, dsf = _grad_inputs(d, dtype, seed=T + 11)
    got = run_bwd(d, do, dsf)
    check_bwd(f"bwd {dtype} {dk}x{dv} T{T}", dtype, got, oracle_bwd(d, do, dsf))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_bwd_scale_no_state_no_final_grad(dtype):
    d = gi.generate(B=1, T=77, Hqk=2, Hv=4, dk=64, dv=64, dtype=dtype, mu=2.0, s0_std=0.0, seed=3)
    assert d["s0"] is None
    do, _ = _grad_inputs(d, dtype, seed=4, with_dsf=False)
    got = run_bwd(d, do, None, scale=0.125)
    check_bwd(f"bwd {dtype} scale", dtype, got, oracle_bwd(d, do, None, scale=0.125))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_bwd_strong_decay_and_identical_keys(dtype):
    """Gates near 0 and 1 (mu = -2 and 8) and one key repeated (a dense A in every chunk)."""
    for mu in (-2.0, 8.0):
        d = gi.generate(B=1, T=96, Hqk=1, Hv=2, dk=64, dv=64, dtype=dtype, mu=mu, s0_std=0.05, seed=9)
        d["k"][:] = d["k"][:, :1]
        do, dsf = _grad_inputs(d, dtype, seed=10)
        check_bwd(f"bwd {dtype} mu={mu} identical keys", dtype, run_bwd(d, do, dsf), oracle_bwd(d, do, dsf))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", ["alpha0_some", "alpha_tiny", "alpha1", "beta0", "beta1"])
def test_chunk_bwd_gate_limits(case, dtype):
    """The gate limits of "Gated Attention Architectures", section 3 (alpha -> 0 clears the
    memory, alpha = 1 is the pure delta rule) and the write strength's ends (beta = 0 and 1),
    through the backward, with an initial state, several chunks and a ragged tail."""
    d = gi.generate(B=2, T=133, Hqk=2, Hv=4, dk=128, dv=64, dtype=dtype, mu=3.0, s0_std=0.05,
                    seed=sum(map(ord, case)))
    rng = np.random.Generator(np.random.PCG64(sum(map(ord, case)) + 1))
    if case == "alpha0_some":      # alpha = 0 (g = -inf) on about a quarter of the tokens
        d["g"][rng.random(d["g"].shape) < 0.25] = -np.inf
    elif case == "alpha_tiny":     # alpha = e^-60 everywhere
        d["g"][:] = -60.0
    elif case == "alpha1":
        d["g"][:] = 0.0
    elif case == "beta0":
        d["beta"][:] = 0.0
    else:
        d["beta"][:] = 1.0
    do, dsf = _grad_inputs(d, dtype, seed=17)
    got = run_bwd(d, do, dsf)
    for kk in KEYS:
        assert np.isfinite(got[kk]).all(), kk
    ref = oracle_bwd(d, do, dsf)
    if case == "alpha_tiny":
        # dg and dS0 are O(alpha) = O(e^-60) here.  The chunkwise form reaches dg as a difference
        # of O(1) terms whose O(alpha) remainder lies below their rounding (the float64
        # oracle.chunked_bwd misses it as well), and the float16 operands of the bf16 passes flush
        # e^-60 to zero; so those two are held to an absolute bound far below the O(1) gradients.
        for kk in ("dg", "ds0"):
            err = float(np.abs(got[kk] - ref[kk]).max())
            say(f"bwd {dtype} {case}: max |{kk} - ref| = {err:.2e} (|ref| <= {np.abs(ref[kk]).max():.1e})")
            assert err <= 1e-6, kk
        check_bwd(f"bwd {dtype} {case}", dtype, got, ref, keys=("dq", "dk", "dv", "dbeta"))
    else:
        check_bwd(f"bwd {dtype} {case}", dtype, got, ref)


def test_chunk_bwd_empty_and_no_initial_grad():
    d = gi.generate(B=2, T=40, Hqk=1, Hv=2, dk=32, dv=32, dtype="f32", mu=3.0, s0_std=0.05, seed=12)
    do, dsf = _grad_inputs(d, "f32", seed=13)
    t = dev(d)
    gdo = gi.to_torch(do, None, "cuda:0")
    gdsf = gi.to_torch(dsf, None, "cuda:0")
    r = gdn.gdn_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], gdo, t["s0"], gdsf, want_grad_initial_state=False)
    full = gdn.gdn_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], gdo, t["s0"], gdsf)
    torch.cuda.synchronize()
    assert r["ds0"] is None
    for kk in ("dq", "dk", "dv", "dg", "dbeta"):
        assert torch.equal(r[kk], full[kk]), kk
    # T == 0: only the initial state's gradient, equal to the final state's
    e = {n: (x[:, :0].contiguous() if n != "s0" else x) for n, x in t.items()}
    r0 = gdn.gdn_chunk_bwd(e["q"], e["k"], e["v"], e["g"], e["beta"], gdo[:, :0].contiguous(), e["s0"], gdsf)
    torch.cuda.synchronize()
    assert torch.equal(r0["ds0"], gdsf)


def test_chunk_bwd_deterministic():
    d = gi.generate(B=1, T=200, Hqk=2, Hv=4, dk=128, dv=128, dtype="bf16", mu=3.0, s0_std=0.02, seed=14)
    do, dsf = _grad_inputs(d, "bf16", seed=15)
    a, b = run_bwd(d, do, dsf), run_bwd(d, do, dsf)
    for kk in KEYS:
        assert np.array_equal(a[kk], b[kk]), kk


def test_chunk_bwd_qwen3next_sampled():
    """The Qwen3-Next shape at full size; the oracle recomputes two query/key heads with all
    the value heads of their groups (a head group's dq, dk need every value head of it)."""
    cfg = gi.CONFIGS["qwen3next_prefill"]
    say(f"bwd full {cfg}")
    d = gi.generate(cfg)
    do, dsf = _grad_inputs(d, "bf16", seed=cfg.seed + 3)
    got = run_bwd(d, do, dsf)
    grp = cfg.Hv // cfg.Hqk
    for i in (0, 11):
        js = list(range(i * grp, (i + 1) * grp))
        sub = {"q": d["q"][:, :, i:i + 1], "k": d["k"][:, :, i:i + 1], "v": d["v"][:, :, js], "g": d["g"][:, :, js],
               "beta": d["beta"][:, :, js], "s0": None if d["s0"] is None else d["s0"][:, js]}
        ref = oracle_bwd(sub, do[:, :, js], None if dsf is None else dsf[:, js])
        sel = {"dq": got["dq"][:, :, i:i + 1], "dk": got["dk"][:, :, i:i + 1], "dv": got["dv"][:, :, js],
               "dg": got["dg"][:, :, js], "dbeta": got["dbeta"][:, :, js], "ds0": got["ds0"][:, js]}
        check_bwd(f"bwd qwen3next head group {i}", "bf16", sel, ref)
