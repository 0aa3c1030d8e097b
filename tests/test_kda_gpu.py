"""Parity of the HIP Kimi Delta Attention prefill (gdn_kda_chunk_fwd) against the float64 KDA
oracle (oracle.kda_recurrent) on the same seeded inputs, element by element over whole tensors,
for both routes (float32 vector kernel, chunks 16 and 32; matrix-core kernels, chunk 64):
several chunks with a ragged tail, grouped heads, scale, strong per-channel decays, in-place
state, empty inputs; the routes against each other and the equal-decay case against the Gated
DeltaNet kernels; the Qwen3-Next-shaped KDA workload at full size over whole tensors."""
import numpy as np
import pytest

import gdn_inputs as gi
import oracle
from gpu_util import check, dev, f64, host, say

gdn = pytest.importorskip("gated_deltanet_linear_delta_amd")
torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def run_kda(d, chunk=32, scale=1.0, want_state=True):
    t = dev(d)
    o, sf = gdn.gdn_kda_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["s0"], output_final_state=want_state,
                                  chunk=chunk, scale=scale)
    torch.cuda.synchronize()
    return host(o), (None if sf is None else host(sf))


def oracle_kda(d, scale=1.0):
    return oracle.kda_recurrent(f64(d["q"]), f64(d["k"]), f64(d["v"]), d["g"], d["beta"], d["s0"], scale=scale)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [16, 32])
@pytest.mark.parametrize("dk,dv,T,Hqk,Hv", [(32, 32, 100, 1, 1), (64, 128, 65, 1, 2), (128, 64, 32, 2, 2),
                                           (128, 128, 97, 2, 4), (32, 128, 1, 2, 6)])
def test_kda_small(dtype, chunk, dk, dv, T, Hqk, Hv):
    say(f"kda {dtype} C={chunk} dk={dk} dv={dv} T={T} Hqk={Hqk} Hv={Hv}")
    d = gi.generate_kda(B=2, T=T, Hqk=Hqk, Hv=Hv, dk=dk, dv=dv, dtype=dtype, mu=2.0, s0_std=0.05, seed=T + dk + Hv)
    o, s = run_kda(d, chunk)
    o_ref, s_ref = oracle_kda(d)
    check(f"kda {dtype} C{chunk}", dtype, o, o_ref, s, s_ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_kda_strong_channel_decay_and_scale(dtype):
    """Some channels nearly cleared every token (mu = -3), others nearly kept (mu = 8)."""
    for mu in (-3.0, 8.0):
        d = gi.generate_kda(B=1, T=80, Hqk=2, Hv=2, dk=64, dv=64, dtype=dtype, mu=mu, s0_std=0.05, seed=21)
        o, s = run_kda(d, 32, scale=0.3)
        o_ref, s_ref = oracle_kda(d, scale=0.3)
        check(f"kda {dtype} mu={mu}", dtype, o, o_ref, s, s_ref)


def test_kda_equal_decay_matches_gated_deltanet():
    """One decay per head copied to every channel: the KDA kernel and the Gated DeltaNet float32
    kernel compute the same recurrence (GPU against GPU, float32 tolerance)."""
    d = gi.generate(B=2, T=90, Hqk=2, Hv=4, dk=64, dv=128, dtype="f32", mu=3.0, s0_std=0.05, seed=22)
    dk_ = d["q"].shape[3]
    dd = dict(d)
    dd["g"] = np.ascontiguousarray(np.repeat(d["g"][..., None], dk_, axis=-1))
    o_k, s_k = run_kda(dd, 32)
    t = dev(d)
    o_g, s_g = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["s0"], chunk=32)
    torch.cuda.synchronize()
    check("kda == gdn (equal decays)", "f32", o_k, host(o_g), s_k, host(s_g))


def test_kda_in_place_resume_and_empty():
    d = gi.generate_kda(B=1, T=70, Hqk=1, Hv=2, dk=32, dv=32, dtype="f32", mu=2.0, s0_std=0.05, seed=23)
    t = dev(d)
    o_full, s_full = gdn.gdn_kda_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["s0"])
    st = t["s0"].clone()
    half = {n: (x[:, :33].contiguous() if n != "s0" else x) for n, x in t.items()}
    rest = {n: (x[:, 33:].contiguous() if n != "s0" else x) for n, x in t.items()}
    oa, _ = gdn.gdn_kda_chunk_fwd(half["q"], half["k"], half["v"], half["g"], half["beta"], st, final_state=st)
    ob, _ = gdn.gdn_kda_chunk_fwd(rest["q"], rest["k"], rest["v"], rest["g"], rest["beta"], st, final_state=st)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_kda(d)
    check("kda resume in place", "f32", np.concatenate([host(oa), host(ob)], axis=1), o_ref, host(st), s_ref)
    e = {n: (x[:, :0].contiguous() if n != "s0" else x) for n, x in t.items()}
    o0, s0 = gdn.gdn_kda_chunk_fwd(e["q"], e["k"], e["v"], e["g"], e["beta"], e["s0"])
    torch.cuda.synchronize()
    assert o0.numel() == 0 and torch.equal(s0, t["s0"])


def test_kda_prefill_full():
    """The KDA workload (B1 T4096, 32 query/key and 32 value heads, d 128, bf16) at full size on
    the float32 vector route, against the oracle over whole tensors."""
    cfg = gi.CONFIGS["kda_prefill"]
    say(f"kda full {cfg}")
    d = gi.generate_kda(cfg.B, cfg.T, cfg.Hqk, cfg.Hv, cfg.dk, cfg.dv, dtype=cfg.dtype, mu=cfg.mu,
                        s0_std=cfg.s0_std, seed=cfg.seed)
    o, s = run_kda(d, 32)
    o_ref, s_ref = oracle_kda(d)
    check("kda_prefill", "bf16", o, o_ref, s, s_ref)


# ------------------------------------------------------------- matrix-core route (chunk 64)

@pytest.mark.parametrize("dk,dv,T,Hqk,Hv", [(128, 128, 200, 2, 4), (64, 128, 65, 1, 2), (128, 64, 64, 2, 2),
                                           (64, 64, 130, 1, 3), (128, 128, 1, 1, 1)])
def test_kda_mfma_small(dk, dv, T, Hqk, Hv):
    say(f"kda mfma dk={dk} dv={dv} T={T} Hqk={Hqk} Hv={Hv}")
    d = gi.generate_kda(B=2, T=T, Hqk=Hqk, Hv=Hv, dk=dk, dv=dv, dtype="bf16", mu=2.0, s0_std=0.05, seed=T + dk + Hv + 7)
    o, s = run_kda(d, 64)
    o_ref, s_ref = oracle_kda(d)
    check("kda mfma", "bf16", o, o_ref, s, s_ref)


def test_kda_mfma_strong_decay_scale_and_resume():
    for mu in (-3.0, 8.0):
        d = gi.generate_kda(B=1, T=150, Hqk=2, Hv=2, dk=128, dv=128, dtype="bf16", mu=mu, s0_std=0.05, seed=31)
        o, s = run_kda(d, 64, scale=0.3)
        o_ref, s_ref = oracle_kda(d, scale=0.3)
        check(f"kda mfma mu={mu}", "bf16", o, o_ref, s, s_ref)
    # continuation with the state updated in place
    d = gi.generate_kda(B=1, T=160, Hqk=1, Hv=2, dk=64, dv=64, dtype="bf16", mu=2.0, s0_std=0.05, seed=32)
    t = dev(d)
    st = t["s0"].clone()
    parts = []
    for a, b in ((0, 70), (70, 160)):
        x = {n: (y[:, a:b].contiguous() if n != "s0" else y) for n, y in t.items()}
        oo, _ = gdn.gdn_kda_chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], st, final_state=st, chunk=64)
        parts.append(host(oo))
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_kda(d)
    check("kda mfma resume in place", "bf16", np.concatenate(parts, axis=1), o_ref, host(st), s_ref)


def test_kda_mfma_matches_vector_kernel_and_gdn():
    """The matrix-core and vector routes agree; with one decay per head copied to every channel
    the matrix-core KDA also agrees with the Gated DeltaNet matrix-core kernel."""
    d = gi.generate_kda(B=2, T=257, Hqk=2, Hv=4, dk=128, dv=128, dtype="bf16", mu=3.0, s0_std=0.02, seed=33)
    o64, s64 = run_kda(d, 64)
    o32, s32 = run_kda(d, 32)
    check("kda mfma vs vector", "bf16", o64, o32, s64, s32)
    g = gi.generate(B=2, T=257, Hqk=2, Hv=4, dk=128, dv=128, dtype="bf16", mu=3.0, s0_std=0.02, seed=34)
    dd = dict(g)
    dd["g"] = np.ascontiguousarray(np.repeat(g["g"][..., None], 128, axis=-1))
    ok, sk = run_kda(dd, 64)
    t = dev(g)
    og, sg = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["s0"], chunk=64)
    torch.cuda.synchronize()
    check("kda mfma == gdn (equal decays)", "bf16", ok, host(og), sk, host(sg))


def test_kda_mfma_prefill_full():
    """The KDA workload at full size on the matrix-core route (chunk 64), whole tensors."""
    cfg = gi.CONFIGS["kda_prefill"]
    say(f"kda mfma full {cfg}")
    d = gi.generate_kda(cfg.B, cfg.T, cfg.Hqk, cfg.Hv, cfg.dk, cfg.dv, dtype=cfg.dtype, mu=cfg.mu,
                        s0_std=cfg.s0_std, seed=cfg.seed)
    o, s = run_kda(d, 64)
    o_ref, s_ref = oracle_kda(d)
    check("kda_prefill mfma", "bf16", o, o_ref, s, s_ref)


@pytest.mark.parametrize("mu", [6.0, 1.0])
@pytest.mark.parametrize("keys", ["identical", "correlated"])
def test_kda_mfma_dense_solve(keys, mu):
    """All keys of a head equal (or close: a shared unit key plus 0.3 of a random one, renormalised)
    and beta near 1: the strictly-lower A of every chunk is dense with entries near beta, so the
    blocks of the blockwise (I + A)^{-1} off its diagonal carry large entries.  Slow channel decay
    (mu = 6) keeps those entries near one; mu = 1 mixes slow and fast channels.  Checked against the
    float64 oracle and against the float32 vector kernel (chunk 32)."""
    say(f"kda mfma dense solve keys={keys} mu={mu}")
    d = gi.generate_kda(B=1, T=256, Hqk=2, Hv=4, dk=128, dv=128, dtype="bf16", mu=mu, s0_std=0.05, seed=35)
    k = f64(d["k"])
    if keys == "identical":
        k[:] = k[:, :1]
    else:
        rng = np.random.default_rng(36)
        r = rng.standard_normal(k.shape)
        r /= np.linalg.norm(r, axis=-1, keepdims=True)
        k = k[:, :1] + 0.3 * r
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    d["k"] = gi.bf16_bits(k.astype(np.float32))
    d["beta"][:] = 0.97
    o, s = run_kda(d, 64)
    o_ref, s_ref = oracle_kda(d)
    check(f"kda mfma dense keys={keys} mu={mu}", "bf16", o, o_ref, s, s_ref)
    o32, s32 = run_kda(d, 32)
    check(f"kda mfma vs vector, dense keys={keys} mu={mu}", "bf16", o, o32, s, s32)
