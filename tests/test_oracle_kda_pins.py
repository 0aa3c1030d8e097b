"""Pins of the KDA oracle (oracle.kda_recurrent in C; kda_brute_force and kda_chunked in numpy) to
things other than themselves: the pages' statement that KDA reduces to Gated DeltaNet when the
decay is one scalar per head (against the pinned Gated DeltaNet oracle), the equation with its
dense transition matrices, closed forms (no writes; one-hot keys), and chunked == recurrent.
Then plausible mistakes are planted in copies of the C oracle and of the chunked form (on the
CPU) and each must fail a pin."""
import ctypes
import os
import subprocess
import types

import numpy as np
import pytest

import oracle

SRC_KDA = os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle_kda.c")


def _problem(seed, B=2, T=9, Hqk=1, Hv=2, dk=5, dv=4, s0=True, gmax=2.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, Hqk, dk))
    k = rng.standard_normal((B, T, Hqk, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, Hv, dv))
    g = -rng.uniform(0.0, gmax, (B, T, Hv, dk))
    beta = rng.uniform(0.1, 0.9, (B, T, Hv))
    S0 = rng.standard_normal((B, Hv, dk, dv)) if s0 else None
    return q, k, v, g, beta, S0


def test_kda_scalar_decay_is_gated_deltanet(m=oracle):
    """With every key channel of a head decaying alike, KDA is Gated DeltaNet ("Gated Attention
    Architectures", section 8 states the reduction): equal to the Gated DeltaNet oracle."""
    q, k, v, g, beta, s0 = _problem(1, Hqk=2, Hv=4, T=30)
    gs = g[..., 0]
    g1 = np.repeat(gs[..., None], q.shape[3], axis=-1)
    o, sf = m.kda_recurrent(q, k, v, g1, beta, s0, scale=0.8)
    og, sg = m.recurrent(q, k, v, gs, beta, s0, scale=0.8)
    assert np.allclose(o, og, rtol=1e-12, atol=1e-13) and np.allclose(sf, sg, rtol=1e-12, atol=1e-13)


def test_kda_dense_transitions(m=oracle):
    """The equation as printed, S_t = (I - beta k k^T) D_t S_{t-1} + beta k v^T, with every
    matrix formed densely, for tiny T, grouped heads, scale, with and without S0."""
    for seed, kw in ((2, {}), (3, dict(Hqk=2, Hv=6, s0=False, dk=3, dv=7))):
        q, k, v, g, beta, s0 = _problem(seed, T=7, **kw)
        o, sf = m.kda_recurrent(q, k, v, g, beta, s0, scale=1.3)
        ob, sb = m.kda_brute_force(q, k, v, g, beta, s0, scale=1.3)
        assert np.allclose(o, ob, rtol=1e-12, atol=1e-13) and np.allclose(sf, sb, rtol=1e-12, atol=1e-13)


def test_kda_no_writes_is_channelwise_decay(m=oracle):
    """beta = 0: nothing is written, S_t = diag(exp(G_t)) S0 with G_t the running sum of g per
    key channel, so o_t = S0^T (exp(G_t) * q_t)."""
    q, k, v, g, beta, s0 = _problem(4, B=1, Hv=1, T=11)
    beta[:] = 0.0
    o, sf = m.kda_recurrent(q, k, v, g, beta, s0)
    G = np.cumsum(g[0, :, 0], axis=0)
    for t in range(11):
        assert np.allclose(o[0, t, 0], s0[0, 0].T @ (np.exp(G[t]) * q[0, t, 0]), rtol=1e-12, atol=1e-13)
    assert np.allclose(sf[0, 0], np.exp(G[-1])[:, None] * s0[0, 0], rtol=1e-12, atol=1e-14)


def test_kda_one_hot_keys(m=oracle):
    """k_t = e_c: row c becomes alpha_c (1 - beta) row_c + beta v_t, every other row m only
    decays by alpha_m (the erase and the write touch key channel c alone)."""
    rng = np.random.default_rng(5)
    dk, dv, T = 4, 3, 10
    q, k, v, g, beta, s0 = _problem(5, B=1, Hv=1, T=T, dk=dk, dv=dv)
    cs = rng.integers(0, dk, T)
    k[:] = 0.0
    k[0, np.arange(T), 0, cs] = 1.0
    _, sf = m.kda_recurrent(q, k, v, g, beta, s0)
    h = s0[0, 0].copy()
    for t in range(T):
        a = np.exp(g[0, t, 0])
        h = a[:, None] * h
        c = cs[t]
        h[c] = (1 - beta[0, t, 0]) * h[c] + beta[0, t, 0] * v[0, t, 0]
    assert np.allclose(sf[0, 0], h, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("T", [37, 70])
def test_kda_chunked_equals_recurrent(T, m=oracle):
    """The chunk algebra (numpy) against the recurrence (C), chunks 1..32, a ragged tail, grouped
    heads, and strong per-channel decays (some channels near 0 within a chunk)."""
    q, k, v, g, beta, s0 = _problem(6 + T, T=T, Hqk=1, Hv=2, dk=8, dv=6, gmax=4.0)
    o, sf = m.kda_recurrent(q, k, v, g, beta, s0, scale=0.6)
    for C in (1, 4, 16, 32):
        oc, sc = m.kda_chunked(q, k, v, g, beta, s0, chunk=C, scale=0.6)
        assert np.abs(oc - o).max() <= 1e-11 * np.abs(o).max(), C
        assert np.abs(sc - sf).max() <= 1e-11 * np.abs(sf).max(), C


def test_kda_resume(m=oracle):
    """One call over T tokens equals two calls over its halves with the state carried."""
    q, k, v, g, beta, s0 = _problem(7, T=20)
    o, sf = m.kda_recurrent(q, k, v, g, beta, s0)
    oa, sa = m.kda_recurrent(q[:, :8], k[:, :8], v[:, :8], g[:, :8], beta[:, :8], s0)
    ob, sb = m.kda_recurrent(q[:, 8:], k[:, 8:], v[:, 8:], g[:, 8:], beta[:, 8:], sa)
    assert np.allclose(np.concatenate([oa, ob], axis=1), o, rtol=1e-12, atol=1e-13)
    assert np.allclose(sb, sf, rtol=1e-12, atol=1e-13)


PINS = [test_kda_scalar_decay_is_gated_deltanet, test_kda_dense_transitions, test_kda_no_writes_is_channelwise_decay,
        test_kda_one_hot_keys]

C_MUTANTS = [
    ("decay_after_erase",
     [("            /* h <- D_t h: key row m decays by alpha_t[m] */\n            for (int r = 0; r < dk; ++r) {\n                const double a = exp(gt[r]);\n                for (int cc = 0; cc < dv; ++cc) h[(size_t)r * dv + cc] *= a;\n            }\n", ""),
      ("            /* o_t = h^T (scale q) */", "            for (int r = 0; r < dk; ++r) { const double a = exp(gt[r]); for (int cc = 0; cc < dv; ++cc) h[(size_t)r * dv + cc] *= a; }\n            /* o_t = h^T (scale q) */")]),
    ("decay_on_value_axis", [("for (int cc = 0; cc < dv; ++cc) h[(size_t)r * dv + cc] *= a;",
                              "for (int cc = 0; cc < dv; ++cc) h[(size_t)r * dv + cc] *= exp(gt[cc % dk]);")]),
    ("log_decay_not_exponentiated", [("const double a = exp(gt[r]);", "const double a = 1.0 + gt[r];")]),
    ("beta_dropped", [("u[cc] = bt * (vt[cc] - u[cc]);", "u[cc] = vt[cc] - u[cc];")]),
    ("channel_index_shifted", [("const double a = exp(gt[r]);", "const double a = exp(gt[(r + 1) % dk]);")]),
    ("erase_not_decayed", [("for (int cc = 0; cc < dv; ++cc) u[cc] += h[(size_t)r * dv + cc] * kt[r];",
                            "for (int cc = 0; cc < dv; ++cc) u[cc] += h[(size_t)r * dv + cc] * kt[r] / exp(gt[r]);")]),
]


@pytest.mark.parametrize("mut", C_MUTANTS, ids=[m[0] for m in C_MUTANTS])
def test_pins_reject_kda_mutant(mut, tmp_path, monkeypatch):
    src = open(SRC_KDA).read()
    for old, new in mut[1]:
        assert src.count(old) == 1, mut[0]
        src = src.replace(old, new)
    (tmp_path / "kda.c").write_text(src)
    base = os.path.dirname(SRC_KDA)
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-fopenmp", os.path.join(base, "gdn_oracle.c"),
                    str(tmp_path / "kda.c"), "-o", str(lib), "-lm"], check=True)
    mlib = ctypes.CDLL(str(lib))
    real = oracle.load()
    for fn in ("gdn_oracle_recurrent", "gdn_oracle_kda_recurrent"):
        getattr(mlib, fn).argtypes = getattr(real, fn).argtypes
        getattr(mlib, fn).restype = ctypes.c_int
    monkeypatch.setattr(oracle, "_lib", mlib)
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin rejects mutant {mut[0]}"


PY_MUTANTS = [
    ("decay_pair_uses_sum", "diff = gc[:, None, :] - gc[None, :, :]", "diff = gc[:, None, :] + 0 * gc[None, :, :]"),
    ("entry_decay_dropped", "rhs = bt[:, None] * V - bt[:, None] * ((np.exp(gc) * K) @ h)", "rhs = bt[:, None] * V - bt[:, None] * (K @ h)"),
    ("exit_decay_scalar", "h = np.exp(gL)[:, None] * h +", "h = np.exp(gL.mean()) * h +"),
    ("output_mask_strict", "Aqk = np.tril(np.einsum(\"rc,ic,ric->ri\", Q, K, E))", "Aqk = np.tril(np.einsum(\"rc,ic,ric->ri\", Q, K, E), -1)"),
]


@pytest.mark.parametrize("mut", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_kda_chunked_pin_rejects_mutant(mut):
    src = open(oracle.__file__).read()
    assert src.count(mut[1]) == 1, mut[0]
    mod = types.ModuleType("oracle_mutant")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(mut[1], mut[2]), "oracle_mutant", "exec"), mod.__dict__)
    m = types.SimpleNamespace(kda_recurrent=oracle.kda_recurrent, kda_chunked=mod.kda_chunked)
    with pytest.raises(AssertionError):
        with np.errstate(all="ignore"):
            test_kda_chunked_equals_recurrent(37, m=m)
