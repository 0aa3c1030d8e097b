"""Pins of the backward-pass oracle (oracle.recurrent_bwd in C, oracle.chunked_bwd in numpy) to
things other than themselves: central finite differences of the forward oracle, torch autograd
of the Gated DeltaNet equation written out here in its literal matrix form, and a closed form
(beta = 0).  Then plausible mistakes are planted in copies of both backward implementations (on
the CPU) and each must fail at least one pin."""
import ctypes
import os
import subprocess
import types

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(oracle.__file__)
SRC = os.path.join(HERE, "gdn_oracle.c")
SRC_BWD = os.path.join(HERE, "gdn_oracle_bwd.c")


def _problem(seed, B=1, T=7, Hqk=1, Hv=2, dk=3, dv=2, s0=True, dsf=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, Hqk, dk))
    k = rng.standard_normal((B, T, Hqk, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, Hv, dv))
    g = -rng.uniform(0.02, 0.5, (B, T, Hv))
    beta = rng.uniform(0.1, 0.9, (B, T, Hv))
    S0 = rng.standard_normal((B, Hv, dk, dv)) if s0 else None
    do = rng.standard_normal((B, T, Hv, dv))
    dS = rng.standard_normal((B, Hv, dk, dv)) if dsf else None
    return dict(q=q, k=k, v=v, g=g, beta=beta, s0=S0), do, dS


def _loss(x, do, dsf, scale):
    o, sf = oracle.recurrent(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], scale=scale)
    return float((o * do).sum() + (0.0 if dsf is None else (sf * dsf).sum()))


NAMES = (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"), ("s0", "ds0"))


def test_bwd_finite_differences(m=oracle):
    """Every gradient element against a central difference of the forward oracle (float64,
    step 1e-6: truncation ~1e-12, rounding ~1e-10)."""
    for seed, kw in ((1, {}), (2, dict(T=4, s0=False, dsf=False, Hv=1))):
        x, do, dsf = _problem(seed, **kw)
        scale = 0.7
        gr = m.recurrent_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], do, dsf, scale=scale)
        for name, key in NAMES:
            if x[name] is None:
                continue
            fd = np.zeros_like(x[name])
            for idx in np.ndindex(x[name].shape):
                xp = dict(x)
                xp[name] = x[name].copy()
                xp[name][idx] += 1e-6
                lp = _loss(xp, do, dsf, scale)
                xp[name][idx] -= 2e-6
                lm = _loss(xp, do, dsf, scale)
                fd[idx] = (lp - lm) / 2e-6
            err = np.abs(fd - gr[key]).max() / max(1.0, np.abs(fd).max())
            assert err < 1e-7, (seed, name, err)


def _torch_grads(x, do, dsf, scale):
    """Autograd through S_t = S_{t-1} (alpha_t (I - beta_t k_t k_t^T)) + beta_t v_t k_t^T, o_t = S_t q_t
    with S in R^{dv x dk} (the equation as printed, not the erase/write form the oracle uses)."""
    torch = pytest.importorskip("torch")
    t = {n: (None if a is None else torch.tensor(a, dtype=torch.float64, requires_grad=True)) for n, a in x.items()}
    B, T, Hqk, dk = x["q"].shape
    Hv, dv = x["v"].shape[2], x["v"].shape[3]
    grp = Hv // Hqk
    L = torch.zeros((), dtype=torch.float64)
    eye = torch.eye(dk, dtype=torch.float64)
    for b in range(B):
        for j in range(Hv):
            i = j // grp
            S = torch.zeros((dv, dk), dtype=torch.float64) if t["s0"] is None else t["s0"][b, j].T
            for s in range(T):
                kt = t["k"][b, s, i][:, None]
                M = torch.exp(t["g"][b, s, j]) * (eye - t["beta"][b, s, j] * (kt @ kt.T))
                S = S @ M + t["beta"][b, s, j] * (t["v"][b, s, j][:, None] @ kt.T)
                o = S @ (scale * t["q"][b, s, i])
                L = L + (o * torch.tensor(do[b, s, j])).sum()
            if dsf is not None:
                L = L + (S.T * torch.tensor(dsf[b, j])).sum()
    L.backward()
    return {key: t[name].grad.numpy() for name, key in NAMES if t[name] is not None}


def test_bwd_matches_autograd_of_the_equation(m=oracle):
    x, do, dsf = _problem(3, B=2, T=23, Hqk=2, Hv=4, dk=5, dv=4)
    ref = _torch_grads(x, do, dsf, 1.3)
    gr = m.recurrent_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], do, dsf, scale=1.3)
    for key, r in ref.items():
        assert np.allclose(gr[key], r, rtol=1e-10, atol=1e-11), key


def test_bwd_beta_zero_closed_form(m=oracle):
    """beta = 0: nothing is written, h_t = (prod_{s<=t} a_s) S0 and o_t = h_t^T (scale q_t), so
    dv = 0, dq_t = scale P_t S0 do_t and dS0 = sum_t P_t scale q_t do_t^T + P_T dsf (P_t the
    running decay product)."""
    x, do, dsf = _problem(4, T=9, Hv=1, dk=4, dv=3)
    x["beta"] = np.zeros_like(x["beta"])
    scale = 0.5
    gr = m.recurrent_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], do, dsf, scale=scale)
    P = np.exp(np.cumsum(x["g"][0, :, 0]))
    S0 = x["s0"][0, 0]
    assert np.allclose(gr["dv"], 0.0, atol=1e-15)
    for t in range(9):
        assert np.allclose(gr["dq"][0, t, 0], scale * P[t] * (S0 @ do[0, t, 0]), rtol=1e-12, atol=1e-14)
    ds0 = sum(P[t] * scale * np.outer(x["q"][0, t, 0], do[0, t, 0]) for t in range(9)) + P[-1] * dsf[0, 0]
    assert np.allclose(gr["ds0"][0, 0], ds0, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("T", [37, 150])
def test_bwd_chunked_equals_recurrent(T, m=oracle):
    """The chunk algebra of the backward (numpy) equals the token adjoint (C) for every chunk
    size, a ragged tail, grouped heads and, at T = 150, several checkpoint segments."""
    x, do, dsf = _problem(5 + T, B=2, T=T, Hqk=1, Hv=2, dk=8, dv=6)
    r = m.recurrent_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], do, dsf, scale=0.6)
    for C in (1, 4, 16, 64):
        c = m.chunked_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], do, dsf, chunk=C, scale=0.6)
        for key in r:
            err = np.abs(c[key] - r[key]).max() / np.abs(r[key]).max()
            assert err < 1e-12, (C, key, err)


def test_bwd_long_sequence_sampled_finite_differences(m=oracle):
    """Past several checkpoint segments (T = 140): sampled gradient elements against central
    differences."""
    x, do, dsf = _problem(6, T=140, Hv=1, dk=4, dv=3)
    gr = m.recurrent_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], do, dsf, scale=1.0)
    rng = np.random.default_rng(0)
    for name, key in NAMES:
        for _ in range(3):
            idx = tuple(int(rng.integers(0, n)) for n in x[name].shape)
            xp = dict(x)
            xp[name] = x[name].copy()
            xp[name][idx] += 1e-6
            lp = _loss(xp, do, dsf, 1.0)
            xp[name][idx] -= 2e-6
            lm = _loss(xp, do, dsf, 1.0)
            fd = (lp - lm) / 2e-6
            assert abs(fd - gr[key][idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, gr[key][idx])


PINS = [test_bwd_finite_differences, test_bwd_matches_autograd_of_the_equation, test_bwd_beta_zero_closed_form,
        test_bwd_long_sequence_sampled_finite_differences]

# ------------------------------------------------------------------------ C mutants

C_MUTANTS = [
    ("readout_grad_from_old_state", "acc += hn[(size_t)r * dv + cc] * dot[cc];", "acc += hp[(size_t)r * dv + cc] * dot[cc];"),
    ("decay_grad_from_new_state", "da += x * hp[(size_t)r * dv + cc];", "da += x * hn[(size_t)r * dv + cc];"),
    ("erase_grad_sign", "du[cc] = -bt * a * dd[cc];", "du[cc] = bt * a * dd[cc];"),
    ("dg_missing_alpha", "dg[tv] = a * da;", "dg[tv] = da;"),
    ("dv_missing_beta", "dvv[tv * dv + cc] = bt * dd[cc];", "dvv[tv * dv + cc] = dd[cc];"),
    ("state_grad_not_decayed", "dh[(size_t)r * dv + cc] = a * dh[(size_t)r * dv + cc] + kt[r] * du[cc];",
     "dh[(size_t)r * dv + cc] = dh[(size_t)r * dv + cc] + kt[r] * du[cc];"),
    ("erase_path_dropped_from_dk", "dkt[r] += acc;", "dkt[r] += 0.0 * acc;"),
    ("dbeta_missing_decay", "db += dd[cc] * (vt[cc] - a * u[cc]);", "db += dd[cc] * vt[cc];"),
    ("checkpoint_off_by_one", "if (t % SEG == 0) memcpy(", "if (t % SEG == 1) memcpy("),
    ("dq_missing_scale", "dqt[r] = scale * acc;", "dqt[r] = acc;"),
]


@pytest.mark.parametrize("mut", C_MUTANTS, ids=[m[0] for m in C_MUTANTS])
def test_pins_reject_bwd_mutant(mut, tmp_path, monkeypatch):
    src = open(SRC_BWD).read()
    assert src.count(mut[1]) == 1, mut[0]
    (tmp_path / "bwd.c").write_text(src.replace(mut[1], mut[2]))
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-fopenmp", SRC, str(tmp_path / "bwd.c"), "-o", str(lib), "-lm"],
                   check=True)
    mlib = ctypes.CDLL(str(lib))
    real = oracle.load()
    for fn in ("gdn_oracle_recurrent", "gdn_oracle_recurrent_bwd"):
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


# ------------------------------------------------------------------- numpy mutants

PY_MUTANTS = [
    ("exit_gate_grad_dropped", "                dgc[-1] += dgL\n", "\n"),
    ("inverse_grad_untransposed", "dA = np.tril(-Tm.T @ dT @ Tm.T, -1)", "dA = np.tril(-Tm @ dT @ Tm, -1)"),
    ("gram_grad_one_sided", "dK += Dk @ K + Dk.T @ K", "dK += Dk @ K"),
    ("output_mask_exclusive", "dM = np.tril(dO @ D.T)", "dM = np.tril(dO @ D.T, -1)"),
    ("state_grad_missing_correction", "- W.T @ dD", "+ 0 * W.T @ dD"),
    ("dg_forward_cumsum", "np.cumsum(dgc[::-1])[::-1]", "np.cumsum(dgc)"),
]


@pytest.mark.parametrize("mut", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_chunked_pin_rejects_mutant(mut):
    src = open(oracle.__file__).read()
    assert src.count(mut[1]) == 1, mut[0]
    mod = types.ModuleType("oracle_mutant")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(mut[1], mut[2]), "oracle_mutant", "exec"), mod.__dict__)
    m = types.SimpleNamespace(recurrent_bwd=oracle.recurrent_bwd, chunked_bwd=mod.chunked_bwd)
    with pytest.raises(AssertionError):
        with np.errstate(all="ignore"):
            test_bwd_chunked_equals_recurrent(37, m=m)
