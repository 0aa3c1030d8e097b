"""Pins of oracle.transport (the affine state map of a stretch of tokens) to things other than
itself: the affine law against the recurrence from other entry states, composition of two
stretches into one, the single-step closed form written from the equation, the no-write closed
form, and a segmented run (maps composed into entry states, then each segment from its own)
equal to one run.  Then plausible mistakes are planted in copies of the function and each must
fail a pin."""
import types

import numpy as np
import pytest

import oracle


def _problem(seed, B=2, T=23, Hqk=1, Hv=2, dk=6, dv=5, gmax=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, Hqk, dk))
    k = rng.standard_normal((B, T, Hqk, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, Hv, dv))
    g = -rng.uniform(0.0, gmax, (B, T, Hv))
    beta = rng.uniform(0.1, 0.9, (B, T, Hv))
    return q, k, v, g, beta


def test_transport_affine_law(m=oracle):
    """For entry states other than those used to form the map, the recurrence ends at M h0 + N."""
    q, k, v, g, beta = _problem(1, Hqk=2, Hv=4)
    M, N = m.transport(k, v, g, beta)
    rng = np.random.default_rng(2)
    for _ in range(2):
        h0 = rng.standard_normal((2, 4, 6, 5))
        _, sf = oracle.recurrent(q, k, v, g, beta, h0)
        assert np.allclose(np.einsum("bjmn,bjnc->bjmc", M, h0) + N, sf, rtol=1e-12, atol=1e-12)


def test_transport_single_step_closed_form(m=oracle):
    """T = 1: h1 = alpha (I - beta k k^T) h0 + beta k v^T, so M = alpha (I - beta k k^T), N = beta k v^T."""
    q, k, v, g, beta = _problem(3, B=1, T=1, Hv=1, dk=4, dv=3)
    M, N = m.transport(k, v, g, beta)
    kk, vv, a, bt = k[0, 0, 0], v[0, 0, 0], np.exp(g[0, 0, 0]), beta[0, 0, 0]
    assert np.allclose(M[0, 0], a * (np.eye(4) - bt * np.outer(kk, kk)), rtol=1e-13, atol=1e-14)
    assert np.allclose(N[0, 0], bt * np.outer(kk, vv), rtol=1e-13, atol=1e-14)


def test_transport_no_writes(m=oracle):
    """beta = 0: the state only decays, M = exp(sum g) I and N = 0."""
    q, k, v, g, beta = _problem(4, T=9)
    beta[:] = 0.0
    M, N = m.transport(k, v, g, beta)
    decay = np.exp(g.sum(axis=1))                      # [B, Hv]
    assert np.allclose(M, decay[..., None, None] * np.eye(6), rtol=1e-13, atol=1e-15)
    assert np.abs(N).max() == 0.0


def test_transport_composes(m=oracle):
    """The map of tokens [0, T) is that of [T1, T) after that of [0, T1): (M2 M1, M2 N1 + N2)."""
    q, k, v, g, beta = _problem(5, T=30, Hqk=1, Hv=3)
    M, N = m.transport(k, v, g, beta)
    M1, N1 = m.transport(k[:, :11], v[:, :11], g[:, :11], beta[:, :11])
    M2, N2 = m.transport(k[:, 11:], v[:, 11:], g[:, 11:], beta[:, 11:])
    assert np.allclose(np.einsum("bjmn,bjnk->bjmk", M2, M1), M, rtol=1e-12, atol=1e-13)
    assert np.allclose(np.einsum("bjmn,bjnc->bjmc", M2, N1) + N2, N, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("cuts", [(7,), (5, 12, 13, 20), (1, 2, 3)])
def test_segmented_run_equals_one_run(cuts, m=oracle):
    """The scan: each segment's map formed alone, entry states composed from them, then every
    segment run from its entry state; outputs and the final state equal one run."""
    q, k, v, g, beta = _problem(6, T=24, Hqk=1, Hv=2)
    s0 = np.random.default_rng(7).standard_normal((2, 2, 6, 5))
    o_ref, sf_ref = oracle.recurrent(q, k, v, g, beta, s0, scale=0.7)
    edges = (0,) + cuts + (24,)
    h = s0
    outs = []
    for a, b in zip(edges[:-1], edges[1:]):
        M, N = m.transport(k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b])
        o, _ = oracle.recurrent(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b], h, scale=0.7)
        outs.append(o)
        h = np.einsum("bjmn,bjnc->bjmc", M, h) + N
    assert np.allclose(np.concatenate(outs, axis=1), o_ref, rtol=1e-11, atol=1e-12)
    assert np.allclose(h, sf_ref, rtol=1e-11, atol=1e-12)


PINS = [test_transport_affine_law, test_transport_single_step_closed_form, test_transport_no_writes,
        test_transport_composes]

MUTANTS = [
    ("writes_kept_in_M", "np.zeros((B, T, Hv, dk)), g, beta, unit", "np.ones((B, T, Hv, dk)), g, beta, unit"),
    ("unit_entry_missing", "np.broadcast_to(np.eye(dk), (B, Hv, dk, dk))", "np.zeros((B, Hv, dk, dk))"),
    ("M_transposed", "    return M, N\n", "    return np.swapaxes(M, -1, -2), N\n"),
    ("N_from_unit_entry", "_, N = recurrent(k, k, v, g, beta, None, threads=threads)",
     "_, N = recurrent(k, k, v, g, beta, np.ones((B, Hv, dk, v.shape[3])), threads=threads)"),
    ("decay_dropped_from_M", "np.zeros((B, T, Hv, dk)), g, beta, unit", "np.zeros((B, T, Hv, dk)), 0 * g, beta, unit"),
]


@pytest.mark.parametrize("mut", MUTANTS, ids=[x[0] for x in MUTANTS])
def test_transport_pins_reject_mutant(mut):
    src = open(oracle.__file__).read()
    assert src.count(mut[1]) >= 1, mut[0]
    start = src.index("def transport(")
    end = src.index("\ndef ", start + 10)
    fn_src = src[start:end]
    assert fn_src.count(mut[1]) == 1, mut[0]
    mod = types.ModuleType("oracle_transport_mutant")
    mod.__dict__.update(np=np, recurrent=oracle.recurrent, _f64=lambda x: np.ascontiguousarray(x, dtype=np.float64))
    exec(compile(fn_src.replace(mut[1], mut[2]), "oracle_transport_mutant", "exec"), mod.__dict__)
    m = types.SimpleNamespace(transport=mod.transport)
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(m=m)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin rejects mutant {mut[0]}"
