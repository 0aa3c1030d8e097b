"""Pins of the float64 CPU oracle against what the pages and the mathematics fix.

None of these checks re-types the oracle's own loop: each one uses a closed form, an invariant,
a special case, a hand-worked example, or a different code path (dense transition matrices,
the chunkwise refactoring).  Each names the passage it rests on."""
import json
import os

import numpy as np
import pytest

import gdn_inputs as gi
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_inputs(B=1, T=16, Hqk=1, Hv=1, dk=8, dv=6, mu=3.0, s0_std=0.0, seed=0):
    d = gi.generate(B=B, T=T, Hqk=Hqk, Hv=Hv, dk=dk, dv=dv, dtype="f32", mu=mu, s0_std=s0_std, seed=seed)
    return {n: (None if a is None else a.astype(np.float64)) for n, a in d.items()}


def run(d, **kw):
    return oracle.recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"], d.get("s0"), **kw)


def test_hand_worked_example():
    """Two steps worked by hand from the Gated DeltaNet equation (tests/golden/hand_worked_dk2.json)."""
    with open(os.path.join(GOLDEN, "hand_worked_dk2.json")) as f:
        ex = json.load(f)
    q = np.array(ex["q"])[None, :, None, :]
    k = np.array(ex["k"])[None, :, None, :]
    v = np.array(ex["v"])[None, :, None, :]
    g = np.array(ex["g"])[None, :, None]
    beta = np.array(ex["beta"])[None, :, None]
    o, sf = oracle.recurrent(q, k, v, g, beta)
    np.testing.assert_allclose(o[0, :, 0], np.array(ex["o"]), atol=1e-14)
    np.testing.assert_allclose(sf[0, 0], np.array(ex["h_final"]), atol=1e-14)


def test_p1_beta_zero_pure_decay():
    """beta = 0: nothing is written; the state only decays (Gated DeltaNet equation with beta_t = 0).
    h_t = exp(G_t) h_0 and o_t = exp(G_t) h_0^T q_t with G_t the inclusive cumsum of log alpha."""
    d = rand_inputs(B=2, T=40, Hqk=1, Hv=2, s0_std=0.5, seed=1)
    d["beta"][:] = 0.0
    o, sf = run(d)
    G = np.cumsum(d["g"], axis=1)  # [B,T,Hv]
    h0 = d["s0"]
    grp = 2
    for b in range(2):
        for j in range(2):
            for t in range(40):
                exp_o = np.exp(G[b, t, j]) * (h0[b, j].T @ d["q"][b, t, j // grp])
                np.testing.assert_allclose(o[b, t, j], exp_o, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(sf[b, j], np.exp(G[b, -1, j]) * h0[b, j], rtol=1e-12, atol=1e-15)


def test_p2_unit_key_writes_value_exactly():
    """alpha = 1, beta = 1, k = e_r: the erase/write decomposition (section on DeltaNet in
    "Architecture Thread I") replaces the memory at key e_r by v exactly: row r of h = S^T is v_t,
    the other rows are untouched."""
    rng = np.random.default_rng(2)
    dk, dv, T = 5, 4, 6
    s0 = rng.standard_normal((1, 1, dk, dv))
    rows = [0, 3, 3, 1, 4, 0]
    k = np.zeros((1, T, 1, dk))
    for t, r in enumerate(rows):
        k[0, t, 0, r] = 1.0
    v = rng.standard_normal((1, T, 1, dv))
    q = rng.standard_normal((1, T, 1, dk))
    g = np.zeros((1, T, 1))
    beta = np.ones((1, T, 1))
    h = s0[0, 0].copy()
    for t in range(T):
        o, sf = oracle.recurrent(q[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1], g[:, t:t + 1],
                                 beta[:, t:t + 1], h[None, None])
        expect = h.copy()
        expect[rows[t]] = v[0, t, 0]
        np.testing.assert_allclose(sf[0, 0], expect, rtol=0, atol=1e-15)
        np.testing.assert_allclose(o[0, 0, 0], expect.T @ q[0, t, 0], rtol=1e-13, atol=1e-14)
        h = sf[0, 0]


def test_p3_single_step_invariants():
    """For a unit key and beta in [0,1]:
    (i)  the memory read at k_t after the step is alpha(1-beta) h^T k + beta v (erase/write);
    (ii) directions orthogonal to k_t are only decayed (eigenvector argument of "Architecture
         Thread I", section "Modern Architecture Improvements": I - beta k k^T is 1 off k);
    (iii) ||h_t||_F <= alpha ||h_{t-1}||_F + beta ||v_t||  (eigenvalues of I - beta k k^T in [0,1])."""
    rng = np.random.default_rng(3)
    dk, dv = 16, 12
    for trial in range(20):
        h0 = rng.standard_normal((dk, dv))
        k = rng.standard_normal(dk)
        k /= np.linalg.norm(k)
        q = rng.standard_normal(dk)
        v = rng.standard_normal(dv)
        alpha = rng.uniform(0.01, 1.0)
        beta = rng.uniform(0.0, 1.0)
        x = rng.standard_normal(dk)
        x -= (x @ k) * k
        _, sf = oracle.recurrent(q[None, None, None], k[None, None, None], v[None, None, None],
                                 np.full((1, 1, 1), np.log(alpha)), np.full((1, 1, 1), beta), h0[None, None])
        h1 = sf[0, 0]
        np.testing.assert_allclose(h1.T @ k, alpha * (1 - beta) * (h0.T @ k) + beta * v, atol=1e-12)
        np.testing.assert_allclose(h1.T @ x, alpha * (h0.T @ x), atol=1e-12)
        assert np.linalg.norm(h1) <= alpha * np.linalg.norm(h0) + beta * np.linalg.norm(v) + 1e-12


def test_p4_online_objective_stationary():
    """The step minimises ||S - alpha S_{t-1}||_F^2 - 2 <S k_t, beta (v_t - alpha S_{t-1} k_t)>
    ("Gated Attention Architectures", section 3, online-learning objective).  Its gradient
    2 (S - alpha S_{t-1}) - 2 beta (v - alpha S_{t-1} k) k^T vanishes at the oracle's S_t.
    An elementwise (Hadamard) reading of (I - beta k k^T) fails this."""
    d = rand_inputs(T=1, dk=12, dv=12, s0_std=1.0, seed=4)
    _, sf = run(d)
    Sp = d["s0"][0, 0].T
    S = sf[0, 0].T
    k = d["k"][0, 0, 0]
    v = d["v"][0, 0, 0]
    a = np.exp(d["g"][0, 0, 0])
    b = d["beta"][0, 0, 0]
    grad = 2 * (S - a * Sp) - 2 * b * np.outer(v - a * Sp @ k, k)
    assert np.abs(grad).max() < 1e-13
    had = a * Sp * (1 - b * np.outer(k, k)) + b * np.outer(v, k)  # the Hadamard variant
    assert np.abs(had - S).max() > 1e-3


def test_p5_identical_unit_keys_closed_form():
    """k_t = k for all t (unit): h_t = exp(G_t)(I - k k^T) h_0 + k m_t^T with the scalar-gain EMA
    m_t = alpha_t (1 - beta_t) m_{t-1} + beta_t v_t, m_0 = h_0^T k.  Derived from the Gated
    DeltaNet equation; here the chunk matrix A is dense, so the chunked form's solve is exercised."""
    rng = np.random.default_rng(5)
    dk, dv, T = 10, 7, 37
    k = rng.standard_normal(dk)
    k /= np.linalg.norm(k)
    d = rand_inputs(T=T, dk=dk, dv=dv, s0_std=0.7, seed=5)
    d["k"][:] = k
    o, sf = run(d)
    h0 = d["s0"][0, 0]
    P = np.eye(dk) - np.outer(k, k)
    m = h0.T @ k
    G = 0.0
    for t in range(T):
        a = np.exp(d["g"][0, t, 0])
        b = d["beta"][0, t, 0]
        G += d["g"][0, t, 0]
        m = a * (1 - b) * m + b * d["v"][0, t, 0]
        h = np.exp(G) * (P @ h0) + np.outer(k, m)
        np.testing.assert_allclose(o[0, t, 0], h.T @ d["q"][0, t, 0], atol=1e-12)
    np.testing.assert_allclose(sf[0, 0], h, atol=1e-12)
    for C in (4, 16, 64):
        oc, sc = oracle.chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], chunk=C)
        np.testing.assert_allclose(oc, o, atol=1e-12)
        np.testing.assert_allclose(sc, sf, atol=1e-12)


def test_p6_orthonormal_keys_decayed_linear_attention():
    """Orthonormal keys, S_0 = 0: the erase term never fires and the output is the decayed
    linear-attention parallel form o_t = sum_{i<=t} exp(G_t - G_i) beta_i (k_i . q_t) v_i (RetNet's
    parallel form in "Gated Attention Architectures", section 4, with a data-dependent decay whose
    indexing d_ij = sum_{l=j+1}^{i} log f_l is FoX's, section 6)."""
    rng = np.random.default_rng(6)
    dk, dv, T = 32, 5, 32
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    d = rand_inputs(T=T, dk=dk, dv=dv, seed=6)
    d["k"][0, :, 0] = Qm.T[:T]
    o, _ = run(d)
    G = np.cumsum(d["g"][0, :, 0])
    for t in range(T):
        acc = np.zeros(dv)
        for i in range(t + 1):
            acc += np.exp(G[t] - G[i]) * d["beta"][0, i, 0] * (d["k"][0, i, 0] @ d["q"][0, t, 0]) * d["v"][0, i, 0]
        np.testing.assert_allclose(o[0, t, 0], acc, atol=1e-13)
    oc, _ = oracle.chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], None, chunk=16)
    np.testing.assert_allclose(oc, o, atol=1e-13)


@pytest.mark.parametrize("seed", [7, 8, 9])
def test_p7_brute_force_dense_transitions(seed):
    """T <= 8: dense M_t = alpha_t (I - beta_t k_t k_t^T), S_t = S_{t-1} M_t + beta_t v_t k_t^T."""
    d = rand_inputs(B=2, T=8, Hqk=2, Hv=4, dk=6, dv=5, s0_std=0.3, seed=seed)
    o, sf = run(d)
    ob, sb = oracle.brute_force(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"])
    np.testing.assert_allclose(o, ob, atol=1e-13)
    np.testing.assert_allclose(sf, sb, atol=1e-13)


@pytest.mark.parametrize("C,T", [(1, 9), (4, 33), (16, 16), (16, 50), (64, 130), (32, 31)])
def test_p8_chunked_equals_recurrent(C, T):
    """The chunkwise refactoring reaches the recurrence's result (fp64, 1e-12), including a
    ragged last chunk, grouped heads and a nonzero initial state."""
    d = rand_inputs(B=2, T=T, Hqk=2, Hv=4, dk=16, dv=8, s0_std=0.1, seed=C * 100 + T)
    o, sf = run(d)
    oc, sc = oracle.chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], chunk=C)
    np.testing.assert_allclose(oc, o, atol=1e-12)
    np.testing.assert_allclose(sc, sf, atol=1e-12)


def test_p9_gqa_equals_repeated_heads():
    """Value head j reads query/key head floor(j / (Hv/Hqk)): equal to repeating q, k per group."""
    d = rand_inputs(B=2, T=12, Hqk=2, Hv=6, dk=8, dv=4, s0_std=0.2, seed=10)
    o, sf = run(d)
    qr = np.repeat(d["q"], 3, axis=2)
    kr = np.repeat(d["k"], 3, axis=2)
    o2, sf2 = oracle.recurrent(qr, kr, d["v"], d["g"], d["beta"], d["s0"])
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(sf, sf2)


def test_p9_resume_split_and_decode_steps():
    """The state is the whole memory: splitting T and feeding final -> initial equals one call;
    T single-token steps equal one prefill."""
    d = rand_inputs(B=1, T=20, Hqk=1, Hv=2, dk=8, dv=4, s0_std=0.2, seed=11)
    o, sf = run(d)
    sl = lambda a, s: a[:, s]
    o1, s1 = oracle.recurrent(*(sl(d[n], slice(0, 7)) for n in ("q", "k", "v", "g", "beta")), d["s0"])
    o2, s2 = oracle.recurrent(*(sl(d[n], slice(7, 20)) for n in ("q", "k", "v", "g", "beta")), s1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o, atol=1e-14)
    np.testing.assert_allclose(s2, sf, atol=1e-14)
    tr = lambda a: np.moveaxis(a, 1, 0)
    od, sd = oracle.decode(tr(d["q"]), tr(d["k"]), tr(d["v"]), tr(d["g"]), tr(d["beta"]), d["s0"])
    np.testing.assert_allclose(tr(od), o, atol=1e-14)
    np.testing.assert_allclose(sd, sf, atol=1e-14)


def test_p9_value_columns_independent():
    """Each value column of the state evolves on its own: running a subset of v's columns gives
    the same columns of o and of the state."""
    d = rand_inputs(T=15, dk=8, dv=6, s0_std=0.2, seed=12)
    o, sf = run(d)
    cols = [1, 4, 5]
    o2, s2 = oracle.recurrent(d["q"], d["k"], d["v"][..., cols], d["g"], d["beta"], d["s0"][..., cols])
    np.testing.assert_allclose(o2, o[..., cols], atol=1e-14)
    np.testing.assert_allclose(s2, sf[..., cols], atol=1e-14)


def test_p9_ungated_equals_delta_loop():
    """alpha = 1 reduces to the plain delta rule of "Decoding Next-Generation LLM Architectures",
    section 3.2: S (d_k x d_v) <- S - beta outer(k, k S) then S <- S + beta outer(k, v); y = q S."""
    d = rand_inputs(T=10, dk=6, dv=5, seed=13)
    d["g"][:] = 0.0
    o, sf = run(d)
    S = np.zeros((6, 5))
    for t in range(10):
        k, v, q, b = d["k"][0, t, 0], d["v"][0, t, 0], d["q"][0, t, 0], d["beta"][0, t, 0]
        S = S - b * np.outer(k, k @ S)
        S = S + b * np.outer(k, v)
        np.testing.assert_allclose(o[0, t, 0], q @ S, atol=1e-14)
    np.testing.assert_allclose(sf[0, 0], S, atol=1e-14)


def test_gate_limit_alpha_zero_clears_state():
    """alpha -> 0 clears the state ("Gated Attention Architectures", section 3): with alpha = 0
    each step keeps only beta v k^T, so o_t = beta_t (k_t . q_t) v_t."""
    d = rand_inputs(T=9, dk=6, dv=5, s0_std=1.0, seed=14)
    d["g"][:] = -np.inf
    o, sf = run(d)
    for t in range(9):
        k, v, q, b = d["k"][0, t, 0], d["v"][0, t, 0], d["q"][0, t, 0], d["beta"][0, t, 0]
        np.testing.assert_allclose(o[0, t, 0], b * (k @ q) * v, atol=1e-14)
    np.testing.assert_allclose(sf[0, 0], d["beta"][0, -1, 0] * np.outer(d["k"][0, -1, 0], d["v"][0, -1, 0]), atol=1e-14)


def test_scale_multiplies_q():
    d = rand_inputs(T=11, dk=8, dv=4, s0_std=0.1, seed=15)
    o, sf = run(d, scale=0.37)
    d2 = dict(d)
    d2["q"] = d["q"] * 0.37
    o2, sf2 = run(d2)
    np.testing.assert_allclose(o, o2, rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(sf, sf2)


def test_generator_recipe():
    """The synthetic inputs follow the stated recipe: unit q, k rows; beta in (0,1); g < 0."""
    d = gi.generate(gi.CONFIGS["tiny_f32"])
    assert d["q"].shape == (1, 128, 2, 32) and d["v"].shape == (1, 128, 2, 32)
    np.testing.assert_allclose(np.linalg.norm(d["k"], axis=-1), 1.0, atol=1e-6)
    assert (d["beta"] > 0).all() and (d["beta"] < 1).all() and (d["g"] < 0).all()
    assert d["s0"] is None
    bits = gi.bf16_bits(np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-39], dtype=np.float32))
    back = gi.bf16_bits_to_f32(bits)
    # 1 + 2^-8 is a tie and rounds to even (1.0); 1 + 3*2^-8 rounds up to 1 + 2^-6
    np.testing.assert_array_equal(back[:4], np.array([1.0, 1.0, 1.015625, -2.5], dtype=np.float32))
    d2 = gi.generate(gi.CONFIGS["tiny_f32"])
    np.testing.assert_array_equal(d["q"], d2["q"])
