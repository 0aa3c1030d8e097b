"""Pins of the layer-step oracle (oracle/layer_ops.py) to things other than itself: a library
convolution, closed forms, hand-worked values and invariants.  Then plausible mistakes are planted
in copies of the oracle (on the CPU) and each must fail at least one pin."""
import math
import os
import types

import numpy as np
import pytest

import oracle
import oracle.layer_ops as LO

SRC = LO.__file__


def _rng(seed=7):
    return np.random.default_rng(seed)


def _inputs(rng, B=2, T=9, Hqk=2, Hv=4, dk=8, dv=6, W=4, state=True):
    q = rng.standard_normal((B, T, Hqk, dk))
    k = rng.standard_normal((B, T, Hqk, dk))
    v = rng.standard_normal((B, T, Hv, dv))
    wq = rng.standard_normal((Hqk * dk, W))
    wk = rng.standard_normal((Hqk * dk, W))
    wv = rng.standard_normal((Hv * dv, W))
    st = rng.standard_normal((B, 2 * Hqk * dk + Hv * dv, W - 1)) if state else None
    return q, k, v, wq, wk, wv, st


# ---------------------------------------------------------------------------------- pins


def test_silu_closed_forms(m=LO):
    assert m.silu(0.0) == 0.0
    assert math.isclose(float(m.silu(1.0)), 1.0 / (1.0 + math.exp(-1.0)), rel_tol=1e-15)
    a = np.linspace(-6, 6, 25)
    assert np.allclose(m.silu(a) - m.silu(-a), a, atol=1e-14)     # odd part of a * sigmoid(a)
    assert math.isclose(float(m.silu(40.0)), 40.0, rel_tol=1e-15)
    assert abs(float(m.silu(-40.0))) < 1e-15


def test_conv_matches_numpy_convolve(m=LO):
    """The value path (no norm) is silu of numpy's full convolution with the reversed taps,
    history prepended."""
    rng = _rng(1)
    q, k, v, wq, wk, wv, st = _inputs(rng)
    _, _, vo, _ = m.qkv_prologue(q, k, v, wq, wk, wv, st)
    B, T, Hv, dv = v.shape
    W = wq.shape[1]
    cq = q.shape[2] * q.shape[3]
    for b in range(B):
        for h in range(Hv):
            for c in range(dv):
                ch = h * dv + c
                x = np.concatenate([st[b, 2 * cq + ch], v[b, :, h, c]])
                a = np.convolve(x, wv[ch][::-1])[W - 1:W - 1 + T]
                assert np.allclose(vo[b, :, h, c], a / (1 + np.exp(-a)), rtol=1e-13, atol=1e-13)


def test_hand_worked_prologue(m=LO):
    """Two channels, two tokens, W = 2, no history: channel 0 taps (1, 1), channel 1 taps (0, 2)."""
    q_in = np.array([[[[1.0, 2.0]], [[3.0, -1.0]]]])            # [1, 2, 1, 2]
    w = np.array([[1.0, 1.0], [0.0, 2.0]])
    q, k, v, st = m.qkv_prologue(q_in, q_in, q_in, w, w, w, None, eps=0.0)
    s = lambda a: a / (1 + math.exp(-a))
    pre = [[1.0, 4.0], [4.0, -2.0]]                              # conv by hand
    for t in range(2):
        y = [s(pre[t][0]), s(pre[t][1])]
        nrm = math.sqrt(y[0] ** 2 + y[1] ** 2)
        assert np.allclose(q[0, t, 0], [y[0] / nrm, y[1] / nrm], rtol=1e-14)
    assert np.allclose(st[0, :2, 0], [3.0, -1.0])               # the last input of q's channels


def test_delta_taps_identity_and_shift(m=LO):
    rng = _rng(2)
    q, k, v, wq, wk, wv, st = _inputs(rng, W=4)
    e3 = np.zeros_like(wv)
    e3[:, 3] = 1.0
    e2 = np.zeros_like(wv)
    e2[:, 2] = 1.0
    _, _, vo, _ = m.qkv_prologue(q, k, v, np.zeros_like(wq), np.zeros_like(wk), e3, st)
    assert np.allclose(vo, v / (1 + np.exp(-v)), rtol=1e-14, atol=1e-15)
    _, _, vs, _ = m.qkv_prologue(q, k, v, np.zeros_like(wq), np.zeros_like(wk), e2, st)
    assert np.allclose(vs[:, 1:], (v / (1 + np.exp(-v)))[:, :-1], rtol=1e-14, atol=1e-15)
    cq = q.shape[2] * q.shape[3]
    last = st[:, 2 * cq:, -1].reshape(v.shape[0], v.shape[2], v.shape[3])   # the input just before token 0
    assert np.allclose(vs[:, 0], last / (1 + np.exp(-last)), rtol=1e-14, atol=1e-15)


def test_l2_norm_per_head_unit_and_parallel(m=LO):
    """With q's and v's inputs and taps equal, q is v's output scaled to unit norm, head by head."""
    rng = _rng(3)
    B, T, H, d, W = 2, 7, 3, 8, 3
    x = rng.standard_normal((B, T, H, d))
    w = rng.standard_normal((H * d, W))
    q, k, v, _ = m.qkv_prologue(x, x, x, w, w, w, None, eps=0.0)
    assert np.allclose(np.linalg.norm(q, axis=-1), 1.0, atol=1e-13)
    assert np.allclose(q * np.linalg.norm(v, axis=-1, keepdims=True), v, rtol=1e-12, atol=1e-13)
    assert np.allclose(k, q)


def test_conv_state_continuation(m=LO):
    """One call over T tokens equals two calls over its halves with the state carried."""
    rng = _rng(4)
    q, k, v, wq, wk, wv, st = _inputs(rng, T=11)
    full = m.qkv_prologue(q, k, v, wq, wk, wv, st)
    for t1 in (1, 2, 5, 10):
        a = m.qkv_prologue(q[:, :t1], k[:, :t1], v[:, :t1], wq, wk, wv, st)
        b = m.qkv_prologue(q[:, t1:], k[:, t1:], v[:, t1:], wq, wk, wv, a[3])
        for i in range(3):
            assert np.allclose(np.concatenate([a[i], b[i]], axis=1), full[i], rtol=1e-13, atol=1e-14)
        assert np.allclose(b[3], full[3])


def test_conv_state_out_is_last_inputs(m=LO):
    rng = _rng(5)
    for T in (1, 2, 3, 6):
        q, k, v, wq, wk, wv, st = _inputs(rng, T=T, W=4)
        *_, so = m.qkv_prologue(q, k, v, wq, wk, wv, st)
        B, cq = q.shape[0], q.shape[2] * q.shape[3]
        x = np.concatenate([q.reshape(B, T, -1), k.reshape(B, T, -1), v.reshape(B, T, -1)], axis=2)
        hx = np.concatenate([np.transpose(st, (0, 2, 1)), x], axis=1)
        assert np.array_equal(so, np.transpose(hx[:, -3:], (0, 2, 1)))


def test_hand_worked_rmsnorm(m=LO):
    o = np.array([3.0, 4.0]).reshape(1, 1, 1, 2)
    z = np.array([50.0, 0.0]).reshape(1, 1, 1, 2)
    w = np.array([2.0, 5.0])
    y = m.gated_rmsnorm(o, z, w, eps=0.0)
    r = 1.0 / math.sqrt((9.0 + 16.0) / 2.0)
    assert math.isclose(float(y[0, 0, 0, 0]), 3.0 * r * 2.0 * 50.0 / (1 + math.exp(-50.0)), rel_tol=1e-14)
    assert y[0, 0, 0, 1] == 0.0                                  # silu(0) = 0


def test_rmsnorm_invariants(m=LO):
    rng = _rng(6)
    B, T, Hv, dv = 2, 5, 3, 16
    o = rng.standard_normal((B, T, Hv, dv))
    z = rng.standard_normal((B, T, Hv, dv))
    w = rng.uniform(0.5, 2.0, dv)
    y = m.gated_rmsnorm(o, z, w, eps=0.0)
    n = y / (w * (z / (1 + np.exp(-z))))
    assert np.allclose(np.mean(n * n, axis=-1), 1.0, rtol=1e-12)           # RMS 1 per head
    assert np.allclose(m.gated_rmsnorm(3.7 * o, z, w, eps=0.0), y, rtol=1e-12)
    assert np.allclose(m.gated_rmsnorm(-o, z, w, eps=0.0), -y, rtol=1e-12)
    c = np.full((1, 1, 1, dv), -2.5)
    zz = z[:1, :1, :1]
    assert np.allclose(m.gated_rmsnorm(c, zz, w, eps=0.0), -w * zz / (1 + np.exp(-zz)), rtol=1e-13)
    wh = np.stack([w * (j + 1) for j in range(Hv)])               # per-head weights
    yh = m.gated_rmsnorm(o, z, wh, eps=0.0)
    for j in range(Hv):
        assert np.allclose(yh[:, :, j], (j + 1) * y[:, :, j], rtol=1e-12)


PINS = [test_silu_closed_forms, test_conv_matches_numpy_convolve, test_hand_worked_prologue,
        test_delta_taps_identity_and_shift, test_l2_norm_per_head_unit_and_parallel,
        test_conv_state_continuation, test_conv_state_out_is_last_inputs, test_hand_worked_rmsnorm,
        test_rmsnorm_invariants]

# ------------------------------------------------------------------------------- mutants

MUTANTS = [
    ("taps_reversed", "a += w[:, j][None, None, :] * xp[:, j:j + T, :]",
     "a += w[:, W - 1 - j][None, None, :] * xp[:, j:j + T, :]"),
    ("history_ignored", "xp = np.concatenate([hist, x], axis=1)", "xp = np.concatenate([0 * hist, x], axis=1)"),
    ("sigmoid_not_silu", "return a / (1.0 + np.exp(-a))", "return 1.0 / (1.0 + np.exp(-a))"),
    ("l2_over_all_heads", "q = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + eps)",
     "q = q / np.sqrt(np.sum(q * q, axis=(-2, -1), keepdims=True) + eps)"),
    ("l2_without_sqrt", "k = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + eps)",
     "k = k / (np.sum(k * k, axis=-1, keepdims=True) + eps)"),
    ("v_normalised_too", "    state_out = np.transpose", "    v = v / np.linalg.norm(v, axis=-1, keepdims=True)\n    state_out = np.transpose"),
    ("state_slice_off_by_one", "xp[:, T:T + W - 1, :]", "xp[:, T - 1:T + W - 2, :]"),
    ("rms_sum_not_mean", "np.mean(o * o, axis=-1, keepdims=True)", "np.sum(o * o, axis=-1, keepdims=True)"),
    ("rms_wrong_axis", "np.mean(o * o, axis=-1, keepdims=True)", "np.mean(o * o, axis=-2, keepdims=True)"),
    ("gate_sigmoid", "return o * r * w * silu(z)", "return o * r * w / (1.0 + np.exp(-z))"),
    ("weight_dropped", "return o * r * w * silu(z)", "return o * r * silu(z)"),
]


def _mutant_module(edit):
    src = open(SRC).read()
    old, new = edit
    assert src.count(old) == 1, old
    mod = types.ModuleType("layer_ops_mutant")
    exec(compile(src.replace(old, new), "layer_ops_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("mut", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_layer_mutant(mut):
    mod = _mutant_module(mut[1:])
    failed = []
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin rejects mutant {mut[0]}"


def test_oracle_package_exports():
    assert oracle.qkv_prologue is LO.qkv_prologue and oracle.gated_rmsnorm is LO.gated_rmsnorm
