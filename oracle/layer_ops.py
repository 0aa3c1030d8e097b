"""Oracle for the steps either side of the recurrence in a Gated DeltaNet layer: plain float64
numpy, written from the definitions.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
may import this module.  Nothing here is shared with the HIP library, and nothing here imports it.

* :func:`qkv_prologue` -- short causal depthwise convolution over time, SiLU, and L2
  normalisation of q and k ("Architecture Thread I: Gated Attention, DeltaNet, and Hybrid
  Models", section "Modern Architecture Improvements": query/key go Linear -> Short Conv -> SiLU
  -> L2 Norm, value Linear -> Short Conv -> SiLU).
* :func:`gated_rmsnorm` -- RMSNorm over each value head's channels (same section, output
  normalisation) times SiLU of the gate projection (the output gate of the Gated DeltaNet block,
  "Gated Attention Architectures"; "gated RMSNorm" in "The Transformer Isn't Alone Anymore").

Readings where the pages leave a step open: the convolution is depthwise and causal with W taps
and no bias, tap W-1 multiplying the current token and history before token 0 taken from a
conv state (zeros when none); the L2 norm is y / sqrt(sum y^2 + eps); RMSNorm is
o / sqrt(mean o^2 + eps) times a per-channel weight; SiLU(a) = a / (1 + e^-a).
"""
from __future__ import annotations

import numpy as np

__all__ = ["silu", "qkv_prologue", "gated_rmsnorm"]


def silu(a):
    """SiLU(a) = a * sigmoid(a) = a / (1 + exp(-a))."""
    a = np.asarray(a, dtype=np.float64)
    return a / (1.0 + np.exp(-a))


def _causal_conv(x, w, hist):
    """x [B, T, C] inputs, w [C, W] taps, hist [B, W-1, C] inputs before token 0.
    Returns a [B, T, C] with a[t] = sum_j w[:, j] * x[t - (W-1) + j]."""
    B, T, C = x.shape
    W = w.shape[1]
    xp = np.concatenate([hist, x], axis=1)   # token t of x is row t + W - 1
    a = np.zeros((B, T, C))
    for j in range(W):
        a += w[:, j][None, None, :] * xp[:, j:j + T, :]
    return a, xp


def qkv_prologue(q_in, k_in, v_in, conv_q, conv_k, conv_v, conv_state_in=None, eps: float = 1e-6):
    """q_in, k_in [B,T,Hqk,dk]; v_in [B,T,Hv,dv]; conv_q, conv_k [Hqk*dk, W]; conv_v [Hv*dv, W];
    conv_state_in [B, 2*Hqk*dk + Hv*dv, W-1] (channels q, then k, then v; oldest first) or None.
    Returns (q, k, v, conv_state_out) in float64, conv_state_out the last W-1 inputs."""
    q_in, k_in, v_in = (np.asarray(a, dtype=np.float64) for a in (q_in, k_in, v_in))
    wq, wk, wv = (np.asarray(a, dtype=np.float64) for a in (conv_q, conv_k, conv_v))
    B, T, Hqk, dk = q_in.shape
    Hv, dv = v_in.shape[2], v_in.shape[3]
    W = wq.shape[1]
    cq, cv = Hqk * dk, Hv * dv
    x = np.concatenate([q_in.reshape(B, T, cq), k_in.reshape(B, T, cq), v_in.reshape(B, T, cv)], axis=2)
    w = np.concatenate([wq, wk, wv], axis=0)
    if conv_state_in is None:
        hist = np.zeros((B, W - 1, 2 * cq + cv))
    else:
        hist = np.transpose(np.asarray(conv_state_in, dtype=np.float64), (0, 2, 1))
    a, xp = _causal_conv(x, w, hist)
    y = silu(a)
    q = y[:, :, :cq].reshape(B, T, Hqk, dk)
    k = y[:, :, cq:2 * cq].reshape(B, T, Hqk, dk)
    v = y[:, :, 2 * cq:].reshape(B, T, Hv, dv)
    q = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + eps)
    k = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + eps)
    state_out = np.transpose(xp[:, T:T + W - 1, :], (0, 2, 1)).copy()
    return q, k, v, state_out


def gated_rmsnorm(o, z, weight, eps: float = 1e-6):
    """o, z [B,T,Hv,dv]; weight [dv] (shared by the heads) or [Hv, dv].
    Returns o / sqrt(mean over dv of o^2 + eps) * weight * silu(z) in float64."""
    o, z, w = (np.asarray(a, dtype=np.float64) for a in (o, z, weight))
    r = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return o * r * w * silu(z)
