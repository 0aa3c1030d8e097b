"""Oracle for the gated delta rule: plain float64 CPU implementations.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
may import this package.  Nothing here is shared with the HIP library, and nothing here imports it.

* :func:`recurrent` -- the definition, token by token, in C (``gdn_oracle.c``), float64, OpenMP
  over independent (batch, value-head) chains.  This is the oracle every GPU result is compared to.
* :func:`decode` -- the same recurrence applied once per call over a sequence of decode steps.
* :func:`recurrent_bwd` -- its reverse-mode adjoint, token by token, in C, float64: the gradients
  of a loss through o and the final state with respect to q, k, v, g, beta and S0.
* :func:`chunked_bwd` -- the gradients through the chunkwise form, in numpy float64: the chunk
  algebra of the backward pass the GPU implements, pinned against :func:`recurrent_bwd`.
* :func:`brute_force` -- the recurrence with every transition matrix written out densely
  (numpy), for tiny inputs; an independent code path used to pin :func:`recurrent`.
* :func:`chunked` -- the chunkwise (WY / UT-transform) refactoring of the same recurrence in
  numpy float64, used to pin the chunk algebra the GPU implements.
* :func:`kda_recurrent` (C), :func:`kda_brute_force`, :func:`kda_chunked` (numpy) -- Kimi Delta
  Attention, the delta rule with one decay per key channel ("Gated Attention Architectures",
  section 8): the definition, its dense transition matrices, and its chunkwise form.
* :func:`transport` -- the affine state map (M, N) of a stretch of tokens, from the definition:
  the state reached from a zero entry state, and the states reached from unit entry states with
  the writes removed.
* :func:`qkv_prologue`, :func:`gated_rmsnorm` (module ``layer_ops``) -- the layer steps either
  side of the recurrence: short causal conv, SiLU and q/k L2 norm; gated RMSNorm of the output.

Citations name the page and the section/equation followed.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

from .layer_ops import gated_rmsnorm, qkv_prologue, silu

__all__ = ["transport", "kda_recurrent", "kda_brute_force", "kda_chunked", "recurrent", "recurrent_bwd", "decode", "brute_force", "chunked", "chunked_bwd", "max_threads",
           "load", "qkv_prologue", "gated_rmsnorm", "silu"]

_lib = None


def load():
    """Load (building if needed) the C oracle library."""
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.gdn_oracle_recurrent.argtypes = [dp] * 8 + [ctypes.c_int] * 6 + [ctypes.c_double, ctypes.c_int]
        lib.gdn_oracle_recurrent.restype = ctypes.c_int
        lib.gdn_oracle_max_threads.restype = ctypes.c_int
        lib.gdn_oracle_recurrent_bwd.argtypes = [dp] * 14 + [ctypes.c_int] * 6 + [ctypes.c_double, ctypes.c_int]
        lib.gdn_oracle_recurrent_bwd.restype = ctypes.c_int
        lib.gdn_oracle_kda_recurrent.argtypes = [dp] * 8 + [ctypes.c_int] * 6 + [ctypes.c_double, ctypes.c_int]
        lib.gdn_oracle_kda_recurrent.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(load().gdn_oracle_max_threads())


def _f64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    if x is None:
        return ctypes.POINTER(ctypes.c_double)()
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def recurrent(q, k, v, g, beta, s0=None, scale: float = 1.0, threads: int = 0):
    """Token-by-token float64 gated delta rule (the definition).

    S_t = S_{t-1}(alpha_t (I - beta_t k_t k_t^T)) + beta_t v_t k_t^T, o_t = S_t q_t
    ("Architecture Thread I", section "Gated DeltaNet"; "Gated Attention Architectures",
    section 3), stored transposed as h = S^T [B,Hv,dk,dv].

    q, k: [B,T,Hqk,dk]; v: [B,T,Hv,dv]; g = log alpha, beta: [B,T,Hv]; s0: [B,Hv,dk,dv] or None.
    Returns (o [B,T,Hv,dv], s_final [B,Hv,dk,dv]) in float64."""
    q, k, v, g, beta, s0 = map(_f64, (q, k, v, g, beta, s0))
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    assert k.shape == q.shape and v.shape[:2] == (B, T) and g.shape == (B, T, Hv) == beta.shape
    if s0 is not None:
        assert s0.shape == (B, Hv, dk, dv)
    o = np.empty((B, T, Hv, dv), dtype=np.float64)
    sf = np.empty((B, Hv, dk, dv), dtype=np.float64)
    rc = load().gdn_oracle_recurrent(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0),
                                     _ptr(o), _ptr(sf), B, T, Hqk, Hv, dk, dv, float(scale), int(threads))
    if rc != 0:
        raise ValueError("oracle rejected the sizes")
    return o, sf


def transport(k, v, g, beta, threads: int = 0):
    """The affine state map of T tokens per (batch, value head): after them the stored state is
    M h0 + N for any entry state h0.

    Every step of the recurrence, h <- alpha (I - beta k k^T) h + beta k v^T in the stored
    orientation h = S^T ("Gated Attention Architectures", section 3, Mathematical Formulation),
    is affine in h, so the whole stretch is too.  N is the state reached from h0 = 0.  The linear
    part acts on each value column of h alike, so M [dk, dk] is the state reached from h0 = I with
    every write removed (v = 0), one unit entry column per key channel.  Both are runs of
    :func:`recurrent` (q does not enter the state; k stands in for it).

    k: [B,T,Hqk,dk]; v: [B,T,Hv,dv]; g, beta: [B,T,Hv].  Returns (M [B,Hv,dk,dk],
    N [B,Hv,dk,dv]) float64."""
    k, v = _f64(k), _f64(v)
    B, T, Hqk, dk = k.shape
    Hv = v.shape[2]
    _, N = recurrent(k, k, v, g, beta, None, threads=threads)
    unit = np.ascontiguousarray(np.broadcast_to(np.eye(dk), (B, Hv, dk, dk)))
    _, M = recurrent(k, k, np.zeros((B, T, Hv, dk)), g, beta, unit, threads=threads)
    return M, N


def recurrent_bwd(q, k, v, g, beta, s0, do, dsf=None, scale: float = 1.0, threads: int = 0):
    """Gradients of L = <do, o> + <dsf, s_final> through :func:`recurrent` (reverse-mode adjoint
    of each step of the recurrence, in C, float64).

    Returns dict(dq, dk [B,T,Hqk,dk], dv [B,T,Hv,dv], dg, dbeta [B,T,Hv], ds0 [B,Hv,dk,dv]); the
    gradient of a query/key head sums the contributions of the value heads of its group."""
    q, k, v, g, beta, s0, do, dsf = map(_f64, (q, k, v, g, beta, s0, do, dsf))
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    assert do.shape == (B, T, Hv, dv)
    dq_v = np.empty((B, T, Hv, dk))
    dk_v = np.empty((B, T, Hv, dk))
    dvv = np.empty((B, T, Hv, dv))
    dg = np.empty((B, T, Hv))
    dbeta = np.empty((B, T, Hv))
    ds0 = np.empty((B, Hv, dk, dv))
    rc = load().gdn_oracle_recurrent_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0), _ptr(do),
                                         _ptr(dsf), _ptr(dq_v), _ptr(dk_v), _ptr(dvv), _ptr(dg), _ptr(dbeta),
                                         _ptr(ds0), B, T, Hqk, Hv, dk, dv, float(scale), int(threads))
    if rc != 0:
        raise ValueError("oracle rejected the sizes")
    grp = Hv // Hqk
    dq = dq_v.reshape(B, T, Hqk, grp, dk).sum(axis=3)
    dkk = dk_v.reshape(B, T, Hqk, grp, dk).sum(axis=3)
    return dict(dq=dq, dk=dkk, dv=dvv, dg=dg, dbeta=dbeta, ds0=ds0)


def decode(q, k, v, g, beta, s0, scale: float = 1.0, threads: int = 0):
    """Decode: one recurrence step per call, ``steps`` calls in a row, state carried over.

    q, k: [steps,B,Hqk,dk]; v: [steps,B,Hv,dv]; g, beta: [steps,B,Hv]; s0: [B,Hv,dk,dv] or None.
    Returns (o [steps,B,Hv,dv], s_final [B,Hv,dk,dv])."""
    steps = q.shape[0]
    h = None if s0 is None else _f64(s0)
    outs = []
    for s in range(steps):
        o, h = recurrent(q[s][:, None], k[s][:, None], v[s][:, None], g[s][:, None],
                         beta[s][:, None], h, scale, threads)
        outs.append(o[:, 0])
    if h is None:  # steps == 0
        B, Hv, dk, dv = q.shape[1], v.shape[2], q.shape[3], v.shape[3]
        h = np.zeros((B, Hv, dk, dv))
    return np.stack(outs) if outs else np.zeros((0,) + v.shape[1:]), h


def brute_force(q, k, v, g, beta, s0=None, scale: float = 1.0):
    """The recurrence with each transition written out as a dense matrix (numpy, tiny T only).

    Follows the Gated DeltaNet equation literally in math orientation S in R^{dv x dk}:
    M_t = alpha_t (I - beta_t k_t k_t^T) (dk x dk), S_t = S_{t-1} M_t + beta_t v_t k_t^T,
    o_t = S_t q_t ("Architecture Thread I", section "Gated DeltaNet")."""
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    grp = Hv // Hqk
    o = np.zeros((B, T, Hv, dv))
    sf = np.zeros((B, Hv, dk, dv))
    for b in range(B):
        for j in range(Hv):
            i = j // grp
            S = np.zeros((dv, dk)) if s0 is None else np.array(s0[b, j], dtype=np.float64).T.copy()
            for t in range(T):
                kt = k[b, t, i][:, None]
                M = np.exp(g[b, t, j]) * (np.eye(dk) - beta[b, t, j] * (kt @ kt.T))
                S = S @ M + beta[b, t, j] * (v[b, t, j][:, None] @ kt.T)
                o[b, t, j] = S @ (scale * q[b, t, i])
            sf[b, j] = S.T
    return o, sf


def chunked(q, k, v, g, beta, s0=None, chunk: int = 64, scale: float = 1.0):
    """Chunkwise form of the same recurrence (numpy float64).

    "Gated Attention Architectures", section 3, names the hardware-efficient algorithm: the
    DeltaNet WY representation (section 2: I - beta k k^T is a generalised Householder matrix)
    extended with per-chunk cumulative decay products gamma_j = prod_{i=chunk start}^{j} alpha_i.
    The pages give no further algebra; the steps below are derived from the recurrence.  Per chunk
    of C positions with entry state h0 (= S^T), log-decay cumsum gc_r = sum_{i<=r} g_i:

      A     = strictly-lower( diag(beta) (K K^T * Gamma) ),  Gamma_ri = exp(gc_r - gc_i)
      Delta = (I + A)^{-1} ( diag(beta) V - diag(beta exp(gc)) K h0 )
      O     = diag(exp(gc)) Q h0 + ( lower-incl(Q K^T * Gamma) ) Delta
      h1    = exp(gc_C) h0 + Ktilde^T Delta,   Ktilde_i = exp(gc_C - gc_i) k_i

    The output step has the shape of GLA's chunkwise parallel form ("Gated Attention
    Architectures", section 1) with V replaced by the state-corrected Delta.
    The triangular solve is done with numpy.linalg.solve (a library primitive)."""
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    grp = Hv // Hqk
    o = np.zeros((B, T, Hv, dv))
    sf = np.zeros((B, Hv, dk, dv))
    for b in range(B):
        for j in range(Hv):
            i = j // grp
            h = np.zeros((dk, dv)) if s0 is None else np.array(s0[b, j], dtype=np.float64)
            for c0 in range(0, T, chunk):
                c1 = min(T, c0 + chunk)
                K = k[b, c0:c1, i]
                Q = scale * q[b, c0:c1, i]
                V = v[b, c0:c1, j]
                bt = beta[b, c0:c1, j]
                gc = np.cumsum(g[b, c0:c1, j])
                Gam = np.exp(gc[:, None] - gc[None, :])
                A = np.tril(bt[:, None] * (K @ K.T) * Gam, -1)
                rhs = bt[:, None] * V - (bt * np.exp(gc))[:, None] * (K @ h)
                Delta = np.linalg.solve(np.eye(c1 - c0) + A, rhs)
                o[b, c0:c1, j] = np.exp(gc)[:, None] * (Q @ h) + np.tril(Q @ K.T * Gam) @ Delta
                Kt = np.exp(gc[-1] - gc)[:, None] * K
                h = np.exp(gc[-1]) * h + Kt.T @ Delta
            sf[b, j] = h
    return o, sf


def chunked_bwd(q, k, v, g, beta, s0, do, dsf=None, chunk: int = 64, scale: float = 1.0):
    """Gradients of L = <do, o> + <dsf, s_final> through the chunkwise form (numpy float64).

    Per chunk, with the forward quantities of :func:`chunked` (A, T = (I + A)^{-1},
    W = T diag(beta e^gc) K, U = T diag(beta) V, Delta = U - W h, M = lower-incl(Q K^T * Gamma),
    O = diag(e^gc) Q h + M Delta, h' = e^gL h + (diag(e^(gL - gc)) K)^T Delta, gL the last gc),
    and the gradient dh' of the chunk's exit state, the steps of the forward are differentiated in
    reverse order (derived from those equations; the pages give none of it):

      dDelta = diag(e^(gL-gc)) K dh' + M^T dO
      dh     = e^gL dh' + Q^T diag(e^gc) dO - W^T dDelta      (the entry state's gradient)
      dW = -dDelta h^T,  dU = dDelta,  dT = dU (diag(beta) V)^T + dW (diag(beta e^gc) K)^T
      dA = -T^T dT T^T  (strictly lower part),  and the gates' and keys' terms of each product

    and dg is the reverse cumulative sum of dgc inside the chunk.  The forward state entering
    every chunk is kept from a first pass.  q, k gradients sum over the value heads of a group.
    The inverse of the unit lower-triangular I + A is numpy.linalg.inv (a library primitive)."""
    q, k, v, g, beta, s0, do, dsf = map(_f64, (q, k, v, g, beta, s0, do, dsf))
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    grp = Hv // Hqk
    out = dict(dq=np.zeros((B, T, Hqk, dk)), dk=np.zeros((B, T, Hqk, dk)), dv=np.zeros((B, T, Hv, dv)),
               dg=np.zeros((B, T, Hv)), dbeta=np.zeros((B, T, Hv)), ds0=np.zeros((B, Hv, dk, dv)))
    starts = list(range(0, T, chunk))
    for b in range(B):
        for j in range(Hv):
            i = j // grp
            h = np.zeros((dk, dv)) if s0 is None else np.array(s0[b, j], dtype=np.float64)

            def parts(c0, h):
                c1 = min(T, c0 + chunk)
                n = c1 - c0
                K, Q, V = k[b, c0:c1, i], scale * q[b, c0:c1, i], v[b, c0:c1, j]
                bt = beta[b, c0:c1, j]
                gc = np.cumsum(g[b, c0:c1, j])
                eg, gL = np.exp(gc), gc[-1]
                ed = np.exp(gL - gc)
                Gam = np.exp(np.tril(gc[:, None] - gc[None, :]))
                KK = K @ K.T
                A = np.tril(bt[:, None] * KK * Gam, -1)
                Tm = np.linalg.inv(np.eye(n) + A)
                KB = (bt * eg)[:, None] * K
                W = Tm @ KB
                U = Tm @ (bt[:, None] * V)
                D = U - W @ h
                M = np.tril((Q @ K.T) * Gam)
                return dict(c1=c1, n=n, K=K, Q=Q, V=V, bt=bt, gc=gc, eg=eg, gL=gL, ed=ed, Gam=Gam, KK=KK, A=A,
                            Tm=Tm, KB=KB, W=W, U=U, D=D, M=M)

            hs = []
            for c0 in starts:
                hs.append(h)
                f = parts(c0, h)
                h = np.exp(f["gL"]) * h + (f["ed"][:, None] * f["K"]).T @ f["D"]
            dh = np.zeros((dk, dv)) if dsf is None else np.array(dsf[b, j], dtype=np.float64)
            for ci in range(len(starts) - 1, -1, -1):
                c0 = starts[ci]
                h = hs[ci]
                f = parts(c0, h)
                c1, K, Q, V, bt, gc, eg, gL, ed, Gam = (f[x] for x in ("c1", "K", "Q", "V", "bt", "gc", "eg", "gL", "ed", "Gam"))
                KK, A, Tm, KB, W, D, M = (f[x] for x in ("KK", "A", "Tm", "KB", "W", "D", "M"))
                dO = do[b, c0:c1, j]
                dK = np.zeros_like(K)
                dQ = np.zeros_like(Q)
                dgc = np.zeros_like(gc)
                dbt = np.zeros_like(bt)
                # h' = e^gL h + (diag(ed) K)^T D
                dD = (ed[:, None] * K) @ dh + M.T @ dO
                X = D @ dh.T                                  # d(diag(ed) K)
                dK += ed[:, None] * X
                t_ed = ed * np.sum(K * X, axis=1)             # d(ed_r) * ed_r
                dgc -= t_ed
                dgL = np.exp(gL) * np.sum(dh * h) + np.sum(t_ed)
                # O = diag(eg) Q h + M D
                Oi = eg[:, None] * (Q @ h)
                dgc += np.sum(dO * Oi, axis=1)
                dQ += eg[:, None] * (dO @ h.T)
                dM = np.tril(dO @ D.T)
                E = dM * Gam
                dQ += E @ K
                dK += E.T @ Q
                PM = dM * M
                dgc += PM.sum(axis=1) - PM.sum(axis=0)
                # state gradient for the previous chunk
                dh_prev = np.exp(gL) * dh + Q.T @ (eg[:, None] * dO) - W.T @ dD
                # D = U - W h
                dW = -dD @ h.T
                dU = dD
                # U = T diag(bt) V, W = T KB
                TdU = Tm.T @ dU
                out["dv"][b, c0:c1, j] = bt[:, None] * TdU
                dbt += np.sum(V * TdU, axis=1)
                dKB = Tm.T @ dW
                dK += (bt * eg)[:, None] * dKB
                kb = np.sum(K * dKB, axis=1)
                dbt += eg * kb
                dgc += bt * eg * kb
                dT = dU @ (bt[:, None] * V).T + dW @ KB.T
                # T = (I + A)^{-1}
                dA = np.tril(-Tm.T @ dT @ Tm.T, -1)
                # A = strictly-lower(diag(bt) (KK * Gam))
                G = KK * Gam
                dbt += np.sum(np.tril(dA * G, -1), axis=1)
                PA = np.tril(dA * A, -1)
                dgc += PA.sum(axis=1) - PA.sum(axis=0)
                Dk = np.tril(dA * bt[:, None] * Gam, -1)
                dK += Dk @ K + Dk.T @ K
                dgc[-1] += dgL
                out["dq"][b, c0:c1, i] += scale * dQ
                out["dk"][b, c0:c1, i] += dK
                out["dbeta"][b, c0:c1, j] = dbt
                out["dg"][b, c0:c1, j] = np.cumsum(dgc[::-1])[::-1]
                dh = dh_prev
            out["ds0"][b, j] = dh
    return out


def kda_recurrent(q, k, v, g, beta, s0=None, scale: float = 1.0, threads: int = 0):
    """Kimi Delta Attention, token by token (C, float64): S_t = (I - beta_t k_t k_t^T) D_t S_{t-1}
    + beta_t v_t k_t^T, o_t = S_t^T q_t with D_t = diag(exp(g_t)) over the key channels
    ("Gated Attention Architectures", section 8, Mathematical Formulation); S stored [dk, dv].

    q, k: [B,T,Hqk,dk]; v: [B,T,Hv,dv]; g = log alpha: [B,T,Hv,dk]; beta: [B,T,Hv];
    s0: [B,Hv,dk,dv] or None.  Returns (o [B,T,Hv,dv], s_final [B,Hv,dk,dv])."""
    q, k, v, g, beta, s0 = map(_f64, (q, k, v, g, beta, s0))
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    assert g.shape == (B, T, Hv, dk) and beta.shape == (B, T, Hv)
    o = np.empty((B, T, Hv, dv))
    sf = np.empty((B, Hv, dk, dv))
    rc = load().gdn_oracle_kda_recurrent(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0), _ptr(o),
                                         _ptr(sf), B, T, Hqk, Hv, dk, dv, float(scale), int(threads))
    if rc != 0:
        raise ValueError("oracle rejected the sizes")
    return o, sf


def kda_brute_force(q, k, v, g, beta, s0=None, scale: float = 1.0):
    """The KDA equation with its transition written out densely (numpy, tiny T only):
    S_t = (I - beta_t k_t k_t^T) diag(alpha_t) S_{t-1} + beta_t k_t v_t^T, S in R^{dk x dv}."""
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    grp = Hv // Hqk
    o = np.zeros((B, T, Hv, dv))
    sf = np.zeros((B, Hv, dk, dv))
    for b in range(B):
        for j in range(Hv):
            i = j // grp
            S = np.zeros((dk, dv)) if s0 is None else np.array(s0[b, j], dtype=np.float64)
            for t in range(T):
                kt = k[b, t, i][:, None]
                P = np.eye(dk) - beta[b, t, j] * (kt @ kt.T)
                S = P @ np.diag(np.exp(g[b, t, j])) @ S + beta[b, t, j] * (kt @ v[b, t, j][None, :])
                o[b, t, j] = S.T @ (scale * q[b, t, i])
            sf[b, j] = S
    return o, sf


def kda_chunked(q, k, v, g, beta, s0=None, chunk: int = 32, scale: float = 1.0):
    """Chunkwise form of KDA (numpy float64), derived from the recurrence: with gc the in-chunk
    cumulative log decay per key channel (gc_r = g_1 + ... + g_r, a vector) and
    E_ri = exp(gc_r - gc_i) for i <= r (elementwise over channels, never above 1):

      A     = strictly-lower( beta_r sum_c k_rc k_ic E_ric )
      Delta = (I + A)^{-1} ( diag(beta) V - diag(beta) (e^gc * K) h0 )
      O     = (e^gc * scale Q) h0 + lower-incl( sum_c q_rc k_ic E_ric ) Delta
      h1    = diag(e^gL) h0 + ((e^(gL - gc) * K))^T Delta,   gL the chunk's last gc

    ("Gated Attention Architectures", section 8, names a chunkwise WY-based algorithm for KDA;
    the pairwise decays are formed from differences so nothing overflows.)  The solve is
    numpy.linalg.solve."""
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    grp = Hv // Hqk
    o = np.zeros((B, T, Hv, dv))
    sf = np.zeros((B, Hv, dk, dv))
    for b in range(B):
        for j in range(Hv):
            i = j // grp
            h = np.zeros((dk, dv)) if s0 is None else np.array(s0[b, j], dtype=np.float64)
            for c0 in range(0, T, chunk):
                c1 = min(T, c0 + chunk)
                n = c1 - c0
                K = k[b, c0:c1, i]
                Q = scale * q[b, c0:c1, i]
                V = v[b, c0:c1, j]
                bt = beta[b, c0:c1, j]
                gc = np.cumsum(g[b, c0:c1, j], axis=0)                 # [n, dk]
                diff = gc[:, None, :] - gc[None, :, :]                  # [n, n, dk]
                E = np.exp(np.where(np.tril(np.ones((n, n)))[:, :, None] > 0, diff, -np.inf))
                A = np.tril(bt[:, None] * np.einsum("rc,ic,ric->ri", K, K, E), -1)
                Aqk = np.tril(np.einsum("rc,ic,ric->ri", Q, K, E))
                rhs = bt[:, None] * V - bt[:, None] * ((np.exp(gc) * K) @ h)
                Delta = np.linalg.solve(np.eye(n) + A, rhs)
                o[b, c0:c1, j] = (np.exp(gc) * Q) @ h + Aqk @ Delta
                gL = gc[-1]
                h = np.exp(gL)[:, None] * h + (np.exp(gL[None, :] - gc) * K).T @ Delta
            sf[b, j] = h
    return o, sf
