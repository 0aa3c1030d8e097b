"""Seeded synthetic inputs for the gated delta rule (shared by the oracle side and the HIP side).

This module only draws random numbers and shapes them into the tensors the gated delta rule
consumes; it holds none of the rule's arithmetic.  The recipe follows the workloads the pages
describe (Qwen3-Next's Gated DeltaNet layer: 16 query/key heads, 32 value heads, head dim 128,
from "Qwen3-Next's Gated Attention: why one sigmoid gate kills the attention sink", spec table;
Qwen3.6-27B's 16 query/key and 48 value heads, from "The Transformer Isn't Alone Anymore",
section "The architecture hidden inside Qwen"):

* q, k ~ N(0, 1), then L2-normalised per (batch, token, head) over the head dim, in float32 with
  eps 1e-12 (the block structure puts an L2 norm on q and k before the delta rule:
  "Architecture Thread I", section "Modern Architecture Improvements").
* v ~ N(0, 1).
* beta = sigmoid(N(0, 1)) and g = log(alpha) = logsigmoid(N(mu, 1)), both computed in float64
  and stored as float32 (one scalar per token and value head).
* Optional initial state S0 = std * N(0, 1), float32, layout [B, Hv, dk, dv].
* bf16 tensors are rounded from float32 with round-to-nearest-even and kept as uint16 bit
  patterns (numpy has no bfloat16).

Draw order from numpy.random.Generator(PCG64(seed)): q, k, v, beta-logits, alpha-logits, S0.

The layer steps either side of the recurrence (:func:`generate_layer`) take the projections'
outputs before the short convolution: q_in, k_in, v_in ~ N(0, 1); conv taps ~ N(0, 1) / sqrt(W)
float32 [channels, W]; an optional conv state ~ N(0, 1) float32 [B, channels, W - 1]; the
recurrence output o ~ N(0, 0.25) and the gate projection z ~ N(0, 1); the RMSNorm weight
1 + 0.1 N(0, 1) float32.  Draw order: q_in, k_in, v_in, conv_q, conv_k, conv_v, state, o, z, w.
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = [
    "Config", "CONFIGS", "bf16_bits", "bf16_bits_to_f32", "generate", "generate_decode",
    "to_torch", "generate_torch", "generate_layer",
]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    B: int
    T: int
    Hqk: int
    Hv: int
    dk: int
    dv: int
    chunk: int
    dtype: str          # "f32" or "bf16": dtype of q, k, v and o
    mu: float           # mean of the alpha logit
    s0_std: float       # 0 -> zero initial state
    seed: int
    steps: int = 0      # >0: decode workload, T == 1 per step


CONFIGS = {
    "tiny_f32": Config("tiny_f32", B=1, T=128, Hqk=2, Hv=2, dk=32, dv=32, chunk=16,
                       dtype="f32", mu=3.0, s0_std=0.0, seed=1001),
    "qwen3next_prefill": Config("qwen3next_prefill", B=1, T=4096, Hqk=16, Hv=32, dk=128, dv=128,
                                chunk=64, dtype="bf16", mu=3.0, s0_std=0.0, seed=1002),
    "batched_prefill": Config("batched_prefill", B=8, T=8192, Hqk=16, Hv=32, dk=128, dv=128,
                              chunk=64, dtype="bf16", mu=3.0, s0_std=0.02, seed=1003),
    "qwen36_long_prefill": Config("qwen36_long_prefill", B=1, T=65536, Hqk=16, Hv=48, dk=128,
                                  dv=128, chunk=64, dtype="bf16", mu=4.0, s0_std=0.0, seed=1004),
    # one GPU's share of the Qwen3.6-27B-shaped 64K-token prefill when its heads are split eight
    # ways (2 query/key, 6 value heads): few chains, the case the affine chunk scan is for
    "qwen36_long_prefill_tp8": Config("qwen36_long_prefill_tp8", B=1, T=65536, Hqk=2, Hv=6, dk=128,
                                      dv=128, chunk=64, dtype="bf16", mu=4.0, s0_std=0.0, seed=1007),
    "decode": Config("decode", B=256, T=1, Hqk=16, Hv=32, dk=128, dv=128, chunk=64,
                     dtype="bf16", mu=3.0, s0_std=0.02, seed=1005, steps=64),
    # Kimi Delta Attention (per-key-channel decay; inputs from generate_kda): the Qwen3-Next
    # layer's size with as many query/key heads as value heads
    "kda_prefill": Config("kda_prefill", B=1, T=4096, Hqk=32, Hv=32, dk=128, dv=128, chunk=64,
                          dtype="bf16", mu=3.0, s0_std=0.0, seed=1006),
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32, exact."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _l2norm(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / np.maximum(n, np.float32(1e-12))).astype(np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def _draw(rng, lead, B, T, Hqk, Hv, dk, dv, dtype, mu, s0_std):
    shp = tuple(lead)
    q = _l2norm(rng.standard_normal(shp + (B, T, Hqk, dk), dtype=np.float32))
    k = _l2norm(rng.standard_normal(shp + (B, T, Hqk, dk), dtype=np.float32))
    v = rng.standard_normal(shp + (B, T, Hv, dv), dtype=np.float32)
    bl = rng.standard_normal(shp + (B, T, Hv)).astype(np.float64)
    al = rng.standard_normal(shp + (B, T, Hv)).astype(np.float64) + mu
    beta = (1.0 / (1.0 + np.exp(-bl))).astype(np.float32)
    g = (-np.logaddexp(0.0, -al)).astype(np.float32)
    s0 = None
    if s0_std > 0:
        s0 = (s0_std * rng.standard_normal((B, Hv, dk, dv), dtype=np.float32)).astype(np.float32)
    return dict(q=_store(q, dtype), k=_store(k, dtype), v=_store(v, dtype), g=g, beta=beta, s0=s0)


def generate(cfg: Config | None = None, *, B=None, T=None, Hqk=None, Hv=None, dk=None, dv=None,
             dtype=None, mu=None, s0_std=None, seed=None) -> dict:
    """Prefill inputs.  Keyword arguments override the fields of ``cfg`` (or define a shape).

    Returns q, k [B,T,Hqk,dk], v [B,T,Hv,dv] (float32 or bf16 bits), g, beta [B,T,Hv] float32
    and s0 [B,Hv,dk,dv] float32 or None."""
    c = cfg
    B = B if B is not None else c.B
    T = T if T is not None else c.T
    Hqk = Hqk if Hqk is not None else c.Hqk
    Hv = Hv if Hv is not None else c.Hv
    dk = dk if dk is not None else c.dk
    dv = dv if dv is not None else c.dv
    dtype = dtype if dtype is not None else c.dtype
    mu = mu if mu is not None else c.mu
    s0_std = s0_std if s0_std is not None else c.s0_std
    seed = seed if seed is not None else c.seed
    rng = np.random.Generator(np.random.PCG64(seed))
    return _draw(rng, (), B, T, Hqk, Hv, dk, dv, dtype, mu, s0_std)


def generate_decode(cfg: Config, *, B=None, steps=None, seed=None) -> dict:
    """Decode inputs: a leading [steps] axis on q, k, v, g, beta (T == 1 is squeezed):
    q, k [steps,B,Hqk,dk], v [steps,B,Hv,dv], g, beta [steps,B,Hv], s0 [B,Hv,dk,dv]."""
    B = B if B is not None else cfg.B
    steps = steps if steps is not None else cfg.steps
    seed = seed if seed is not None else cfg.seed
    rng = np.random.Generator(np.random.PCG64(seed))
    d = _draw(rng, (steps,), B, 1, cfg.Hqk, cfg.Hv, cfg.dk, cfg.dv, cfg.dtype, cfg.mu, cfg.s0_std)
    for n in ("q", "k", "v", "g", "beta"):
        d[n] = np.ascontiguousarray(d[n][:, :, 0])
    return d


def generate_gate(B, T, Hv, dv, dtype="bf16", seed=3001, w_per_head=False) -> dict:
    """Inputs of the output gate alone (same recipe as generate_layer's z and weight):
    z [B,T,Hv,dv] (dtype) ~ N(0, 1); weight [dv] or [Hv, dv] float32 = 1 + 0.1 N(0, 1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    f = np.float32
    z = rng.standard_normal((B, T, Hv, dv), dtype=f)
    w = (1.0 + 0.1 * rng.standard_normal((Hv, dv) if w_per_head else (dv,))).astype(f)
    return dict(z=_store(z, dtype), weight=w)


def generate_kda(B, T, Hqk, Hv, dk, dv, dtype="bf16", mu=3.0, s0_std=0.0, seed=4001) -> dict:
    """Kimi Delta Attention inputs: q, k, v, beta and S0 as :func:`generate` (same draws and
    order), then g = log alpha per key channel [B,T,Hv,dk] = logsigmoid(N(mu + m_c, 1)) with a
    per-(head, channel) offset m_c ~ N(0, 1) drawn once, so channels decay at different rates."""
    rng = np.random.Generator(np.random.PCG64(seed))
    d = _draw(rng, (), B, T, Hqk, Hv, dk, dv, dtype, mu, s0_std)
    off = rng.standard_normal((Hv, dk))
    x = rng.standard_normal((B, T, Hv, dk)) + mu + off[None, None]
    d["g"] = (-np.logaddexp(0.0, -x)).astype(np.float32)
    return d


def varlen_lengths(n=64, lo=64, hi=2048, seed=5001) -> np.ndarray:
    """Sequence lengths of a packed batch: n draws uniform in [lo, hi] (int32, seeded)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(lo, hi + 1, n).astype(np.int32)


def to_torch(x: np.ndarray | None, dtype: str, device):
    """numpy array (float32, or uint16 bf16 bits) -> torch tensor on ``device``."""
    import torch
    if x is None:
        return None
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def generate_torch(cfg: Config, device, seed: int | None = None, decode_steps: int | None = None):
    """Same recipe drawn with torch's generator on ``device`` (fast, for timing runs only;
    parity runs use :func:`generate`).  Returns torch tensors in the same layouts."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(cfg.seed if seed is None else seed)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    lead = () if decode_steps is None else (decode_steps,)
    T = () if decode_steps is not None else (cfg.T,)

    def nrm(shape):
        return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)

    def l2(x):
        return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)

    q = l2(nrm(lead + (cfg.B,) + T + (cfg.Hqk, cfg.dk))).to(tdt)
    k = l2(nrm(lead + (cfg.B,) + T + (cfg.Hqk, cfg.dk))).to(tdt)
    v = nrm(lead + (cfg.B,) + T + (cfg.Hv, cfg.dv)).to(tdt)
    bl = nrm(lead + (cfg.B,) + T + (cfg.Hv,)).double()
    al = nrm(lead + (cfg.B,) + T + (cfg.Hv,)).double() + cfg.mu
    beta = torch.sigmoid(bl).float()
    g = (-torch.nn.functional.softplus(-al)).float()
    s0 = None
    if cfg.s0_std > 0:
        s0 = cfg.s0_std * nrm((cfg.B, cfg.Hv, cfg.dk, cfg.dv))
    return dict(q=q.contiguous(), k=k.contiguous(), v=v.contiguous(), g=g.contiguous(),
                beta=beta.contiguous(), s0=s0)


def generate_layer(B, T, Hqk, Hv, dk, dv, W=4, dtype="bf16", seed=2001, state=True, w_per_head=False) -> dict:
    """Inputs of the layer steps: q_in, k_in [B,T,Hqk,dk], v_in [B,T,Hv,dv] (dtype), conv_q,
    conv_k [Hqk*dk, W], conv_v [Hv*dv, W] float32, conv_state [B, 2*Hqk*dk + Hv*dv, W-1] float32
    or None; o, z [B,T,Hv,dv] (dtype); weight [dv] or [Hv, dv] float32."""
    rng = np.random.Generator(np.random.PCG64(seed))
    f = np.float32
    q_in = rng.standard_normal((B, T, Hqk, dk), dtype=f)
    k_in = rng.standard_normal((B, T, Hqk, dk), dtype=f)
    v_in = rng.standard_normal((B, T, Hv, dv), dtype=f)
    sc = f(1.0 / np.sqrt(W))
    conv_q = (rng.standard_normal((Hqk * dk, W), dtype=f) * sc).astype(f)
    conv_k = (rng.standard_normal((Hqk * dk, W), dtype=f) * sc).astype(f)
    conv_v = (rng.standard_normal((Hv * dv, W), dtype=f) * sc).astype(f)
    st = rng.standard_normal((B, 2 * Hqk * dk + Hv * dv, W - 1), dtype=f) if state else None
    o = (rng.standard_normal((B, T, Hv, dv), dtype=f) * f(0.5)).astype(f)
    z = rng.standard_normal((B, T, Hv, dv), dtype=f)
    w = (1.0 + 0.1 * rng.standard_normal((Hv, dv) if w_per_head else (dv,))).astype(f)
    return dict(q_in=_store(q_in, dtype), k_in=_store(k_in, dtype), v_in=_store(v_in, dtype), conv_q=conv_q,
                conv_k=conv_k, conv_v=conv_v, conv_state=st, o=_store(o, dtype), z=_store(z, dtype), weight=w)
