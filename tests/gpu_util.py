"""Helpers for the GPU parity tests: move seeded inputs to the device, call the HIP library,
compare with the float64 oracle at the stated tolerances."""
import sys

import numpy as np

import gdn_inputs as gi

DEV = "cuda:0"

# Tolerances: float32 inputs -> relative L2 <= 1e-4 on O and on the final state;
# bf16 inputs -> relative L2 <= 1e-2 on O and on the final state, and max |O - O_ref| <= 5e-2.
TOL = {"f32": dict(rel=1e-4, max_abs=None), "bf16": dict(rel=1e-2, max_abs=5e-2)}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def f64(a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return gi.bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def dev(d):
    import torch  # noqa: F401
    return {n: gi.to_torch(a, None, DEV) for n, a in d.items()}


def host(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def rel_l2(x, ref):
    den = np.linalg.norm(ref)
    return np.linalg.norm(x - ref) / (den if den > 0 else 1.0)


def check(name, dtype, o, o_ref, s=None, s_ref=None):
    tol = TOL[dtype]
    ro = rel_l2(o, o_ref)
    msg = f"{name}: rel_l2(o)={ro:.3e}"
    ok = ro <= tol["rel"]
    if tol["max_abs"] is not None:
        ma = float(np.abs(o - o_ref).max()) if o.size else 0.0
        msg += f" max_abs(o)={ma:.3e}"
        ok &= ma <= tol["max_abs"]
    if s is not None:
        rs = rel_l2(s, s_ref)
        msg += f" rel_l2(S)={rs:.3e}"
        ok &= rs <= tol["rel"]
    say(msg)
    assert ok, msg + f" exceeds tolerance {tol}"


def sample_chains(d, chains, Hqk, Hv):
    """Cut the inputs of the (b, value head) chains listed into a batch of single-head problems
    (for the oracle): q, k [n,T,1,dk], v [n,T,1,dv], g, beta [n,T,1], s0 [n,1,dk,dv]."""
    grp = Hv // Hqk
    out = {}
    for n in ("q", "k"):
        out[n] = np.stack([d[n][b, :, j // grp] for b, j in chains])[:, :, None]
    out["v"] = np.stack([d["v"][b, :, j] for b, j in chains])[:, :, None]
    for n in ("g", "beta"):
        out[n] = np.stack([d[n][b, :, j] for b, j in chains])[:, :, None]
    out["s0"] = None if d["s0"] is None else np.stack([d["s0"][b, j] for b, j in chains])[:, None]
    return out


class Guarded:
    """An output tensor with guard bands: `t` is a view into a larger buffer whose GUARD elements
    before and after it hold a fill pattern; `check()` asserts that no kernel wrote past either
    end of `t`."""
    GUARD = 1024

    def __init__(self, shape, dtype, fill=-7.75):
        import torch
        n = 1
        for x in shape:
            n *= int(x)
        self.n = n
        self.fill = fill
        self.buf = torch.full((n + 2 * self.GUARD,), fill, dtype=dtype, device=DEV)
        self.t = self.buf[self.GUARD:self.GUARD + n].view(*shape)

    def check(self, name=""):
        import torch
        lo, hi = self.buf[:self.GUARD], self.buf[self.GUARD + self.n:]
        ref = torch.full_like(lo, self.fill)
        assert torch.equal(lo, ref) and torch.equal(hi, ref), f"{name}: a kernel wrote outside its output"
