"""Shared pieces of the GPU parity tests: seeded inputs as host tensors in the
device precision, their device copies, the oracle on sampled slices, and the
error metric (relative Frobenius error per head, max over heads)."""
from __future__ import annotations

import numpy as np
import torch

import vdn_synth
from oracle import vdn_oracle as orc

PREC_DTYPE = {"fp32": torch.float32, "bf16": torch.bfloat16, "bf16_fp8qk": torch.bfloat16, "fp8": torch.bfloat16}
TOL = {"fp32": 1e-4, "bf16": 1e-2, "bf16_fp8qk": 5e-2}


class Inputs:
    """q, k, v (host tensors in the I/O dtype, [F, N, H, d]), beta, gate, and their
    device copies.  The oracle reads the host tensors, i.e. exactly the values the
    device sees."""

    def __init__(self, F, N, H, d, precision, seed=0, q_std=1.0, k_override=None):
        self.F, self.N, self.H, self.d, self.precision = F, N, H, d, precision
        dt = PREC_DTYPE[precision]

        def make(name, **kw):
            out = torch.empty((F, N, H, d), dtype=dt)
            vdn_synth.tensor(name, F, N, H, d, seed=seed, out=out,
                             convert=lambda b: torch.from_numpy(b).to(dt), **kw)
            return out

        self.q = make("q", q_std=q_std)
        self.k = make("k") if k_override is None else k_override.to(dt)
        self.v = make("v")
        self.beta = torch.from_numpy(vdn_synth.beta(F, H, seed=seed))
        self.gate = torch.from_numpy(vdn_synth.gate(H, d, seed=seed))
        self.dq = self.q.cuda()
        self.dk = self.k.cuda()
        self.dv = self.v.cuda()
        self.dbeta = self.beta.cuda()
        self.dgate = self.gate.cuda()

    def host64(self, name, frames=None, heads=None, tokens=None):
        x = getattr(self, name)
        if frames is not None:
            x = x[list(frames)]
        if tokens is not None:
            x = x[:, list(tokens)]
        if heads is not None:
            x = x[:, :, list(heads)]
        return x.to(torch.float64).numpy()


def rel_err(x, ref, head_axis=2):
    """max over heads of ||x - ref||_F / ||ref||_F (x, ref arrays with a head axis)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    worst = 0.0
    for h in range(ref.shape[head_axis]):
        a = np.take(x, h, axis=head_axis)
        b = np.take(ref, h, axis=head_axis)
        nb = np.linalg.norm(b)
        e = np.linalg.norm(a - b) / nb if nb > 0 else np.linalg.norm(a - b)
        if not np.isfinite(e):
            return float("inf")      # NaN / Inf anywhere fails (max() would skip a NaN)
        worst = max(worst, e)
    return worst


def oracle_slices(inp: Inputs, frames, heads, tokens=None, fp8=False, fp8v=False):
    """Oracle O_soft, O_lin (ungated) and O on the sampled frames / tokens / heads.
    With fp8=True the softmax uses the E4M3-quantised q and k (the oracle's fp8
    operands: per-head power-of-two scales, q carrying the base-2 temperature),
    isolating the kernel's error from the quantisation."""
    q = inp.host64("q", heads=heads)
    k = inp.host64("k", heads=heads)
    v = inp.host64("v", heads=heads)
    beta = inp.beta.numpy().astype(np.float64)[:, heads]
    gate = inp.gate.numpy().astype(np.float64)[heads]
    qs, ks = q, k
    vs = v
    if fp8:
        qs, ks = orc.fp8_qk_operands(q, k, q.shape[-1])
    if fp8v:
        vs = orc.fp8_v_operand(v)
    O_soft = orc.softmax_branch(qs, ks, vs, frames=frames, tokens=tokens)
    Sf, Sb = orc.vda_states(k, v, beta)
    qt = q if tokens is None else q[:, list(tokens)]
    O_lin = orc.linear_branch(qt, Sf, Sb, frames=frames)
    O = orc.merge(O_soft, O_lin, gate)
    return O_soft, O_lin, O, Sf, Sb
