"""GPU parity of the layer with extra (text / audio) tokens: vdn_hybrid_attn_mixed
(through the C ABI) against the fp64 oracle on the same seeded inputs.

The video rows are checked per branch: with the gate at zero the layer returns the
softmax branch there (the readout adds g (.) O_lin = 0), and with the real gate the
merged output.  The extra rows (plain softmax over every token) are checked in
both calls and must not depend on the gate.  Tolerances as in test_gpu_parity:
max over heads of the relative Frobenius error, 1e-2 for bf16, and for the fp8
q.k variant 1e-2 against the oracle fed the same E4M3 codes, 5e-2 against the
unquantised oracle."""
import sys

import numpy as np
import pytest
import torch

import hybrid_sparse_linear_chunked_amd as vdn
import vdn_synth
from oracle import vdn_oracle as orc
from vdn_testlib import PREC_DTYPE, rel_err

pytestmark = pytest.mark.gpu

PREC = {"bf16": vdn.PREC_BF16, "bf16_fp8qk": vdn.PREC_BF16_FP8QK}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    vdn.load()


class MixedInputs:
    """q, k, v [F*N + T, H, d] in the I/O dtype (video tokens frame-major, then the
    extra tokens), beta, gate, and their device copies."""

    def __init__(self, F, N, T, H, d, precision, seed=0, q_std=1.0):
        self.F, self.N, self.T, self.H, self.d = F, N, T, H, d
        dt = PREC_DTYPE[precision]

        def make(name, **kw):
            vid = torch.empty((F, N, H, d), dtype=dt)
            vdn_synth.tensor(name, F, N, H, d, seed=seed, out=vid,
                             convert=lambda b: torch.from_numpy(b).to(dt), **kw)
            ext = torch.from_numpy(vdn_synth.extra(name, T, H, d, seed=seed, **kw)).to(dt)
            return torch.cat([vid.reshape(F * N, H, d), ext], dim=0).contiguous()

        self.q = make("q", q_std=q_std)
        self.k = make("k")
        self.v = make("v")
        self.beta = torch.from_numpy(vdn_synth.beta(F, H, seed=seed))
        self.gate = torch.from_numpy(vdn_synth.gate(H, d, seed=seed))
        self.dq, self.dk, self.dv = self.q.cuda(), self.k.cuda(), self.v.cuda()
        self.dbeta, self.dgate = self.beta.cuda(), self.gate.cuda()

    def host64(self, name, heads):
        """(video [F, N, Hs, d], extra [T, Hs, d]) as float64."""
        x = getattr(self, name)[:, list(heads)].to(torch.float64).numpy()
        F, N = self.F, self.N
        return x[:F * N].reshape(F, N, len(heads), self.d), x[F * N:]


def oracle_mixed(inp, frames, heads, tokens=None, xtokens=None, fp8=False):
    """Oracle (O_soft video, O video, O extra) on the sampled frames / tokens /
    extra tokens / heads; with fp8=True the softmax sees the oracle's fp8 q, k
    operands (per-head power-of-two scales over all F*N + T tokens)."""
    q, qx = inp.host64("q", heads)
    k, kx = inp.host64("k", heads)
    v, vx = inp.host64("v", heads)
    beta = inp.beta.numpy().astype(np.float64)[:, heads]
    gate = inp.gate.numpy().astype(np.float64)[heads]
    qs, ks, qxs, kxs = q, k, qx, kx
    if fp8:
        n = q.shape[0] * q.shape[1]
        allq = np.concatenate([q.reshape(-1, *q.shape[2:]), qx], axis=0)
        allk = np.concatenate([k.reshape(-1, *k.shape[2:]), kx], axis=0)
        qe, ke = orc.fp8_qk_operands(allq, allk, q.shape[-1])
        qs, qxs = qe[:n].reshape(q.shape), qe[n:]
        ks, kxs = ke[:n].reshape(k.shape), ke[n:]
    O_soft = orc.softmax_branch_mixed(qs, ks, v, kxs, vx, frames=frames, tokens=tokens)
    O_x = orc.softmax_extra_rows(ks, v, qxs, kxs, vx, xtokens=xtokens)
    Sf, Sb = orc.vda_states(k, v, beta)
    qt = q if tokens is None else q[:, list(tokens)]
    O_lin = orc.linear_branch(qt, Sf, Sb, frames=frames)
    return O_soft, orc.merge(O_soft, O_lin, gate), O_x


def check(name, got, ref, tol, head_axis=2):
    e = rel_err(got, ref, head_axis=head_axis)
    say(f"  {name}: rel_F err {e:.3e} (tol {tol:.0e})")
    assert e <= tol, f"{name}: {e} > {tol}"


def run_and_check(inp, precision, frames, heads, tokens=None, xtokens=None):
    F, N = inp.F, inp.N
    p = PREC[precision]
    O = vdn.hybrid_attn_mixed(inp.dq, inp.dk, inp.dv, inp.dbeta, inp.dgate, F, N, precision=p)
    O0 = vdn.hybrid_attn_mixed(inp.dq, inp.dk, inp.dv, inp.dbeta, torch.zeros_like(inp.dgate), F, N,
                               precision=p)
    torch.cuda.synchronize()
    say("  device done")
    # the extra rows do not depend on the gate
    assert torch.equal(O[F * N:].view(torch.int16), O0[F * N:].view(torch.int16))
    hs = list(heads)
    vid = lambda X: X[:F * N].reshape(F, N, inp.H, inp.d)[list(frames)][:, tokens if tokens is not None else slice(None)][:, :, hs]
    ext = lambda X: X[F * N:][xtokens if xtokens is not None else slice(None)][:, hs]
    host = lambda X: X.to(torch.float64).cpu().numpy()
    fp8 = precision == "bf16_fp8qk"
    rOs, rO, rOx = oracle_mixed(inp, frames, hs, tokens, xtokens, fp8=fp8)
    say("  oracle done")
    check("O_soft (video rows)", host(vid(O0)), rOs, 1e-2)
    check("O (video rows)", host(vid(O)), rO, 1e-2)
    if inp.T > 0:
        check("O (extra rows)", host(ext(O)), rOx, 1e-2, head_axis=1)
    if fp8:
        uOs, uO, uOx = oracle_mixed(inp, frames, hs, tokens, xtokens, fp8=False)
        check("O_soft vs unquantised", host(vid(O0)), uOs, 5e-2)
        check("O vs unquantised", host(vid(O)), uO, 5e-2)
        if inp.T > 0:
            check("O (extra rows) vs unquantised", host(ext(O)), uOx, 5e-2, head_axis=1)


@pytest.mark.parametrize("cfg", [
    (22, 100, 77, 2, 64, "bf16"),        # partial last chunk; ragged video and extra tiles
    (30, 256, 300, 4, 128, "bf16"),      # extra rows over two query tiles
    (7, 40, 5, 2, 32, "bf16"),           # every window sees every frame
    (23, 37, 130, 3, 32, "bf16"),        # d = 32 with linear states
    (2, 33, 20, 1, 64, "bf16"),          # anchors only
    (1, 5, 3, 1, 32, "bf16"),            # a single frame
    (31, 48, 64, 2, 64, "bf16_fp8qk"),   # exactly one extra key tile
    (24, 50, 200, 2, 128, "bf16_fp8qk"),
])
def test_mixed_small(cfg):
    F, N, T, H, d, prec = cfg
    say(f"case mixed F={F} N={N} T={T} H={H} d={d} {prec}")
    inp = MixedInputs(F, N, T, H, d, prec, seed=2)
    run_and_check(inp, prec, list(range(F)), list(range(H)))


def test_mixed_sharp_softmax():
    # logits at standard deviation ~4: the online maximum moves between video
    # and extra tiles
    F, N, T, H, d = 22, 64, 100, 2, 64
    say(f"case mixed sharp F={F} N={N} T={T} H={H} d={d}")
    inp = MixedInputs(F, N, T, H, d, "bf16", seed=3, q_std=4.0 * d ** 0.5)
    run_and_check(inp, "bf16", list(range(F)), list(range(H)))


def test_mixed_without_extras_is_the_video_layer():
    F, N, H, d = 22, 100, 2, 64
    say(f"case mixed T=0 F={F} N={N} H={H} d={d}")
    inp = MixedInputs(F, N, 0, H, d, "bf16", seed=4)
    O = vdn.hybrid_attn_mixed(inp.dq, inp.dk, inp.dv, inp.dbeta, inp.dgate, F, N)
    R = vdn.hybrid_attn(inp.dq.view(F, N, H, d), inp.dk.view(F, N, H, d), inp.dv.view(F, N, H, d),
                        inp.dbeta, inp.dgate)
    torch.cuda.synchronize()
    assert torch.equal(O.view(torch.int16).reshape(-1), R.view(torch.int16).reshape(-1))


def test_mixed_headline_sampled():
    # the headline video shape with 512 extra tokens; sampled outputs
    F, N, T, H, d = 90, 4032, 512, 24, 128
    say(f"case mixed full-size F={F} N={N} T={T} H={H} d={d} bf16")
    inp = MixedInputs(F, N, T, H, d, "bf16")
    frames = [0, 1, 7, 12, F // 2, F - 9, F - 2, F - 1]
    tokens = list(range(0, N, 97)) + [N - 1]
    xtokens = [0, 1, 63, 64, 255, 256, T - 1]
    run_and_check(inp, "bf16", frames, [0, H - 1], tokens, xtokens)
