"""GPU parity of the output projections (vdn_hybrid_attn_proj, vdn_out_proj, through
the C ABI) against the fp64 oracle on the same seeded inputs.

The GEMM alone is compared with the fp64 product of the same bf16 operands, and
must leave everything past Y[M, N] untouched.  The layer's projections are checked
per branch (W_l = 0 leaves the softmax branch's projection, W_s = 0 the gated
linear branch's) and together.  At the headline shape the weights are nonzero on
two heads' columns only, so the oracle needs those two heads.  Tolerance: relative
Frobenius error <= 1e-2 for the layer (bf16 inputs and output), 4e-3 for the GEMM
alone (one bf16 rounding of the output)."""
import sys

import numpy as np
import pytest
import torch

import hybrid_sparse_linear_chunked_amd as vdn
import vdn_synth
from oracle import vdn_oracle as orc
from vdn_testlib import Inputs

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    vdn.load()


def relF(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    return np.linalg.norm(x - ref) / np.linalg.norm(ref)


@pytest.mark.parametrize("M,K,N", [
    (1, 64, 8),          # one row, one K step, a partial N tile
    (300, 128, 200),     # ragged M and N tiles
    (513, 192, 264),
    (1024, 6144, 512),   # the layer's K at d = 128, H = 24
    (1300, 128, 520),    # 6 M tiles: one full group of 4 and a partial one; ragged N
])
def test_gemm_alone(M, K, N):
    say(f"case gemm M={M} K={K} N={N}")
    g = torch.Generator().manual_seed(M * 7 + K + N)
    A = torch.randn(M, K, generator=g).to(torch.bfloat16)
    B = (torch.randn(N, K, generator=g) / K ** 0.5).to(torch.bfloat16)
    guard = 4096
    Ybuf = torch.full((M * N + guard,), 7.0, dtype=torch.bfloat16, device="cuda")
    Y = Ybuf[:M * N].view(M, N)
    vdn.out_proj(A.cuda(), B.cuda(), out=Y)
    torch.cuda.synchronize()
    ref = A.double().numpy() @ B.double().numpy().T
    e = relF(Y.double().cpu().numpy(), ref)
    say(f"  rel_F err {e:.3e}")
    assert e <= 4e-3
    assert torch.all(Ybuf[M * N:] == 7.0), "writes past Y"


def _proj_check(inp, Wp, precision, tag):
    F, N, H, d = inp.F, inp.N, inp.H, inp.d
    Hd = H * d
    p = {"bf16": vdn.PREC_BF16, "bf16_fp8qk": vdn.PREC_BF16_FP8QK}[precision]
    W = torch.from_numpy(Wp).to(torch.bfloat16)
    Wd = W.cuda()
    zero = torch.zeros_like(Wd[:, :Hd])
    Ws_only = torch.cat([Wd[:, :Hd], zero], dim=1).contiguous()
    Wl_only = torch.cat([zero, Wd[:, Hd:]], dim=1).contiguous()
    outs = [vdn.hybrid_attn_proj(inp.dq, inp.dk, inp.dv, inp.dbeta, inp.dgate, w, precision=p)
            for w in (Ws_only, Wl_only, Wd)]
    torch.cuda.synchronize()
    Wf = W.double().numpy()
    q, k, v = inp.host64("q"), inp.host64("k"), inp.host64("v")
    beta = inp.beta.numpy().astype(np.float64)
    gate = inp.gate.numpy().astype(np.float64)
    qs, ks = q, k
    if precision == "bf16_fp8qk":
        qs, ks = orc.fp8_qk_operands(q, k, q.shape[-1])
    Os = orc.softmax_branch(qs, ks, v)
    Sf, Sb = orc.vda_states(k, v, beta)
    Ol = orc.linear_branch(q, Sf, Sb)
    Zs = np.zeros_like(Wf[:, :Hd])
    refs = [orc.output_projection(Os, Ol, gate, Wf[:, :Hd], Zs),
            orc.output_projection(Os, Ol, gate, Zs, Wf[:, Hd:]),
            orc.output_projection(Os, Ol, gate, Wf[:, :Hd], Wf[:, Hd:])]
    for name, Y, R in zip(("softmax branch projected", "linear branch projected", "both"), outs, refs):
        if tag == "no-linear" and name == "linear branch projected":
            assert not Y.float().abs().max().item()
            continue
        e = relF(Y.double().cpu().numpy(), R.reshape(F * N, -1))
        say(f"  {name}: rel_F err {e:.3e}")
        assert e <= 1e-2, f"{name}: {e}"


@pytest.mark.parametrize("cfg", [
    (22, 100, 2, 64, 96, "bf16", ""),           # partial last chunk, ragged tiles, partial N tile
    (30, 256, 4, 128, 264, "bf16", ""),
    (23, 37, 3, 32, 40, "bf16", ""),            # d = 32
    (7, 40, 2, 32, 64, "bf16", "no-linear"),    # every window sees every frame: O_lin = 0
    (31, 48, 2, 64, 64, "bf16_fp8qk", ""),
])
def test_layer_projection_small(cfg):
    F, N, H, d, D, prec, tag = cfg
    say(f"case proj F={F} N={N} H={H} d={d} D={D} {prec}")
    inp = Inputs(F, N, H, d, prec, seed=5)
    _proj_check(inp, vdn_synth.proj_weights(D, H * d, seed=5), prec, tag)


def test_layer_projection_headline_sampled():
    F, N, H, d, D = 90, 4032, 24, 128, 3072
    Hd = H * d
    say(f"case proj full-size F={F} N={N} H={H} d={d} D={D} bf16 (weights on heads 0 and {H - 1})")
    inp = Inputs(F, N, H, d, "bf16")
    heads = [0, H - 1]
    Wp = vdn_synth.proj_weights(D, Hd)
    mask = np.zeros(Hd, dtype=bool)
    for h in heads:
        mask[h * d:(h + 1) * d] = True
    Wp[:, :Hd][:, ~mask] = 0.0
    Wp[:, Hd:][:, ~mask] = 0.0
    W = torch.from_numpy(Wp).to(torch.bfloat16)
    Y = vdn.hybrid_attn_proj(inp.dq, inp.dk, inp.dv, inp.dbeta, inp.dgate, W.cuda())
    torch.cuda.synchronize()
    say("  device done")
    frames = [0, 1, 7, 12, F // 2, F - 9, F - 2, F - 1]
    tokens = list(range(0, N, 97)) + [N - 1]
    q, k, v = (inp.host64(n, heads=heads) for n in ("q", "k", "v"))
    beta = inp.beta.numpy().astype(np.float64)[:, heads]
    gate = inp.gate.numpy().astype(np.float64)[heads]
    Os = orc.softmax_branch(q, k, v, frames=frames, tokens=tokens)
    Sf, Sb = orc.vda_states(k, v, beta)
    Ol = orc.linear_branch(q[:, tokens], Sf, Sb, frames=frames)
    cols = np.concatenate([np.arange(h * d, (h + 1) * d) for h in heads])
    Wf = W.double().numpy()
    R = orc.output_projection(Os, Ol, gate, Wf[:, :Hd][:, cols], Wf[:, Hd:][:, cols])
    rows = [f * N + t for f in frames for t in tokens]
    got = Y[rows].double().cpu().numpy().reshape(len(frames), len(tokens), D)
    say("  oracle done")
    e = relF(got, R)
    say(f"  Y (sampled rows): rel_F err {e:.3e}")
    assert e <= 1e-2
