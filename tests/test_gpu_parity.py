"""GPU parity: the HIP path (called through the C ABI) against the fp64 oracle on
the same seeded inputs, per branch and for the merged output.

Tolerances (max over heads of the relative Frobenius error): 1e-4 fp32, 1e-2 bf16,
5e-2 for the fp8 (E4M3 q.k) softmax variant against the unquantised oracle and
1e-2 against the oracle fed the same E4M3 codes.  Integer work (the partition,
the E4M3 codes) is compared bit for bit."""
import os
import sys

import numpy as np
import pytest
import torch

import hybrid_sparse_linear_chunked_amd as vdn
from oracle import vdn_oracle as orc
from vdn_testlib import TOL, Inputs, oracle_slices, rel_err

pytestmark = pytest.mark.gpu

PREC = {"fp32": vdn.PREC_FP32, "bf16": vdn.PREC_BF16, "bf16_fp8qk": vdn.PREC_BF16_FP8QK}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    vdn.load()


def run_all(inp: Inputs, precision):
    """(O, O_soft, O_lin, S_fwd, S_bwd) from the library, on the host as float64."""
    p = PREC[precision]
    O = vdn.hybrid_attn(inp.dq, inp.dk, inp.dv, inp.dbeta, inp.dgate, precision=p)
    Os = vdn.softmax_branch(inp.dq, inp.dk, inp.dv, precision=p)
    Sf, Sb = vdn.vda_states(inp.dk, inp.dv, inp.dbeta, precision=p)
    Ol = vdn.vda_linear(inp.dq, Sf, Sb, precision=p)
    torch.cuda.synchronize()
    return O, Os, Ol, Sf, Sb


def host(x, frames=None, tokens=None, heads=None):
    if frames is not None:
        x = x[list(frames)]
    if tokens is not None:
        x = x[:, list(tokens)]
    if heads is not None:
        x = x[:, :, list(heads)]
    return x.to(torch.float64).cpu().numpy()


def check(name, got, ref, tol):
    e = rel_err(got, ref)
    say(f"  {name}: rel_F err {e:.3e} (tol {tol:.0e})")
    assert e <= tol, f"{name}: {e} > {tol}"


def _states_err(S, R):
    # states [C, H, d, d]: per-head relative error, max over heads
    S = S.to(torch.float64).cpu().numpy()
    return rel_err(S, R, head_axis=1)


def compare_full(inp, got, ref, precision, soft_tol=None):
    O, Os, Ol, Sf, Sb = got
    rOs, rOl, rO, rSf, rSb = ref
    tol = TOL[precision]
    es = _states_err(Sf, rSf)
    eb = _states_err(Sb, rSb)
    say(f"  S_fwd {es:.3e}  S_bwd {eb:.3e}")
    assert es <= tol and eb <= tol
    check("O_soft", host(Os), rOs, soft_tol or tol)
    check("O_lin", host(Ol), rOl, tol)
    check("O", host(O), rO, soft_tol or tol)


# ------------------------------------------------------------------ whole small configs

@pytest.mark.parametrize("cfg", [
    (20, 16, 2, 32, "fp32"),      # tiny fp32 workload
    (30, 256, 8, 64, "bf16"),     # small bf16 workload
])
def test_small_configs_full(cfg):
    F, N, H, d, prec = cfg
    say(f"case F={F} N={N} H={H} d={d} {prec}")
    inp = Inputs(F, N, H, d, prec)
    got = run_all(inp, prec)
    ref = oracle_slices(inp, list(range(F)), list(range(H)))
    compare_full(inp, got, (ref[0], ref[1], ref[2], ref[3], ref[4]), prec)


@pytest.mark.parametrize("cfg", [
    (22, 100, 2, 64, "bf16"),     # partial last chunk, ragged 64-key tiles, ragged query tile
    (7, 40, 2, 32, "bf16"),       # every chunk sees every frame: no linear states
    (3, 70, 1, 128, "bf16"),      # one non-anchor frame
    (2, 33, 2, 64, "bf16"),       # anchors only
    (1, 5, 1, 32, "bf16"),        # a single frame
    (16, 24, 3, 32, "fp32"),
    (26, 65, 2, 128, "fp32"),
    (31, 48, 2, 64, "bf16_fp8qk"),
    (23, 37, 3, 32, "bf16"),      # d = 32 with linear states: partial load of the readout weights
    (24, 50, 2, 128, "bf16_fp8qk"),
])
def test_edge_shapes(cfg):
    F, N, H, d, prec = cfg
    say(f"case F={F} N={N} H={H} d={d} {prec}")
    inp = Inputs(F, N, H, d, prec, seed=1)
    got = run_all(inp, prec)
    ref = oracle_slices(inp, list(range(F)), list(range(H)), fp8=prec == "bf16_fp8qk")
    compare_full(inp, got, ref, "bf16" if prec == "bf16_fp8qk" else prec)


def test_sharp_softmax_bf16():
    # logits with standard deviation ~4 exercise the running-max rescaling
    F, N, H, d = 25, 192, 2, 128
    say(f"case sharp F={F} N={N} H={H} d={d}")
    inp = Inputs(F, N, H, d, "bf16", seed=2, q_std=4.0 * np.sqrt(d))
    got = run_all(inp, "bf16")
    ref = oracle_slices(inp, list(range(F)), list(range(H)))
    compare_full(inp, got, ref, "bf16")


def test_identity_keys_ema_states():
    # K_t = I: the states are exponential moving averages of V (closed form pinned
    # in the oracle tests); checks the scan order and every snapshot index
    F, H, d = 32, 2, 32
    N = d
    k = torch.zeros((F, N, H, d))
    for n in range(N):
        k[:, n, :, n] = 1.0
    for prec in ("fp32", "bf16"):
        say(f"case identity keys F={F} d={d} {prec}")
        inp = Inputs(F, N, H, d, prec, seed=3, k_override=k)
        got = run_all(inp, prec)
        ref = oracle_slices(inp, list(range(F)), list(range(H)))
        compare_full(inp, got, ref, prec)


def test_mid_config_sampled_frames():
    # F=45, N=1024, H=16, d=128 bf16: every head's states, sampled query frames
    F, N, H, d = 45, 1024, 16, 128
    say(f"case mid F={F} N={N} H={H} d={d}")
    inp = Inputs(F, N, H, d, "bf16")
    O, Os, Ol, Sf, Sb = run_all(inp, "bf16")
    heads = [0, 7, 15]
    frames = [0, 1, 4, 5, 12, 22, 37, 40, 43, 44]
    tokens = list(range(0, N, 7))
    rOs, rOl, rO, rSf, rSb = oracle_slices(inp, frames, heads, tokens)
    assert _states_err(Sf[:, heads], rSf) <= 1e-2 and _states_err(Sb[:, heads], rSb) <= 1e-2
    check("O_soft", host(Os, frames, tokens, heads), rOs, 1e-2)
    check("O_lin", host(Ol, frames, tokens, heads), rOl, 1e-2)
    check("O", host(O, frames, tokens, heads), rO, 1e-2)


def test_determinism():
    F, N, H, d = 30, 256, 4, 64
    inp = Inputs(F, N, H, d, "bf16", seed=5)
    a = vdn.hybrid_attn(inp.dq, inp.dk, inp.dv, inp.dbeta, inp.dgate)
    b = vdn.hybrid_attn(inp.dq, inp.dk, inp.dv, inp.dbeta, inp.dgate)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_fp8_codes_bit_exact():
    F, N, H, d = 12, 333, 3, 128
    inp = Inputs(F, N, H, d, "bf16", seed=6)
    codes, amax = vdn.fp8_quantize(inp.dq)
    torch.cuda.synchronize()
    x = inp.q.to(torch.float32).numpy()
    ram = orc.fp8_head_scales(x)
    np.testing.assert_array_equal(amax.cpu().numpy(), ram)
    ref = orc.fp8_quantize(x, ram)
    ref_bits = torch.from_numpy(ref.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codes.cpu().numpy(), ref_bits)


def test_gate_zero_gives_softmax_branch():
    F, N, H, d = 20, 128, 2, 64
    inp = Inputs(F, N, H, d, "bf16", seed=7)
    O = vdn.hybrid_attn(inp.dq, inp.dk, inp.dv, inp.dbeta, torch.zeros_like(inp.dgate))
    Os = vdn.softmax_branch(inp.dq, inp.dk, inp.dv)
    torch.cuda.synchronize()
    assert torch.equal(O.view(torch.int16), Os.view(torch.int16))


# ------------------------------------------------------------------ full-size workloads

def sampled_full_size(F, N, H, d, precision):
    say(f"case full-size F={F} N={N} H={H} d={d} {precision}")
    inp = Inputs(F, N, H, d, precision)
    p = PREC[precision]
    O = vdn.hybrid_attn(inp.dq, inp.dk, inp.dv, inp.dbeta, inp.dgate, precision=p)
    Os = vdn.softmax_branch(inp.dq, inp.dk, inp.dv, precision=p)
    Sf, Sb = vdn.vda_states(inp.dk, inp.dv, inp.dbeta, precision=p)
    torch.cuda.synchronize()
    say("  device done")
    heads = [0, H - 1]
    C = (F + 4) // 5
    frames = [0, 1, 7, 12, F // 2, F - 9, F - 2, F - 1]       # anchor, edge, next-to-edge, interior
    tokens = list(range(0, N, 97)) + [N - 1]
    fp8 = precision == "bf16_fp8qk"
    rOs, rOl, rO, rSf, rSb = oracle_slices(inp, frames, heads, tokens, fp8=fp8)
    say("  oracle done")
    es = _states_err(Sf[:, heads], rSf)
    eb = _states_err(Sb[:, heads], rSb)
    say(f"  S_fwd {es:.3e}  S_bwd {eb:.3e}")
    assert es <= 1e-2 and eb <= 1e-2
    check("O_soft", host(Os, frames, tokens, heads), rOs, 1e-2)
    check("O", host(O, frames, tokens, heads), rO, 1e-2)
    if fp8:
        # against the unquantised oracle: the pages' tolerance for the fp8 variant
        uOs, _, uO, _, _ = oracle_slices(inp, frames, heads, tokens, fp8=False)
        check("O_soft vs unquantised", host(Os, frames, tokens, heads), uOs, 5e-2)
        check("O vs unquantised", host(O, frames, tokens, heads), uO, 5e-2)


def test_headline_config_sampled():
    sampled_full_size(90, 4032, 24, 128, "bf16")


def test_long_stream_fp8_sampled():
    sampled_full_size(180, 4032, 24, 128, "bf16_fp8qk")
