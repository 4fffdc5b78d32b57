"""GPU parity: the HIP path (called through the C ABI) against the fp64 oracle on
the same seeded inputs, per branch and for the merged output.

Tolerances (max over heads of the relative Frobenius error): 1e-4 fp32, 1e-2 bf16,
5e-2 for the fp8 (E4M3 q.k) softmax variant against the unquantised oracle and
1e-2 against the oracle fed the same E4M3 codes.  The VDA states are fp32 in every
precision (the oracle sees the same rounded k and v), so they are held to 1e-5.
Integer work (the partition, the E4M3 codes) is compared bit for bit.

In the bf16 and fp8 layers the readout and gated merge run in the softmax kernel's
epilogue, and at these input distributions the gated linear term dominates O
(|O_soft| is well under 1 % of |O|).  The softmax half of that fused output is
therefore isolated on its own: with g = 0 the layer must equal the softmax branch
bit for bit, and with a small gate (so that O_soft carries most of |O|) the layer
must match the oracle."""
import math
import os
import sys

import numpy as np
import pytest
import torch

import hybrid_sparse_linear_chunked_amd as vdn
from oracle import vdn_oracle as orc
from vdn_testlib import TOL, Inputs, oracle_slices, rel_err

pytestmark = pytest.mark.gpu

PREC = {"fp32": vdn.PREC_FP32, "bf16": vdn.PREC_BF16, "bf16_fp8qk": vdn.PREC_BF16_FP8QK, "fp8": vdn.PREC_FP8}

# The full-fp8 layer (VDN_PREC_FP8) also rounds the probabilities to E4M3 after the
# running-max shift, which the oracle does not model: each weight moves by at most
# half a step of a 3-bit mantissa (2^-4 relative), so O_soft is held to 5e-2 of the
# oracle fed the same E4M3 q, k, v (measured 2.2-2.3 % on these inputs) and 8e-2 of
# the unquantised one.
FP8PV_SOFT_TOL, FP8PV_SOFT_TOL_UNQ = 5e-2, 8e-2


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


STATE_TOL = 1e-5        # fp32 states from the same rounded inputs as the oracle's


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
    assert es <= STATE_TOL and eb <= STATE_TOL
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


@pytest.mark.parametrize("d", [64, 128])
def test_ill_conditioned_keys_states(d):
    # Every token of a frame carries one key direction plus 1e-3 noise, so A_t =
    # I + beta_t G_t has a condition number near 1 + beta_t N (about 200 here): the
    # per-frame factorisation in fp32 loses accuracy in proportion to it (relative
    # error of order kappa 2^-24 in M_t, and so in the states).  The states are held
    # to 32 kappa 2^-24, kappa the largest over frames and heads.
    F, N, H = 14, 256, 2
    rng = np.random.default_rng(5)
    base = rng.standard_normal((F, 1, H, d))
    k = base + 1e-3 * rng.standard_normal((F, N, H, d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    for prec in ("fp32", "bf16"):
        inp = Inputs(F, N, H, d, prec, seed=5, k_override=torch.from_numpy(k))
        k64 = inp.host64("k")
        beta = inp.beta.numpy().astype(np.float64)
        kappa = max(np.linalg.cond(np.eye(d) + beta[t, h] * k64[t, :, h, :].T @ k64[t, :, h, :])
                    for t in range(1, F - 1) for h in range(H))
        tol = 32 * kappa * 2.0 ** -24
        say(f"case ill-conditioned keys F={F} N={N} d={d} {prec}: kappa {kappa:.0f}, tol {tol:.2e}")
        Sf, Sb = vdn.vda_states(inp.dk, inp.dv, inp.dbeta, precision=PREC[prec])
        torch.cuda.synchronize()
        rSf, rSb = orc.vda_states(k64, inp.host64("v"), beta)
        es, eb = _states_err(Sf, rSf), _states_err(Sb, rSb)
        say(f"  S_fwd {es:.3e}  S_bwd {eb:.3e}")
        assert kappa > 100        # the case is what it says
        assert es <= tol and eb <= tol


MID = (45, 1024, 16, 128)


@pytest.fixture(scope="module")
def mid_layer():
    """The F=45, N=1024, H=16, d=128 bf16 workload, every output on the host."""
    F, N, H, d = MID
    say(f"case mid F={F} N={N} H={H} d={d} (device)")
    inp = Inputs(F, N, H, d, "bf16")
    O, Os, Ol, Sf, Sb = run_all(inp, "bf16")
    out = dict(inp=inp, O=O.cpu(), Os=Os.cpu(), Ol=Ol.cpu(), Sf=Sf.cpu(), Sb=Sb.cpu())
    del O, Os, Ol, Sf, Sb
    return out


@pytest.mark.parametrize("heads", [[0, 1, 2, 3], [4, 5, 6, 7], [8, 9, 10, 11], [12, 13, 14, 15]])
def test_mid_config_full(mid_layer, heads):
    # every frame, token and channel of four heads per case (the oracle needs about
    # 10 s per head here), states of those heads
    F, N, H, d = MID
    say(f"case mid full, heads {heads}")
    m = mid_layer
    frames = list(range(F))
    rOs, rOl, rO, rSf, rSb = oracle_slices(m["inp"], frames, heads)
    es = _states_err(m["Sf"][:, heads], rSf)
    eb = _states_err(m["Sb"][:, heads], rSb)
    say(f"  S_fwd {es:.3e}  S_bwd {eb:.3e}")
    assert es <= STATE_TOL and eb <= STATE_TOL
    check("O_soft", host(m["Os"], heads=heads), rOs, 1e-2)
    check("O_lin", host(m["Ol"], heads=heads), rOl, 1e-2)
    check("O", host(m["O"], heads=heads), rO, 1e-2)


# ------------------------------------------------------------------ the fused epilogue's softmax half, d = 128

def _fused_softmax_half(inp, precision, frames, heads, tokens, gate_scale=3e-3):
    """(i) g = 0: the layer equals the softmax branch bit for bit; (ii) a small gate,
    so that O_soft carries most of |O|: the layer matches the oracle (fp8 q.k: within
    1e-2 of the oracle fed the same E4M3 codes and 5e-2 of the unquantised one; full
    fp8: the O_soft tolerances above)."""
    p = PREC[precision]
    fp8 = precision in ("bf16_fp8qk", "fp8")
    fp8v = precision == "fp8"
    O0 = vdn.hybrid_attn(inp.dq, inp.dk, inp.dv, inp.dbeta, torch.zeros_like(inp.dgate), precision=p)
    Os = vdn.softmax_branch(inp.dq, inp.dk, inp.dv, precision=p)
    torch.cuda.synchronize()
    assert torch.equal(O0.view(torch.int16), Os.view(torch.int16)), "g = 0 layer differs from the softmax branch"
    say("  g = 0: layer == softmax branch (bitwise)")
    del O0, Os
    small = inp.dgate * gate_scale
    O = vdn.hybrid_attn(inp.dq, inp.dk, inp.dv, inp.dbeta, small, precision=p)
    torch.cuda.synchronize()
    got = host(O, frames, tokens, heads)
    del O
    g = inp.gate.numpy().astype(np.float64)[heads] * np.float64(np.float32(gate_scale))
    for quant in ((True, False) if fp8 else (False,)):
        rOs, rOl, _, _, _ = oracle_slices(inp, frames, heads, tokens, fp8=quant, fp8v=quant and fp8v)
        rO = orc.merge(rOs, rOl, g)
        soft_share = np.linalg.norm(rOs) / np.linalg.norm(rO)
        lin_share = np.linalg.norm(g[None, None] * rOl) / np.linalg.norm(rO)
        say(f"  small gate: |O_soft| / |O| = {soft_share:.3f}, |g O_lin| / |O| = {lin_share:.3f}")
        assert soft_share >= 0.3 and lin_share >= 0.1
        if fp8v:
            tol = FP8PV_SOFT_TOL if quant else FP8PV_SOFT_TOL_UNQ
        else:
            tol = 1e-2 if (quant or not fp8) else 5e-2
        check("O (small gate)" + (" vs E4M3 oracle" if quant else ""), got, rO, tol)


@pytest.mark.parametrize("precision", ["bf16", "bf16_fp8qk", "fp8"])
def test_fused_softmax_half_mid(precision):
    F, N, H, d = 25, 1024, 3, 128
    say(f"case fused epilogue F={F} N={N} H={H} d={d} {precision}")
    inp = Inputs(F, N, H, d, precision, seed=11)
    _fused_softmax_half(inp, precision, list(range(F)), list(range(H)), None)


@pytest.mark.parametrize("precision", ["bf16", "bf16_fp8qk"])
def test_w64_kernel_opt_in(precision, monkeypatch):
    # the opt-in 64-queries-per-wave attention kernel (VDN_ATTN_W64=1): a ragged
    # shape against the oracle in full, and the fused softmax half at N = 1024
    monkeypatch.setenv("VDN_ATTN_W64", "1")
    fp8 = precision == "bf16_fp8qk"
    F, N, H, d = 24, 50, 2, 128
    say(f"case w64 F={F} N={N} H={H} d={d} {precision}")
    inp = Inputs(F, N, H, d, precision, seed=1)
    got = run_all(inp, precision)
    ref = oracle_slices(inp, list(range(F)), list(range(H)), fp8=fp8)
    compare_full(inp, got, ref, "bf16")
    F, N, H, d = 25, 1024, 3, 128
    say(f"case w64 fused epilogue F={F} N={N} H={H} d={d} {precision}")
    inp = Inputs(F, N, H, d, precision, seed=11)
    _fused_softmax_half(inp, precision, list(range(F)), list(range(H)), None)


@pytest.mark.parametrize("cfg", [
    (24, 50, 2, 128),     # ragged 64-key tiles and query tile
    (31, 48, 2, 64),      # d = 64, partial last chunk
    (7, 40, 2, 128),      # every chunk sees every frame: no linear states
    (1, 20, 1, 64),       # one frame, one partial tile: a segment loop of two passes
    (2, 64, 2, 128),      # two anchor frames, one whole tile each
    (16, 300, 1, 64),     # several tiles per frame, ragged last tile and query tile
])
def test_full_fp8_layer(cfg):
    F, N, H, d = cfg
    say(f"case full fp8 F={F} N={N} H={H} d={d}")
    inp = Inputs(F, N, H, d, "fp8", seed=1)
    O, Os, Ol, Sf, Sb = run_all(inp, "fp8")
    fr, hs = list(range(F)), list(range(H))
    rOs, rOl, rO, rSf, rSb = oracle_slices(inp, fr, hs, fp8=True, fp8v=True)
    es, eb = _states_err(Sf, rSf), _states_err(Sb, rSb)
    say(f"  S_fwd {es:.3e}  S_bwd {eb:.3e}")
    assert es <= STATE_TOL and eb <= STATE_TOL
    check("O_lin", host(Ol), rOl, 1e-2)
    check("O_soft vs E4M3 q, k, v oracle", host(Os), rOs, FP8PV_SOFT_TOL)
    # (with no linear states, as at F = 7, O is O_soft: its tolerance)
    check("O vs E4M3 q, k, v oracle", host(O), rO, FP8PV_SOFT_TOL)
    uOs = oracle_slices(inp, fr, hs)[0]
    check("O_soft vs unquantised oracle", host(Os), uOs, FP8PV_SOFT_TOL_UNQ)


def test_determinism():
    F, N, H, d = 30, 256, 4, 64
    inp = Inputs(F, N, H, d, "bf16", seed=5)
    a = vdn.hybrid_attn(inp.dq, inp.dk, inp.dv, inp.dbeta, inp.dgate)
    b = vdn.hybrid_attn(inp.dq, inp.dk, inp.dv, inp.dbeta, inp.dgate)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("magnitude, temperature", [(1.0, False), (1.0, True), (3e-30, False), (2e4, True)])
def test_fp8_codes_bit_exact(magnitude, temperature):
    # codes and power-of-two scale exponents bit for bit against the oracle's
    # quantiser, with and without the base-2 temperature as prescale, at magnitudes
    # that take the exponents far below and above zero
    F, N, H, d = 12, 333, 3, 128
    inp = Inputs(F, N, H, d, "bf16", seed=6)
    xb = (inp.q.to(torch.float32) * magnitude).to(torch.bfloat16)
    pre = np.float32(np.float32(math.log2(math.e)) / np.sqrt(np.float32(d))) if temperature else np.float32(1.0)
    codes, sexp = vdn.fp8_quantize(xb.to("cuda"), float(pre))
    torch.cuda.synchronize()
    y = (xb.to(torch.float32).numpy() * pre).astype(np.float32)
    e = orc.fp8_scale_exponent(orc.fp8_head_scales(y))
    say(f"  magnitude {magnitude:g}: scale exponents {e.tolist()}")
    np.testing.assert_array_equal(sexp.cpu().numpy(), e)
    ref = orc.fp8_quantize(y, e)
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
    fp8 = precision in ("bf16_fp8qk", "fp8")
    fp8v = precision == "fp8"
    rOs, rOl, rO, rSf, rSb = oracle_slices(inp, frames, heads, tokens, fp8=fp8, fp8v=fp8v)
    say("  oracle done")
    es = _states_err(Sf[:, heads], rSf)
    eb = _states_err(Sb[:, heads], rSb)
    say(f"  S_fwd {es:.3e}  S_bwd {eb:.3e}")
    assert es <= STATE_TOL and eb <= STATE_TOL
    check("O_soft", host(Os, frames, tokens, heads), rOs, FP8PV_SOFT_TOL if fp8v else 1e-2)
    check("O", host(O, frames, tokens, heads), rO, 1e-2)
    if fp8:
        # against the unquantised oracle
        uOs, _, uO, _, _ = oracle_slices(inp, frames, heads, tokens, fp8=False)
        check("O_soft vs unquantised", host(Os, frames, tokens, heads), uOs, FP8PV_SOFT_TOL_UNQ if fp8v else 5e-2)
        check("O vs unquantised", host(O, frames, tokens, heads), uO, 5e-2)
    del O, Os, Sf, Sb
    # the softmax half of the fused output, at this shape and launch configuration
    _fused_softmax_half(inp, precision, frames, heads, tokens)


def test_headline_config_sampled():
    sampled_full_size(90, 4032, 24, 128, "bf16")


def test_long_stream_fp8_sampled():
    sampled_full_size(180, 4032, 24, 128, "bf16_fp8qk")


def test_long_stream_full_fp8_sampled():
    sampled_full_size(180, 4032, 24, 128, "fp8")


def test_binding_rejects_aliasing():
    # outputs must not alias inputs, and the workspace must alias neither: the
    # binding refuses such calls before anything is launched
    F, N, H, d = 12, 32, 2, 64
    inp = Inputs(F, N, H, d, "bf16", seed=12)
    with pytest.raises(ValueError):
        vdn.hybrid_attn(inp.dq, inp.dk, inp.dv, inp.dbeta, inp.dgate, out=inp.dq)
    with pytest.raises(ValueError):
        vdn.softmax_branch(inp.dq, inp.dk, inp.dv, out=inp.dv)
    need = vdn.workspace_bytes(F, N, H, d, vdn.PREC_BF16)
    ws = torch.empty(need + inp.dq.numel() * 2, dtype=torch.uint8, device="cuda")
    inside = ws[-inp.dq.numel() * 2:].view(torch.bfloat16).view(F, N, H, d)
    with pytest.raises(ValueError):
        vdn.hybrid_attn(inp.dq, inp.dk, inp.dv, inp.dbeta, inp.dgate, out=inside, workspace=ws)
    ok = vdn.hybrid_attn(inp.dq, inp.dk, inp.dv, inp.dbeta, inp.dgate, workspace=ws[:need])
    torch.cuda.synchronize()
    assert ok.shape == inp.dq.shape
