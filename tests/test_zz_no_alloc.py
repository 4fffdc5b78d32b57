"""The no-allocation entry point (vdn_hybrid_attn_noalloc, workspace in the
library's static device array) against the workspace entry point
(vdn_hybrid_attn): same kernels, so the outputs must agree bit for bit; both are
also checked against the fp64 oracle.  Two calls in a row on one GPU, the second
with a smaller input, so stale scratch contents from the first cannot leak into
the second."""
import sys

import numpy as np
import pytest
import torch

import hybrid_sparse_linear_chunked_amd as vdn
from vdn_testlib import TOL, Inputs, oracle_slices, rel_err

pytestmark = pytest.mark.gpu

PREC = {"fp32": vdn.PREC_FP32, "bf16": vdn.PREC_BF16, "bf16_fp8qk": vdn.PREC_BF16_FP8QK, "fp8": vdn.PREC_FP8}
# O against the oracle fed the same E4M3 operands (full fp8: the probabilities'
# E4M3 rounding bound, as in the full-fp8 parity tests)
O_TOL = {"fp32": TOL["fp32"], "bf16": TOL["bf16"], "bf16_fp8qk": TOL["bf16"], "fp8": 5e-2}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    vdn.load()


def _one(cfg, seed):
    F, N, H, d, prec = cfg
    say(f"case noalloc F={F} N={N} H={H} d={d} {prec}")
    assert vdn.workspace_bytes(F, N, H, d, PREC[prec]) <= vdn.NOALLOC_SCRATCH_BYTES
    inp = Inputs(F, N, H, d, prec, seed=seed)
    p = PREC[prec]
    out = torch.full_like(inp.dq, float("nan"))
    got = vdn.hybrid_attn_noalloc(inp.dq, inp.dk, inp.dv, inp.dbeta, inp.dgate, precision=p, out=out)
    ref = vdn.hybrid_attn(inp.dq, inp.dk, inp.dv, inp.dbeta, inp.dgate, precision=p)
    torch.cuda.synchronize()
    bits = torch.int32 if prec == "fp32" else torch.int16
    assert torch.equal(got.view(bits), ref.view(bits)), "no-allocation output differs from vdn_hybrid_attn"
    rOs, rOl, rO, _, _ = oracle_slices(inp, list(range(F)), list(range(H)), fp8=prec in ("bf16_fp8qk", "fp8"),
                                       fp8v=prec == "fp8")
    e = rel_err(got.to(torch.float64).cpu().numpy(), rO)
    say(f"  bitwise equal to vdn_hybrid_attn; O rel_F err {e:.3e}")
    assert e <= O_TOL[prec]


@pytest.mark.parametrize("pair", [
    ((30, 256, 8, 64, "bf16"), (22, 100, 2, 64, "bf16")),
    ((31, 48, 2, 64, "bf16_fp8qk"), (12, 40, 1, 64, "bf16_fp8qk")),
    ((26, 65, 2, 128, "fp32"), (20, 16, 2, 32, "fp32")),
    ((24, 50, 2, 128, "fp8"), (9, 30, 1, 64, "fp8")),
])
def test_noalloc_matches_workspace_entry_two_calls(pair):
    big, small = pair
    _one(big, seed=21)
    _one(small, seed=22)


def test_noalloc_rejects_too_large():
    F, N, H, d = 45, 1024, 16, 128
    assert vdn.workspace_bytes(F, N, H, d, vdn.PREC_BF16) > vdn.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((F, N, H, d), dtype=torch.bfloat16, device="cuda")
    beta = torch.full((F, H), 0.5, device="cuda")
    gate = torch.ones((H, d), device="cuda")
    with pytest.raises(vdn.VdnError) as ei:
        vdn.hybrid_attn_noalloc(x, x, x, beta, gate)
    assert ei.value.status == vdn.ERR_TOO_LARGE
