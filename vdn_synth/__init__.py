"""Seeded synthetic inputs for the Video DeltaNet hybrid video-to-video attention layer.

This module is shared by the fp64 oracle's tests and by the GPU path's tests and
benchmark.  It draws random numbers and lays them out; it holds none of the layer's
arithmetic.

Recipe (every configuration):
  * q, k, v ~ N(0, 1) in float32, one independent block of N x d values per
    (tensor, frame, head), drawn from NumPy PCG64 seeded with
    SeedSequence([seed, tensor_id, frame, head]) with tensor_id q=0, k=1, v=2;
  * every key vector (one token, one head) is scaled to unit L2 norm in float32;
  * beta ~ U(0.2, 0.8) per (frame, head) from SeedSequence([seed, 3]);
  * gate = sigmoid(N(0, 1)) per (head, channel) from SeedSequence([seed, 4]);
  * q_std scales q (the "sharp" variant uses q_std = 4 * sqrt(d), which puts the
    attention logits at standard deviation ~4);
  * extra (text / audio) tokens, when a layer has them: q, k, v of T tokens, the
    same distributions, one T x d block per (tensor, head) from
    SeedSequence([seed, 5 + tensor_id, head]), laid out [T, H, d];
  * output projection weights [W_s | W_l], N(0, 1/(H*d)), from SeedSequence([seed, 8]).

Block seeding lets a test regenerate only the frames and heads it samples.
Tensors are laid out [F, N, H, d] (token-major, one token = H*d contiguous values).
"""
from __future__ import annotations

import concurrent.futures as _cf
import os

import numpy as np

TENSOR_ID = {"q": 0, "k": 1, "v": 2}

# The five workloads: (F, N, H, d, precision name).
CONFIGS = {
    0: dict(F=20, N=16, H=2, d=32, precision="fp32"),
    1: dict(F=30, N=256, H=8, d=64, precision="bf16"),
    2: dict(F=45, N=1024, H=16, d=128, precision="bf16"),
    3: dict(F=90, N=4032, H=24, d=128, precision="bf16"),
    4: dict(F=180, N=4032, H=24, d=128, precision="bf16_fp8qk"),
}


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def block(name: str, frame: int, head: int, N: int, d: int, seed: int = 0,
          q_std: float = 1.0) -> np.ndarray:
    """One (frame, head) block of q, k or v: float32 array of shape (N, d)."""
    x = _rng(seed, TENSOR_ID[name], frame, head).standard_normal((N, d), dtype=np.float32)
    if name == "k":
        nrm = np.sqrt(np.sum(x * x, axis=1, dtype=np.float32), dtype=np.float32)
        x = x / nrm[:, None]
    elif name == "q" and q_std != 1.0:
        x = x * np.float32(q_std)
    return x


def extra(name: str, T: int, H: int, d: int, seed: int = 0, q_std: float = 1.0) -> np.ndarray:
    """q, k or v of T extra tokens: float32 [T, H, d]."""
    out = np.empty((T, H, d), dtype=np.float32)
    for h in range(H):
        x = _rng(seed, 5 + TENSOR_ID[name], h).standard_normal((T, d), dtype=np.float32)
        if name == "k":
            nrm = np.sqrt(np.sum(x * x, axis=1, dtype=np.float32), dtype=np.float32)
            x = x / nrm[:, None]
        elif name == "q" and q_std != 1.0:
            x = x * np.float32(q_std)
        out[:, h, :] = x
    return out


def proj_weights(D: int, Hd: int, seed: int = 0) -> np.ndarray:
    """Output projections of the two branches side by side, [W_s | W_l]: float32
    [D, 2*Hd], N(0, 1/Hd) entries from SeedSequence([seed, 8])."""
    return (_rng(seed, 8).standard_normal((D, 2 * Hd), dtype=np.float32) / np.float32(np.sqrt(Hd))).astype(np.float32)


def beta(F: int, H: int, seed: int = 0) -> np.ndarray:
    """float32 [F, H], uniform on (0.2, 0.8)."""
    return _rng(seed, 3).uniform(0.2, 0.8, size=(F, H)).astype(np.float32)


def gate(H: int, d: int, seed: int = 0) -> np.ndarray:
    """float32 [H, d], sigmoid of a standard normal."""
    z = _rng(seed, 4).standard_normal((H, d))
    return (1.0 / (1.0 + np.exp(-z))).astype(np.float32)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def tensor(name: str, F: int, N: int, H: int, d: int, seed: int = 0, q_std: float = 1.0,
           frames=None, heads=None, out=None, convert=None) -> np.ndarray:
    """Fill a [len(frames), N, len(heads), d] tensor block by block.

    `convert` (optional) maps each float32 block to the stored representation
    (e.g. bf16 rounding); `out` is an optional preallocated array-like with a
    numpy-compatible __setitem__ (a CPU torch tensor works).
    """
    frames = list(range(F)) if frames is None else list(frames)
    heads = list(range(H)) if heads is None else list(heads)
    if out is None:
        out = np.empty((len(frames), N, len(heads), d), dtype=np.float32)

    def gen(fi_hi):
        fi, hi = fi_hi
        return block(name, frames[fi], heads[hi], N, d, seed, q_std)

    nh = len(heads)
    if len(frames) * nh * N * d < (1 << 22):
        for fi in range(len(frames)):
            for hi in range(nh):
                b = gen((fi, hi))
                out[fi, :, hi, :] = convert(b) if convert is not None else b
    else:
        # worker threads only draw the float32 blocks (NumPy); `convert` and the
        # stores into `out` (possibly torch calls, not safe to run from many
        # threads at once) stay on the calling thread, one frame (all heads) per
        # call, while the workers draw the next two frames
        with _cf.ThreadPoolExecutor(_workers()) as ex:
            pending = {}
            ahead = 2
            for fi in range(min(ahead, len(frames))):
                pending[fi] = [ex.submit(gen, (fi, hi)) for hi in range(nh)]
            for fi in range(len(frames)):
                if fi + ahead < len(frames):
                    pending[fi + ahead] = [ex.submit(gen, (fi + ahead, hi)) for hi in range(nh)]
                blk = np.stack([f.result() for f in pending.pop(fi)], axis=1)      # [N, heads, d]
                out[fi] = convert(blk) if convert is not None else blk
    return out
