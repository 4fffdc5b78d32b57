"""fp64 CPU oracle of the Video DeltaNet (VDN) hybrid video-to-video attention layer.

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's CPU
baseline may import this module; the library and its Python binding never do,
and this module imports nothing from them.

It computes, in float64 with NumPy, exactly what the layer is defined to compute:

  * the frame partition of every query frame into a softmax key set S(i), a
    forward linear set Phi(i) and a backward linear set Psi(i)
    [sd114.wiki article "VDN-Minimax-H3 ...", sections 双向滑动窗口Softmax分支 and
    双向线性注意力分支; ananclaw note "Video DeltaNet ... critical read", section
    一、方法拆解];
  * the softmax branch: softmax(q k^T / sqrt(d)) v over all tokens of S(i)
    [same sd114.wiki section 双向滑动窗口Softmax分支];
  * the Video Delta Attention (VDA) state update, once per frame, with all of
    the frame's tokens jointly solving one update that is non-expansive
    [besthub article "VDN-H3 Generates 14-Second 768p Video ...", section
    Video Delta Attention (VDA); arXiv abstract page "Video DeltaNet: A
    Video-Native Hybrid Attention ...", Abstract].  The pages do not print the
    algebra; the form used is the proximal least-squares step
    S_t = (S_{t-1} + beta V_t K_t^T)(I + beta K_t K_t^T)^-1;
  * the bidirectional readout o = S_fwd q + S_bwd q (the query reads both states
    and the results are added) [sd114.wiki section 双向线性注意力分支];
  * the gated merge O = O_soft + g * O_lin [arXiv abstract: separate output
    projections and learnable gates calibrate the two branches; besthub section
    Hybrid Attention Architecture: outputs merged by a gating mechanism];
  * with extra (text / audio) tokens in the layer, plain softmax for every
    interaction that involves one of them [arXiv abstract; ananclaw note,
    section 一、方法拆解];
  * separate output projections of the two branches, the gate on the linear
    branch [same abstract and note section].

Tensor layout: q, k, v are [F, N, H, d] (frame, token-in-frame, head, channel);
beta is [F, H]; gate is [H, d]; states are [C, H, d, d] with C = ceil(F / 5),
row index = value channel, column index = key channel.

Readings taken where the pages are silent (each is listed with its reason in the
design notes): initial state zero; forward scan starts at frame 1 and the
backward scan at frame F-2 (anchors excluded); the same beta in both directions;
edge chunks see only the chunks that exist (no inward shift); softmax scale
1/sqrt(d); anchor query frames have no linear output; additive merge with a
per-(head, channel) gate; no normaliser in the linear readout; the fp8 variant's
quantiser (OCP E4M3, one power-of-two scale per head, q multiplied by the base-2
softmax temperature before quantisation: fp8_qk_operands).

Parity unpinned: that the VDA algebra above is the authors' update (the pages do
not give it), and that the fp8 (e4m3) variant is the authors' (the pages name FP8
without its format or scaling); the quantiser and operands are pinned against
their own definition only.
"""
from __future__ import annotations

import math

import numpy as np

CHUNK_FRAMES = 5          # five latent frames per chunk
E4M3_MAX = 448.0          # largest finite OCP E4M3 ("FN") value


# --------------------------------------------------------------------------
# Frame partition
# --------------------------------------------------------------------------

def chunk_of(i: int) -> int:
    return i // CHUNK_FRAMES


def num_chunks(F: int) -> int:
    return (F + CHUNK_FRAMES - 1) // CHUNK_FRAMES


def is_anchor(i: int, F: int) -> bool:
    """First and last frame are the boundary anchors."""
    return i == 0 or i == F - 1


def window_frames(c: int, F: int) -> list[int]:
    """Frames of chunk c and of its previous and next chunk (those that exist)."""
    return [j for j in range(F) if abs(chunk_of(j) - c) <= 1]


def softmax_frames(i: int, F: int) -> list[int]:
    """Key frames whose tokens query frame i attends to with softmax.

    Anchor query frames (first, last) see every frame; any other frame sees its
    chunk window plus all tokens of the first and last frames.
    """
    if is_anchor(i, F):
        return list(range(F))
    return sorted(set(window_frames(chunk_of(i), F)) | {0, F - 1})


def forward_frames(i: int, F: int) -> list[int]:
    """Frames summarised by the forward state of query frame i, ascending:
    all frames before its window that are not anchors."""
    if is_anchor(i, F):
        return []
    first = min(window_frames(chunk_of(i), F))
    return [j for j in range(F) if j < first and not is_anchor(j, F)]


def backward_frames(i: int, F: int) -> list[int]:
    """Frames summarised by the backward state of query frame i, ascending:
    all frames after its window that are not anchors."""
    if is_anchor(i, F):
        return []
    last = max(window_frames(chunk_of(i), F))
    return [j for j in range(F) if j > last and not is_anchor(j, F)]


def frame_mask(F: int) -> np.ndarray:
    """Boolean [F, F]: entry (i, j) is True when query frame i attends key frame j."""
    m = np.zeros((F, F), dtype=bool)
    for i in range(F):
        m[i, softmax_frames(i, F)] = True
    return m


# --------------------------------------------------------------------------
# Softmax branch
# --------------------------------------------------------------------------

def _softmax_rows(s: np.ndarray) -> np.ndarray:
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    return p / p.sum(axis=-1, keepdims=True)


def softmax_branch(q, k, v, frames=None, heads=None, tokens=None) -> np.ndarray:
    """Windowed + anchored softmax attention, one query frame at a time.

    Returns float64 [len(frames), len(tokens), len(heads), d] for the requested
    query frames, query tokens within a frame and heads (all by default).
    q, k, v: [F, N, H, d].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    F, N, H, d = q.shape
    frames = list(range(F)) if frames is None else list(frames)
    heads = list(range(H)) if heads is None else list(heads)
    tokens = list(range(N)) if tokens is None else list(tokens)
    out = np.zeros((len(frames), len(tokens), len(heads), d))
    for a, h in enumerate(heads):
        for b, i in enumerate(frames):
            keys = np.concatenate([k[j, :, h, :] for j in softmax_frames(i, F)], axis=0)
            vals = np.concatenate([v[j, :, h, :] for j in softmax_frames(i, F)], axis=0)
            p = _softmax_rows(q[i, tokens, h, :] @ keys.T / math.sqrt(d))
            out[b, :, a, :] = p @ vals
    return out


def softmax_branch_dense(q, k, v) -> np.ndarray:
    """Same branch as dense attention over all F*N tokens under the explicit
    token mask expanded from frame_mask (small inputs only)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    F, N, H, d = q.shape
    tok_mask = np.kron(frame_mask(F), np.ones((N, N), dtype=bool)).astype(bool)
    out = np.zeros_like(q)
    for h in range(H):
        Q = q[:, :, h, :].reshape(F * N, d)
        K = k[:, :, h, :].reshape(F * N, d)
        V = v[:, :, h, :].reshape(F * N, d)
        s = np.where(tok_mask, Q @ K.T / math.sqrt(d), -np.inf)
        out[:, :, h, :] = (_softmax_rows(s) @ V).reshape(F, N, d)
    return out


# --------------------------------------------------------------------------
# Video Delta Attention (linear branch)
# --------------------------------------------------------------------------

def vda_update(S, K, V, beta) -> np.ndarray:
    """One frame's state update.

    S: [dv, dk] state; K: [dk, Nt] keys of the frame as columns; V: [dv, Nt]
    values as columns; beta: scalar.  Returns (S + beta V K^T)(I + beta K K^T)^-1,
    the minimiser of beta * ||X K - V||^2 + ||X - S||^2.
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    return vda_update_grams(S, K @ K.T, V @ K.T, beta)


def vda_update_grams(S, G, B, beta) -> np.ndarray:
    """vda_update given the frame's Grams G = K K^T and B = V K^T."""
    d = G.shape[0]
    A = np.eye(d) + beta * G            # symmetric positive definite
    R = np.asarray(S, dtype=np.float64) + beta * B
    # X A = R  <=>  A X^T = R^T  (A = A^T)
    return np.linalg.solve(A, R.T).T


def vda_states(k, v, beta, heads=None):
    """Forward and backward states of every chunk.

    For chunk c, take any non-anchor query frame i of the chunk (all of them
    have the same window and hence the same Phi and Psi).  S_fwd[c] applies the
    update over forward_frames(i) in ascending time, starting from zero;
    S_bwd[c] applies it over backward_frames(i) in descending time (latest frame
    first), starting from zero.  Chunks with no non-anchor frame keep zeros.

    Returns (S_fwd, S_bwd), each float64 [C, len(heads), d, d].
    """
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    F, N, H, d = k.shape
    heads = list(range(H)) if heads is None else list(heads)
    C = num_chunks(F)
    S_fwd = np.zeros((C, len(heads), d, d))
    S_bwd = np.zeros((C, len(heads), d, d))
    for a, h in enumerate(heads):
        grams = {}

        def gram(t):
            if t not in grams:
                Kt = k[t, :, h, :].T          # [d, N]
                Vt = v[t, :, h, :].T
                grams[t] = (Kt @ Kt.T, Vt @ Kt.T)
            return grams[t]

        for c in range(C):
            members = [i for i in range(F) if chunk_of(i) == c and not is_anchor(i, F)]
            if not members:
                continue
            i = members[0]
            S = np.zeros((d, d))
            for t in forward_frames(i, F):
                G, B = gram(t)
                S = vda_update_grams(S, G, B, beta[t, h])
            S_fwd[c, a] = S
            S = np.zeros((d, d))
            for t in reversed(backward_frames(i, F)):
                G, B = gram(t)
                S = vda_update_grams(S, G, B, beta[t, h])
            S_bwd[c, a] = S
    return S_fwd, S_bwd


def linear_branch(q, S_fwd, S_bwd, frames=None) -> np.ndarray:
    """o = S_fwd q + S_bwd q for every token of a non-anchor frame; 0 on anchors.

    S_fwd, S_bwd: [C, Hs, d, d] for the heads present in q's head axis.
    Returns float64 [len(frames), N, Hs, d].
    """
    q = np.asarray(q, dtype=np.float64)
    F, N, Hs, d = q.shape
    frames = list(range(F)) if frames is None else list(frames)
    out = np.zeros((len(frames), N, Hs, d))
    for b, i in enumerate(frames):
        if is_anchor(i, F):
            continue
        c = chunk_of(i)
        for h in range(Hs):
            x = q[i, :, h, :].T                      # [d, N]
            out[b, :, h, :] = (S_fwd[c, h] @ x + S_bwd[c, h] @ x).T
    return out


def merge(O_soft, O_lin, gate) -> np.ndarray:
    """O = O_soft + g * O_lin with g per (head, channel); gate: [Hs, d]."""
    return np.asarray(O_soft, np.float64) + np.asarray(gate, np.float64)[None, None] * O_lin


def hybrid(q, k, v, beta, gate, dense=False):
    """The whole layer.  Returns (O, O_soft, O_lin), each float64 [F, N, H, d]."""
    O_soft = softmax_branch_dense(q, k, v) if dense else softmax_branch(q, k, v)
    S_fwd, S_bwd = vda_states(k, v, beta)
    O_lin = linear_branch(q, S_fwd, S_bwd)
    return merge(O_soft, O_lin, gate), O_soft, O_lin


# --------------------------------------------------------------------------
# Separate output projections of the two branches
# --------------------------------------------------------------------------
# Each branch has its own output projection, and learnable gates set the linear
# branch's share [arXiv abstract page, Abstract; ananclaw note, section 一、方法拆解].
# With W_s, W_l in R^{D x H*d} (per token, the H*d head outputs flattened head-major)
# and the per-(head, channel) gate g of the merge:
#     Y = O_soft W_s^T + (g * O_lin) W_l^T.
# W_s = W_l = W gives merge(O_soft, O_lin, g) W^T.

def output_projection(O_soft, O_lin, gate, W_s, W_l) -> np.ndarray:
    """Y [F, N, D] from O_soft, O_lin [F, N, H, d], gate [H, d], W_s, W_l [D, H*d]."""
    O_soft = np.asarray(O_soft, np.float64)
    F, N, H, d = O_soft.shape
    lin = np.asarray(gate, np.float64)[None, None] * np.asarray(O_lin, np.float64)
    Ws = np.asarray(W_s, np.float64)
    Wl = np.asarray(W_l, np.float64)
    return O_soft.reshape(F, N, H * d) @ Ws.T + lin.reshape(F, N, H * d) @ Wl.T


def hybrid_proj(q, k, v, beta, gate, W_s, W_l):
    """The layer followed by the two output projections.  Returns (Y, O_soft, O_lin)."""
    O_soft = softmax_branch(q, k, v)
    S_fwd, S_bwd = vda_states(k, v, beta)
    O_lin = linear_branch(q, S_fwd, S_bwd)
    return output_projection(O_soft, O_lin, gate, W_s, W_l), O_soft, O_lin


# --------------------------------------------------------------------------
# Extra (text / audio) tokens in the same layer
# --------------------------------------------------------------------------
# The hybrid replaces only video-to-video interactions; every interaction that
# involves a text or audio token stays plain softmax [arXiv abstract page, Abstract;
# ananclaw note, section 一、方法拆解].  With T such tokens (qx, kx, vx: [T, H, d]):
#   * a video query of frame i attends, in one softmax, to the tokens of its key
#     frames S(i) and to all T extra tokens;
#   * an extra query attends to every video token and every extra token;
#   * the linear branch and the merge concern video tokens only; an extra token's
#     output is its softmax output.

def softmax_branch_mixed(q, k, v, kx, vx, frames=None, heads=None, tokens=None) -> np.ndarray:
    """Video query rows of the softmax branch with extra key tokens.

    Same return layout as softmax_branch; kx, vx: [T, H, d]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    kx = np.asarray(kx, dtype=np.float64)
    vx = np.asarray(vx, dtype=np.float64)
    F, N, H, d = q.shape
    frames = list(range(F)) if frames is None else list(frames)
    heads = list(range(H)) if heads is None else list(heads)
    tokens = list(range(N)) if tokens is None else list(tokens)
    out = np.zeros((len(frames), len(tokens), len(heads), d))
    for a, h in enumerate(heads):
        for b, i in enumerate(frames):
            keys = np.concatenate([k[j, :, h, :] for j in softmax_frames(i, F)] + [kx[:, h, :]], axis=0)
            vals = np.concatenate([v[j, :, h, :] for j in softmax_frames(i, F)] + [vx[:, h, :]], axis=0)
            p = _softmax_rows(q[i, tokens, h, :] @ keys.T / math.sqrt(d))
            out[b, :, a, :] = p @ vals
    return out


def softmax_extra_rows(k, v, qx, kx, vx, heads=None, xtokens=None) -> np.ndarray:
    """Extra query rows: softmax over all F*N video tokens and all T extra tokens.

    Returns float64 [len(xtokens), len(heads), d]."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    qx = np.asarray(qx, dtype=np.float64)
    kx = np.asarray(kx, dtype=np.float64)
    vx = np.asarray(vx, dtype=np.float64)
    F, N, H, d = k.shape
    T = qx.shape[0]
    heads = list(range(H)) if heads is None else list(heads)
    xtokens = list(range(T)) if xtokens is None else list(xtokens)
    out = np.zeros((len(xtokens), len(heads), d))
    for a, h in enumerate(heads):
        keys = np.concatenate([k[:, :, h, :].reshape(F * N, d), kx[:, h, :]], axis=0)
        vals = np.concatenate([v[:, :, h, :].reshape(F * N, d), vx[:, h, :]], axis=0)
        p = _softmax_rows(qx[xtokens, h, :] @ keys.T / math.sqrt(d))
        out[:, a, :] = p @ vals
    return out


def token_mask_mixed(F: int, N: int, T: int) -> np.ndarray:
    """Boolean [F*N+T, F*N+T] over video tokens (frame-major) then extra tokens:
    video-video entries follow frame_mask, every entry in an extra row or column
    is True."""
    L = F * N
    m = np.ones((L + T, L + T), dtype=bool)
    m[:L, :L] = np.kron(frame_mask(F), np.ones((N, N), dtype=bool)).astype(bool)
    return m


def softmax_mixed_dense(q, k, v, qx, kx, vx):
    """Both kinds of rows as one dense attention over F*N+T tokens under
    token_mask_mixed (small inputs only).  Returns (O_video [F, N, H, d],
    O_extra [T, H, d])."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    F, N, H, d = q.shape
    T = np.asarray(qx).shape[0]
    mask = token_mask_mixed(F, N, T)
    ov = np.zeros_like(q)
    ox = np.zeros((T, H, d))
    for h in range(H):
        Q = np.concatenate([q[:, :, h, :].reshape(F * N, d), np.asarray(qx, np.float64)[:, h, :]], axis=0)
        K = np.concatenate([k[:, :, h, :].reshape(F * N, d), np.asarray(kx, np.float64)[:, h, :]], axis=0)
        V = np.concatenate([v[:, :, h, :].reshape(F * N, d), np.asarray(vx, np.float64)[:, h, :]], axis=0)
        s = np.where(mask, Q @ K.T / math.sqrt(d), -np.inf)
        o = _softmax_rows(s) @ V
        ov[:, :, h, :] = o[:F * N].reshape(F, N, d)
        ox[:, h, :] = o[F * N:]
    return ov, ox


def hybrid_mixed(q, k, v, qx, kx, vx, beta, gate, dense=False):
    """The layer with T extra tokens.  Returns (O_video, O_extra, O_soft_video,
    O_lin): video rows O = O_soft + g * O_lin, extra rows their softmax output."""
    if dense:
        O_soft, O_x = softmax_mixed_dense(q, k, v, qx, kx, vx)
    else:
        O_soft = softmax_branch_mixed(q, k, v, kx, vx)
        O_x = softmax_extra_rows(k, v, qx, kx, vx)
    S_fwd, S_bwd = vda_states(k, v, beta)
    O_lin = linear_branch(q, S_fwd, S_bwd)
    return merge(O_soft, O_lin, gate), O_x, O_soft, O_lin


# --------------------------------------------------------------------------
# fp8 (OCP E4M3, "FN": no infinities, max 448) quantiser for the fp8 softmax variant
# --------------------------------------------------------------------------

def e4m3_round(x) -> np.ndarray:
    """Round float values to the nearest E4M3 value, ties to even, saturating at +-448.

    E4M3: 1 sign, 4 exponent (bias 7) and 3 mantissa bits; normal values
    2^(e-7) * (1 + m/8), subnormals 2^-6 * m/8.  The spacing of representable
    values around |x| is 2^(max(floor(log2|x|), -6) - 3).
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    quantum = np.exp2(e - 3.0)
    r = np.round(a / quantum) * quantum          # np.round: ties to even
    r = np.minimum(r, E4M3_MAX)
    return np.sign(x) * r


def fp8_head_scales(x) -> np.ndarray:
    """Per-head amax of x [..., H, d] (head axis -2) over all tokens and channels,
    float32 [H]."""
    x = np.asarray(x, dtype=np.float32)
    axes = tuple(a for a in range(x.ndim) if a != x.ndim - 2)
    return np.max(np.abs(x), axis=axes).astype(np.float32)


def fp8_scale_exponent(amax) -> np.ndarray:
    """Power-of-two quantiser scale per head: the smallest integer e with
    amax <= 448 * 2^e, clamped to [-127, 127] (0 where amax is 0), int64 [H].
    Found from the binary exponent of amax (exact; no logarithm is rounded)."""
    out = []
    for a in np.asarray(amax, dtype=np.float64).ravel():
        if not a > 0:
            out.append(0)
            continue
        e = -200
        while not a <= E4M3_MAX * 2.0 ** e:      # 448 * 2^e is exact in float64
            e += 1
        out.append(min(max(e, -127), 127))
    return np.asarray(out, dtype=np.int64)


def fp8_quantize(x, e) -> np.ndarray:
    """E4M3 codes (as float64 values) of x [..., H, d] with per-head power-of-two
    scales 2^e [H]: code = e4m3_round(fp32(x * 2^-e)).  The product is a float32
    operation (exact unless it falls below the float32 normal range), so the
    rounding decision is taken in the same precision as the device."""
    x = np.asarray(x, dtype=np.float32)
    inv = np.exp2(-np.asarray(e, dtype=np.float64)).astype(np.float32)
    scaled = (x * inv.reshape((-1, 1))).astype(np.float32)
    return e4m3_round(scaled)


def fp8_temperature(d: int) -> np.float32:
    """The softmax temperature in base-2 units, log2(e) / sqrt(d), as the float32
    value fp32(fp32(log2 e) / fp32(sqrt d))."""
    return np.float32(np.float32(math.log2(math.e)) / np.sqrt(np.float32(d)))


def fp8_qk_operands(q, k, d: int):
    """(q_eff, k_eff), float64, such that the plain softmax branch on q_eff, k_eff
    is the fp8 (E4M3) Q.K^T variant of the layer.

    Reading (the pages name FP8 inference without giving its quantiser): q is
    first multiplied by the base-2 temperature c = fp8_temperature(d) (float32),
    then each of q' = fp32(q c) and k is quantised per head to E4M3 with the
    power-of-two scale 2^e of fp8_scale_exponent over all of its tokens.  A score
    in base-2 units is then 2^(e_q + e_k) * sum(code_q * code_k), and the
    probabilities are 2^(that score - its row max).  In the units of the plain
    branch (natural exponent of q.k / sqrt(d)) that is q_eff = code_q 2^e_q
    sqrt(d) ln 2 and k_eff = code_k 2^e_k.  q, k: [..., H, d] (head axis -2)."""
    c = fp8_temperature(d)
    qp = (np.asarray(q, dtype=np.float32) * c).astype(np.float32)
    kf = np.asarray(k, dtype=np.float32)
    eq = fp8_scale_exponent(fp8_head_scales(qp))
    ek = fp8_scale_exponent(fp8_head_scales(kf))
    sq = np.exp2(eq.astype(np.float64)) * math.sqrt(d) * math.log(2.0)
    sk = np.exp2(ek.astype(np.float64))
    q_eff = fp8_quantize(qp, eq) * sq.reshape((-1, 1))
    k_eff = fp8_quantize(kf, ek) * sk.reshape((-1, 1))
    return q_eff, k_eff


def fp8_v_operand(v) -> np.ndarray:
    """v as the full-fp8 variant's P.V sees it, float64: per head, E4M3 codes of v
    with the power-of-two scale of fp8_scale_exponent over all tokens (no
    prescale), times that scale.  v: [..., H, d] (head axis -2).

    Reading (as for fp8_qk_operands, the pages name FP8 inference without its
    format): v is coded like k; the probabilities are also rounded to E4M3 in that
    variant, after the shift by the kernel's running maximum, which this oracle
    does not model (the rounding depends on the running maximum's history), so the
    variant is compared within the probabilities' rounding bound."""
    vf = np.asarray(v, dtype=np.float32)
    ev = fp8_scale_exponent(fp8_head_scales(vf))
    return fp8_quantize(vf, ev) * np.exp2(ev.astype(np.float64)).reshape((-1, 1))

