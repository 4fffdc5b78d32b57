"""Pins of the fp64 oracle against facts fixed outside the oracle itself:
hand-written partitions from the pages, library routines (torch SDPA,
numpy lstsq, torch's float8 cast), textbook identities (Sherman-Morrison),
closed forms (uniform attention, an exponential moving average) and invariants
(disjoint partition, time reversal, non-expansiveness)."""
import math
import os

import numpy as np
import pytest
import torch

import vdn_synth
from oracle import vdn_oracle as orc
from conftest import GOLDEN, load_partition


def small_inputs(F, N, H, d, seed=0, q_std=1.0):
    q = vdn_synth.tensor("q", F, N, H, d, seed=seed, q_std=q_std).astype(np.float64)
    k = vdn_synth.tensor("k", F, N, H, d, seed=seed).astype(np.float64)
    v = vdn_synth.tensor("v", F, N, H, d, seed=seed).astype(np.float64)
    return q, k, v


# ---------------------------------------------------------------- partition

@pytest.mark.parametrize("F", [12, 20, 22, 30])
def test_partition_matches_hand_written_tables(F):
    table = load_partition(F)
    for i in range(F):
        s, f, b = table[i]
        assert orc.softmax_frames(i, F) == s, i
        assert orc.forward_frames(i, F) == f, i
        assert orc.backward_frames(i, F) == b, i


@pytest.mark.parametrize("F", range(1, 61))
def test_partition_disjoint_and_complete(F):
    # sd114.wiki, section 双向线性注意力分支: the forward and backward ranges do not
    # overlap each other nor the frames the window and the anchors cover; together
    # they are every frame, so nothing is computed twice and nothing is dropped.
    for i in range(F):
        s = set(orc.softmax_frames(i, F))
        f = set(orc.forward_frames(i, F))
        b = set(orc.backward_frames(i, F))
        assert not (s & f) and not (s & b) and not (f & b)
        assert s | f | b == set(range(F))
        assert {0, F - 1} <= s
        assert all(j < min(s - {0}, default=F) for j in f)
        assert all(j > max(s - {F - 1}, default=-1) for j in b)


def test_pair_counts():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "pair_counts.txt"))
            if l.strip() and not l.startswith("#")]
    for F, P, W in ((int(a), int(b), int(c)) for a, b, c in rows):
        m = orc.frame_mask(F)
        assert m.sum() == P
        win = sum(len(orc.window_frames(orc.chunk_of(i), F)) for i in range(F))
        assert win == W


def test_anchor_density_increment_near_printed_value():
    # The sd114.wiki article (section 双向滑动窗口Softmax分支) prints a 3.57% density
    # increment for the anchors without the frame count; a weak check that some
    # length near the headline one reproduces it to within 0.01 points.
    best = min(abs(100.0 * (orc.frame_mask(F).sum()
                            - sum(len(orc.window_frames(orc.chunk_of(i), F)) for i in range(F)))
                   / F ** 2 - 3.57) for F in range(90, 111))
    assert best < 0.01


# ---------------------------------------------------------------- softmax branch

def _sdpa(q, k, v, mask=None):
    """torch's scaled_dot_product_attention on float64 [L, d] per head."""
    Q = torch.from_numpy(q)[None]
    K = torch.from_numpy(k)[None]
    V = torch.from_numpy(v)[None]
    m = None if mask is None else torch.from_numpy(mask)[None]
    return torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=m)[0].numpy()


@pytest.mark.parametrize("F", [1, 2, 5, 7, 10])
def test_short_video_is_full_attention(F):
    # F <= 10: every chunk's window covers the whole video, so the softmax branch is
    # plain full attention and the linear branch is empty.
    N, H, d = 6, 2, 8
    q, k, v = small_inputs(F, N, H, d, seed=F)
    out = orc.softmax_branch(q, k, v)
    for h in range(H):
        ref = _sdpa(q[:, :, h].reshape(-1, d), k[:, :, h].reshape(-1, d), v[:, :, h].reshape(-1, d))
        np.testing.assert_allclose(out[:, :, h].reshape(-1, d), ref, rtol=1e-12, atol=1e-12)
    beta = vdn_synth.beta(F, H)
    Sf, Sb = orc.vda_states(k, v, beta)
    assert not Sf.any() and not Sb.any()


@pytest.mark.parametrize("F", [20, 22])
def test_softmax_equals_masked_sdpa(F):
    N, H, d = 3, 2, 8
    q, k, v = small_inputs(F, N, H, d, seed=1, q_std=4.0)
    table = load_partition(F)
    fmask = np.zeros((F, F), dtype=bool)
    for i in range(F):
        fmask[i, table[i][0]] = True
    tmask = np.kron(fmask, np.ones((N, N), dtype=bool)).astype(bool)
    gathered = orc.softmax_branch(q, k, v)
    dense = orc.softmax_branch_dense(q, k, v)
    for h in range(H):
        ref = _sdpa(q[:, :, h].reshape(-1, d), k[:, :, h].reshape(-1, d),
                    v[:, :, h].reshape(-1, d), tmask)
        np.testing.assert_allclose(gathered[:, :, h].reshape(-1, d), ref, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(dense[:, :, h].reshape(-1, d), ref, rtol=1e-11, atol=1e-12)


def test_zero_query_gives_mean_of_visible_values():
    # q = 0 makes every visible key equally weighted: the output is the mean of v
    # over the key frames of the hand-written table.
    F, N, H, d = 20, 4, 2, 8
    _, k, v = small_inputs(F, N, H, d, seed=2)
    q = np.zeros_like(k)
    out = orc.softmax_branch(q, k, v)
    table = load_partition(F)
    for i in range(F):
        ref = v[table[i][0]].mean(axis=(0, 1))          # [H, d]
        np.testing.assert_allclose(out[i], np.broadcast_to(ref, (N, H, d)), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- extra (text / audio) tokens

def small_extra(T, H, d, seed=0, q_std=1.0):
    return tuple(vdn_synth.extra(n, T, H, d, seed=seed, q_std=q_std).astype(np.float64)
                 for n in ("q", "k", "v"))


@pytest.mark.parametrize("F,T", [(1, 3), (4, 5), (10, 7)])
def test_short_video_with_extras_is_full_attention(F, T):
    # F <= 10: the video part is full attention, and extra tokens add plain softmax
    # keys and rows, so the whole branch is unmasked attention over F*N+T tokens.
    N, H, d = 5, 2, 8
    q, k, v = small_inputs(F, N, H, d, seed=F)
    qx, kx, vx = small_extra(T, H, d, seed=F)
    ov = orc.softmax_branch_mixed(q, k, v, kx, vx)
    ox = orc.softmax_extra_rows(k, v, qx, kx, vx)
    dv, dx = orc.softmax_mixed_dense(q, k, v, qx, kx, vx)
    for h in range(H):
        cat = lambda a, ax: np.concatenate([a[:, :, h].reshape(-1, d), ax[:, h]], axis=0)
        ref = _sdpa(cat(q, qx), cat(k, kx), cat(v, vx))
        for got_v, got_x in ((ov, ox), (dv, dx)):
            np.testing.assert_allclose(got_v[:, :, h].reshape(-1, d), ref[:F * N], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(got_x[:, h], ref[F * N:], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("F,T", [(20, 6), (22, 9)])
def test_mixed_softmax_equals_masked_sdpa(F, T):
    # the hand-written frame table for video-video pairs, every pair with an extra
    # token allowed
    N, H, d = 3, 2, 8
    q, k, v = small_inputs(F, N, H, d, seed=3, q_std=4.0)
    qx, kx, vx = small_extra(T, H, d, seed=3, q_std=4.0)
    table = load_partition(F)
    fmask = np.zeros((F, F), dtype=bool)
    for i in range(F):
        fmask[i, table[i][0]] = True
    tmask = np.ones((F * N + T, F * N + T), dtype=bool)
    tmask[:F * N, :F * N] = np.kron(fmask, np.ones((N, N), dtype=bool))
    ov = orc.softmax_branch_mixed(q, k, v, kx, vx)
    ox = orc.softmax_extra_rows(k, v, qx, kx, vx)
    dv, dx = orc.softmax_mixed_dense(q, k, v, qx, kx, vx)
    for h in range(H):
        cat = lambda a, ax: np.concatenate([a[:, :, h].reshape(-1, d), ax[:, h]], axis=0)
        ref = _sdpa(cat(q, qx), cat(k, kx), cat(v, vx), tmask)
        for got_v, got_x in ((ov, ox), (dv, dx)):
            np.testing.assert_allclose(got_v[:, :, h].reshape(-1, d), ref[:F * N], rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(got_x[:, h], ref[F * N:], rtol=1e-11, atol=1e-12)


def test_mixed_zero_query_gives_mean_of_visible_values():
    # q = 0: a video row of frame i averages v over its table frames and all extra
    # tokens; an extra row averages v over every token
    F, N, T, H, d = 20, 4, 6, 2, 8
    _, k, v = small_inputs(F, N, H, d, seed=4)
    _, kx, vx = small_extra(T, H, d, seed=4)
    ov = orc.softmax_branch_mixed(np.zeros_like(k), k, v, kx, vx)
    ox = orc.softmax_extra_rows(k, v, np.zeros_like(kx), kx, vx)
    table = load_partition(F)
    for i in range(F):
        vis = np.concatenate([v[table[i][0]].reshape(-1, H, d), vx], axis=0)
        np.testing.assert_allclose(ov[i], np.broadcast_to(vis.mean(axis=0), (N, H, d)), rtol=1e-12, atol=1e-13)
    allv = np.concatenate([v.reshape(-1, H, d), vx], axis=0).mean(axis=0)
    np.testing.assert_allclose(ox, np.broadcast_to(allv, (T, H, d)), rtol=1e-12, atol=1e-13)


def test_mixed_layer_linear_branch_is_video_only():
    # extra tokens change neither the states nor O_lin, and with T = 0 the mixed
    # layer is the video layer
    F, N, T, H, d = 22, 3, 4, 2, 8
    q, k, v = small_inputs(F, N, H, d, seed=5)
    qx, kx, vx = small_extra(T, H, d, seed=5)
    beta, gate = vdn_synth.beta(F, H, seed=5), vdn_synth.gate(H, d, seed=5)
    O, Ox, Os, Ol = orc.hybrid_mixed(q, k, v, qx, kx, vx, beta, gate)
    O0, Os0, Ol0 = orc.hybrid(q, k, v, beta, gate)
    np.testing.assert_array_equal(Ol, Ol0)
    np.testing.assert_allclose(O - Os, O0 - Os0, rtol=1e-12, atol=1e-12)
    e = np.zeros((0, H, d))
    Oe, Oxe, Ose, _ = orc.hybrid_mixed(q, k, v, e, e, e, beta, gate)
    np.testing.assert_allclose(Oe, O0, rtol=1e-12, atol=1e-13)
    assert Oxe.shape == (0, H, d)


# ---------------------------------------------------------------- output projections

def test_projection_special_weights():
    # identity and zero weights reduce the projection to each branch alone, shared
    # weights to the merged layer followed by one projection, and the result is
    # linear in each weight matrix
    F, N, H, d = 22, 3, 2, 8
    Hd = H * d
    q, k, v = small_inputs(F, N, H, d, seed=6)
    beta, gate = vdn_synth.beta(F, H, seed=6), vdn_synth.gate(H, d, seed=6)
    O, Os, Ol = orc.hybrid(q, k, v, beta, gate)
    I, Z = np.eye(Hd), np.zeros((Hd, Hd))
    Y, Ys, Yl = orc.hybrid_proj(q, k, v, beta, gate, I, Z)
    np.testing.assert_allclose(Y, Os.reshape(F, N, Hd), rtol=1e-12, atol=1e-14)
    Y, _, _ = orc.hybrid_proj(q, k, v, beta, gate, Z, I)
    np.testing.assert_allclose(Y, (gate[None, None] * Ol).reshape(F, N, Hd), rtol=1e-12, atol=1e-14)
    Wp = vdn_synth.proj_weights(5, Hd, seed=6).astype(np.float64)
    W1, W2 = Wp[:, :Hd], Wp[:, Hd:]
    Y, _, _ = orc.hybrid_proj(q, k, v, beta, gate, W1, W1)
    np.testing.assert_allclose(Y, O.reshape(F, N, Hd) @ W1.T, rtol=1e-11, atol=1e-12)
    Ya, _, _ = orc.hybrid_proj(q, k, v, beta, gate, W1, W2)
    Yb, _, _ = orc.hybrid_proj(q, k, v, beta, gate, W1 + W2, W2)
    Yc, _, _ = orc.hybrid_proj(q, k, v, beta, gate, W2, np.zeros_like(W2))
    np.testing.assert_allclose(Yb, Ya + Yc, rtol=1e-10, atol=1e-12)
    # one output channel by hand: a plain sum over heads and channels
    t_f, t_n, c = 13, 1, 3
    ref = sum(Os[t_f, t_n, h, e] * W1[c, h * d + e] + gate[h, e] * Ol[t_f, t_n, h, e] * W2[c, h * d + e]
              for h in range(H) for e in range(d))
    assert abs(Ya[t_f, t_n, c] - ref) <= 1e-12 * max(1.0, abs(ref))


# ---------------------------------------------------------------- VDA update

def test_update_is_least_squares_minimiser():
    # argmin_X beta ||X K - V||^2 + ||X - S||^2, row by row: stack [sqrt(beta) K^T; I] x = [sqrt(beta) v_r; s_r]
    rng = np.random.default_rng(5)
    for (d, n) in [(8, 3), (8, 20), (16, 16)]:
        K = rng.standard_normal((d, n))
        V = rng.standard_normal((d, n))
        S = rng.standard_normal((d, d))
        beta = 0.37
        X = orc.vda_update(S, K, V, beta)
        A = np.vstack([math.sqrt(beta) * K.T, np.eye(d)])
        for r in range(d):
            rhs = np.concatenate([math.sqrt(beta) * V[r], S[r]])
            x, *_ = np.linalg.lstsq(A, rhs, rcond=None)
            np.testing.assert_allclose(X[r], x, rtol=1e-10, atol=1e-12)


def test_update_single_token_sherman_morrison():
    # N = 1: (S + b v k^T)(I + b k k^T)^-1 = S + b/(1 + b |k|^2) (v - S k) k^T
    rng = np.random.default_rng(6)
    d = 12
    k = rng.standard_normal((d, 1))
    v = rng.standard_normal((d, 1))
    S = rng.standard_normal((d, d))
    b = 0.6
    ref = S + b / (1.0 + b * float((k.T @ k)[0, 0])) * (v - S @ k) @ k.T
    np.testing.assert_allclose(orc.vda_update(S, k, v, b), ref, rtol=1e-12, atol=1e-12)


def test_update_non_expansive():
    rng = np.random.default_rng(7)
    d, n = 16, 40
    for _ in range(20):
        K = rng.standard_normal((d, n))
        V = rng.standard_normal((d, n))
        S1 = rng.standard_normal((d, d))
        S2 = rng.standard_normal((d, d))
        b = rng.uniform(0.01, 1.0)
        lhs = np.linalg.norm(orc.vda_update(S1, K, V, b) - orc.vda_update(S2, K, V, b))
        assert lhs <= np.linalg.norm(S1 - S2) * (1 + 1e-12)


def _identity_key_inputs(F, H, d, seed):
    """K_t = I (N = d tokens, token n has key e_n): A_t = (1 + b) I and the update is
    the exponential moving average S <- (S + b V_t) / (1 + b)."""
    N = d
    k = np.zeros((F, N, H, d))
    for n in range(N):
        k[:, n, :, n] = 1.0
    v = vdn_synth.tensor("v", F, N, H, d, seed=seed).astype(np.float64)
    q = vdn_synth.tensor("q", F, N, H, d, seed=seed).astype(np.float64)
    beta = vdn_synth.beta(F, H, seed=seed).astype(np.float64)
    return q, k, v, beta


@pytest.mark.parametrize("F", [20, 22, 30])
def test_states_equal_ema_closed_form(F):
    H, d = 2, 6
    q, k, v, beta = _identity_key_inputs(F, H, d, seed=3)
    Sf, Sb = orc.vda_states(k, v, beta)
    table = load_partition(F) if os.path.exists(os.path.join(GOLDEN, f"partition_F{F}.txt")) else None
    for c in range(orc.num_chunks(F)):
        members = [i for i in range(F) if i // 5 == c and i not in (0, F - 1)]
        if not members:
            continue
        i = members[0]
        fwd = table[i][1] if table else orc.forward_frames(i, F)
        bwd = table[i][2] if table else orc.backward_frames(i, F)
        for h in range(H):
            # V_t as [d, N]: column n is v[t, n, h, :]
            ref_f = np.zeros((d, d))
            for t in fwd:                         # oldest first: weight b_t prod_{u > t} 1/(1+b_u)
                w = beta[t, h] / np.prod([1.0 + beta[u, h] for u in fwd if u >= t])
                ref_f += w * v[t, :, h, :].T
            ref_b = np.zeros((d, d))
            for t in bwd:                         # absorbed latest first
                w = beta[t, h] / np.prod([1.0 + beta[u, h] for u in bwd if u <= t])
                ref_b += w * v[t, :, h, :].T
            np.testing.assert_allclose(Sf[c, h], ref_f, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(Sb[c, h], ref_b, rtol=1e-12, atol=1e-14)
    # and the readout: o = (S_fwd + S_bwd) q on non-anchor frames, 0 on anchors
    Ol = orc.linear_branch(q, Sf, Sb)
    assert not Ol[0].any() and not Ol[F - 1].any()
    i = F // 2
    c = i // 5
    np.testing.assert_allclose(Ol[i, 3, 1], (Sf[c, 1] + Sb[c, 1]) @ q[i, 3, 1], rtol=1e-12)


def _ema_weights(frames, beta_h, latest_first):
    """Weight of each absorbed frame in the state after the identity-key updates
    S <- (S + b_t V_t) / (1 + b_t) over `frames`, in absorption order: frame t
    keeps b_t / prod(1 + b_u) over itself and every frame absorbed after it."""
    order = sorted(frames, reverse=latest_first)
    w = {}
    for pos, t in enumerate(order):
        w[t] = beta_h[t] / np.prod([1.0 + beta_h[u] for u in order[pos:]])
    return w


@pytest.mark.parametrize("F", [20, 22, 30])
def test_linear_branch_closed_form_every_frame(F):
    # Identity keys (K_t = I, N = d) turn every state into an exponential moving
    # average of the value blocks, and a one-hot query e_m reads column m of
    # S_fwd + S_bwd, i.e. row m of each absorbed value block, weighted as above.
    # So O_lin of every token of every non-anchor frame has a closed form over the
    # hand-written forward / backward sets (sd114.wiki, 双向线性注意力分支: the query
    # reads both states and adds them; anchor frames read nothing); the one-hot
    # index varies with frame, token and head, so a readout that took another
    # chunk's states, another head or another query column would not match.
    H, d = 2, 6
    N = d
    _, k, v, beta = _identity_key_inputs(F, H, d, seed=9)
    q = np.zeros((F, N, H, d))
    onehot = lambda i, n, h: (n + 3 * i + 5 * h) % d
    for i in range(F):
        for n in range(N):
            for h in range(H):
                q[i, n, h, onehot(i, n, h)] = 1.0
    table = load_partition(F)
    Sf, Sb = orc.vda_states(k, v, beta)
    got = orc.linear_branch(q, Sf, Sb)
    for i in range(F):
        _, fwd, bwd = table[i]
        for h in range(H):
            wf = _ema_weights(fwd, beta[:, h], latest_first=False)
            wb = _ema_weights(bwd, beta[:, h], latest_first=True)
            for n in range(N):
                m = onehot(i, n, h)
                ref = np.zeros(d)
                if i not in (0, F - 1):
                    for t, w in list(wf.items()) + list(wb.items()):
                        ref += w * v[t, m, h, :]
                np.testing.assert_allclose(got[i, n, h], ref, rtol=1e-12, atol=1e-14)
    assert np.abs(got).max() > 1e-2          # both directions contribute somewhere


def test_time_reversal_swaps_directions():
    # F a multiple of 5: reversing the frame axis maps chunks to chunks and the
    # forward state of one input to the backward state of the other.
    F, N, H, d = 30, 5, 2, 6
    q, k, v = small_inputs(F, N, H, d, seed=4)
    beta = vdn_synth.beta(F, H, seed=4).astype(np.float64)
    gate = vdn_synth.gate(H, d, seed=4).astype(np.float64)
    O, Os, Ol = orc.hybrid(q, k, v, beta, gate)
    Or, Osr, Olr = orc.hybrid(q[::-1], k[::-1], v[::-1], beta[::-1], gate)
    np.testing.assert_allclose(Or[::-1], O, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(Olr[::-1], Ol, rtol=1e-10, atol=1e-12)
    assert np.abs(Ol).max() > 1e-3          # the linear branch is active here


def test_beta_zero_and_gate_zero():
    F, N, H, d = 25, 4, 2, 8
    q, k, v = small_inputs(F, N, H, d, seed=8)
    gate = vdn_synth.gate(H, d).astype(np.float64)
    O, Os, Ol = orc.hybrid(q, k, v, np.zeros((F, H)), gate)
    assert not Ol.any()
    np.testing.assert_array_equal(O, Os)
    beta = vdn_synth.beta(F, H).astype(np.float64)
    O, Os, Ol = orc.hybrid(q, k, v, beta, np.zeros((H, d)))
    np.testing.assert_array_equal(O, Os)
    # small beta: the linear output shrinks linearly
    _, _, Ol1 = orc.hybrid(q, k, v, 1e-6 * np.ones((F, H)), gate)
    _, _, Ol2 = orc.hybrid(q, k, v, 2e-6 * np.ones((F, H)), gate)
    assert np.abs(Ol1).max() > 0
    assert np.linalg.norm(Ol2 - 2 * Ol1) <= 1e-4 * np.linalg.norm(2 * Ol1)


# ---------------------------------------------------------------- fp8 quantiser

def test_e4m3_round_matches_torch_float8():
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1.0, 30.0, 300.0)])
    x = np.concatenate([x, [0.0, 448.0, -448.0, 450.0, 2.0 ** -9, 2.0 ** -10, 1.0625, 1.1875, 240.0, 248.0]])
    x = x.astype(np.float32)
    x = x[np.abs(x) <= 448.0]                    # torch's cast does not saturate above 448
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(orc.e4m3_round(x), ref)


def test_fp8_scale_exponent_is_the_smallest_power_of_two():
    # hand-worked values: 448 * 2^e is the first bound at or above amax
    f32 = np.float32
    table = [(448.0, 0), (float(np.nextafter(f32(448.0), f32(1e9))), 1), (224.0, -1),
             (float(np.nextafter(f32(224.0), f32(1e9))), 0), (1.0, -8), (1.75, -8), (1.7500001, -7),
             (0.0, 0), (3.0e38, 120), (1e-44, -127), (448.0 * 2.0 ** 100, 100)]
    got = orc.fp8_scale_exponent(np.array([a for a, _ in table], dtype=np.float32))
    assert got.tolist() == [e for _, e in table]
    # and the defining property over a wide random range
    rng = np.random.default_rng(3)
    a = (10.0 ** rng.uniform(-30, 30, 5000)).astype(np.float32).astype(np.float64)
    e = orc.fp8_scale_exponent(a.astype(np.float32)).astype(np.float64)
    assert np.all(a <= 448.0 * np.exp2(e))
    assert np.all(a > 448.0 * np.exp2(e - 1))


def test_fp8_quantize_power_of_two_codes():
    # codes of x / 2^e: every head reaches [224, 448], and code * 2^e is within half
    # an E4M3 step of x (relative 2^-4 in the normal range, 2^-10 * 2^e below it)
    F, N, H, d = 10, 8, 3, 16
    q, _, _ = small_inputs(F, N, H, d)
    x = (q * np.array([1e-3, 1.0, 5e3])[None, None, :, None]).astype(np.float32)
    e = orc.fp8_scale_exponent(orc.fp8_head_scales(x))
    codes = orc.fp8_quantize(x, e)
    back = codes * np.exp2(e.astype(np.float64))[:, None]
    for h in range(H):
        m = np.abs(codes[:, :, h]).max()
        assert 224.0 <= m <= 448.0     # (the top may round down to 224)
    xs = x.astype(np.float64)
    step = np.maximum(2.0 ** -4 * np.abs(xs), 2.0 ** -10 * np.exp2(e.astype(np.float64))[:, None])
    assert np.all(np.abs(back - xs) <= step * (1 + 1e-12))


def test_fp8_temperature_and_operands():
    d = 128
    c = orc.fp8_temperature(d)
    assert c.dtype == np.float32
    assert abs(float(c) - math.log2(math.e) / math.sqrt(d)) <= 2.0 ** -23 * float(c)
    F, N, H = 6, 10, 2
    rng = np.random.default_rng(4)
    # k on the E4M3 grid times 2^5 with a head maximum of exactly 448 * 2^5: exact
    grid = orc.e4m3_round(rng.uniform(-448, 448, (F, N, H, d)))
    grid[0, 0, :, 0] = 448.0
    k = grid * 32.0
    q = rng.standard_normal((F, N, H, d)) * np.array([0.02, 30.0])[None, None, :, None]
    q = q.astype(np.float32).astype(np.float64)
    q_eff, k_eff = orc.fp8_qk_operands(q, k, d)
    np.testing.assert_array_equal(k_eff, k)
    # q_eff stands for q in the units of the plain branch: within half an E4M3 step
    # of q (the temperature is divided out again, up to its float32 rounding)
    eq = orc.fp8_scale_exponent(orc.fp8_head_scales((q.astype(np.float32) * c).astype(np.float32)))
    unit = np.exp2(eq.astype(np.float64)) / float(c)        # value of one code unit, in q units
    step = np.maximum(2.0 ** -4 * np.abs(q), 2.0 ** -10 * unit[:, None])
    assert np.all(np.abs(q_eff - q) <= step * (1 + 1e-5) + 1e-6 * np.abs(q))
    # and the scores: the plain softmax on (q_eff, k_eff) sees q.k within the same bound
    s_eff = np.einsum("fnhd,gmhd->hfngm", q_eff, k_eff)
    s_ref = np.einsum("fnhd,gmhd->hfngm", q, k)
    bound = np.einsum("fnhd,gmhd->hfngm", np.abs(q) * 2.0 ** -4 + 2.0 ** -10 * unit[None, None, :, None], np.abs(k))
    assert np.all(np.abs(s_eff - s_ref) <= bound * (1 + 1e-5) + 1e-9)


def test_fp8_v_operand():
    # v on the E4M3 grid times 2^-3 with a head maximum of 448 * 2^-3: exact; any v:
    # within half an E4M3 step, every head reaching [224, 448] code units
    rng = np.random.default_rng(8)
    F, N, H, d = 5, 12, 3, 32
    grid = orc.e4m3_round(rng.uniform(-448, 448, (F, N, H, d)))
    grid[1, 2, :, 3] = -448.0
    v = grid / 8.0
    np.testing.assert_array_equal(orc.fp8_v_operand(v), v)
    v = (rng.standard_normal((F, N, H, d)) * np.array([1e-4, 1.0, 300.0])[None, None, :, None]).astype(np.float32)
    ve = orc.fp8_v_operand(v)
    e = orc.fp8_scale_exponent(orc.fp8_head_scales(v)).astype(np.float64)
    unit = np.exp2(e)[:, None]
    vs = v.astype(np.float64)
    step = np.maximum(2.0 ** -4 * np.abs(vs), 2.0 ** -10 * unit)
    assert np.all(np.abs(ve - vs) <= step * (1 + 1e-12))
    for h in range(H):
        assert 224.0 <= np.abs(ve[:, :, h]).max() / unit[h, 0] <= 448.0   # (the top may round down to 224)

