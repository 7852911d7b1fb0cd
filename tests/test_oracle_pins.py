"""Pins of the CPU oracle to facts outside itself (CPU only).

Each test checks the oracle against something the pages or the mathematics
fix: the least-squares objective the closed form minimises, the textbook
token-wise delta rule it reduces to, closed-form evidence weights, library
attention, brute-force mask enumeration, and values the pages print.
"""
import itertools
import os

import numpy as np
import pytest
import torch

from oracle import vdn_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split()[:2]
            vals[key] = float(val)
    return vals


def _objective(S, S_bar, k, v, beta):
    r = S @ k.T - v.T                         # [d_v, n]
    return np.sum((S - S_bar) ** 2) + np.sum(beta * np.sum(r * r, axis=0))


def _rand_inputs(rng, lay, beta_scale=1.0):
    B, H, d, N, L, T = lay.batch, lay.heads, lay.head_dim, lay.video_tokens, lay.text_tokens, lay.frames
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    return dict(
        q=rng.standard_normal((B, N, H, d)),
        k=unit(rng.standard_normal((B, N, H, d))),
        v=rng.standard_normal((B, N, H, d)),
        text_k=unit(rng.standard_normal((B, L, H, d))),
        text_v=rng.standard_normal((B, L, H, d)),
        beta=beta_scale / (1 + np.exp(-rng.standard_normal((B, N + L, H)))),
        alpha=rng.uniform(0.9, 1.0, size=(B, T, H)),
        gate_logits=rng.standard_normal((B, N, H, 2)),
    )


# --------------------------------------------------------------------------
# V1: the closed form is the minimiser of the regularised objective
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_closed_form_minimises_objective(seed):
    rng = np.random.default_rng(seed)
    d_k, d_v, n = 6, 5, 9
    k = rng.standard_normal((n, d_k))
    v = rng.standard_normal((n, d_v))
    beta = rng.uniform(0.05, 3.0, size=n)
    S_bar = rng.standard_normal((d_v, d_k))
    A, B = O.frame_stats(k, v, beta)
    U = O.vda_update(S_bar, A, B)
    # gradient of ||S-S_bar||^2 + sum_i beta_i ||S k_i - v_i||^2 vanishes at U
    grad = 2 * (U - S_bar) + 2 * ((U @ k.T - v.T) * beta) @ k
    assert np.max(np.abs(grad)) < 1e-10
    J0 = _objective(U, S_bar, k, v, beta)
    for _ in range(20):
        E = rng.standard_normal(U.shape)
        for eps in (1e-3, 1e-1, 1.0):
            assert _objective(U + eps * E, S_bar, k, v, beta) >= J0 - 1e-12


def test_text_write_is_ridge_regression_solution():
    """S_x from the zero state equals the least-squares solution of the stacked
    system [I; sqrt(beta) k^T] (numpy lstsq, a different route)."""
    rng = np.random.default_rng(5)
    d, n = 7, 12
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    beta = rng.uniform(0.1, 2.0, size=n)
    S_x = O.text_prior(k, v, beta)
    # rows of S solve min ||s||^2 + sum beta (s.k - v_r)^2
    Aug = np.concatenate([np.eye(d), np.sqrt(beta)[:, None] * k], axis=0)
    rhs = np.concatenate([np.zeros((d, d)), np.sqrt(beta)[:, None] * v], axis=0)
    S_ls = np.linalg.lstsq(Aug, rhs, rcond=None)[0].T
    assert np.allclose(S_x, S_ls, atol=1e-12)


# --------------------------------------------------------------------------
# V2: one token per frame is the textbook gated delta rule
# --------------------------------------------------------------------------
def test_single_token_frames_reduce_to_gated_delta_rule():
    rng = np.random.default_rng(11)
    lay = O.Layout(batch=1, heads=1, head_dim=6, frames=23, tokens_per_frame=1,
                   text_tokens=3, chunk_frames=2, window_chunks=1)
    inp = _rand_inputs(rng, lay, beta_scale=2.0)
    N = lay.video_tokens
    k, v = inp["k"][0, :, 0], inp["v"][0, :, 0]
    beta, alpha = inp["beta"][0, :, 0], inp["alpha"][0, :, 0]
    S0 = O.initial_state(inp["text_k"][0, :, 0], inp["text_v"][0, :, 0], beta[N:], 6, 6)
    A_st = {f: O.frame_stats(k[f:f + 1], v[f:f + 1], beta[f:f + 1]) for f in range(lay.frames)}
    for t in range(lay.frames):
        for direction, frames in (("f", O.far_forward(lay, t)), ("b", O.far_backward(lay, t))):
            # textbook gated delta rule, token by token:
            #   S <- alpha S (I - b' k k^T) + b' v k^T,  b' = beta / (1 + beta |k|^2)
            S = S0.copy()
            for f in frames:
                kk, vv, bb = k[f], v[f], beta[f]
                bp = bb / (1.0 + bb * kk @ kk)
                S = alpha[f] * S @ (np.eye(6) - bp * np.outer(kk, kk)) + bp * np.outer(vv, kk)
            fn = O.forward_state if direction == "f" else O.backward_state
            got = fn(S0, lay, t, A_st, alpha)
            assert np.max(np.abs(got - S)) < 1e-12


# --------------------------------------------------------------------------
# V3 / V3': evidence weights
# --------------------------------------------------------------------------
@pytest.mark.parametrize("n", [1, 10, 100, 1000])
def test_repeated_evidence_weight_approaches_but_never_passes_one(n):
    rng = np.random.default_rng(n)
    d = 8
    kv = rng.standard_normal(d)
    kv /= np.linalg.norm(kv)
    vv = rng.standard_normal(d)
    k = np.tile(kv, (n, 1))
    v = np.tile(vv, (n, 1))
    A, B = O.frame_stats(k, v, np.ones(n))
    S = O.vda_update(np.zeros((d, d)), A, B)
    read = S @ kv
    w = read @ vv / (vv @ vv)
    assert abs(w - n / (1.0 + n)) < 1e-12
    assert np.allclose(read, w * vv, atol=1e-12)
    assert w < 1.0


def test_hundred_patches_golden():
    g = _golden("window_and_evidence.txt")
    n = int(g["evidence_tokens"])
    d = 16
    e = np.zeros(d); e[3] = 1.0
    v = np.arange(d, dtype=float)
    A, B = O.frame_stats(np.tile(e, (n, 1)), np.tile(v, (n, 1)), np.ones(n))
    w = (O.vda_update(np.zeros((d, d)), A, B) @ e) @ v / (v @ v)
    assert 0.98 < w < g["evidence_weight_upper_bound"]


def test_independent_directions_keep_full_strength():
    rng = np.random.default_rng(3)
    d, n = 10, 4
    Q, _ = np.linalg.qr(rng.standard_normal((d, n)))
    k = Q.T                                    # orthonormal keys
    v = rng.standard_normal((n, d))
    beta = rng.uniform(0.1, 5.0, size=n)
    A, B = O.frame_stats(k, v, beta)
    S = O.vda_update(np.zeros((d, d)), A, B)
    for i in range(n):
        assert np.allclose(S @ k[i], beta[i] / (1 + beta[i]) * v[i], atol=1e-12)
        # the same weight as a frame that holds token i alone
        Ai, Bi = O.frame_stats(k[i:i + 1], v[i:i + 1], beta[i:i + 1])
        assert np.allclose(O.vda_update(np.zeros((d, d)), Ai, Bi) @ k[i], S @ k[i], atol=1e-12)


# --------------------------------------------------------------------------
# V4: the transition is non-expansive
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [0, 1])
def test_transition_is_non_expansive(seed):
    rng = np.random.default_rng(seed)
    d, n = 12, 40
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    beta = rng.uniform(0.0, 10.0, size=n)
    A, B = O.frame_stats(k, v, beta)
    G = O.vda_update(np.eye(d), A, np.zeros((d, d)))   # (I + A)^-1
    assert np.linalg.norm(G, 2) <= 1.0 + 1e-12
    lam = np.linalg.eigvalsh(A)
    assert np.allclose(np.sort(np.linalg.eigvalsh((G + G.T) / 2)), np.sort(1 / (1 + lam)), atol=1e-12)
    for _ in range(10):
        S = rng.standard_normal((d, d))
        a = rng.uniform(0.3, 1.0)
        assert np.linalg.norm(O.vda_update(a * S, A, np.zeros((d, d)))) <= a * np.linalg.norm(S) + 1e-12


# --------------------------------------------------------------------------
# V5: order independence inside a frame
# --------------------------------------------------------------------------
def test_permuting_tokens_within_a_frame_permutes_output():
    rng = np.random.default_rng(21)
    lay = O.Layout(batch=1, heads=2, head_dim=4, frames=13, tokens_per_frame=5,
                   text_tokens=3, chunk_frames=2, window_chunks=1)
    inp = _rand_inputs(rng, lay)
    out = O.hybrid_attn(inp, lay)
    P = lay.tokens_per_frame
    for f in (0, 6, 12):
        perm = np.arange(lay.video_tokens)
        perm[f * P:(f + 1) * P] = f * P + rng.permutation(P)
        pin = dict(inp)
        for key in ("q", "k", "v", "gate_logits"):
            pin[key] = inp[key][:, perm]
        beta = inp["beta"].copy()
        beta[:, :lay.video_tokens] = inp["beta"][:, perm]
        pin["beta"] = beta
        out_p = O.hybrid_attn(pin, lay)
        assert np.allclose(out_p, out[:, perm], atol=1e-12)


# --------------------------------------------------------------------------
# X1 / X2: the text counts exactly once
# --------------------------------------------------------------------------
def test_text_counted_once_every_frame():
    rng = np.random.default_rng(8)
    lay = O.Layout(batch=1, heads=1, head_dim=5, frames=17, tokens_per_frame=3,
                   text_tokens=6, chunk_frames=3, window_chunks=1)
    inp = _rand_inputs(rng, lay)
    inp["beta"][:, :lay.video_tokens] = 0.0      # video writes vanish
    inp["alpha"][:] = 1.0
    N = lay.video_tokens
    tk, tv, tb = inp["text_k"][0, :, 0], inp["text_v"][0, :, 0], inp["beta"][0, N:, 0]
    # S_x as the solution of the stacked least-squares system
    d = lay.head_dim
    Aug = np.concatenate([np.eye(d), np.sqrt(tb)[:, None] * tk], axis=0)
    rhs = np.concatenate([np.zeros((d, d)), np.sqrt(tb)[:, None] * tv], axis=0)
    S_x = np.linalg.lstsq(Aug, rhs, rcond=None)[0].T
    _, _, o_lin, _ = O.hybrid_attn_rows(inp, lay, 0, 0, np.arange(N), parts=True)
    expect = inp["q"][0, :, 0] @ S_x.T
    assert np.allclose(o_lin, expect, atol=1e-12)     # anchors included


def test_text_prior_propagates_through_affine_scan():
    rng = np.random.default_rng(9)
    lay = O.Layout(batch=1, heads=1, head_dim=4, frames=19, tokens_per_frame=3,
                   text_tokens=5, chunk_frames=2, window_chunks=1)
    inp = _rand_inputs(rng, lay)
    inp["v"][:] = 0.0                            # video writes are zero: the scan is linear
    N, P, d = lay.video_tokens, lay.tokens_per_frame, lay.head_dim
    k, beta, alpha = inp["k"][0, :, 0], inp["beta"][0, :, 0], inp["alpha"][0, :, 0]
    tk, tv, tb = inp["text_k"][0, :, 0], inp["text_v"][0, :, 0], beta[N:]
    Ax = (tk * tb[:, None]).T @ tk
    S_x = ((tv * tb[:, None]).T @ tk) @ np.linalg.inv(np.eye(d) + Ax)
    G = {f: np.linalg.inv(np.eye(d) + (k[f * P:(f + 1) * P] * beta[f * P:(f + 1) * P, None]).T @ k[f * P:(f + 1) * P])
         for f in range(lay.frames)}
    _, _, o_lin, _ = O.hybrid_attn_rows(inp, lay, 0, 0, np.arange(N), parts=True)
    for t in range(lay.frames):
        Pf, Pb = np.eye(d), np.eye(d)
        for f in O.far_forward(lay, t):
            Pf = Pf @ (alpha[f] * G[f])
        for f in O.far_backward(lay, t):
            Pb = Pb @ (alpha[f] * G[f])
        R = 0.5 * S_x @ (Pf + Pb)
        rows = slice(t * P, (t + 1) * P)
        assert np.allclose(o_lin[rows], inp["q"][0, rows, 0] @ R.T, atol=1e-12)


# --------------------------------------------------------------------------
# S3: the window / anchor / far masks partition every frame pair once
# --------------------------------------------------------------------------
@pytest.mark.parametrize("C,w", [(5, 1), (2, 1), (3, 2), (1, 1), (4, 0)])
@pytest.mark.parametrize("anchors", [(True, True), (False, False), (True, False)])
def test_masks_partition_every_pair(C, w, anchors):
    for T in range(1, 41):
        lay = O.Layout(batch=1, heads=1, head_dim=4, frames=T, tokens_per_frame=1,
                       text_tokens=0, chunk_frames=C, window_chunks=w,
                       anchor_first=anchors[0], anchor_last=anchors[1])
        A = O.anchor_frames(lay)
        for t in range(T):
            vis = set(O.visible_frames(lay, t))
            ff, fb = O.far_forward(lay, t), O.far_backward(lay, t)
            assert ff == sorted(ff) and fb == sorted(fb, reverse=True)
            assert all(f < t for f in ff) and all(f > t for f in fb)
            parts = [vis, set(ff), set(fb)]
            for x, y in itertools.combinations(parts, 2):
                assert not (x & y)
            assert vis | set(ff) | set(fb) == set(range(T))
            assert t in vis
            assert not (A & (set(ff) | set(fb)))      # anchors are never written
            for f in range(T):
                cls = O.pair_class(lay, t, f)
                # brute force: chunk distance, then anchor membership
                near = abs(t // C - f // C) <= w
                anch = (f in A) or (t in A)
                exp = "window" if near else ("anchor" if anch else "far")
                assert cls == exp
                assert (cls != "far") == (f in vis)


def test_interior_window_covers_fifteen_frames():
    g = _golden("window_and_evidence.txt")
    lay = O.Layout(batch=1, heads=1, head_dim=4, frames=60, tokens_per_frame=1, text_tokens=0,
                   chunk_frames=int(g["chunk_frames"]))
    for t in range(5, 55):
        assert len(O.window_frames(lay, t)) == int(g["interior_window_frames"])


def test_anchor_density_increment_matches_printed_value():
    g = _golden("anchor_density.txt")
    lay = O.Layout(batch=1, heads=1, head_dim=4, frames=int(g["frames"]), tokens_per_frame=1,
                   text_tokens=0, chunk_frames=int(g["chunk_frames"]),
                   window_chunks=int(g["window_chunks"]))
    inc = 100 * (O.softmax_density(lay, True) - O.softmax_density(lay, False))
    assert g["increment_percent"] <= inc < g["increment_percent"] + g["print_resolution_percent"]


def test_density_falls_with_length():
    g = _golden("window_and_evidence.txt")
    d42 = O.softmax_density(O.Layout(1, 1, 4, 42, 1, 0))
    d102 = O.softmax_density(O.Layout(1, 1, 4, 102, 1, 0))
    assert d102 < d42
    # the video-only share stays below the printed totals (text/audio keys add to them)
    assert 100 * d42 < g["density_42_percent"] and 100 * d102 < g["density_102_percent"]


# --------------------------------------------------------------------------
# Softmax branch against library attention
# --------------------------------------------------------------------------
def _sdpa(qm, km, vm, mask):
    """Library attention with its default scale 1/sqrt(d) (reading R1)."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qm)[None], torch.from_numpy(km)[None], torch.from_numpy(vm)[None],
        attn_mask=None if mask is None else torch.from_numpy(mask)[None])[0].numpy()


def test_softmax_branch_matches_masked_library_attention():
    rng = np.random.default_rng(4)
    lay = O.Layout(batch=2, heads=2, head_dim=8, frames=14, tokens_per_frame=3,
                   text_tokens=4, chunk_frames=3, window_chunks=1)
    inp = _rand_inputs(rng, lay)
    got = O.softmax_branch(inp["q"], inp["k"], inp["v"], inp["text_k"], inp["text_v"], lay)
    N, P, L = lay.video_tokens, lay.tokens_per_frame, lay.text_tokens
    mask = np.zeros((N, N + L), dtype=bool)
    for i in range(N):
        for j in range(N):
            mask[i, j] = O.pair_class(lay, i // P, j // P) != "far"
        mask[i, N:] = True
    for b in range(2):
        for h in range(2):
            km = np.concatenate([inp["k"][b, :, h], inp["text_k"][b, :, h]])
            vm = np.concatenate([inp["v"][b, :, h], inp["text_v"][b, :, h]])
            ref = _sdpa(inp["q"][b, :, h], km, vm, mask)
            assert np.allclose(got[b, :, h], ref, atol=1e-12)


def test_dense_window_reduces_to_dense_attention_and_text_read():
    rng = np.random.default_rng(6)
    lay = O.Layout(batch=1, heads=1, head_dim=6, frames=11, tokens_per_frame=4,
                   text_tokens=5, chunk_frames=2, window_chunks=6)
    inp = _rand_inputs(rng, lay)
    N = lay.video_tokens
    out, o_soft, o_lin, _ = O.hybrid_attn_rows(inp, lay, 0, 0, np.arange(N), parts=True)
    km = np.concatenate([inp["k"][0, :, 0], inp["text_k"][0, :, 0]])
    vm = np.concatenate([inp["v"][0, :, 0], inp["text_v"][0, :, 0]])
    assert np.allclose(o_soft, _sdpa(inp["q"][0, :, 0], km, vm, None), atol=1e-12)
    tb = inp["beta"][0, N:, 0]
    S_x = O.text_prior(inp["text_k"][0, :, 0], inp["text_v"][0, :, 0], tb)
    assert np.allclose(o_lin, inp["q"][0, :, 0] @ S_x.T, atol=1e-12)


# --------------------------------------------------------------------------
# G1: gates isolate the branches; the linear branch is RMS-normalised
# --------------------------------------------------------------------------
def test_gates_isolate_branches():
    rng = np.random.default_rng(12)
    lay = O.Layout(batch=1, heads=1, head_dim=8, frames=12, tokens_per_frame=2,
                   text_tokens=3, chunk_frames=2, window_chunks=1)
    inp = _rand_inputs(rng, lay)
    N = lay.video_tokens
    g = inp["gate_logits"]
    g[..., 1] = -40.0
    out, o_soft, _, _ = O.hybrid_attn_rows(inp, lay, 0, 0, np.arange(N), parts=True)
    sig0 = 1 / (1 + np.exp(-g[0, :, 0, 0]))
    assert np.allclose(out, sig0[:, None] * o_soft, atol=1e-15)
    g[..., 0] = -40.0
    g[..., 1] = 40.0
    out, _, o_lin, n_lin = O.hybrid_attn_rows(inp, lay, 0, 0, np.arange(N), parts=True)
    rms = np.sqrt(np.mean(out ** 2, axis=-1))
    ms = np.mean(o_lin ** 2, axis=-1)
    assert np.allclose(rms, np.sqrt(ms / (ms + lay.rms_eps)), atol=1e-12)
    assert np.all(np.abs(rms - 1) < 1e-3)


def test_readings_alternatives_differ_only_where_expected():
    """R5/R7 alternatives change the result; R6's alternative only matters
    when an anchor lies on the far side of the window."""
    rng = np.random.default_rng(13)
    lay = O.Layout(batch=1, heads=1, head_dim=4, frames=16, tokens_per_frame=2,
                   text_tokens=3, chunk_frames=2, window_chunks=1)
    inp = _rand_inputs(rng, lay)
    N = lay.video_tokens
    base = O.hybrid_attn(inp, lay)
    alt5 = O.hybrid_attn(inp, lay, O.Readings(anchor_read="zero"))
    P = lay.tokens_per_frame
    assert np.allclose(base[:, P:N - P], alt5[:, P:N - P])
    assert not np.allclose(base[:, :P], alt5[:, :P])
    alt7 = O.hybrid_attn(inp, lay, O.Readings(half_write="raw"))
    assert not np.allclose(base, alt7)
    alt6 = O.hybrid_attn(inp, lay, O.Readings(anchor_decay=True))
    assert not np.allclose(base, alt6)


# --------------------------------------------------------------------------
# Alternative readings, each pinned outside its own formula
# --------------------------------------------------------------------------
def test_r5_zero_anchor_read_leaves_the_gated_dense_softmax():
    """R5 alternative (anchor frames read nothing from the linear branch):
    RMSNorm of a zero read is zero, so an anchor row is sigmoid(l0) times
    dense attention over every video and text key (an anchor frame sees the
    whole sequence), computed here by library attention; other rows keep the
    primary reading's values."""
    rng = np.random.default_rng(21)
    lay = O.Layout(batch=1, heads=2, head_dim=6, frames=11, tokens_per_frame=3,
                   text_tokens=4, chunk_frames=2, window_chunks=1)
    inp = _rand_inputs(rng, lay)
    N, P = lay.video_tokens, lay.tokens_per_frame
    alt = O.hybrid_attn(inp, lay, O.Readings(anchor_read="zero"))
    base = O.hybrid_attn(inp, lay)
    anchor_rows = np.r_[0:P, N - P:N]
    for h in range(lay.heads):
        km = np.concatenate([inp["k"][0, :, h], inp["text_k"][0, :, h]])
        vm = np.concatenate([inp["v"][0, :, h], inp["text_v"][0, :, h]])
        dense = _sdpa(inp["q"][0, anchor_rows, h], km, vm, None)
        sig0 = 1.0 / (1.0 + np.exp(-inp["gate_logits"][0, anchor_rows, h, 0]))
        assert np.allclose(alt[0, anchor_rows, h], sig0[:, None] * dense, atol=1e-12)
    assert np.allclose(alt[:, P:N - P], base[:, P:N - P], atol=0)


def _rank_one_update(S_bar, k, v, beta):
    """One token's joint update by Sherman-Morrison:
    (S_bar + b v k^T)(I + b k k^T)^-1 = S_bar + b'(v - S_bar k) k^T, b' = b/(1 + b|k|^2)."""
    bp = beta / (1.0 + beta * (k @ k))
    return S_bar + bp * np.outer(v - S_bar @ k, k)


def test_r6_decay_without_write_matches_token_loop():
    """R6 alternative (an anchor frame on the far side of a window decays the
    state but writes nothing).  With one token per frame and one text token
    every update is rank one, so both states follow from a plain loop over
    frames with chunk arithmetic: the forward state of query frame t starts at
    half the text write, decays by alpha_0 at anchor frame 0 when some frame
    lies before the window, then takes the token update of every frame before
    the window; the backward state mirrors this from frame T-1 down."""
    rng = np.random.default_rng(22)
    C, w, T, d = 2, 1, 15, 5
    lay = O.Layout(batch=1, heads=1, head_dim=d, frames=T, tokens_per_frame=1,
                   text_tokens=1, chunk_frames=C, window_chunks=w)
    inp = _rand_inputs(rng, lay, beta_scale=3.0)
    inp["alpha"][:] = rng.uniform(0.3, 0.9, size=inp["alpha"].shape)   # decay far from 1
    k, v, q = inp["k"][0, :, 0], inp["v"][0, :, 0], inp["q"][0, :, 0]
    beta, alpha = inp["beta"][0, :, 0], inp["alpha"][0, :, 0]
    S_x = _rank_one_update(np.zeros((d, d)), inp["text_k"][0, 0, 0], inp["text_v"][0, 0, 0], beta[T])
    _, _, o_lin, _ = O.hybrid_attn_rows(inp, lay, 0, 0, np.arange(T),
                                        O.Readings(anchor_decay=True), parts=True)
    for t in range(T):
        if t in (0, T - 1):
            assert np.allclose(o_lin[t], S_x @ q[t], atol=1e-12)
            continue
        c = t // C
        lo, hi = max(0, (c - w) * C), min(T, (c + w + 1) * C) - 1
        Sf = 0.5 * S_x
        if lo > 1:                          # frames 1 .. lo-1 are far
            Sf = alpha[0] * Sf
            for f in range(1, lo):
                Sf = _rank_one_update(alpha[f] * Sf, k[f], v[f], beta[f])
        Sb = 0.5 * S_x
        if hi < T - 2:                      # frames hi+1 .. T-2 are far
            Sb = alpha[T - 1] * Sb
            for f in range(T - 2, hi, -1):
                Sb = _rank_one_update(alpha[f] * Sb, k[f], v[f], beta[f])
        assert np.allclose(o_lin[t], (Sf + Sb) @ q[t], atol=1e-12)


def test_r7_raw_half_write_closed_form():
    """R7: with orthonormal text keys, video tokens that write nothing
    (beta = 0) and no decay (alpha = 1), every frame reads twice its start
    state.  Reading a text key k_j then gives beta_j v_j under the raw half
    write (0.5 * B_x) and beta_j / (1 + beta_j) v_j under the primary one (the
    joint update from zero): the evidence weight of an independent direction."""
    rng = np.random.default_rng(23)
    d, L = 7, 3
    lay = O.Layout(batch=1, heads=1, head_dim=d, frames=9, tokens_per_frame=L,
                   text_tokens=L, chunk_frames=2, window_chunks=1)
    inp = _rand_inputs(rng, lay)
    Qm, _ = np.linalg.qr(rng.standard_normal((d, L)))
    inp["text_k"][0, :, 0] = Qm.T
    N = lay.video_tokens
    inp["beta"][0, :N, 0] = 0.0
    inp["beta"][0, N:, 0] = rng.uniform(0.2, 4.0, size=L)
    inp["alpha"][:] = 1.0
    bt, tv = inp["beta"][0, N:, 0], inp["text_v"][0, :, 0]
    for t in range(lay.frames):
        inp["q"][0, t * L:(t + 1) * L, 0] = Qm.T        # frame t's queries are the text keys
    toks = np.arange(N)
    for reading, weight in (("raw", bt), ("vda", bt / (1 + bt))):
        _, _, o_lin, _ = O.hybrid_attn_rows(inp, lay, 0, 0, toks, O.Readings(half_write=reading),
                                            parts=True)
        want = np.tile(weight[:, None] * tv, (lay.frames, 1))
        assert np.allclose(o_lin, want, atol=1e-12), reading
