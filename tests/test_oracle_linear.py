"""Pins for the linear-branch and fusion part of the CPU oracle
(``phi``, ``linear_key_frames``, ``linear_mask``, ``linear_branch``,
``rms_norm``, ``hybrid_fuse``).  Each check compares the oracle with
something other than itself: the softmax mask (the two branches split the
(query, key) pairs between them), a pair-by-pair weighted sum over the
explicit mask with the feature map taken from torch, torch's own RMSNorm,
closed forms and values derived by hand from the block rule.  The mutation
tests at the end plant plausible mistakes and check that a pin catches
each."""

import numpy as np
import pytest
import torch

import oracle
from oracle import local_attn as OL

SWEEP = [(F, T, N, Bf)
         for F in (1, 2, 3, 5, 6, 10, 11, 12, 16, 20, 21)
         for T in (1, 3)
         for N in (0, 4)
         for Bf in (1, 2, 5, 7)]


# ------------------------------------------------------------------ key set


@pytest.mark.parametrize("F,T,N,Bf", SWEEP)
def test_linear_mask_is_the_softmax_complement(F, T, N, Bf):
    # the linear branch leaves out exactly what the softmax branch covers
    soft = OL.allowed_mask(F, T, N, Bf)
    lin = oracle.linear_mask(F, T, N, Bf)
    assert not np.any(soft & lin)
    assert np.all(soft | lin)


@pytest.mark.parametrize("F,T,N,Bf", SWEEP)
def test_linear_key_frames_equal_mask_rows(F, T, N, Bf):
    lin = oracle.linear_mask(F, T, N, Bf)
    S = F * T + N
    for beta in range(oracle.num_frame_blocks(F, Bf)):
        cols = np.zeros(S, dtype=bool)
        for f in oracle.linear_key_frames(beta, F, Bf):
            cols[f * T:(f + 1) * T] = True
        r0, r1 = beta * Bf * T, min(F, (beta + 1) * Bf) * T
        for i in range(r0, r1):
            assert np.array_equal(lin[i], cols), (beta, i)
    # text rows have no linear keys
    assert not np.any(lin[F * T:])


def test_linear_key_frames_768p_hand_derived():
    # 20 frames in blocks of 5, anchors 0 and 19: block 0's window is frames
    # 0-9, so it sums frames 10-18; block 1 (window 0-14) frames 15-18;
    # block 2 (window 5-19) frames 1-4; block 3 (window 10-19) frames 1-9
    assert [oracle.linear_key_frames(b, 20, 5) for b in range(4)] == [
        list(range(10, 19)), [15, 16, 17, 18], [1, 2, 3, 4], list(range(1, 10))]
    # 42 frames (ragged last block of 2 frames): block 4 (frames 20-24,
    # window 15-29) sums 1-14 and 30-40
    assert oracle.linear_key_frames(4, 42, 5) == list(range(1, 15)) + list(range(30, 41))
    # 11 frames: blocks 0 and 1 have nothing outside their windows but the
    # anchor frame 10; block 2 (frame 10, window 5-10) sums frames 1-4
    assert [oracle.linear_key_frames(b, 11, 5) for b in range(3)] == [[], [], [1, 2, 3, 4]]


def test_768p_pair_split():
    # share of (query, key) pairs on each branch at the 768p shape; pair
    # counts from the block rule: 4 blocks x 5040 rows see 9, 4, 4 and 9
    # frames of 1008 keys on the linear side
    F, T, N, Bf = 20, 1008, 512, 5
    S = F * T + N
    lin_pairs = 5040 * 1008 * (9 + 4 + 4 + 9)
    soft_pairs, _ = oracle.count_pairs(F, T, N, Bf)
    assert soft_pairs + lin_pairs == S * S


# ------------------------------------------------------------------- values


def test_phi_values():
    x = np.array([-50.0, -1.0, -1e-3, 0.0, 1e-3, 0.5, 3.0])
    # torch's elu(x) + 1 cancels for very negative x; phi keeps exp(x)
    ref = torch.nn.functional.elu(torch.tensor(x, dtype=torch.float64)).numpy() + 1.0
    np.testing.assert_allclose(oracle.phi(x), ref, rtol=1e-15, atol=1e-16)
    assert oracle.phi(np.array([-50.0]))[0] == np.exp(-50.0)
    assert oracle.phi(np.array([0.0]))[0] == 1.0
    assert oracle.phi(np.array([2.0]))[0] == 3.0
    assert np.all(oracle.phi(np.linspace(-30, 30, 101)) > 0)


def _qkv(seed, B, H, D, F, T, N, v_offset=0.0):
    rng = np.random.default_rng(seed)
    S = F * T + N
    q = rng.standard_normal((B, S, H, D))
    k = rng.standard_normal((B, S, H, D))
    v = rng.standard_normal((B, S, H, D))
    if v_offset:
        # a per-frame offset so that the output depends on which frames are
        # summed, not only on their number
        frame = np.minimum(np.arange(S) // T, F)
        v = v + v_offset * frame[None, :, None, None]
    return q, k, v


def _pairwise(q, k, v, mask):
    """Pair-by-pair weighted average over the explicit mask, with the feature
    map taken from torch's elu: a route through no state and no frame sums."""
    fq = torch.nn.functional.elu(torch.tensor(q, dtype=torch.float64)).numpy() + 1.0
    fk = torch.nn.functional.elu(torch.tensor(k, dtype=torch.float64)).numpy() + 1.0
    B, S, H, D = q.shape
    out = np.zeros_like(q)
    for b in range(B):
        for h in range(H):
            w = (fq[b, :, h, :] @ fk[b, :, h, :].T) * mask
            den = w.sum(axis=1)
            num = w @ v[b, :, h, :]
            ok = den > 0
            out[b, ok, h, :] = num[ok] / den[ok, None]
    return out


CASES = [
    # (seed, B, H, D, F, T, N, Bf)
    (1, 1, 2, 8, 20, 3, 4, 5),
    (2, 2, 1, 4, 11, 4, 3, 5),
    (3, 1, 1, 8, 13, 2, 0, 3),
    (4, 1, 2, 4, 21, 2, 5, 5),
    (5, 1, 1, 6, 7, 3, 2, 1),
    (6, 1, 1, 4, 42, 1, 2, 5),
]


@pytest.mark.parametrize("case", CASES)
def test_linear_branch_equals_pairwise_sum(case):
    seed, B, H, D, F, T, N, Bf = case
    q, k, v = _qkv(seed, B, H, D, F, T, N, v_offset=0.3)
    got = oracle.linear_branch(q, k, v, F, T, N, Bf)
    ref = _pairwise(q, k, v, oracle.linear_mask(F, T, N, Bf))
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_constant_values_pass_through():
    # every key carries the same value vector: each video query with at least
    # one linear key returns it exactly; text rows and empty blocks are zero
    F, T, N, Bf, D = 11, 3, 4, 5, 6
    q, k, _ = _qkv(7, 1, 1, D, F, T, N)
    S = F * T + N
    c = np.linspace(-2, 3, D)
    v = np.broadcast_to(c, (1, S, 1, D)).copy()
    out = oracle.linear_branch(q, k, v, F, T, N, Bf)
    # blocks 0 and 1 (frames 0-9) see only the anchor frame 10 outside their
    # windows; block 2 (frame 10) sums frames 1-4
    assert np.all(out[0, :30] == 0.0)
    np.testing.assert_allclose(out[0, 30:33, 0, :], np.broadcast_to(c, (3, D)), rtol=1e-13)
    assert np.all(out[0, 33:] == 0.0)


def test_zero_queries_weight_keys_by_feature_sums():
    # q = 0 gives phi(q) = 1, so key j weighs sum_d phi(k_j)_d: written out
    # with the key frames taken from the hand-derived list for 768p-like
    # blocks (20 frames of 2 tokens, blocks of 5)
    F, T, N, Bf, D = 20, 2, 3, 5, 4
    _, k, v = _qkv(8, 1, 1, D, F, T, N)
    S = F * T + N
    q = np.zeros((1, S, 1, D))
    out = oracle.linear_branch(q, k, v, F, T, N, Bf)
    frames = {0: range(10, 19), 1: range(15, 19), 2: range(1, 5), 3: range(1, 10)}
    for beta, fr in frames.items():
        keys = np.concatenate([np.arange(f * T, (f + 1) * T) for f in fr])
        w = np.where(k[0, keys, 0, :] > 0, k[0, keys, 0, :] + 1, np.exp(k[0, keys, 0, :])).sum(axis=1)
        want = (w[:, None] * v[0, keys, 0, :]).sum(axis=0) / w.sum()
        for i in range(beta * Bf * T, (beta + 1) * Bf * T):
            np.testing.assert_allclose(out[0, i, 0, :], want, rtol=1e-12)


def test_output_is_a_convex_combination():
    # positive weights: every coordinate lies between the smallest and the
    # largest value over the summed keys
    F, T, N, Bf, D = 16, 3, 2, 5, 5
    q, k, v = _qkv(9, 1, 1, D, F, T, N)
    out = oracle.linear_branch(q, k, v, F, T, N, Bf)
    for beta in range(oracle.num_frame_blocks(F, Bf)):
        fr = oracle.linear_key_frames(beta, F, Bf)
        if not fr:
            continue
        keys = np.concatenate([np.arange(f * T, (f + 1) * T) for f in fr])
        lo, hi = v[0, keys, 0, :].min(axis=0), v[0, keys, 0, :].max(axis=0)
        r0, r1 = beta * Bf * T, min(F, (beta + 1) * Bf) * T
        assert np.all(out[0, r0:r1, 0, :] >= lo - 1e-12)
        assert np.all(out[0, r0:r1, 0, :] <= hi + 1e-12)


# ------------------------------------------------------------------- fusion


def test_rms_norm_equals_torch():
    rng = np.random.default_rng(10)
    B, S, H, D = 2, 5, 3, 4
    x = rng.standard_normal((B, S, H, D)) * 3
    w = rng.standard_normal((H, D))
    for eps in (0.0, 1e-6, 0.5):
        ref = torch.nn.functional.rms_norm(torch.tensor(x.reshape(B, S, H * D)), (H * D,),
                                           weight=torch.tensor(w.reshape(H * D)), eps=eps)
        np.testing.assert_allclose(oracle.rms_norm(x, w, eps), ref.numpy().reshape(B, S, H, D),
                                   rtol=1e-13, atol=1e-15)


def test_rms_norm_scale_invariance_and_unit_rms():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((1, 4, 2, 8))
    ones = np.ones((2, 8))
    y = oracle.rms_norm(x, ones, 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=(-2, -1)), 1.0, rtol=1e-13)
    np.testing.assert_allclose(oracle.rms_norm(7.5 * x, ones, 0.0), y, rtol=1e-13)


def test_hybrid_fuse_closed_forms():
    rng = np.random.default_rng(12)
    B, S, H, D = 1, 6, 2, 4
    soft = rng.standard_normal((B, S, H, D))
    lin = rng.standard_normal((B, S, H, D))
    w = rng.standard_normal((H, D))
    g = rng.standard_normal((B, S, H))
    # gate logit 0 -> weight one half
    half = oracle.hybrid_fuse(soft, lin, np.zeros((B, S, H)), w, 1e-6)
    np.testing.assert_allclose(half, soft + 0.5 * oracle.rms_norm(lin, w, 1e-6), rtol=1e-14)
    # a closed gate leaves the softmax branch alone
    np.testing.assert_allclose(oracle.hybrid_fuse(soft, lin, np.full((B, S, H), -700.0), w, 1e-6),
                               soft, rtol=0, atol=0)
    # zero linear output with eps > 0 adds nothing
    np.testing.assert_array_equal(oracle.hybrid_fuse(soft, np.zeros_like(lin), g, w, 1e-6), soft)
    # a token whose linear output is c on every channel: the norm gives w
    lin1 = np.full((B, S, H, D), -3.0)
    want = soft + (1 / (1 + np.exp(-g)))[..., None] * (-w)[None, None]
    np.testing.assert_allclose(oracle.hybrid_fuse(soft, lin1, g, w, 0.0), want, rtol=1e-13)


# ---------------------------------------------------------- mutation tests


def _pins():
    for c in CASES[:2]:
        test_linear_branch_equals_pairwise_sum(c)
    test_constant_values_pass_through()
    test_zero_queries_weight_keys_by_feature_sums()
    test_linear_key_frames_768p_hand_derived()
    test_rms_norm_equals_torch()
    test_hybrid_fuse_closed_forms()


@pytest.mark.parametrize("mutant", ["anchors_in", "window_edge", "phi_exp", "no_normaliser",
                                    "norm_per_head", "gate_sign"])
def test_linear_mutants_are_caught(monkeypatch, mutant):
    if mutant == "anchors_in":
        def bad(beta, F, Bf):
            lo, hi = OL.window_frames(beta, F, Bf)
            return [f for f in range(F) if f < lo or f >= hi]
        monkeypatch.setattr(OL, "linear_key_frames", bad)
        monkeypatch.setattr(oracle, "linear_key_frames", bad)
    elif mutant == "window_edge":
        def bad(beta, F, Bf):
            lo, hi = OL.window_frames(beta, F, Bf)
            return [f for f in range(F) if (f < lo or f > hi) and f != 0 and f != F - 1]
        monkeypatch.setattr(OL, "linear_key_frames", bad)
        monkeypatch.setattr(oracle, "linear_key_frames", bad)
    elif mutant == "phi_exp":
        monkeypatch.setattr(OL, "phi", lambda x: np.exp(np.asarray(x, dtype=np.float64)))
    elif mutant == "no_normaliser":
        orig = OL.linear_branch

        def bad(q, k, v, F, T, N, Bf):
            out = orig(q, k, v, F, T, N, Bf)
            return out * 1.01
        monkeypatch.setattr(oracle, "linear_branch", bad)
    elif mutant == "norm_per_head":
        def bad(x, weight, eps):
            x = np.asarray(x, dtype=np.float64)
            r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
            return x / r * np.asarray(weight)[None, None]
        monkeypatch.setattr(OL, "rms_norm", bad)
        monkeypatch.setattr(oracle, "rms_norm", bad)
    elif mutant == "gate_sign":
        monkeypatch.setattr(OL, "sigmoid", lambda g: 1.0 / (1.0 + np.exp(np.asarray(g, dtype=np.float64))))
    with pytest.raises(AssertionError):
        _pins()
