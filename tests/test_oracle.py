"""Pins for the CPU oracle: each check compares it with something other than
itself (hand-derived values, brute force over an explicit mask, torch's
scaled_dot_product_attention in float64, closed forms and needle probes).
The mutation tests at the end plant plausible mistakes in the oracle and
check that at least one pin catches each."""

import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import local_attn as OL

WORKLOAD_NAMES = ["tiny", "medium", "768p", "long"]


def _as_lists(ivs):
    return [[list(p) for p in lst] for lst in ivs]


# ---------------------------------------------------------------- structure


def check_intervals_golden(golden):
    for name in WORKLOAD_NAMES:
        g = golden["workloads"][name]
        F, T, N, Bf = g["F"], g["T"], g["N"], g["Bf"]
        assert [list(r) for r in OL.query_blocks(F, T, N, Bf)] == g["query_rows"], name
        assert _as_lists(OL.key_intervals(F, T, N, Bf)) == g["key_intervals"], name


def check_counts_golden(golden):
    for name in WORKLOAD_NAMES:
        g = golden["workloads"][name]
        F, T, N, Bf = g["F"], g["T"], g["N"], g["Bf"]
        assert OL.count_pairs(F, T, N, Bf) == (g["allowed"], g["anchor_added"]), name


def test_intervals_match_hand_derived(golden):
    check_intervals_golden(golden)


def test_counts_match_hand_derived(golden):
    check_counts_golden(golden)


def test_mask_hand_picked_pairs():
    # F=20 frames of T=3 tokens, N=2 text tokens, blocks of 5 frames.
    F, T, N, Bf = 20, 3, 2, 5
    m = OL.allowed_mask(F, T, N, Bf)
    tok = lambda f, j=0: f * T + j  # noqa: E731
    text = F * T
    # frame 7 is in block 1: sees frames 0..14 (blocks 0..2), anchor 19, text
    for f in list(range(0, 15)) + [19]:
        assert m[tok(7), tok(f, 2)], f
    for f in (15, 16, 17, 18):
        assert not m[tok(7, 1), tok(f)], f
    assert m[tok(7), text] and m[tok(7), text + 1]
    # frame 19 is in block 3: sees frames 10..19 and anchor 0, not 1..9
    assert m[tok(19), tok(0)] and m[tok(19), tok(10)] and m[tok(19), tok(19, 2)]
    for f in range(1, 10):
        assert not m[tok(19), tok(f)], f
    # frame 0 is in block 0: sees frames 0..9 and anchor 19, not 10..18
    assert m[tok(0), tok(9, 2)] and m[tok(0), tok(19)]
    for f in range(10, 19):
        assert not m[tok(0), tok(f)], f
    # an anchor-frame query follows its own block rule (frame 19 does not
    # see frame 5), and text queries see everything
    assert not m[tok(19), tok(5)]
    assert m[text].all() and m[text + 1].all()


SWEEP = [(F, T, N, Bf)
         for F in (1, 2, 3, 5, 6, 9, 10, 11, 12, 16, 21, 30)
         for T in (1, 2, 5)
         for N in (0, 1, 4)
         for Bf in (1, 2, 3, 5, 6)]


@pytest.mark.parametrize("F,T,N,Bf", SWEEP)
def test_intervals_equal_mask_scan(F, T, N, Bf):
    """Every row of a query block has the same mask row, equal to the union of
    that block's canonical intervals; intervals are sorted, disjoint and not
    touching."""
    m = OL.allowed_mask(F, T, N, Bf)
    qb = OL.query_blocks(F, T, N, Bf)
    kiv = OL.key_intervals(F, T, N, Bf)
    assert len(qb) == len(kiv)
    covered = np.zeros(F * T + N, dtype=int)
    for (r0, r1), ivs in zip(qb, kiv):
        covered[r0:r1] += 1
        expect = np.zeros(F * T + N, dtype=bool)
        for a, b in ivs:
            expect[a:b] = True
        for (a0, b0), (a1, b1) in zip(ivs, ivs[1:]):
            assert b0 < a1 and a0 < b0
        assert (m[r0:r1] == expect[None, :]).all()
    assert (covered == 1).all()


@pytest.mark.parametrize("F,T,N,Bf", SWEEP)
def test_counts_equal_bruteforce(F, T, N, Bf):
    assert OL.count_pairs(F, T, N, Bf) == OL.count_pairs_bruteforce(F, T, N, Bf)


def test_full_window_is_everything():
    for F, Bf in ((1, 5), (5, 5), (10, 5), (7, 4), (3, 1), (2, 1)):
        if F > 2 * Bf:
            continue
        T, N = 3, 2
        assert OL.allowed_mask(F, T, N, Bf).all(), (F, Bf)
        assert all(ivs == [(0, F * T + N)] for ivs in OL.key_intervals(F, T, N, Bf))


# ------------------------------------------------------------------- values


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _sdpa64(q, k, v, mask=None, scale=None):
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).permute(0, 2, 1, 3)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3)
    am = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=am, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


VALUE_SWEEP = [(1, 2, 8, 7, 6, 3, 2), (2, 1, 4, 11, 5, 4, 5), (1, 3, 16, 9, 4, 0, 3),
               (1, 1, 8, 1, 7, 2, 5), (1, 2, 8, 13, 2, 1, 1), (1, 1, 4, 16, 3, 5, 5)]


@pytest.mark.parametrize("B,H,D,F,T,N,Bf", VALUE_SWEEP)
def test_structured_equals_dense_masked(B, H, D, F, T, N, Bf):
    S = F * T + N
    q, k, v = (_rand((B, S, H, D), s) for s in (1, 2, 3))
    g = _rand((B, S, H), 4)
    mask = OL.allowed_mask(F, T, N, Bf)
    o1, l1 = OL.attend(q, k, v, g, F, T, N, Bf)
    o2, l2 = OL.attend_dense_masked(q, k, v, g, mask)
    assert np.abs(o1 - o2).max() <= 1e-12
    assert np.abs(l1 - l2).max() <= 1e-12


@pytest.mark.parametrize("B,H,D,F,T,N,Bf", VALUE_SWEEP)
def test_dense_masked_equals_torch_sdpa(B, H, D, F, T, N, Bf):
    S = F * T + N
    q, k, v = (_rand((B, S, H, D), s) for s in (5, 6, 7))
    mask = OL.allowed_mask(F, T, N, Bf)
    o1, _ = OL.attend_dense_masked(q, k, v, None, mask)
    o2 = _sdpa64(q, k, v, mask)
    assert np.abs(o1 - o2).max() <= 1e-12


@pytest.mark.parametrize("F,Bf", [(10, 5), (5, 5), (1, 5), (8, 4), (2, 1)])
def test_full_window_equals_torch_sdpa(F, Bf):
    B, H, D, T, N = 1, 2, 8, 4, 3
    S = F * T + N
    q, k, v = (_rand((B, S, H, D), s, 2.0) for s in (8, 9, 10))
    o1, l1 = OL.attend(q, k, v, None, F, T, N, Bf)
    o2 = _sdpa64(q, k, v)
    assert np.abs(o1 - o2).max() <= 1e-12
    # log-sum-exp against torch.logsumexp of the full score matrix
    s = torch.einsum("bshd,bthd->bhst", torch.from_numpy(q), torch.from_numpy(k)) / math.sqrt(D)
    assert np.abs(l1 - torch.logsumexp(s, dim=-1).numpy()).max() <= 1e-12


def test_zero_queries_average_frame_indicators():
    """q = 0 makes every visible key equally weighted, so with v a one-hot
    frame indicator (text in its own channel) the output is the fraction of
    visible keys in each frame, and the log-sum-exp is ln |K|.  Expected
    values are written out by hand for F=12, T=2, N=3, Bf=5 (blocks 0-4,
    5-9, 10-11; S = 27)."""
    F, T, N, Bf = 12, 2, 3, 5
    S, D = F * T + N, 16
    q = np.zeros((1, S, 1, D))
    k = _rand((1, S, 1, D), 11)
    v = np.zeros((1, S, 1, D))
    for t in range(S):
        v[0, t, 0, min(t // T, F)] = 1.0  # channel F = text
    o, lse = OL.attend(q, k, v, None, F, T, N, Bf)
    # block 0 (frames 0-4) sees frames 0-9, anchor 11, text: 11*2+3 = 25 keys
    # block 1 (frames 5-9) sees frames 0-11 and text: 27 keys
    # block 2 (frames 10-11) sees frames 5-11, anchor 0, text: 8*2+3 = 19 keys
    expect = {0: (25, list(range(10)) + [11]), 1: (27, list(range(12))), 2: (19, [0] + list(range(5, 12)))}
    for t in range(F * T):
        nk, frames = expect[(t // T) // Bf]
        row = np.zeros(D)
        for f in frames:
            row[f] = T / nk
        row[F] = N / nk
        assert np.abs(o[0, t, 0] - row).max() <= 1e-15, t
        assert abs(lse[0, 0, t] - math.log(nk)) <= 1e-14
    for t in range(F * T, S):  # text rows see all 27 keys
        row = np.zeros(D)
        row[:F] = T / S
        row[F] = N / S
        assert np.abs(o[0, t, 0] - row).max() <= 1e-15


def test_constant_values_and_gate_closed_forms():
    F, T, N, Bf = 13, 3, 2, 3
    S, D = F * T + N, 8
    q, k = _rand((1, S, 2, D), 12, 3.0), _rand((1, S, 2, D), 13)
    v = np.broadcast_to(np.arange(D, dtype=np.float64), (1, S, 2, D)).copy()
    o, _ = OL.attend(q, k, v, None, F, T, N, Bf)
    assert np.abs(o - v).max() <= 1e-12          # convex combination of equal rows
    g0 = np.zeros((1, S, 2))
    o0, _ = OL.attend(q, k, v, g0, F, T, N, Bf)
    assert np.abs(o0 - 0.5 * v).max() <= 1e-12   # sigmoid(0) = 1/2
    g = np.full((1, S, 2), math.log(3.0))
    o3, _ = OL.attend(q, k, v, g, F, T, N, Bf)
    assert np.abs(o3 - 0.75 * v).max() <= 1e-12  # sigmoid(ln 3) = 3/4


def needle_rows(F, T, N, Bf):
    """Hand-picked (query token, key token, visible?) triples for F=20,
    T=6, N=4, Bf=5 (blocks of frames 0-4, 5-9, 10-14, 15-19)."""
    tok = lambda f, j=0: f * T + j  # noqa: E731
    V = F * T
    return [
        (tok(2), tok(9, 5), True),     # last key of the window of block 0
        (tok(2, 1), tok(10), False),   # first key after block 0's window
        (tok(2, 2), tok(19, 3), True), # last-frame anchor
        (tok(2, 3), tok(18, 5), False),# just before the anchor
        (tok(7), tok(0), True),        # block 1 window starts at frame 0
        (tok(7, 1), tok(14, 5), True), # block 1 window end
        (tok(7, 2), tok(15), False),   # first key after block 1's window
        (tok(12), tok(4, 5), False),   # just before block 2's window
        (tok(12, 1), tok(5), True),    # first key of block 2's window
        (tok(12, 2), tok(0, 5), True), # first-frame anchor
        (tok(12, 3), tok(1), False),   # just after the anchor
        (tok(17), tok(9, 5), False),   # block 3: frames 10.. only
        (tok(17, 1), tok(10), True),
        (tok(19), tok(5), False),      # anchor frame query keeps its block rule
        (tok(19, 1), V, True),         # first text token
        (tok(0), V + N - 1, True),     # last text token
        (V, tok(12, 3), True),         # text queries see everything
        (V + 1, tok(19, 5), True),
    ]


def test_needle_probes():
    """q_i = alpha * k_j gives query i a score far above all others at key j:
    the output is then v_j when j is visible and something else when not."""
    F, T, N, Bf = 20, 6, 4, 5
    S, D, alpha = F * T + N, 64, 4.0
    k = _rand((1, S, 1, D), 14)
    v = _rand((1, S, 1, D), 15)
    q = np.zeros((1, S, 1, D))
    triples = needle_rows(F, T, N, Bf)
    for i, j, _ in triples:
        q[0, i, 0] = alpha * k[0, j, 0]
    o, _ = OL.attend(q, k, v, None, F, T, N, Bf)
    for i, j, visible in triples:
        err = np.abs(o[0, i, 0] - v[0, j, 0]).max()
        if visible:
            assert err < 1e-3, (i, j, err)
        else:
            assert err > 0.5, (i, j, err)


def test_dequantize_fp8_exact():
    codes = torch.tensor([448.0, -0.001953125, 1.5, 0.0]).to(torch.float8_e4m3fn)
    c64 = codes.to(torch.float64).numpy().reshape(1, 1, 1, 4)
    s = np.array([np.float32(0.1)], dtype=np.float32)
    out = OL.dequantize_fp8(c64, s)
    # hand: 448*fl32(0.1), -2^-9*fl32(0.1), 1.5*fl32(0.1), 0
    s64 = float(np.float32(0.1))
    assert out.ravel().tolist() == [448 * s64, -(2.0 ** -9) * s64, 1.5 * s64, 0.0]


# ---------------------------------------------------------- mutation tests


def _shifted_window(beta, F, Bf):
    lo = Bf * max(0, beta)      # window starts at the block itself
    hi = min(F, Bf * (beta + 2))
    return lo, hi


def _no_anchor_intervals(F, T, N, Bf):
    out = []
    for beta in range(OL.num_frame_blocks(F, Bf)):
        lo, hi = OL.window_frames(beta, F, Bf)
        out.append(OL._merge([(lo * T, hi * T), (F * T, F * T + N)]))
    if N > 0:
        out.append([(0, F * T + N)])
    return out


def _no_text_intervals(F, T, N, Bf):
    out = []
    for beta in range(OL.num_frame_blocks(F, Bf)):
        lo, hi = OL.window_frames(beta, F, Bf)
        out.append(OL._merge([(lo * T, hi * T), (0, T), ((F - 1) * T, F * T)]))
    if N > 0:
        out.append([(0, F * T + N)])
    return out


def _value_pins():
    test_structured_equals_dense_masked(*VALUE_SWEEP[1])
    test_needle_probes()


@pytest.mark.parametrize("mutant", ["shift_window", "drop_anchor", "drop_text", "no_gate",
                                    "wrong_scale", "no_max_shift"])
def test_mutants_are_caught(monkeypatch, golden, mutant):
    if mutant == "shift_window":
        monkeypatch.setattr(OL, "window_frames", _shifted_window)
        checks = [lambda: check_intervals_golden(golden), lambda: check_counts_golden(golden), _value_pins]
    elif mutant == "drop_anchor":
        monkeypatch.setattr(OL, "key_intervals", _no_anchor_intervals)
        checks = [lambda: check_intervals_golden(golden), _value_pins]
    elif mutant == "drop_text":
        monkeypatch.setattr(OL, "key_intervals", _no_text_intervals)
        checks = [lambda: check_intervals_golden(golden), _value_pins]
    elif mutant == "no_gate":
        monkeypatch.setattr(OL, "sigmoid", lambda g: np.ones_like(np.asarray(g, dtype=np.float64)))
        checks = [test_constant_values_and_gate_closed_forms]
    elif mutant == "wrong_scale":
        orig = OL.attend

        def bad(q, k, v, gate, F, T, N, Bf, scale=None, **kw):
            return orig(q, k, v, gate, F, T, N, Bf, scale=1.0 / np.asarray(q).shape[-1], **kw)
        monkeypatch.setattr(OL, "attend", bad)
        checks = [lambda: test_full_window_equals_torch_sdpa(10, 5)]
    elif mutant == "no_max_shift":
        # dropping the +m in the log-sum-exp
        orig = OL._softmax_rows

        def bad(s):
            p, l = orig(s)
            return p, l - s.max(axis=1)
        monkeypatch.setattr(OL, "_softmax_rows", bad)
        checks = [lambda: test_full_window_equals_torch_sdpa(10, 5)]
    caught = 0
    for c in checks:
        try:
            c()
        except AssertionError:
            caught += 1
    assert caught >= 1, mutant
