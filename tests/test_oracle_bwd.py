"""Pins for the backward part of the CPU oracle (``key_blocks`` and
``attend_backward``).  Each check compares the oracle with something other
than itself: a column scan of the explicit mask, torch autograd (float64)
through dense masked attention, central finite differences, and closed
forms.  The mutation tests at the end plant plausible mistakes in the
backward oracle and check that at least one pin catches each."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import local_attn as OL

# ---------------------------------------------------------------- key side

KB_SWEEP = [(F, T, N, Bf)
            for F in (1, 2, 3, 5, 6, 10, 11, 12, 20, 21)
            for T in (1, 3, 8)
            for N in (0, 1, 5)
            for Bf in (1, 2, 5, 7)]


@pytest.mark.parametrize("F,T,N,Bf", KB_SWEEP)
def test_key_blocks_equal_mask_columns(F, T, N, Bf):
    mask = OL.allowed_mask(F, T, N, Bf)
    S = F * T + N
    seen = np.zeros(S, dtype=int)
    for keys, qivs in oracle.key_blocks(F, T, N, Bf):
        rows = np.zeros(S, dtype=bool)
        for a, b in qivs:
            rows[a:b] = True
        for a, b in keys:
            assert a < b
            for j in range(a, b):
                seen[j] += 1
                assert np.array_equal(mask[:, j], rows), (j, keys, qivs)
    assert np.all(seen == 1)  # the groups partition the keys


def test_key_blocks_768p_hand_derived():
    # frame blocks of 5 frames x 1008 tokens, anchors 0 and 19, text after
    # 20160: block 0 keeps frames 1-4, block 3 frames 15-18
    kb = oracle.key_blocks(20, 1008, 512, 5)
    assert kb == [
        ([(1008, 5040)], [(0, 10080), (20160, 20672)]),
        ([(5040, 10080)], [(0, 15120), (20160, 20672)]),
        ([(10080, 15120)], [(5040, 20672)]),
        ([(15120, 19152)], [(10080, 20672)]),
        ([(0, 1008), (19152, 20672)], [(0, 20672)]),
    ]


# ------------------------------------------------------------------ values


def _inputs(seed, B, H, D, F, T, N, gate=True, scale_v=1.0):
    rng = np.random.default_rng(seed)
    S = F * T + N
    q = rng.standard_normal((B, S, H, D))
    k = rng.standard_normal((B, S, H, D))
    v = rng.standard_normal((B, S, H, D)) * scale_v
    g = rng.standard_normal((B, S, H)) if gate else None
    do = rng.standard_normal((B, S, H, D))
    return q, k, v, g, do


def _torch_grads(q, k, v, g, do, mask, scale):
    """Autograd of dense masked attention (float64): an independent route to
    the same derivatives."""
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    tg = None if g is None else torch.tensor(g, dtype=torch.float64, requires_grad=True)
    m = torch.tensor(mask)
    s = torch.einsum("bihd,bjhd->bhij", tq, tk) * scale
    s = s.masked_fill(~m, float("-inf"))
    p = torch.softmax(s, dim=-1)
    o = torch.einsum("bhij,bjhd->bihd", p, tv)
    if tg is not None:
        o = o * torch.sigmoid(tg)[..., None]
    o.backward(torch.tensor(do, dtype=torch.float64))
    return (tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy(),
            None if tg is None else tg.grad.numpy())


BWD_SWEEP = [
    # (seed, B, H, D, F, T, N, Bf, gate, scale)
    (1, 1, 2, 8, 11, 4, 3, 5, True, None),
    (2, 2, 1, 16, 7, 5, 0, 2, False, None),
    (3, 1, 1, 4, 1, 6, 2, 5, True, 0.7),
    (4, 1, 2, 8, 13, 3, 5, 3, True, None),
    (5, 1, 1, 8, 20, 2, 4, 5, True, None),
    (6, 1, 1, 8, 6, 4, 9, 1, False, 0.25),
]


@pytest.mark.parametrize("case", BWD_SWEEP)
def test_backward_equals_torch_autograd(case):
    seed, B, H, D, F, T, N, Bf, gate, scale = case
    q, k, v, g, do = _inputs(seed, B, H, D, F, T, N, gate)
    mask = OL.allowed_mask(F, T, N, Bf)
    sc = scale if scale else 1.0 / math.sqrt(D)
    dq, dk, dv, dg = oracle.attend_backward(q, k, v, g, do, F, T, N, Bf, scale=scale)
    tq, tk, tv, tg = _torch_grads(q, k, v, g, do, mask, sc)
    np.testing.assert_allclose(dq, tq, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dk, tk, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dv, tv, rtol=1e-10, atol=1e-11)
    if gate:
        np.testing.assert_allclose(dg, tg, rtol=1e-10, atol=1e-11)
    else:
        assert dg is None


def test_backward_equals_finite_differences():
    # directional derivatives of L = sum(dout * out) along random directions,
    # by central differences of the forward oracle (no autograd involved)
    F, T, N, Bf, D = 7, 3, 2, 2, 4
    q, k, v, g, do = _inputs(11, 1, 1, D, F, T, N, True)
    dq, dk, dv, dg = oracle.attend_backward(q, k, v, g, do, F, T, N, Bf)

    def loss(q_, k_, v_, g_):
        o, _ = oracle.attend(q_, k_, v_, g_, F, T, N, Bf)
        return float(np.sum(o * do))

    rng = np.random.default_rng(12)
    eps = 1e-5
    for name, grad in (("q", dq), ("k", dk), ("v", dv), ("g", dg)):
        for _ in range(3):
            args = {"q": q, "k": k, "v": v, "g": g}
            dirn = rng.standard_normal(args[name].shape)
            plus = dict(args)
            minus = dict(args)
            plus[name] = args[name] + eps * dirn
            minus[name] = args[name] - eps * dirn
            fd = (loss(plus["q"], plus["k"], plus["v"], plus["g"])
                  - loss(minus["q"], minus["k"], minus["v"], minus["g"])) / (2 * eps)
            an = float(np.sum(grad * dirn))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_constant_values_give_zero_score_gradients():
    # v_j identical for every key: the output does not depend on the
    # weights, so dq = dk = 0 exactly (up to rounding), and each key's dv is
    # its share of the weights times the upstream gradient
    F, T, N, Bf, D = 11, 4, 3, 5, 8
    q, k, _, g, do = _inputs(21, 1, 1, D, F, T, N, True)
    S = F * T + N
    v = np.broadcast_to(np.linspace(-1, 1, D), (1, S, 1, D)).copy()
    dq, dk, dv, dg = oracle.attend_backward(q, k, v, g, do, F, T, N, Bf)
    assert np.max(np.abs(dq)) < 1e-12 and np.max(np.abs(dk)) < 1e-12
    # gate: out = sg * v, so dg = (do . v) sg (1 - sg)
    sg = 1 / (1 + np.exp(-g[0, :, 0]))
    np.testing.assert_allclose(dg[0, :, 0], (do[0, :, 0, :] @ v[0, 0, 0, :]) * sg * (1 - sg), rtol=1e-12)


def test_zero_queries_spread_dv_evenly():
    # q = 0: every query weighs its |K(i)| keys equally, so
    # dv_j = sum over the queries i that see j of da_i / |K(i)|, written here
    # from the explicit mask
    F, T, N, Bf, D = 10, 3, 4, 2, 6
    _, k, v, g, do = _inputs(31, 1, 1, D, F, T, N, True)
    S = F * T + N
    q = np.zeros((1, S, 1, D))
    dq, dk, dv, dg = oracle.attend_backward(q, k, v, g, do, F, T, N, Bf)
    mask = OL.allowed_mask(F, T, N, Bf).astype(np.float64)
    sg = 1 / (1 + np.exp(-g[0, :, 0]))
    da = do[0, :, 0, :] * sg[:, None]
    w = mask / mask.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(dv[0, :, 0, :], w.T @ da, rtol=1e-12, atol=1e-14)
    # with q = 0 the key gradients vanish (they are scale * ds^T q)
    assert np.max(np.abs(dk)) == 0.0


def test_key_gradients_sum_to_zero():
    # every softmax row's ds sums to zero, so sum_j dk_j = scale sum_i
    # (sum_j ds_ij) q_i = 0 for each (sample, head)
    F, T, N, Bf, D = 13, 3, 5, 3, 8
    q, k, v, g, do = _inputs(41, 2, 2, D, F, T, N, True)
    _, dk, _, _ = oracle.attend_backward(q, k, v, g, do, F, T, N, Bf)
    tot = dk.sum(axis=1)
    assert np.max(np.abs(tot)) < 1e-10 * max(1.0, np.max(np.abs(dk)))


def test_row_and_head_sampling_matches_full():
    F, T, N, Bf, D = 12, 5, 4, 3, 8
    q, k, v, g, do = _inputs(51, 2, 3, D, F, T, N, True)
    full = oracle.attend_backward(q, k, v, g, do, F, T, N, Bf)
    rows = np.array([0, 3, 14, 15, 31, 40, 59, 60, 63])
    part = oracle.attend_backward(q, k, v, g, do, F, T, N, Bf, rows=rows, heads=[1, 2])
    for x, y in ((full[0], part[0]), (full[3], part[3])):
        np.testing.assert_allclose(x[:, rows][:, :, [1, 2]], y[:, rows][:, :, [1, 2]], rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------- mutation tests


def _pins():
    test_backward_equals_torch_autograd(BWD_SWEEP[0])
    test_constant_values_give_zero_score_gradients()
    test_zero_queries_spread_dv_evenly()
    test_key_gradients_sum_to_zero()


@pytest.mark.parametrize("mutant", ["no_centering", "gate_not_in_dv", "dgate_sign", "wrong_scale",
                                    "key_blocks_no_text"])
def test_backward_mutants_are_caught(monkeypatch, mutant):
    if mutant == "no_centering":
        monkeypatch.setattr(OL, "_softmax_backward", lambda p, dp: p * dp)
        checks = [_pins]
    elif mutant == "gate_not_in_dv":
        orig = OL._gate_backward

        def bad(do, a, sg):
            _, dg = orig(do, a, sg)
            return do, dg
        monkeypatch.setattr(OL, "_gate_backward", bad)
        checks = [_pins]
    elif mutant == "dgate_sign":
        monkeypatch.setattr(OL, "_gate_backward",
                            lambda do, a, sg: (do * sg[:, None], np.sum(do * a, axis=1) * sg * (1.0 + sg)))
        checks = [_pins]
    elif mutant == "wrong_scale":
        orig = OL.attend_backward

        def bad(q, k, v, gate, dout, F, T, N, Bf, scale=None, **kw):
            return orig(q, k, v, gate, dout, F, T, N, Bf, scale=1.0 / np.asarray(q).shape[-1], **kw)
        monkeypatch.setattr(oracle, "attend_backward", bad)
        checks = [_pins]
    elif mutant == "key_blocks_no_text":
        orig = OL.key_blocks

        def bad(F, T, N, Bf):
            V = F * T
            return [(keys, [iv for iv in qivs if iv[1] <= V] or qivs) for keys, qivs in orig(F, T, N, Bf)]
        monkeypatch.setattr(oracle, "key_blocks", bad)
        checks = [lambda: test_key_blocks_equal_mask_columns(11, 3, 5, 5),
                  test_key_blocks_768p_hand_derived]
    caught = 0
    for c in checks:
        try:
            c()
        except AssertionError:
            caught += 1
    assert caught >= 1, mutant
