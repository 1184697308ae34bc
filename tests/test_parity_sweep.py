"""Seeded sweep of small random shapes through the GPU entry points (softmax
forward and backward, linear branch, the hybrid output in one call), each
compared in full with the oracle: batches of one or two samples, one to five
heads, both head sizes, ragged frames, videos shorter than a block, no text
or more text than video, one-frame blocks.  Shapes this small give each XCD
only a few tiles, so every one also runs the dealt tile order and the half
tiles."""

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_31_amd import binding as B
from block_sparse_attention_31_amd import synth

from .gpu_util import BF16_LSE_BOUND, compare, gpu_available, oracle_inputs, run_gpu
from .test_parity_bwd import _oracle as bwd_oracle
from .test_parity_bwd import check as bwd_check
from .test_parity_bwd import run_bwd
from .test_parity_linear import DEV
from .test_parity_linear import check as lin_check
from .test_parity_linear import inputs as lin_inputs
from .test_parity_linear import oracle_linear, run_linear, zero_rows

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _shapes(n, seed, max_s):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        F = int(rng.integers(1, 15))
        T = int(rng.choice([1, 2, 7, 16, 33, 48, 64, 70]))
        N = int(rng.choice([0, 0, 1, 5, 40, 130]))
        if F * T + N > max_s:
            continue
        out.append(dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 6)),
                        D=int(rng.choice([64, 128])), F=F, T=T, N=N,
                        Bf=int(rng.integers(1, 7)), gate=bool(rng.integers(0, 2))))
    return out


FWD = _shapes(40, 9001, 700)
BWD = _shapes(20, 9002, 500)
LIN = _shapes(20, 9003, 700)
HYB = _shapes(20, 9004, 600)


def _name(s):
    return "B{B}H{H}D{D}F{F}T{T}N{N}Bf{Bf}g{gate:d}".format(**s)


@pytest.mark.parametrize("s", FWD, ids=[_name(s) for s in FWD])
def test_sweep_forward(s):
    w = synth.random_workload(seed=9100 + len(_name(s)) * 7 + s["F"] * 13 + s["T"], **s)
    inp = synth.make_inputs(w)
    og, lg = run_gpu(inp, w)
    orf, lrf = oracle.attend(*oracle_inputs(inp), w.F, w.T, w.N, w.Bf)
    # rows with a handful of keys: the bf16 rounding of each weight does not
    # average out in the row sum, so the log-sum-exp gets its rigorous bound
    compare(og, lg, orf, lrf, lse_tol=BF16_LSE_BOUND)


@pytest.mark.parametrize("s", BWD, ids=[_name(s) for s in BWD])
def test_sweep_backward(s):
    w = synth.random_workload(seed=9200 + s["F"] * 13 + s["T"], **s)
    inp = synth.make_inputs(w)
    dout = synth.make_dout(w)
    bwd_check(_name(s), run_bwd(inp, dout, w), bwd_oracle(inp, dout, w))


@pytest.mark.parametrize("s", LIN, ids=[_name(s) for s in LIN])
def test_sweep_linear(s):
    w = synth.random_workload(seed=9300 + s["F"] * 13 + s["T"], **{**s, "gate": False})
    q, k, v = lin_inputs(w)
    got = run_linear(q, k, v, w)
    ref = oracle_linear(q, k, v, w)
    assert np.all(got[:, zero_rows(w)] == 0.0)
    if np.any(ref != 0):
        lin_check(_name(s), got, ref)
    else:
        assert np.all(got == 0.0)


@pytest.mark.parametrize("s", HYB, ids=[_name(s) for s in HYB])
def test_sweep_hybrid_one_call(s):
    w = synth.random_workload(seed=9400 + s["F"] * 13 + s["T"], **s)
    inp = synth.make_inputs(w)
    v = synth.with_frame_offsets(inp["v"], w.F, w.T, 0.2)
    fi = synth.make_fuse_inputs(w)
    q, k, vd = (t.to(DEV) for t in (inp["q"], inp["k"], v))
    g = None if inp["gate"] is None else inp["gate"].to(DEV)
    out = B.hybrid_attn_fwd(q, k, vd, g, fi["gate"].to(DEV), fi["weight"].to(DEV), F=w.F,
                            tokens_per_frame=w.T, n_text=w.N, block_frames=w.Bf, eps=1e-6)
    torch.cuda.synchronize()
    qn, kn, vn, gn = oracle_inputs({"q": inp["q"], "k": inp["k"], "v": v, "gate": inp["gate"], "scales": None})
    soft_ref, _ = oracle.attend(qn, kn, vn, gn, w.F, w.T, w.N, w.Bf)
    lin_ref = oracle.linear_branch(qn, kn, vn, w.F, w.T, w.N, w.Bf)
    ref = oracle.hybrid_fuse(soft_ref, lin_ref, fi["gate"].to(torch.float64).numpy(),
                             fi["weight"].to(torch.float64).numpy(), 1e-6)
    lin_check(_name(s), out.cpu().to(torch.float64).numpy(), ref)
