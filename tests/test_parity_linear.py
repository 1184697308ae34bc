"""GPU parity of the complement linear branch and the two-branch fusion
(through the C ABI) against the CPU oracle, on the same seeded inputs.

The bar is relative: with N(0, 1) values the linear branch averages some
thousands of keys, so its outputs are small and absolute bars would say
little.  Per tensor: relative L2 error at most 1e-2, and no element off by
more than 2e-2 of the reference's largest magnitude.  Derivation: phi(q),
phi(k) and the block state are rounded to bf16 (relative 2^-9 each, averaged
over D channels and thousands of keys, and the normaliser uses the same
rounded phi(q)); the output is rounded to bf16 (2^-9 = 2e-3 of each value).
The fusion rounds only its output (and reads bf16 inputs exactly)."""

import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_31_amd import binding as B
from block_sparse_attention_31_amd import synth

from .gpu_util import gpu_available, oracle_inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

REL_L2 = 1e-2
MAX_OVER_PEAK = 2e-2
DEV = torch.device("cuda:0")


def _log(name, stats):
    print(f"[linear-parity] {name}: " + ", ".join(f"{k}={v:.3g}" for k, v in stats.items()), flush=True)


def check(name, got, ref):
    assert np.all(np.isfinite(got)), name
    err = got - ref
    peak = float(np.max(np.abs(ref)))
    stats = {"rel_l2": float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300)),
             "max/peak": float(np.max(np.abs(err))) / max(peak, 1e-300), "peak": peak}
    _log(name, stats)
    assert stats["rel_l2"] <= REL_L2, (name, stats)
    assert stats["max/peak"] <= MAX_OVER_PEAK, (name, stats)
    return stats


def run_linear(q, k, v, w: synth.Workload, ws=None, stream=None):
    """GPU linear branch; out starts as NaN and the workspace as 0xFF bytes,
    so unwritten outputs and reads of stale workspace show."""
    q, k, v = (t.to(DEV) for t in (q, k, v))
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    if ws is None:
        n = B.vdn_linear_branch_workspace_bytes(w.F, w.T, w.N, w.Bf, w.H, w.D, w.B)
        ws = torch.full((max(n, 1),), 255, dtype=torch.uint8, device=DEV)
    B.vdn_linear_branch_fwd(q, k, v, out, w.F, w.T, w.N, w.Bf, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    return out.cpu().to(torch.float64).numpy()


def inputs(w, offset=0.3):
    inp = synth.make_inputs(w)
    v = synth.with_frame_offsets(inp["v"], w.F, w.T, offset) if offset else inp["v"]
    return inp["q"], inp["k"], v


def oracle_linear(q, k, v, w, heads=None):
    qn, kn, vn = (t.to(torch.float64).numpy() for t in (q, k, v))
    if heads is not None:
        qn, kn, vn = (x[:, :, heads] for x in (qn, kn, vn))
    return oracle.linear_branch(qn, kn, vn, w.F, w.T, w.N, w.Bf)


def zero_rows(w):
    """Rows with no linear keys: text rows and rows of blocks whose
    complement is empty (from the oracle's key-frame lists)."""
    rows = [np.arange(w.F * w.T, w.S)]
    for beta in range(oracle.num_frame_blocks(w.F, w.Bf)):
        if not oracle.linear_key_frames(beta, w.F, w.Bf):
            rows.append(np.arange(beta * w.Bf * w.T, min(w.F, (beta + 1) * w.Bf) * w.T))
    return np.concatenate(rows)


# ----------------------------------------------------------- linear branch


def test_tiny_linear():
    # 11 frames in blocks of 5: blocks 0 and 1 have no key outside their
    # windows but the anchor, block 2 (frame 10) sums frames 1-4
    w = synth.WORKLOADS["tiny"]
    q, k, v = inputs(w)
    got = run_linear(q, k, v, w)
    ref = oracle_linear(q, k, v, w)
    zr = zero_rows(w)
    assert np.all(got[:, zr] == 0.0)
    assert np.all(ref[:, zr] == 0.0)
    check("tiny", got, ref)


SHAPES = [
    # (B, H, D, F, T, N, Bf)
    (1, 2, 128, 20, 48, 16, 5),
    (2, 1, 64, 13, 17, 3, 3),     # ragged frames (17 tokens), two samples
    (1, 3, 128, 21, 33, 0, 5),    # ragged last block of one frame, no text
    (1, 1, 64, 7, 100, 5, 1),     # one frame per block
    (1, 2, 64, 12, 1, 2, 2),      # one token per frame
    (1, 1, 128, 3, 40, 4, 5),     # a single block: no key outside the window
    (1, 1, 64, 2, 16, 4, 1),      # anchors only
    (1, 1, 128, 1, 9, 0, 5),      # one frame
    (1, 2, 128, 16, 257, 7, 4),   # tiles of 512 rows within 4-frame blocks
    (2, 2, 64, 42, 8, 5, 5),      # the long-video frame structure, small frames
    (1, 1, 64, 315, 2, 4, 5),     # 63 frame blocks
]


@pytest.mark.parametrize("Bt,H,D,F,T,N,Bf", SHAPES)
def test_linear_shapes(Bt, H, D, F, T, N, Bf):
    w = synth.random_workload(700 + F * 31 + T, B=Bt, H=H, D=D, F=F, T=T, N=N, Bf=Bf, gate=False)
    q, k, v = inputs(w)
    got = run_linear(q, k, v, w)
    ref = oracle_linear(q, k, v, w)
    zr = zero_rows(w)
    assert np.all(got[:, zr] == 0.0)
    if np.any(ref != 0):
        check(f"shape B{Bt} H{H} D{D} F{F} T{T} N{N} Bf{Bf}", got, ref)
    else:
        assert np.all(got == 0.0)


def test_constant_values_pass_through():
    # every key carries the same value vector c: rows with linear keys
    # return c (up to the bf16 roundings of state and output)
    w = synth.random_workload(711, B=1, H=2, D=128, F=20, T=64, N=8, Bf=5, gate=False)
    inp = synth.make_inputs(w)
    c = torch.linspace(-3, 3, w.D)
    v = c.expand(w.B, w.S, w.H, w.D).contiguous().to(torch.bfloat16)
    got = run_linear(inp["q"], inp["k"], v, w)
    cv = v[0, 0, 0].to(torch.float64).numpy()
    rows = np.arange(w.F * w.T)
    np.testing.assert_allclose(got[0, rows], np.broadcast_to(cv, got[0, rows].shape), rtol=8e-3, atol=2e-2)
    assert np.all(got[0, w.F * w.T:] == 0.0)


def test_outliers_and_offsets_medium():
    # medium shape, 2% outlier channels x8 in q, k and v, frame offsets in v
    w = synth.WORKLOADS["medium"]
    q, k, v = inputs(w, offset=0.1)
    got = run_linear(q, k, v, w)
    heads = [0, 7, 15]
    ref = oracle_linear(q, k, v, w, heads=heads)
    check("medium", got[:, :, heads], ref)


@pytest.mark.parametrize("name,heads", [("768p", [0, 13, 31]), ("long", [0, 31])])
def test_workload_heads(name, heads):
    # the full-size launch (all heads), checked against the oracle on some
    # heads in full; N(0,1) values as the benchmark uses
    w = synth.WORKLOADS[name]
    q, k, v = inputs(w, offset=0.0)
    got = run_linear(q, k, v, w)
    ref = oracle_linear(q, k, v, w, heads=heads)
    check(name, got[:, :, heads], ref)
    assert np.all(got[:, zero_rows(w)] == 0.0)
    assert np.all(np.isfinite(got))


def test_workspace_reuse_and_stream():
    # one workspace for two shapes in a row (the second smaller), on a side
    # stream; results equal fresh-workspace runs bit for bit
    w1 = synth.random_workload(721, B=1, H=4, D=128, F=20, T=96, N=8, Bf=5, gate=False)
    w2 = synth.random_workload(722, B=1, H=2, D=64, F=9, T=40, N=3, Bf=2, gate=False)
    n = max(B.vdn_linear_branch_workspace_bytes(w.F, w.T, w.N, w.Bf, w.H, w.D, w.B) for w in (w1, w2))
    ws = torch.full((n,), 255, dtype=torch.uint8, device=DEV)
    s = torch.cuda.Stream()
    for w in (w1, w2):
        q, k, v = inputs(w)
        a = run_linear(q, k, v, w, ws=ws, stream=s.cuda_stream)
        b = run_linear(q, k, v, w)
        assert np.array_equal(a, b)


def test_deterministic():
    w = synth.random_workload(731, B=1, H=2, D=128, F=16, T=200, N=8, Bf=5, gate=False)
    q, k, v = inputs(w)
    assert np.array_equal(run_linear(q, k, v, w), run_linear(q, k, v, w))


def test_bad_arguments_raise():
    w = synth.random_workload(741, B=1, H=2, D=64, F=9, T=16, N=3, Bf=2, gate=False)
    q, k, v = (t.to(DEV) for t in inputs(w))
    out = torch.empty_like(q)
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(B.VdnError):
        B.vdn_linear_branch_fwd(q, k, v, out, w.F, w.T, w.N, w.Bf, workspace=small)
    n = B.vdn_linear_branch_workspace_bytes(w.F, w.T, w.N, w.Bf, w.H, w.D, w.B)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    with pytest.raises(B.VdnError):
        B.vdn_linear_branch_fwd(q, k, v, q, w.F, w.T, w.N, w.Bf, workspace=ws)


# ------------------------------------------------------------------ fusion


def run_fuse(fi, eps, in_place=False):
    soft = fi["soft"].to(DEV)
    lin, gate, weight = fi["lin"].to(DEV), fi["gate"].to(DEV), fi["weight"].to(DEV)
    out = soft if in_place else torch.full_like(soft, float("nan"))
    B.vdn_hybrid_fuse(soft, lin, gate, weight, out, eps)
    torch.cuda.synchronize()
    return out.cpu().to(torch.float64).numpy()


def oracle_fuse(fi, eps, rows=None):
    soft, lin = (fi[n].to(torch.float64).numpy() for n in ("soft", "lin"))
    gate, weight = fi["gate"].to(torch.float64).numpy(), fi["weight"].to(torch.float64).numpy()
    if rows is not None:
        soft, lin, gate = soft[:, rows], lin[:, rows], gate[:, rows]
    return oracle.hybrid_fuse(soft, lin, gate, weight, eps)


@pytest.mark.parametrize("H,D", [(2, 64), (3, 64), (32, 128), (5, 8), (64, 128)])
def test_fuse_shapes(H, D):
    w = synth.random_workload(751 + H + D, B=2, H=H, D=D, F=3, T=5, N=7, Bf=2)
    fi = synth.make_fuse_inputs(w)
    for eps in (1e-6, 0.25):
        check(f"fuse H{H} D{D} eps{eps}", run_fuse(fi, eps), oracle_fuse(fi, eps))


def test_fuse_768p_in_place():
    w = synth.WORKLOADS["768p"]
    fi = synth.make_fuse_inputs(w)
    rng = np.random.default_rng(5)
    rows = np.sort(np.concatenate([[0, 1, w.S - 1], rng.integers(0, w.S, 400)]))
    got = run_fuse(fi, 1e-6, in_place=True)
    check("fuse 768p in place", got[:, rows], oracle_fuse(fi, 1e-6, rows=rows))


def test_fuse_zero_linear_output_keeps_softmax_branch():
    # lin_out = 0 with eps > 0: out = soft_out exactly
    w = synth.random_workload(761, B=1, H=4, D=64, F=3, T=5, N=2, Bf=2)
    fi = synth.make_fuse_inputs(w)
    fi["lin"] = torch.zeros_like(fi["lin"])
    got = run_fuse(fi, 1e-6)
    assert np.array_equal(got, fi["soft"].to(torch.float64).numpy())


# ------------------------------------------------------- the hybrid layer


def test_hybrid_end_to_end():
    # gated softmax branch, linear branch and fusion on the GPU, against the
    # oracle's attend, linear_branch and hybrid_fuse chained in fp64
    w = synth.random_workload(771, B=1, H=2, D=128, F=16, T=40, N=12, Bf=5, gate=True)
    inp = synth.make_inputs(w)
    v = synth.with_frame_offsets(inp["v"], w.F, w.T, 0.2)
    fi = synth.make_fuse_inputs(w)
    q, k, vd, g = (t.to(DEV) for t in (inp["q"], inp["k"], v, inp["gate"]))
    soft = B.local_attn_fwd(q, k, vd, g, F=w.F, tokens_per_frame=w.T, n_text=w.N, block_frames=w.Bf)
    lin = B.linear_branch_fwd(q, k, vd, F=w.F, tokens_per_frame=w.T, n_text=w.N, block_frames=w.Bf)
    out = B.hybrid_fuse(soft, lin, fi["gate"].to(DEV), fi["weight"].to(DEV), 1e-6)
    torch.cuda.synchronize()
    qn, kn, vn, gn = oracle_inputs({"q": inp["q"], "k": inp["k"], "v": v, "gate": inp["gate"], "scales": None})
    soft_ref, _ = oracle.attend(qn, kn, vn, gn, w.F, w.T, w.N, w.Bf)
    lin_ref = oracle.linear_branch(qn, kn, vn, w.F, w.T, w.N, w.Bf)
    ref = oracle.hybrid_fuse(soft_ref, lin_ref, fi["gate"].to(torch.float64).numpy(),
                             fi["weight"].to(torch.float64).numpy(), 1e-6)
    check("hybrid end to end", out.cpu().to(torch.float64).numpy(), ref)
    assert math.isfinite(float(out.float().abs().max()))


@pytest.mark.parametrize("kw", [dict(B=1, H=2, D=128, F=16, T=40, N=12, Bf=5, gate=True),
                                dict(B=2, H=3, D=64, F=11, T=33, N=5, Bf=2, gate=False),
                                dict(B=1, H=4, D=128, F=3, T=20, N=40, Bf=1, gate=True)])
def test_hybrid_one_call(kw):
    # the whole hybrid output from vdn_hybrid_attn_fwd (fusion in the softmax
    # branch's epilogue) against the oracle chain, and against the three-call
    # path (which rounds the softmax branch before the sum); the workspace
    # starts as 0xFF bytes and out as NaN, so stale or unwritten data shows
    w = synth.random_workload(781 + kw["F"], **kw)
    inp = synth.make_inputs(w)
    v = synth.with_frame_offsets(inp["v"], w.F, w.T, 0.2)
    fi = synth.make_fuse_inputs(w)
    q, k, vd = (t.to(DEV) for t in (inp["q"], inp["k"], v))
    g = None if inp["gate"] is None else inp["gate"].to(DEV)
    gl, wt = fi["gate"].to(DEV), fi["weight"].to(DEV)
    n = B.vdn_hybrid_attn_workspace_bytes(w.F, w.T, w.N, w.Bf, w.H, w.D, w.B)
    ws = torch.full((n,), 255, dtype=torch.uint8, device=DEV)
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=DEV)
    B.vdn_hybrid_attn_fwd(q, k, vd, g, gl, wt, out, w.F, w.T, w.N, w.Bf, eps=1e-6, lse=lse, workspace=ws)
    soft = B.local_attn_fwd(q, k, vd, g, F=w.F, tokens_per_frame=w.T, n_text=w.N, block_frames=w.Bf)
    lin = B.linear_branch_fwd(q, k, vd, F=w.F, tokens_per_frame=w.T, n_text=w.N, block_frames=w.Bf)
    three = B.hybrid_fuse(soft, lin, gl, wt, 1e-6)
    torch.cuda.synchronize()
    got = out.cpu().to(torch.float64).numpy()
    qn, kn, vn, gn = oracle_inputs({"q": inp["q"], "k": inp["k"], "v": v, "gate": inp["gate"], "scales": None})
    soft_ref, lse_ref = oracle.attend(qn, kn, vn, gn, w.F, w.T, w.N, w.Bf)
    lin_ref = oracle.linear_branch(qn, kn, vn, w.F, w.T, w.N, w.Bf)
    ref = oracle.hybrid_fuse(soft_ref, lin_ref, fi["gate"].to(torch.float64).numpy(),
                             fi["weight"].to(torch.float64).numpy(), 1e-6)
    check("hybrid one call", got, ref)
    check("hybrid one call vs three calls", got, three.cpu().to(torch.float64).numpy())
    # the log-sum-exp output is the softmax branch's
    assert np.max(np.abs(lse.cpu().numpy() - lse_ref)) <= 2e-3


def _run_one_call(w, seed_offset_step=0.2):
    """vdn_hybrid_attn_fwd on a workload's inputs (v with per-frame offsets);
    returns the GPU output and log-sum-exp and the oracle's fp64 inputs."""
    inp = synth.make_inputs(w)
    v = synth.with_frame_offsets(inp["v"], w.F, w.T, seed_offset_step)
    fi = synth.make_fuse_inputs(w)
    q, k, vd = (t.to(DEV) for t in (inp["q"], inp["k"], v))
    g = None if inp["gate"] is None else inp["gate"].to(DEV)
    n = B.vdn_hybrid_attn_workspace_bytes(w.F, w.T, w.N, w.Bf, w.H, w.D, w.B)
    ws = torch.full((n,), 255, dtype=torch.uint8, device=DEV)
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=DEV)
    B.vdn_hybrid_attn_fwd(q, k, vd, g, fi["gate"].to(DEV), fi["weight"].to(DEV), out, w.F, w.T, w.N, w.Bf,
                          eps=1e-6, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    got = out.cpu().to(torch.float64).numpy()
    del q, k, vd, g, ws, out
    qn, kn, vn, gn = oracle_inputs({"q": inp["q"], "k": inp["k"], "v": v, "gate": inp["gate"], "scales": None})
    return got, lse.cpu().numpy(), (qn, kn, vn, gn), fi


def test_hybrid_one_call_768p_two_heads_full():
    # the size the one-call hybrid is benchmarked at: 32 heads (each token's
    # RMSNorm spans all of them in the fused prologue), whole 256-row tiles
    # (no half tiles at this size) and the peeled last step of every tile;
    # two heads compared element by element against attend -> linear_branch
    # (all 32 heads) -> hybrid_fuse
    w = synth.WORKLOADS["768p"]
    got, lse, (qn, kn, vn, gn), fi = _run_one_call(w)
    heads = [0, 31]
    soft_ref, lse_ref = oracle.attend(qn, kn, vn, gn, w.F, w.T, w.N, w.Bf, heads=heads)
    lin_ref = oracle.linear_branch(qn, kn, vn, w.F, w.T, w.N, w.Bf)
    ref = oracle.hybrid_fuse(soft_ref, lin_ref, fi["gate"].to(torch.float64).numpy(),
                             fi["weight"].to(torch.float64).numpy(), 1e-6)
    check("hybrid one call 768p heads 0,31", got[:, :, heads], ref[:, :, heads])
    assert np.max(np.abs(lse[:, heads] - lse_ref[:, heads])) <= 2e-3


def _in_tile_rows(w, tile=256):
    """Rows at both ends and across the middle of every 256-row tile of every
    query block (tile offsets 0, 1, 127, 128, 129, 200 and 255)."""
    rows = set()
    for lo, hi in oracle.query_blocks(w.F, w.T, w.N, w.Bf):
        for r0 in range(lo, hi, tile):
            rows.update(r for r in (r0, r0 + 1, r0 + 127, r0 + 128, r0 + 129, r0 + 200, r0 + 255) if r < hi)
        rows.update({hi - 2, hi - 1})
    return np.array(sorted(rows))


def test_hybrid_one_call_768p_h4_sampled():
    # one GPU's share of the 768p heads (4): most tiles run whole and the last
    # 16 tiles of each XCD share run as 128-row halves, so both the waves
    # staging rows 128..255 of a whole tile's linear output and the half
    # tiles are exercised; rows at every in-tile offset class of all 4 heads
    w = synth.WORKLOADS["768p-h4"]
    got, lse, (qn, kn, vn, gn), fi = _run_one_call(w)
    rows = _in_tile_rows(w)
    soft_ref, lse_ref = oracle.attend(qn, kn, vn, gn, w.F, w.T, w.N, w.Bf, rows=rows)
    lin_ref = oracle.linear_branch(qn, kn, vn, w.F, w.T, w.N, w.Bf)
    ref = oracle.hybrid_fuse(soft_ref, lin_ref, fi["gate"].to(torch.float64).numpy(),
                             fi["weight"].to(torch.float64).numpy(), 1e-6)
    check(f"hybrid one call 768p-h4, {rows.size} rows", got[:, rows], ref[:, rows])
    assert np.max(np.abs(lse[:, :, rows] - lse_ref[:, :, rows])) <= 2e-3
