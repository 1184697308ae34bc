"""Plain fp64 CPU oracle of the local Softmax branch of VDN-H3 attention,
its backward pass, the complement linear branch and the two-branch fusion.

TEST INFRASTRUCTURE ONLY: used by tests, the smoke check and the benchmark's
CPU-baseline leg.  Shares no code with the HIP path and imports nothing from
the product package.

What the branch computes, restated from the pages:

* openi.cn "VDN-MiniMax-H3", section "technical principles: local exact,
  remote compressed": latent frames are grouped five consecutive frames to a
  block; a block attends with exact softmax to itself and to the blocks right
  before and right after it; the first and last latent frames are boundary
  anchors, and the linear branch leaves out both the window frames and the
  anchors (so the softmax branch is the one that covers the anchors).
* nav.superapi.store "VDN-MiniMax-H3 - OpenVDN's Open-Source Video Generation
  Acceleration Solution", section "Technical Principles", items "Local
  Softmax Branch" (bidirectional block window, first/last frame anchors) and
  "Text Dual-Branch Injection" (in the softmax branch every frame sees all
  text tokens).
* Same two sections, "Gated Fusion" item: each branch output goes through a
  content-dependent sigmoid gate before the (separate) output projection.

Readings where the pages are silent (each listed in the design notes):

* blocks start at frame 0, the last block may be short;
* anchors are keys visible to every query (an anchor-frame *query* follows
  its own block's rule);
* text tokens sit after the F*T video tokens; text *queries* see every key;
* softmax scale 1/sqrt(D) unless given;
* the gate is one logit per (token, head), applied as o * sigmoid(g) after
  normalisation.

Token layout: token t < F*T belongs to frame t // T; tokens [F*T, F*T+N) are
text.  Tensors are [B, S, H, D] (sequence-major), gate [B, S, H], the
log-sum-exp [B, H, S].
"""

from __future__ import annotations

import math

import numpy as np

# --------------------------------------------------------------------------
# Key structure
# --------------------------------------------------------------------------


def num_frame_blocks(F: int, Bf: int) -> int:
    """Number of frame blocks: blocks of Bf consecutive frames from frame 0."""
    return -(-F // Bf)


def window_frames(beta: int, F: int, Bf: int) -> tuple[int, int]:
    """Half-open frame range [lo, hi) of block ``beta`` plus its two
    neighbouring blocks, clipped to the video (the bidirectional block window
    of the local softmax branch)."""
    lo = Bf * max(0, beta - 1)
    hi = min(F, Bf * (beta + 2))
    return lo, hi


def query_blocks(F: int, T: int, N: int, Bf: int) -> list[tuple[int, int]]:
    """Query row ranges: one per frame block, then one for the text tokens
    (omitted when N == 0)."""
    out = []
    for beta in range(num_frame_blocks(F, Bf)):
        f0 = beta * Bf
        f1 = min(F, f0 + Bf)
        out.append((f0 * T, f1 * T))
    V = F * T
    if N > 0:
        out.append((V, V + N))
    return out


def _merge(intervals):
    """Sort and merge touching or overlapping half-open intervals."""
    ivs = sorted((a, b) for a, b in intervals if b > a)
    merged: list[list[int]] = []
    for a, b in ivs:
        if merged and a <= merged[-1][1]:
            merged[-1][1] = max(merged[-1][1], b)
        else:
            merged.append([a, b])
    return [(a, b) for a, b in merged]


def key_intervals(F: int, T: int, N: int, Bf: int) -> list[list[tuple[int, int]]]:
    """Canonical key intervals per query block (same order as
    :func:`query_blocks`): sorted, disjoint, touching intervals merged.

    A video query of block beta sees the window frames, the two anchor frames
    (0 and F-1) and all text tokens.  A text query sees every token."""
    V = F * T
    S = V + N
    lists = []
    for beta in range(num_frame_blocks(F, Bf)):
        lo, hi = window_frames(beta, F, Bf)
        parts = [(lo * T, hi * T), (0, T), ((F - 1) * T, F * T), (V, S)]
        lists.append(_merge(parts))
    if N > 0:
        lists.append([(0, S)])
    return lists


def allowed_mask(F: int, T: int, N: int, Bf: int) -> np.ndarray:
    """Explicit S x S boolean mask, built pair by pair from the rule itself
    (not from the intervals): key j is visible to query i when i is text, or
    j is text, or j's frame is an anchor (first or last frame), or the frame
    blocks of i and j differ by at most one."""
    V = F * T
    S = V + N
    t = np.arange(S)
    is_text = t >= V
    frame = np.where(is_text, -1, t // max(T, 1))
    block = np.where(is_text, -1, frame // Bf)
    qi_text = is_text[:, None]
    kj_text = is_text[None, :]
    anchor_key = ((frame == 0) | (frame == F - 1)) & ~is_text
    near = np.abs(block[:, None] - block[None, :]) <= 1
    return qi_text | kj_text | anchor_key[None, :] | near


def count_pairs(F: int, T: int, N: int, Bf: int) -> tuple[int, int]:
    """Closed-form pair counts per (sample, head): (allowed pairs, pairs added
    by the two anchors beyond the block window).  Text query rows attend to
    all S keys."""
    V = F * T
    S = V + N
    allowed = N * S
    anchor = 0
    for beta in range(num_frame_blocks(F, Bf)):
        lo, hi = window_frames(beta, F, Bf)
        rows = (min(F, (beta + 1) * Bf) - beta * Bf) * T
        extra = int(lo > 0) + int(hi < F)
        allowed += rows * (T * (hi - lo + extra) + N)
        anchor += rows * T * extra
    return allowed, anchor


def count_pairs_bruteforce(F: int, T: int, N: int, Bf: int) -> tuple[int, int]:
    """Counts by summing the explicit mask; anchor-added pairs are video
    query / video key pairs whose blocks are more than one apart but whose key
    frame is an anchor."""
    m = allowed_mask(F, T, N, Bf)
    V = F * T
    S = V + N
    t = np.arange(S)
    frame = t // max(T, 1)
    block = frame // Bf
    vq = (t < V)[:, None]
    vk = (t < V)[None, :]
    far = np.abs(block[:, None] - block[None, :]) > 1
    anchor_key = ((frame == 0) | (frame == F - 1))[None, :]
    return int(m.sum()), int((vq & vk & far & anchor_key).sum())


# --------------------------------------------------------------------------
# Values
# --------------------------------------------------------------------------


def sigmoid(g: np.ndarray) -> np.ndarray:
    """1 / (1 + exp(-g)) in fp64."""
    return 1.0 / (1.0 + np.exp(-np.asarray(g, dtype=np.float64)))


def dequantize_fp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Value of per-head scaled fp8 tensors: codes [B,S,H,D] (already widened
    to fp64, which is exact) times scales[h].  The product of a 4-bit
    significand and a 24-bit fp32 scale is exact in fp64."""
    c = np.asarray(codes, dtype=np.float64)
    s = np.asarray(scales, dtype=np.float64)
    return c * s[None, None, :, None]


def _softmax_rows(s: np.ndarray):
    """Row softmax pieces in fp64: (p / l, log-sum-exp)."""
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    return p / l, (m + np.log(l))[:, 0]


def attend(q, k, v, gate, F: int, T: int, N: int, Bf: int,
           scale: float | None = None, rows=None, heads=None,
           row_chunk: int = 2048):
    """Exact local-window attention in fp64.

    q, k, v: [B, S, H, D] real arrays (fp64 or anything that widens exactly);
    gate: [B, S, H] logits or None.  For every sample b, head h and query i,
    gather the key set of i's query block, form s = scale * q_i . k_j, take
    the softmax over that set, average v with it and multiply by sigmoid(g).

    ``rows`` (optional sorted array of query indices) and ``heads`` restrict
    the work to a sample of the output; unrequested entries are NaN.
    Returns (out [B,S,H,D] fp64, lse [B,H,S] fp64, natural log)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, S, H, D = q.shape
    assert S == F * T + N, (S, F, T, N)
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(D)
    heads = list(range(H)) if heads is None else list(heads)
    out = np.full((B, S, H, D), np.nan)
    lse = np.full((B, H, S), np.nan)
    qblocks = query_blocks(F, T, N, Bf)
    kivs = key_intervals(F, T, N, Bf)
    for (r0, r1), ivs in zip(qblocks, kivs):
        if rows is None:
            qrows = np.arange(r0, r1)
        else:
            rr = np.asarray(rows)
            qrows = rr[(rr >= r0) & (rr < r1)]
        if qrows.size == 0:
            continue
        keys = np.concatenate([np.arange(a, b) for a, b in ivs])
        for b in range(B):
            for h in heads:
                kb = k[b, keys, h, :]
                vb = v[b, keys, h, :]
                for c0 in range(0, qrows.size, row_chunk):
                    qi = qrows[c0:c0 + row_chunk]
                    s = (q[b, qi, h, :] @ kb.T) * scale
                    p, ls = _softmax_rows(s)
                    o = p @ vb
                    if gate is not None:
                        o = o * sigmoid(np.asarray(gate)[b, qi, h])[:, None]
                    out[b, qi, h, :] = o
                    lse[b, h, qi] = ls
    return out, lse


def attend_dense_masked(q, k, v, gate, mask: np.ndarray, scale: float | None = None):
    """Masked attention over the full S x S score matrix (small inputs only):
    disallowed scores are set to -inf before the softmax."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, S, H, D = q.shape
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(D)
    out = np.empty((B, S, H, D))
    lse = np.empty((B, H, S))
    for b in range(B):
        for h in range(H):
            s = (q[b, :, h, :] @ k[b, :, h, :].T) * scale
            s = np.where(mask, s, -np.inf)
            p, ls = _softmax_rows(s)
            o = p @ v[b, :, h, :]
            if gate is not None:
                o = o * sigmoid(np.asarray(gate)[b, :, h])[:, None]
            out[b, :, h, :] = o
            lse[b, h, :] = ls
    return out, lse


# --------------------------------------------------------------------------
# Backward pass (gradients of the forward above)
# --------------------------------------------------------------------------
#
# The pages train low-rank adapters on the attention projections through this
# branch (superapi "Technical Principles", training stages), so gradients
# flow back through it.  They state no formula: the gradient of the forward
# defined above is its derivative, written out here by the chain rule.  With
# p_ij = softmax_j(s_i) over the key set, a_i = sum_j p_ij v_j (before the
# gate), sg_i = sigmoid(g_i) and out_i = sg_i a_i, for an upstream gradient
# dout:
#   da_i    = sg_i dout_i
#   dg_i    = (dout_i . a_i) sg_i (1 - sg_i)
#   dp_ij   = da_i . v_j
#   ds_ij   = p_ij (dp_ij - sum_k p_ik dp_ik)        (softmax derivative)
#   dq_i    = scale sum_j ds_ij k_j
#   dk_j    = scale sum_i ds_ij q_i                  (over queries that see j)
#   dv_j    = sum_i p_ij da_i


def key_blocks(F: int, T: int, N: int, Bf: int) -> list[tuple[list[tuple[int, int]], list[tuple[int, int]]]]:
    """The key side of the key structure: groups of keys that are seen by the
    same query rows, as (key intervals, query intervals), both canonical.

    Read off the rule of :func:`allowed_mask` column-wise: a video key whose
    frame is not an anchor, in frame block b, is seen by the video queries of
    blocks b-1 .. b+1 (the same frame range as :func:`window_frames` of b) and
    by every text query; anchor-frame keys and text keys are seen by every
    query.  One group per frame block (its non-anchor frames; omitted when
    empty), then the group of anchor and text keys (omitted when empty)."""
    V = F * T
    S = V + N
    out = []
    for beta in range(num_frame_blocks(F, Bf)):
        f0, f1 = beta * Bf, min(F, (beta + 1) * Bf)
        frames = [f for f in range(f0, f1) if f != 0 and f != F - 1]
        if not frames or T == 0:
            continue
        keys = _merge([(f * T, (f + 1) * T) for f in frames])
        lo, hi = window_frames(beta, F, Bf)
        out.append((keys, _merge([(lo * T, hi * T), (V, S)])))
    glob = _merge([(0, T), ((F - 1) * T, F * T), (V, S)])
    if glob:
        out.append((glob, [(0, S)]))
    return out


def _gate_backward(do, a, sg):
    """Through out = sg * a: (da, dg) = (sg do, (do . a) sg (1 - sg))."""
    return do * sg[:, None], np.sum(do * a, axis=1) * sg * (1.0 - sg)


def _softmax_backward(p, dp):
    """Through a row softmax p: ds = p (dp - sum_k p_k dp_k)."""
    return p * (dp - np.sum(p * dp, axis=1, keepdims=True))


def attend_backward(q, k, v, gate, dout, F: int, T: int, N: int, Bf: int,
                    scale: float | None = None, row_chunk: int = 2048, rows=None, heads=None):
    """Gradients of :func:`attend` in fp64: returns (dq, dk, dv, dgate) with
    the shapes of q, k, v and gate (dgate is None without a gate).

    Query block by query block: recompute the softmax over the block's key set
    as the forward does, then apply the chain rule written out in the comment
    above; the key gradients are scattered back to the gathered keys.

    ``rows`` (sorted query indices) and ``heads`` restrict the work to a
    sample: dq and dgate of those rows and heads are exact; dk and dv then only
    hold the sampled rows' contributions."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, S, H, D = q.shape
    assert S == F * T + N, (S, F, T, N)
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(D)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dgate = None if gate is None else np.zeros((B, S, H))
    heads = list(range(H)) if heads is None else list(heads)
    for (r0, r1), ivs in zip(query_blocks(F, T, N, Bf), key_intervals(F, T, N, Bf)):
        if rows is None:
            qrows = np.arange(r0, r1)
        else:
            rr = np.asarray(rows)
            qrows = rr[(rr >= r0) & (rr < r1)]
        if qrows.size == 0:
            continue
        keys = np.concatenate([np.arange(a, b) for a, b in ivs])
        for b in range(B):
            for h in heads:
                kb = k[b, keys, h, :]
                vb = v[b, keys, h, :]
                for c0 in range(0, qrows.size, row_chunk):
                    qi = qrows[c0:c0 + row_chunk]
                    s = (q[b, qi, h, :] @ kb.T) * scale
                    p, _ = _softmax_rows(s)
                    a = p @ vb
                    do = dout[b, qi, h, :]
                    if gate is not None:
                        da, dg = _gate_backward(do, a, sigmoid(np.asarray(gate)[b, qi, h]))
                        dgate[b, qi, h] = dg
                    else:
                        da = do
                    dp = da @ vb.T
                    ds = _softmax_backward(p, dp)
                    dq[b, qi, h, :] = scale * (ds @ kb)
                    np.add.at(dk[b, :, h, :], keys, scale * (ds.T @ q[b, qi, h, :]))
                    np.add.at(dv[b, :, h, :], keys, p.T @ da)
    return dq, dk, dv, dgate


# --------------------------------------------------------------------------
# Complement linear branch and the two-branch fusion
# --------------------------------------------------------------------------
#
# openi.cn "VDN-MiniMax-H3", technical principles: the linear branch sums up,
# separately, what lies before and what lies after the current window, and
# deliberately leaves out the window frames and the boundary anchors (so it
# does not repeat the softmax branch); the same section: the linear branch's
# output is RMS-normalised and then gated by its own content-dependent
# sigmoid, and the two branches are summed.  nav.superapi.store
# "VDN-MiniMax-H3 - OpenVDN's Open-Source Video Generation Acceleration
# Solution", Technical Principles, "Hybrid Attention Architecture": long-range
# linear attention with linear complexity.
#
# Readings (the pages fix neither the feature map nor the state update; the
# frame-level normal-equation update they name is not specified and is left
# out): plain linear attention with feature map phi(x) = elu(x) + 1 applied
# elementwise to q and k; a video query of block beta uses the video keys of
# frames outside [lo, hi) other than frames 0 and F-1; text queries get no
# linear-branch output (zero), and text keys are not in the linear state
# (writing text into the linear state is a separate mechanism the pages
# name without defining).  Together with the softmax mask this covers every
# (query, key) pair exactly once.  RMSNorm runs over a token's whole
# linear-branch output (all heads), as the input of the branch's output
# projection; the linear branch's gate is one logit per token and head.


def phi(x):
    """Linear-attention feature map elu(x) + 1 (positive everywhere)."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def linear_key_frames(beta: int, F: int, Bf: int) -> list[int]:
    """Frames whose keys enter the linear branch of frame block ``beta``:
    before and after the block window, anchors excluded."""
    lo, hi = window_frames(beta, F, Bf)
    return [f for f in range(F) if (f < lo or f >= hi) and f != 0 and f != F - 1]


def linear_mask(F: int, T: int, N: int, Bf: int) -> np.ndarray:
    """Explicit S x S mask of the linear branch, pair by pair from the rule
    (video query, video key, key frame outside the query's window, key frame
    not an anchor)."""
    V = F * T
    S = V + N
    t = np.arange(S)
    video = t < V
    frame = np.where(video, t // max(T, 1), -1)
    block = frame // Bf
    lo = Bf * np.maximum(0, block - 1)
    hi = np.minimum(F, Bf * (block + 2))
    kf = frame[None, :]
    outside = (kf < lo[:, None]) | (kf >= hi[:, None])
    not_anchor = (kf != 0) & (kf != F - 1)
    return video[:, None] & video[None, :] & outside & not_anchor


def linear_branch(q, k, v, F: int, T: int, N: int, Bf: int):
    """Linear-branch output in fp64, [B, S, H, D]: for a video query of block
    beta, sum_j (phi(q_i).phi(k_j)) v_j / sum_j phi(q_i).phi(k_j) over the keys
    of :func:`linear_key_frames`, computed through the summed state
    sum_j phi(k_j) v_j^T and normaliser sum_j phi(k_j); zero for text queries
    and for blocks with no such keys."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, S, H, D = q.shape
    assert S == F * T + N, (S, F, T, N)
    out = np.zeros((B, S, H, D))
    for beta in range(num_frame_blocks(F, Bf)):
        frames = linear_key_frames(beta, F, Bf)
        if not frames:
            continue
        keys = np.concatenate([np.arange(f * T, (f + 1) * T) for f in frames])
        r0, r1 = beta * Bf * T, min(F, (beta + 1) * Bf) * T
        for b in range(B):
            for h in range(H):
                pk = phi(k[b, keys, h, :])
                state = pk.T @ v[b, keys, h, :]      # D x D
                z = pk.sum(axis=0)                   # D
                pq = phi(q[b, r0:r1, h, :])
                out[b, r0:r1, h, :] = (pq @ state) / (pq @ z)[:, None]
    return out


def rms_norm(x, weight, eps: float):
    """RMSNorm of each token's whole branch output: x [B, S, H, D] is divided
    by sqrt(mean over all H*D entries of x^2 + eps) and multiplied by
    ``weight`` [H, D] (one weight per hidden channel)."""
    x = np.asarray(x, dtype=np.float64)
    r = np.sqrt(np.mean(x * x, axis=(-2, -1), keepdims=True) + eps)
    return x / r * np.asarray(weight, dtype=np.float64)[None, None]


def hybrid_fuse(soft_out, lin_out, gate_lin, norm_weight, eps: float):
    """The hybrid layer's attention output before the output projections:
    the softmax-branch output (already multiplied by its own gate) plus the
    RMS-normalised linear-branch output times the linear branch's sigmoid
    gate (one logit per token and head, [B, S, H])."""
    return (np.asarray(soft_out, dtype=np.float64)
            + sigmoid(gate_lin)[..., None] * rms_norm(lin_out, norm_weight, eps))
