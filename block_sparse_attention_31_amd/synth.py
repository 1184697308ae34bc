"""Seeded synthetic inputs for the local-window attention path.

This module only draws and encodes inputs; it holds none of the attention
arithmetic.  Both the HIP path (through the tests and the benchmark) and the
CPU oracle receive exactly the tensors produced here.

Workloads follow the shapes of the video latents the pages describe (a dozen
or more latent frames of about a thousand tokens each, plus text tokens;
openi.cn "VDN-MiniMax-H3", technical principles section).  768p latents are a
24 x 42 token grid per frame.  No dataset is involved: values are N(0, 1)
draws, optionally with outlier channels scaled by 8, and fp8 variants are
quantised per head with an fp32 scale (amax / 448, round-to-nearest-even,
saturating to the OCP e4m3fn range).
"""

from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np
import torch

FP8_E4M3_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    D: int
    F: int          # latent frames
    T: int          # tokens per frame
    N: int          # text tokens
    Bf: int = 5     # frames per block
    dtype: str = "bf16"          # "bf16" or "fp8"
    gate: bool = True
    outlier_frac: float = 0.0    # fraction of the H*D channels scaled x8
    seed: int = 0
    per_sample_seed: bool = False

    @property
    def S(self) -> int:
        return self.F * self.T + self.N

    def dense(self) -> "Workload":
        """Same inputs with the window covering every frame."""
        return replace(self, Bf=max(self.F, 1))


WORKLOADS = {
    "tiny": Workload("tiny", B=1, H=2, D=64, F=11, T=64, N=16, gate=False,
                     seed=31001),
    "medium": Workload("medium", B=1, H=16, D=128, F=16, T=1024, N=128,
                       outlier_frac=0.02, seed=31002),
    "768p": Workload("768p", B=1, H=32, D=128, F=20, T=1008, N=512,
                     seed=31003),
    "768p-fp8": Workload("768p-fp8", B=1, H=32, D=128, F=20, T=1008, N=512,
                         dtype="fp8", outlier_frac=0.02, seed=31004),
    # one GPU's share of the 768p shape when 8 GPUs split the 32 heads
    "768p-h4": Workload("768p-h4", B=1, H=4, D=128, F=20, T=1008, N=512,
                        seed=31006),
    "long": Workload("long", B=2, H=32, D=128, F=42, T=1008, N=512,
                     seed=31005, per_sample_seed=True),
}


def _draw_sample(rng: np.random.Generator, w: Workload):
    shape = (w.S, w.H, w.D)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    g = rng.standard_normal((w.S, w.H), dtype=np.float32) if w.gate else None
    return q, k, v, g


def _apply_outliers(rng: np.random.Generator, x: np.ndarray, frac: float):
    """Scale round(frac * H * D) channels, chosen without replacement, by 8
    for every token (x is [B, S, H, D])."""
    H, D = x.shape[2], x.shape[3]
    n = int(round(frac * H * D))
    if n == 0:
        return x
    ch = rng.choice(H * D, size=n, replace=False)
    flat = x.reshape(x.shape[0], x.shape[1], H * D)
    flat[:, :, ch] *= np.float32(8.0)
    return x


def quantize_fp8_per_head(x: torch.Tensor):
    """[B,S,H,D] fp32 -> (e4m3fn codes, fp32 scale per head).  The scale is the
    head's absolute maximum over all tokens divided by 448."""
    amax = x.abs().amax(dim=(0, 1, 3)).clamp_min(1e-30)
    scale = (amax / FP8_E4M3_MAX).to(torch.float32)
    y = (x / scale[None, None, :, None]).clamp(-FP8_E4M3_MAX, FP8_E4M3_MAX)
    return y.to(torch.float8_e4m3fn), scale


def make_inputs(w: Workload) -> dict:
    """Draw the workload's inputs on the CPU.

    Returns a dict with q, k, v ([B,S,H,D] bf16 or float8_e4m3fn), gate
    ([B,S,H] fp32 or None) and scales ([3,H] fp32 for fp8, else None)."""
    if w.per_sample_seed:
        parts = [_draw_sample(np.random.default_rng(w.seed + b), w) for b in range(w.B)]
        orng = np.random.default_rng(w.seed + 1000)
    else:
        rng = np.random.default_rng(w.seed)
        parts = [_draw_sample(rng, w) for _ in range(w.B)]
        orng = rng
    q = np.stack([p[0] for p in parts])
    k = np.stack([p[1] for p in parts])
    v = np.stack([p[2] for p in parts])
    g = np.stack([p[3] for p in parts]) if w.gate else None
    del parts
    if w.outlier_frac > 0:
        for x in (q, k, v):
            _apply_outliers(orng, x, w.outlier_frac)
    out = {"gate": torch.from_numpy(g) if g is not None else None, "scales": None}
    if w.dtype == "bf16":
        for name, x in (("q", q), ("k", k), ("v", v)):
            out[name] = torch.from_numpy(x).to(torch.bfloat16)
    elif w.dtype == "fp8":
        scales = []
        for name, x in (("q", q), ("k", k), ("v", v)):
            codes, s = quantize_fp8_per_head(torch.from_numpy(x))
            out[name] = codes
            scales.append(s)
        out["scales"] = torch.stack(scales).contiguous()
    else:
        raise ValueError(f"unknown dtype {w.dtype}")
    return out


def make_dout(w: Workload) -> torch.Tensor:
    """Upstream gradient for the backward pass: bf16 [B, S, H, D], fp32
    N(0,1) draws (seed + 2000) rounded to nearest even."""
    rng = np.random.default_rng(w.seed + 2000)
    x = rng.standard_normal((w.B, w.S, w.H, w.D), dtype=np.float32)
    return torch.from_numpy(x).to(torch.bfloat16)


def random_workload(seed: int, **overrides) -> Workload:
    """A small seeded workload for sweeps (shape fields can be overridden)."""
    base = dict(name=f"rand{seed}", B=1, H=2, D=64, F=7, T=48, N=8, Bf=2,
                dtype="bf16", gate=True, outlier_frac=0.0, seed=seed)
    base.update(overrides)
    return Workload(**base)


def needle_queries(k: torch.Tensor, pairs, alpha: float) -> torch.Tensor:
    """Queries that point at chosen keys: for each (b, i, h, j) in ``pairs``
    set q[b, i, h] = alpha * k[b, j, h] (other rows zero).  Returns a tensor of
    k's dtype and shape."""
    q = torch.zeros_like(k, dtype=torch.float32)
    kf = k.to(torch.float32)
    for b, i, h, j in pairs:
        q[b, i, h] = alpha * kf[b, j, h]
    return q.to(k.dtype)


def with_frame_offsets(v: torch.Tensor, F: int, T: int, step: float) -> torch.Tensor:
    """Values with a per-frame offset: token t of frame f gets step * f added
    to every channel (text tokens get step * F); re-rounded to bf16.  Makes an
    average over keys depend on which frames it covers, not only on how many."""
    S = v.shape[1]
    frame = torch.clamp(torch.arange(S) // T, max=F).to(torch.float32)
    return (v.to(torch.float32) + step * frame[None, :, None, None]).to(torch.bfloat16)


def make_fuse_inputs(w: Workload) -> dict:
    """Inputs of the two-branch fusion for the workload's shape (seed + 3000):
    soft_out and lin_out [B,S,H,D] bf16 N(0,1), gate_lin [B,S,H] fp32 N(0,1)
    logits and norm_weight [H,D] fp32 drawn as 1 + 0.1 N(0,1)."""
    rng = np.random.default_rng(w.seed + 3000)
    shape = (w.B, w.S, w.H, w.D)
    soft = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(torch.bfloat16)
    lin = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(torch.bfloat16)
    gate = torch.from_numpy(rng.standard_normal((w.B, w.S, w.H), dtype=np.float32))
    weight = torch.from_numpy(1.0 + 0.1 * rng.standard_normal((w.H, w.D), dtype=np.float32))
    return {"soft": soft, "lin": lin, "gate": gate, "weight": weight}
