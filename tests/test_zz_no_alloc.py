"""GPU check of vdn_local_attn_bwd_noalloc (the backward pass on the
library's fixed per-GPU scratch, for callers that cannot allocate) against
vdn_local_attn_bwd with a caller workspace, through the C ABI: two calls in a
row, the second on a smaller input, each bit-identical to the workspace entry
point (the same kernels on the same data)."""

import pytest
import torch

from block_sparse_attention_31_amd import binding as B
from block_sparse_attention_31_amd import synth

from .gpu_util import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = torch.device("cuda:0")

# the first call fills more of the scratch than the second reads
SHAPES = [dict(B=2, H=4, D=128, F=12, T=130, N=70, Bf=3, gate=True),
          dict(B=1, H=2, D=64, F=7, T=48, N=8, Bf=2, gate=False)]


def _grads(w, inp, noalloc):
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    gate = None if inp["gate"] is None else inp["gate"].to(DEV)
    dout = synth.make_dout(w).to(DEV)
    out, lse = B.local_attn_fwd(q, k, v, gate, F=w.F, tokens_per_frame=w.T, n_text=w.N,
                                block_frames=w.Bf, return_lse=True)
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    dgate = None if gate is None else torch.full_like(gate, float("nan"))
    if noalloc:
        B.vdn_local_attn_bwd_noalloc(q, k, v, gate, out, dout, lse, dq, dk, dv, dgate, w.F, w.T, w.N, w.Bf)
    else:
        ws = torch.full((2 * w.B * w.H * w.S,), float("nan"), dtype=torch.float32, device=DEV)
        B.vdn_local_attn_bwd(q, k, v, gate, out, dout, lse, dq, dk, dv, dgate, w.F, w.T, w.N, w.Bf,
                             workspace=ws)
    torch.cuda.synchronize()
    return [None if t is None else t.cpu() for t in (dq, dk, dv, dgate)]


def test_noalloc_backward_matches_workspace_entry_point():
    for i, kw in enumerate(SHAPES):
        w = synth.random_workload(seed=900 + i, **kw)
        inp = synth.make_inputs(w)
        ref = _grads(w, inp, noalloc=False)
        got = _grads(w, inp, noalloc=True)
        for name, g, r in zip(("dq", "dk", "dv", "dgate"), got, ref):
            if r is None:
                assert g is None
                continue
            assert torch.isfinite(g.float()).all(), (i, name)
            assert torch.equal(g, r), (i, name, float((g.float() - r.float()).abs().max()))
        print(f"[no-alloc] call {i}: B{w.B} H{w.H} D{w.D} S{w.S} bit-identical", flush=True)
