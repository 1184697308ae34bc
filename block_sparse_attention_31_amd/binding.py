"""ctypes binding of libvdn_local_attn.so (argument marshalling only).

Every function keeps the C name.  Tensors must be torch tensors on the GPU;
the binding passes their data pointers and the current HIP stream.  There is
no CPU fallback: if the library is missing the call fails.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libvdn_local_attn.so")

VDN_BF16 = 0
VDN_FP8_E4M3 = 1
VDN_MAX_KEY_INTERVALS = 4

STATUS_NAMES = {
    0: "VDN_OK",
    -1: "VDN_ERR_INVALID_ARG",
    -2: "VDN_ERR_UNSUPPORTED",
    -3: "VDN_ERR_ALIGNMENT",
    -4: "VDN_ERR_OVERFLOW",
    -5: "VDN_ERR_HIP",
    -6: "VDN_ERR_CAPACITY",
}

# Every symbol the header declares, with (restype, argtypes).
_i, _f, _p = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
_i64 = ctypes.c_int64
_pi64 = ctypes.POINTER(ctypes.c_int64)
_pi32 = ctypes.POINTER(ctypes.c_int32)
_pint = ctypes.POINTER(ctypes.c_int)
SIGNATURES = {
    "vdn_local_attn_fwd": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _p, _f, _p, _p]),
    "vdn_local_attn_bwd": (_i, [_p] * 11 + [_i] * 7 + [_f, _p, _p]),
    "vdn_local_attn_bwd_noalloc": (_i, [_p] * 11 + [_i] * 7 + [_f, _p]),
    "vdn_local_attn_num_query_blocks": (_i, [_i, _i, _i, _i]),
    "vdn_local_attn_key_intervals": (_i, [_i, _i, _i, _i, _pi64, _pi64, _i, _pint]),
    "vdn_local_attn_count_pairs": (_i, [_i, _i, _i, _i, _pi64, _pi64]),
    "vdn_local_attn_tile_schedule": (_i, [_i, _i, _i, _i, _i, _pi32, _i, _pint]),
    "vdn_local_attn_key_blocks": (_i, [_i, _i, _i, _i, _pi64, _pi64, _i, _pint]),
    "vdn_local_attn_kernel_tile_m": (_i, [_i, _i]),
    "vdn_linear_branch_fwd": (_i, [_p] * 4 + [_i] * 7 + [_p, _i64, _p]),
    "vdn_linear_branch_workspace_bytes": (_i64, [_i] * 7),
    "vdn_hybrid_fuse": (_i, [_p, _p, _p, _p, _f, _p, _i64, _i, _i, _p]),
    "vdn_hybrid_attn_fwd": (_i, [_p] * 6 + [_f, _p] + [_i] * 7 + [_f, _p, _p, _i64, _p]),
    "vdn_hybrid_attn_workspace_bytes": (_i64, [_i] * 7),
    "vdn_last_error": (ctypes.c_char_p, []),
}

_LIB = None


class VdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")


def lib() -> ctypes.CDLL:
    """Load the HIP library (built in-tree by build.build())."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m block_sparse_attention_31_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def vdn_last_error() -> str:
    return lib().vdn_last_error().decode()


def _check(rc: int) -> int:
    if rc < 0:
        raise VdnError(rc, vdn_last_error())
    return rc


# ------------------------------------------------------------ host functions


def vdn_local_attn_num_query_blocks(F: int, tokens_per_frame: int, n_text: int, block_frames: int) -> int:
    return _check(lib().vdn_local_attn_num_query_blocks(F, tokens_per_frame, n_text, block_frames))


def vdn_local_attn_key_intervals(F: int, tokens_per_frame: int, n_text: int, block_frames: int):
    """Returns (query_rows [(lo, hi)], key_intervals [[(lo, hi), ...]])."""
    n = vdn_local_attn_num_query_blocks(F, tokens_per_frame, n_text, block_frames)
    rows = (ctypes.c_int64 * (2 * n))()
    ivs = (ctypes.c_int64 * (2 * VDN_MAX_KEY_INTERVALS * n))()
    got = ctypes.c_int(0)
    _check(lib().vdn_local_attn_key_intervals(F, tokens_per_frame, n_text, block_frames,
                                              rows, ivs, n, ctypes.byref(got)))
    qrows = [(rows[2 * i], rows[2 * i + 1]) for i in range(got.value)]
    lists = []
    for i in range(got.value):
        base = 2 * VDN_MAX_KEY_INTERVALS * i
        lst = []
        for j in range(VDN_MAX_KEY_INTERVALS):
            lo, hi = ivs[base + 2 * j], ivs[base + 2 * j + 1]
            if lo >= 0:
                lst.append((lo, hi))
        lists.append(lst)
    return qrows, lists


def vdn_local_attn_count_pairs(F: int, tokens_per_frame: int, n_text: int, block_frames: int):
    a, x = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(lib().vdn_local_attn_count_pairs(F, tokens_per_frame, n_text, block_frames,
                                            ctypes.byref(a), ctypes.byref(x)))
    return a.value, x.value


def vdn_local_attn_tile_schedule(F: int, tokens_per_frame: int, n_text: int, block_frames: int,
                                 tile_m: int):
    """Returns [(query block, first row, rows, keys)] in launch order."""
    n = ctypes.c_int(0)
    rc = lib().vdn_local_attn_tile_schedule(F, tokens_per_frame, n_text, block_frames, tile_m,
                                            None, 0, ctypes.byref(n))
    if rc not in (0, -6):
        _check(rc)
    buf = (ctypes.c_int32 * (4 * max(n.value, 1)))()
    _check(lib().vdn_local_attn_tile_schedule(F, tokens_per_frame, n_text, block_frames, tile_m,
                                              buf, n.value, ctypes.byref(n)))
    return [tuple(buf[4 * i:4 * i + 4]) for i in range(n.value)]


def vdn_local_attn_key_blocks(F: int, tokens_per_frame: int, n_text: int, block_frames: int):
    """Returns [(key intervals [(lo, hi)], query intervals [(lo, hi)])]."""
    n = ctypes.c_int(0)
    rc = lib().vdn_local_attn_key_blocks(F, tokens_per_frame, n_text, block_frames, None, None, 0,
                                         ctypes.byref(n))
    if rc not in (0, -6):
        _check(rc)
    cap = max(n.value, 1)
    kiv = (ctypes.c_int64 * (2 * VDN_MAX_KEY_INTERVALS * cap))()
    qiv = (ctypes.c_int64 * (2 * VDN_MAX_KEY_INTERVALS * cap))()
    _check(lib().vdn_local_attn_key_blocks(F, tokens_per_frame, n_text, block_frames, kiv, qiv, cap,
                                           ctypes.byref(n)))

    def unpack(buf, i):
        base = 2 * VDN_MAX_KEY_INTERVALS * i
        return [(buf[base + 2 * j], buf[base + 2 * j + 1]) for j in range(VDN_MAX_KEY_INTERVALS)
                if buf[base + 2 * j] >= 0]
    return [(unpack(kiv, i), unpack(qiv, i)) for i in range(n.value)]


def vdn_local_attn_kernel_tile_m(head_dim: int, dtype: int) -> int:
    return _check(lib().vdn_local_attn_kernel_tile_m(head_dim, dtype))


# ------------------------------------------------------------------ forward


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return VDN_BF16
    if t.dtype == torch.float8_e4m3fn:
        return VDN_FP8_E4M3
    raise TypeError(f"unsupported q/k/v dtype {t.dtype} (bfloat16 or float8_e4m3fn)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def vdn_local_attn_fwd(q, k, v, gate, out, F: int, tokens_per_frame: int, n_text: int,
                       block_frames: int = 5, heads: int | None = None,
                       head_dim: int | None = None, dtype: int | None = None,
                       batch: int | None = None, qkv_scales=None, softmax_scale: float = 0.0,
                       lse=None, stream=None) -> None:
    """Enqueue the forward pass on `stream` (default: torch's current stream).

    q, k, v: [B, S, H, D] bf16 or float8_e4m3fn CUDA tensors; gate [B, S, H]
    fp32 or None; out [B, S, H, D] bf16; qkv_scales [3, H] fp32 (fp8 only);
    lse [B, H, S] fp32 or None."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if q.shape != k.shape or q.shape != v.shape or q.shape != out.shape:
        raise ValueError("q, k, v and out must have the same shape")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k and v must share a dtype")
    if out.dtype != torch.bfloat16:
        raise ValueError("out must be bfloat16")
    B, S, H, D = q.shape
    for name, t, shape in (("gate", gate, (B, S, H)), ("lse", lse, (B, H, S)),
                           ("qkv_scales", qkv_scales, (3, H))):
        if t is None:
            continue
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.float32:
            raise ValueError(f"{name} must be a contiguous fp32 GPU tensor")
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must have shape {shape}, got {tuple(t.shape)}")
    code = _dtype_code(q)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib().vdn_local_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(out),
        F, tokens_per_frame, n_text, block_frames,
        H if heads is None else heads, D if head_dim is None else head_dim,
        code if dtype is None else dtype, B if batch is None else batch,
        _ptr(qkv_scales), float(softmax_scale), _ptr(lse), ctypes.c_void_p(stream))
    _check(rc)


def local_attn_fwd(q, k, v, gate=None, *, F: int, tokens_per_frame: int, n_text: int,
                   block_frames: int = 5, qkv_scales=None, softmax_scale: float = 0.0,
                   return_lse: bool = False):
    """Allocating convenience wrapper: returns out (and lse if asked)."""
    import torch
    B, S, H, D = q.shape
    out = torch.empty((B, S, H, D), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device) if return_lse else None
    vdn_local_attn_fwd(q, k, v, gate, out, F, tokens_per_frame, n_text, block_frames,
                       qkv_scales=qkv_scales, softmax_scale=softmax_scale, lse=lse)
    return (out, lse) if return_lse else out


# ----------------------------------------------------------------- backward


def vdn_local_attn_bwd(q, k, v, gate, out, dout, lse, dq, dk, dv, dgate, F: int,
                       tokens_per_frame: int, n_text: int, block_frames: int = 5,
                       softmax_scale: float = 0.0, workspace=None, stream=None) -> None:
    """Enqueue the backward pass on `stream` (default: torch's current stream).

    q, k, v, out, dout, dq, dk, dv: [B, S, H, D] bf16 CUDA tensors; gate and
    dgate [B, S, H] fp32 (both or neither); lse [B, H, S] fp32 (the forward's);
    workspace: fp32 CUDA tensor of at least 2*B*H*S elements."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout),
                    ("dq", dq), ("dk", dk), ("dv", dv)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be a contiguous bf16 GPU tensor")
        if t.shape != q.shape:
            raise ValueError(f"{name} must have the shape of q")
    B, S, H, D = q.shape
    if workspace is None or workspace.numel() < 2 * B * H * S:
        raise ValueError(f"workspace must hold at least {2 * B * H * S} fp32 values")
    for name, t, shape in (("gate", gate, (B, S, H)), ("dgate", dgate, (B, S, H)),
                           ("lse", lse, (B, H, S)), ("workspace", workspace, None)):
        if t is None:
            continue
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.float32:
            raise ValueError(f"{name} must be a contiguous fp32 GPU tensor")
        if shape is not None and tuple(t.shape) != shape:
            raise ValueError(f"{name} must have shape {shape}, got {tuple(t.shape)}")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib().vdn_local_attn_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(out), _ptr(dout), _ptr(lse),
        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dgate), F, tokens_per_frame, n_text, block_frames,
        H, D, B, float(softmax_scale), _ptr(workspace), ctypes.c_void_p(stream))
    _check(rc)


def vdn_local_attn_bwd_noalloc(q, k, v, gate, out, dout, lse, dq, dk, dv, dgate, F: int,
                               tokens_per_frame: int, n_text: int, block_frames: int = 5,
                               softmax_scale: float = 0.0, stream=None) -> None:
    """vdn_local_attn_bwd with the library's fixed per-GPU scratch in place of
    a workspace (the call allocates nothing); tensors as there."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout),
                    ("dq", dq), ("dk", dk), ("dv", dv)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be a contiguous bf16 GPU tensor")
        if t.shape != q.shape:
            raise ValueError(f"{name} must have the shape of q")
    B, S, H, D = q.shape
    for name, t, shape in (("gate", gate, (B, S, H)), ("dgate", dgate, (B, S, H)), ("lse", lse, (B, H, S))):
        if t is None:
            continue
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.float32:
            raise ValueError(f"{name} must be a contiguous fp32 GPU tensor")
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must have shape {shape}, got {tuple(t.shape)}")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib().vdn_local_attn_bwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(out), _ptr(dout), _ptr(lse),
        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dgate), F, tokens_per_frame, n_text, block_frames,
        H, D, B, float(softmax_scale), ctypes.c_void_p(stream))
    _check(rc)


def local_attn_bwd(q, k, v, gate, out, dout, lse, *, F: int, tokens_per_frame: int, n_text: int,
                   block_frames: int = 5, softmax_scale: float = 0.0):
    """Allocating convenience wrapper: returns (dq, dk, dv, dgate or None)."""
    import torch
    B, S, H, D = q.shape
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    dgate = None if gate is None else torch.empty((B, S, H), dtype=torch.float32, device=q.device)
    ws = torch.empty(2 * B * H * S, dtype=torch.float32, device=q.device)
    vdn_local_attn_bwd(q, k, v, gate, out, dout, lse, dq, dk, dv, dgate, F, tokens_per_frame, n_text,
                       block_frames, softmax_scale=softmax_scale, workspace=ws)
    return dq, dk, dv, dgate


# ------------------------------------------------ linear branch and fusion


def vdn_linear_branch_workspace_bytes(F: int, tokens_per_frame: int, n_text: int, block_frames: int,
                                      heads: int, head_dim: int, batch: int) -> int:
    return _check(lib().vdn_linear_branch_workspace_bytes(F, tokens_per_frame, n_text, block_frames,
                                                          heads, head_dim, batch))


def vdn_linear_branch_fwd(q, k, v, out, F: int, tokens_per_frame: int, n_text: int,
                          block_frames: int = 5, workspace=None, stream=None) -> None:
    """Enqueue the linear branch on `stream` (default: torch's current stream).

    q, k, v, out: [B, S, H, D] bf16 CUDA tensors; workspace: a CUDA tensor of
    at least vdn_linear_branch_workspace_bytes(...) bytes."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be a contiguous bf16 GPU tensor")
        if t.shape != q.shape:
            raise ValueError(f"{name} must have the shape of q")
    B, S, H, D = q.shape
    if workspace is None or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    nbytes = workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib().vdn_linear_branch_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), F, tokens_per_frame, n_text, block_frames,
        H, D, B, _ptr(workspace), nbytes, ctypes.c_void_p(stream))
    _check(rc)


def linear_branch_fwd(q, k, v, *, F: int, tokens_per_frame: int, n_text: int, block_frames: int = 5):
    """Allocating convenience wrapper: returns the linear-branch output."""
    import torch
    B, S, H, D = q.shape
    out = torch.empty_like(q)
    nbytes = vdn_linear_branch_workspace_bytes(F, tokens_per_frame, n_text, block_frames, H, D, B)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    vdn_linear_branch_fwd(q, k, v, out, F, tokens_per_frame, n_text, block_frames, workspace=ws)
    return out


def vdn_hybrid_fuse(soft_out, lin_out, gate_lin, norm_weight, out, eps: float = 1e-6, stream=None) -> None:
    """Enqueue the two-branch fusion on `stream`.

    soft_out, lin_out, out: [..., H, D] bf16 CUDA tensors of one shape (out
    may be soft_out); gate_lin [..., H] fp32; norm_weight [H, D] (or H*D) fp32."""
    import torch
    for name, t in (("soft_out", soft_out), ("lin_out", lin_out), ("out", out)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be a contiguous bf16 GPU tensor")
        if t.shape != soft_out.shape:
            raise ValueError(f"{name} must have the shape of soft_out")
    if soft_out.dim() < 2:
        raise ValueError("soft_out must be [..., heads, head_dim]")
    H, D = soft_out.shape[-2], soft_out.shape[-1]
    tokens = soft_out.numel() // (H * D)
    for name, t, n in (("gate_lin", gate_lin, tokens * H), ("norm_weight", norm_weight, H * D)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.float32:
            raise ValueError(f"{name} must be a contiguous fp32 GPU tensor")
        if t.numel() != n:
            raise ValueError(f"{name} must hold {n} values, got {t.numel()}")
    if tuple(gate_lin.shape) != tuple(soft_out.shape[:-1]):
        raise ValueError(f"gate_lin must have shape {tuple(soft_out.shape[:-1])}")
    if stream is None:
        stream = torch.cuda.current_stream(soft_out.device).cuda_stream
    rc = lib().vdn_hybrid_fuse(_ptr(soft_out), _ptr(lin_out), _ptr(gate_lin), _ptr(norm_weight),
                               float(eps), _ptr(out), tokens, H, D, ctypes.c_void_p(stream))
    _check(rc)


def hybrid_fuse(soft_out, lin_out, gate_lin, norm_weight, eps: float = 1e-6):
    """Allocating convenience wrapper: returns the fused output."""
    import torch
    out = torch.empty_like(soft_out)
    vdn_hybrid_fuse(soft_out, lin_out, gate_lin, norm_weight, out, eps)
    return out


def vdn_hybrid_attn_workspace_bytes(F: int, tokens_per_frame: int, n_text: int, block_frames: int,
                                    heads: int, head_dim: int, batch: int) -> int:
    return _check(lib().vdn_hybrid_attn_workspace_bytes(F, tokens_per_frame, n_text, block_frames,
                                                        heads, head_dim, batch))


def vdn_hybrid_attn_fwd(q, k, v, gate, gate_lin, norm_weight, out, F: int, tokens_per_frame: int,
                        n_text: int, block_frames: int = 5, eps: float = 1e-6,
                        softmax_scale: float = 0.0, lse=None, workspace=None, stream=None) -> None:
    """Enqueue the hybrid attention output (linear branch, then the softmax
    branch with the fusion in its epilogue) on `stream`.

    q, k, v, out: [B, S, H, D] bf16 CUDA tensors; gate (or None) and gate_lin
    [B, S, H] fp32; norm_weight [H, D] (or H*D) fp32; lse [B, H, S] fp32 or
    None; workspace: a contiguous GPU tensor of at least
    vdn_hybrid_attn_workspace_bytes bytes."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be a contiguous bf16 GPU tensor")
        if t.shape != q.shape:
            raise ValueError(f"{name} must have the shape of q")
    B, S, H, D = q.shape
    for name, t, shape in (("gate", gate, (B, S, H)), ("gate_lin", gate_lin, (B, S, H)),
                           ("norm_weight", norm_weight, None), ("lse", lse, (B, H, S))):
        if t is None:
            continue
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.float32:
            raise ValueError(f"{name} must be a contiguous fp32 GPU tensor")
        if shape is not None and tuple(t.shape) != shape:
            raise ValueError(f"{name} must have shape {shape}, got {tuple(t.shape)}")
    if gate_lin is None or norm_weight is None:
        raise ValueError("gate_lin and norm_weight are required")
    if norm_weight.numel() != H * D:
        raise ValueError(f"norm_weight must hold {H * D} values, got {norm_weight.numel()}")
    if workspace is None or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    nbytes = workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib().vdn_hybrid_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(gate_lin), _ptr(norm_weight), float(eps),
        _ptr(out), F, tokens_per_frame, n_text, block_frames, H, D, B, float(softmax_scale),
        _ptr(lse), _ptr(workspace), nbytes, ctypes.c_void_p(stream))
    _check(rc)


def hybrid_attn_fwd(q, k, v, gate, gate_lin, norm_weight, *, F: int, tokens_per_frame: int,
                    n_text: int, block_frames: int = 5, eps: float = 1e-6, softmax_scale: float = 0.0):
    """Allocating convenience wrapper: returns the hybrid attention output."""
    import torch
    B, S, H, D = q.shape
    out = torch.empty_like(q)
    nbytes = vdn_hybrid_attn_workspace_bytes(F, tokens_per_frame, n_text, block_frames, H, D, B)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    vdn_hybrid_attn_fwd(q, k, v, gate, gate_lin, norm_weight, out, F, tokens_per_frame, n_text,
                        block_frames, eps=eps, softmax_scale=softmax_scale, workspace=ws)
    return out
