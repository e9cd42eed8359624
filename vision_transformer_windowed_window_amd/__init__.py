"""Fused shifted-window attention for AMD Instinct MI355X -- Python binding of libwattn.so.

This module only marshals arguments: it checks tensor shapes and dtypes, passes device
pointers and the current HIP stream to the C ABI declared in include/wattn.h, and turns a
non-zero status into an exception.  Every step of the computation runs in the HIP
kernels of libwattn.so; there is no fallback.  If the library has not been built, every
call raises.

    out = forward(q, k, v, M=32, shift=16, theta=theta)
    out, lse = forward(q, k, v, M=32, shift=16, theta=theta, return_lse=True)
    dq, dk, dv, dtheta, dbias_u, dbias_v = backward(q, k, v, out, dout, lse, M=32, shift=16, theta=theta)
    blocks, count = select_blocks(gate, tau)                      # gated local path: routing
    local_residual(q, k, v, out, blocks, count, w=8, eps=1e-6)    # out += O_local - O_lin-local
    gated_local_path(q, k, v, out, gate, tau, w=8, eps=1e-6)      # both in one launch, no list

q, k, v: [B, Hgrid, Wgrid, H, 32] contiguous device tensors, bfloat16 or float32.
theta:   [H, 16] float32 device tensor of rotation-pair frequencies, or None (no RoPE).
bias_u, bias_v: [H, M*M, 16] device tensors of the input dtype, or None (no bias).
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "forward",
    "backward",
    "cla_logits",
    "linear",
    "layernorm",
    "patch_merge_norm",
    "stem_conv",
    "token_mean",
    "swin_block",
    "swin_block_workspace",
    "BlockParams",
    "select_blocks",
    "local_residual",
    "gated_local_path",
    "pair_count",
    "abi_version",
    "status_string",
    "library_path",
    "load_library",
    "WattnError",
    "BF16",
    "FP32",
    "BF16_OUT_FP32",
    "STATUS",
]

BF16 = 0
FP32 = 1
BF16_OUT_FP32 = 2
STATUS = {
    0: "WATTN_OK",
    1: "WATTN_ERR_NULL",
    2: "WATTN_ERR_SHAPE",
    3: "WATTN_ERR_SHIFT",
    4: "WATTN_ERR_HEAD_DIM",
    5: "WATTN_ERR_RANK",
    6: "WATTN_ERR_DTYPE",
    7: "WATTN_ERR_ALIAS",
    8: "WATTN_ERR_HIP",
    9: "WATTN_ERR_POINTER",
    10: "WATTN_ERR_VALUE",
    11: "WATTN_ERR_SCRATCH",
}

ACT_NONE = 0
ACT_GELU = 1


class BlockParams(ctypes.Structure):
    """wattn_block_params_t: device pointers of one transformer block's parameters."""

    _fields_ = [(name, ctypes.c_void_p) for name in (
        "ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_proj", "b_proj", "ln2_g", "ln2_b", "w_fc1", "b_fc1", "w_fc2",
        "b_fc2", "theta")]


_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class WattnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def library_path() -> str:
    return os.path.join(_HERE, "libwattn.so")


def load_library() -> ctypes.CDLL:
    """Load libwattn.so (built in-tree).  Raises if it is missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m vision_transformer_windowed_window_amd.build` "
            "(there is no non-HIP fallback)"
        )
    lib = ctypes.CDLL(path)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    lib.wattn_forward.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, vp, vp, vp, ci, ci, vp]
    lib.wattn_forward.restype = ci
    lib.wattn_forward_lse.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, vp, vp, vp, ci, ci, vp]
    lib.wattn_forward_lse.restype = ci
    lib.wattn_backward.argtypes = [vp] * 11 + [ci] * 7 + [vp, vp, vp, ci, vp, vp, ci, vp]
    lib.wattn_backward.restype = ci
    lib.wattn_backward_noalloc.argtypes = [vp] * 10 + [ci] * 7 + [vp, vp, vp, ci, vp, vp, ci, vp]
    lib.wattn_backward_noalloc.restype = ci
    i64 = ctypes.c_int64
    lib.wattn_backward_scratch_bytes.argtypes = [ci] * 5
    lib.wattn_backward_scratch_bytes.restype = i64
    lib.wattn_linear.argtypes = [vp] * 5 + [ci] * 6 + [vp]
    lib.wattn_linear.restype = ci
    lib.wattn_layernorm.argtypes = [vp] * 4 + [i64, ci, ctypes.c_float, vp]
    lib.wattn_layernorm.restype = ci
    lib.wattn_patch_merge_norm.argtypes = [vp] * 4 + [ci] * 4 + [ctypes.c_float, vp]
    lib.wattn_patch_merge_norm.restype = ci
    lib.wattn_stem_conv.argtypes = [vp] * 4 + [ci] * 6 + [vp]
    lib.wattn_stem_conv.restype = ci
    lib.wattn_token_mean.argtypes = [vp, vp, ci, ci, ci, vp]
    lib.wattn_token_mean.restype = ci
    lib.wattn_swin_block_workspace.argtypes = [ci] * 4
    lib.wattn_swin_block_workspace.restype = i64
    lib.wattn_swin_block.argtypes = [vp, ctypes.POINTER(BlockParams), vp, i64] + [ci] * 7 + [vp]
    lib.wattn_swin_block.restype = ci
    lib.wattn_cla_logits.argtypes = [vp] * 6 + [ci] * 5 + [vp]
    lib.wattn_cla_logits.restype = ci
    lib.wattn_forward_gated.argtypes = [vp] * 6 + [ci] * 7 + [vp, vp, vp, ci, ci, vp]
    lib.wattn_forward_gated.restype = ci
    lib.wattn_backward_gated.argtypes = [vp] * 13 + [ci] * 7 + [vp, vp, vp, ci, vp, vp, ci, vp]
    lib.wattn_backward_gated.restype = ci
    lib.wattn_select_blocks.argtypes = [vp, ci, ctypes.c_float, vp, vp, vp]
    lib.wattn_select_blocks.restype = ci
    lib.wattn_local_residual.argtypes = [vp] * 6 + [ci] * 6 + [ctypes.c_float, ci, vp]
    lib.wattn_local_residual.restype = ci
    lib.wattn_gated_local.argtypes = [vp] * 5 + [ctypes.c_float] + [ci] * 6 + [ctypes.c_float, ci, vp]
    lib.wattn_gated_local.restype = ci
    lib.wattn_pair_count.argtypes = [ci] * 6
    lib.wattn_pair_count.restype = ctypes.c_int64
    lib.wattn_status_string.argtypes = [ci]
    lib.wattn_status_string.restype = ctypes.c_char_p
    lib.wattn_abi_version.argtypes = []
    lib.wattn_abi_version.restype = ci
    _LIB = lib
    return lib


def abi_version() -> int:
    return load_library().wattn_abi_version()


def status_string(status: int) -> str:
    return load_library().wattn_status_string(status).decode()


def pair_count(B: int, H: int, Hgrid: int, Wgrid: int, M: int, shift: int) -> int:
    """Number of (query, key) pairs with a finite logit (host arithmetic in the library)."""
    return int(load_library().wattn_pair_count(B, H, Hgrid, Wgrid, M, shift))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def forward(q, k, v, *, M: int, shift: int = 0, theta=None, bias_u=None, bias_v=None, out=None,
            out_dtype=None, stream=None, return_lse: bool = False, gate_z=None):
    """Shifted-window attention of (q, k, v) on the GPU; returns ``out`` ([B, Hg, Wg, H, d]).

    ``out_dtype`` (or the dtype of a given ``out``) may be torch.float32 for bfloat16
    inputs; by default the output has the input dtype.  The call is asynchronous on
    ``stream`` (default: torch's current stream).  With ``return_lse`` (bfloat16 inputs)
    it returns ``(out, lse)``, lse being the float32 [B, Hg, Wg, H] natural-log log-sum-exp
    of every query row that ``backward`` needs.  With ``gate_z`` (gate logits shaped and typed
    like q, bfloat16 inputs only) the output is sigmoid(gate_z) * attention.
    """
    import torch

    lib = load_library()
    if q.dtype == torch.bfloat16:
        dtype = BF16
    elif q.dtype == torch.float32:
        dtype = FP32
    else:
        raise TypeError(f"unsupported dtype {q.dtype} (bfloat16 or float32)")
    if q.dim() != 5:
        raise ValueError("q must be [B, Hgrid, Wgrid, H, d]")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must match q in shape, dtype and device")
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    B, Hg, Wg, H, d = q.shape
    if theta is not None:
        if theta.dtype != torch.float32 or not theta.is_cuda or not theta.is_contiguous():
            raise ValueError("theta must be a contiguous float32 device tensor")
        if tuple(theta.shape) != (H, d // 2):
            raise ValueError(f"theta must be [H, d/2] = [{H}, {d // 2}]")
    r = 0
    if (bias_u is None) != (bias_v is None):
        raise ValueError("bias_u and bias_v go together")
    if bias_u is not None:
        r = bias_u.shape[-1]
        for name, t in (("bias_u", bias_u), ("bias_v", bias_v)):
            if tuple(t.shape) != (H, M * M, r) or t.dtype != q.dtype or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous [H, M*M, r] device tensor of q's dtype")
    if out is not None:
        out_dtype = out.dtype
    elif out_dtype is None:
        out_dtype = q.dtype
    if out_dtype == torch.float32 and dtype == BF16:
        dtype = BF16_OUT_FP32
    elif out_dtype != q.dtype:
        raise TypeError(f"unsupported output dtype {out_dtype} for {q.dtype} inputs")
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    elif out.shape != q.shape or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous device tensor shaped like q")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    lse = torch.empty((B, Hg, Wg, H), dtype=torch.float32, device=q.device) if return_lse else None
    if gate_z is not None:
        if gate_z.shape != q.shape or gate_z.dtype != q.dtype or not gate_z.is_cuda or not gate_z.is_contiguous():
            raise ValueError("gate_z must be a contiguous device tensor shaped and typed like q")
        st = lib.wattn_forward_gated(
            _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(gate_z), B, H, Hg, Wg, M, shift, d,
            _ptr(theta), _ptr(bias_u), _ptr(bias_v), r, dtype, ctypes.c_void_p(stream),
        )
    elif return_lse:
        st = lib.wattn_forward_lse(
            _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Hg, Wg, M, shift, d,
            _ptr(theta), _ptr(bias_u), _ptr(bias_v), r, dtype, ctypes.c_void_p(stream),
        )
    else:
        st = lib.wattn_forward(
            _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, Hg, Wg, M, shift, d,
            _ptr(theta), _ptr(bias_u), _ptr(bias_v), r, dtype, ctypes.c_void_p(stream),
        )
    if st != 0:
        raise WattnError(st, status_string(st))
    return (out, lse) if return_lse else out


def backward(q, k, v, out, dout, lse, *, M: int, shift: int = 0, theta=None, bias_u=None, bias_v=None,
             stream=None, gate_z=None):
    """Gradients of sum(dout * out) for the call ``out, lse = forward(q, k, v, ...,
    return_lse=True)``; returns float32 ``(dq, dk, dv, dtheta, dbias_u, dbias_v)`` (dtheta
    is None without theta, the bias gradients None without a bias).  q, k, v and the bias
    factors are bfloat16; out and dout are both bfloat16 or both float32.  With ``gate_z`` (the
    forward call's gate logits) it returns the float32 gradient of gate_z as a seventh value."""
    import torch

    lib = load_library()
    if q.dtype != torch.bfloat16:
        raise TypeError("backward takes bfloat16 q, k, v")
    for name, t in (("k", k), ("v", v)):
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must match q in shape, dtype and device")
    if out.dtype != dout.dtype or out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out and dout must both be bfloat16 or both float32")
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        if t.shape != q.shape or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor shaped like q")
    B, Hg, Wg, H, d = q.shape
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hg, Wg, H) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, Hg, Wg, H] tensor")
    if theta is not None and (theta.dtype != torch.float32 or tuple(theta.shape) != (H, d // 2)
                              or not theta.is_contiguous()):
        raise ValueError(f"theta must be a contiguous float32 [{H}, {d // 2}] tensor")
    r = 0
    if (bias_u is None) != (bias_v is None):
        raise ValueError("bias_u and bias_v go together")
    if bias_u is not None:
        r = bias_u.shape[-1]
        for name, t in (("bias_u", bias_u), ("bias_v", bias_v)):
            if tuple(t.shape) != (H, M * M, r) or t.dtype != q.dtype or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous [H, M*M, r] bfloat16 device tensor")
    dtype = BF16 if out.dtype == torch.bfloat16 else BF16_OUT_FP32
    f32 = dict(dtype=torch.float32, device=q.device)
    dq, dk, dv = (torch.empty(q.shape, **f32) for _ in range(3))
    scratch = torch.empty(lib.wattn_backward_scratch_bytes(B, H, Hg, Wg, d), dtype=torch.uint8, device=q.device)
    dtheta = None if theta is None else torch.empty((H, d // 2), **f32)
    dbu = None if bias_u is None else torch.empty(bias_u.shape, **f32)
    dbv = None if bias_v is None else torch.empty(bias_v.shape, **f32)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    if gate_z is not None:
        if gate_z.shape != q.shape or gate_z.dtype != q.dtype or not gate_z.is_cuda or not gate_z.is_contiguous():
            raise ValueError("gate_z must be a contiguous device tensor shaped and typed like q")
        dz = torch.empty(q.shape, **f32)
        st = lib.wattn_backward_gated(
            _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(gate_z), _ptr(scratch), _ptr(dq),
            _ptr(dk), _ptr(dv), _ptr(dtheta), _ptr(dz), B, H, Hg, Wg, M, shift, d, _ptr(theta), _ptr(bias_u),
            _ptr(bias_v), r, _ptr(dbu), _ptr(dbv), dtype, ctypes.c_void_p(stream),
        )
        if st != 0:
            raise WattnError(st, status_string(st))
        return dq, dk, dv, dtheta, dbu, dbv, dz
    st = lib.wattn_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(scratch), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(dtheta), B, H, Hg, Wg, M, shift, d, _ptr(theta), _ptr(bias_u), _ptr(bias_v), r, _ptr(dbu), _ptr(dbv),
        dtype, ctypes.c_void_p(stream),
    )
    if st != 0:
        raise WattnError(st, status_string(st))
    return dq, dk, dv, dtheta, dbu, dbv


def select_blocks(gate, tau: float, *, blocks=None, count=None, stream=None):
    """Routing of the gated local path: the ascending indices of the blocks whose gate value
    exceeds ``tau``.  ``gate`` is a float32 device tensor of the per-block gate values
    ([B, Hg/w, Wg/w] or flat); returns ``(blocks, count)``: an int32 device tensor with room
    for every block, of which the first ``count[0]`` entries are valid, and the one-element
    int32 device count.  Nothing is synchronised."""
    import torch

    lib = load_library()
    if gate.dtype != torch.float32 or not gate.is_cuda or not gate.is_contiguous():
        raise ValueError("gate must be a contiguous float32 device tensor")
    n = gate.numel()
    if blocks is None:
        blocks = torch.empty(n, dtype=torch.int32, device=gate.device)
    if count is None:
        count = torch.empty(1, dtype=torch.int32, device=gate.device)
    if blocks.dtype != torch.int32 or blocks.numel() < n or count.dtype != torch.int32 or count.numel() < 1:
        raise ValueError("blocks must be int32 with room for every block, count int32 with one element")
    if stream is None:
        stream = torch.cuda.current_stream(gate.device).cuda_stream
    st = lib.wattn_select_blocks(_ptr(gate), n, ctypes.c_float(tau), _ptr(blocks), _ptr(count),
                                 ctypes.c_void_p(stream))
    if st != 0:
        raise WattnError(st, status_string(st))
    return blocks, count


def local_residual(q, k, v, out, blocks, count, *, w: int, eps: float = 1e-6, stream=None):
    """out += O_local - O_lin-local on the tokens of the listed blocks (in place; ``out``
    holds the global path's output).  q, k, v: bfloat16 [B, Hg, Wg, H, 32]; out: bfloat16 or
    float32 of that shape; blocks, count: as returned by ``select_blocks``.  Returns out."""
    import torch

    lib = load_library()
    if q.dtype != torch.bfloat16 or q.dim() != 5:
        raise TypeError("q, k, v must be bfloat16 [B, Hgrid, Wgrid, H, d]")
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t.shape != q.shape or not t.is_cuda or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous device tensor shaped like q")
    for name, t in (("k", k), ("v", v)):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} must be bfloat16")
    if out.dtype == torch.bfloat16:
        dtype = BF16
    elif out.dtype == torch.float32:
        dtype = BF16_OUT_FP32
    else:
        raise TypeError("out must be bfloat16 or float32")
    if blocks.dtype != torch.int32 or count.dtype != torch.int32 or not blocks.is_cuda or not count.is_cuda:
        raise ValueError("blocks and count must be int32 device tensors")
    B, Hg, Wg, H, d = q.shape
    if blocks.numel() < B * (Hg // w) * (Wg // w):
        raise ValueError("blocks must have room for every block of the grid")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = lib.wattn_local_residual(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(blocks), _ptr(count),
                                  B, H, Hg, Wg, w, d, ctypes.c_float(eps), dtype, ctypes.c_void_p(stream))
    if st != 0:
        raise WattnError(st, status_string(st))
    return out


def gated_local_path(q, k, v, out, gate, tau: float, *, w: int, eps: float = 1e-6, stream=None):
    """Routing and residual correction in one launch: the blocks whose gate value exceeds
    ``tau`` get out += O_local - O_lin-local (in place).  ``gate``: float32 device tensor of
    the B * (Hg/w) * (Wg/w) block gates in block order.  Returns out."""
    import torch

    lib = load_library()
    if q.dtype != torch.bfloat16 or q.dim() != 5:
        raise TypeError("q, k, v must be bfloat16 [B, Hgrid, Wgrid, H, d]")
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t.shape != q.shape or not t.is_cuda or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous device tensor shaped like q")
    for name, t in (("k", k), ("v", v)):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} must be bfloat16")
    if out.dtype == torch.bfloat16:
        dtype = BF16
    elif out.dtype == torch.float32:
        dtype = BF16_OUT_FP32
    else:
        raise TypeError("out must be bfloat16 or float32")
    B, Hg, Wg, H, d = q.shape
    if (gate.dtype != torch.float32 or not gate.is_cuda or not gate.is_contiguous()
            or gate.numel() != B * (Hg // w) * (Wg // w)):
        raise ValueError("gate must be a contiguous float32 device tensor with one value per block")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = lib.wattn_gated_local(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(gate), ctypes.c_float(tau),
                               B, H, Hg, Wg, w, d, ctypes.c_float(eps), dtype, ctypes.c_void_p(stream))
    if st != 0:
        raise WattnError(st, status_string(st))
    return out


def cla_logits(x, w_dw, w_pw, b_dw=None, b_pw=None, *, out=None, stream=None):
    """Gate logits z = PW(DW3x3(x)) of the convolutional gate (zero padding, no activation
    between).  x: bfloat16 [B, Hg, Wg, C] (or [B, Hg, Wg, H, d] with C = H * d); w_dw: float32
    [C, 3, 3]; w_pw: float32 [C, C]; biases float32 [C] or None.  Returns z shaped like x."""
    import torch

    lib = load_library()
    if x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous() or x.dim() < 4:
        raise ValueError("x must be a contiguous bfloat16 device tensor [B, Hg, Wg, C] or [B, Hg, Wg, H, d]")
    B, Hg, Wg = x.shape[:3]
    C = x[0, 0, 0].numel()
    for name, t, shape in (("w_dw", w_dw, (C, 3, 3)), ("w_pw", w_pw, (C, C)), ("b_dw", b_dw, (C,)),
                           ("b_pw", b_pw, (C,))):
        if t is None and name.startswith("b"):
            continue
        if t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 device tensor of shape {shape}")
    if out is None:
        out = torch.empty_like(x)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    st = lib.wattn_cla_logits(_ptr(x), _ptr(w_dw), _ptr(b_dw), _ptr(w_pw), _ptr(b_pw), _ptr(out), B, Hg, Wg, C,
                              BF16, ctypes.c_void_p(stream))
    if st != 0:
        raise WattnError(st, status_string(st))
    return out


def _check(st):
    if st != 0:
        raise WattnError(st, status_string(st))


def _stream(t, stream):
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream if stream is None else stream)


def linear(x, W, bias=None, *, residual=None, act: int = ACT_NONE, split=None, out=None, out_dtype=None,
           stream=None):
    """y = act(x W^T + bias) (+ residual) over the last axis of x (bfloat16, K channels); W:
    bfloat16 [N, K]; bias float32 [N] or None.  ``split`` stores column n in part n // split
    (returns the [N // split, M, split] tensor).  ``out`` may be ``residual`` (in place)."""
    import torch

    K = x.shape[-1]
    M = x.numel() // K
    N = W.shape[0]
    split = N if split is None else split
    odt = torch.bfloat16 if out_dtype is None else out_dtype
    dtype = BF16 if odt == torch.bfloat16 else BF16_OUT_FP32
    if out is None:
        shape = (N // split, M, split) if split != N else tuple(x.shape[:-1]) + (N,)
        out = torch.empty(shape, dtype=odt, device=x.device)
    _check(load_library().wattn_linear(_ptr(x), _ptr(W), _ptr(bias), _ptr(residual), _ptr(out), M, N, K, split,
                                       act, dtype, _stream(x, stream)))
    return out


def layernorm(x, gamma, beta, *, eps: float = 1e-5, out=None, stream=None):
    """Layer norm over the last axis of x (bfloat16); gamma, beta float32."""
    import torch

    C = x.shape[-1]
    out = torch.empty_like(x) if out is None else out
    _check(load_library().wattn_layernorm(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(out), x.numel() // C, C,
                                          ctypes.c_float(eps), _stream(x, stream)))
    return out


def patch_merge_norm(x, gamma, beta, *, eps: float = 1e-5, stream=None):
    """[B, Hg, Wg, C] -> [B, Hg/2, Wg/2, 4C]: 2 x 2 neighbours concatenated and normalised."""
    import torch

    B, Hg, Wg, C = x.shape
    out = torch.empty((B, Hg // 2, Wg // 2, 4 * C), dtype=x.dtype, device=x.device)
    _check(load_library().wattn_patch_merge_norm(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(out), B, Hg, Wg, C,
                                                 ctypes.c_float(eps), _stream(x, stream)))
    return out


def stem_conv(img, W, bias, *, p: int, stream=None):
    """Overlapping stem on an NHWC bfloat16 image: kernel 2p - 1, stride p, padding p - 1."""
    import torch

    B, Hi, Wi, Cin = img.shape
    Cout = W.shape[0]
    out = torch.empty((B, Hi // p, Wi // p, Cout), dtype=torch.bfloat16, device=img.device)
    _check(load_library().wattn_stem_conv(_ptr(img), _ptr(W), _ptr(bias), _ptr(out), B, Hi, Wi, Cin, Cout, p,
                                          _stream(img, stream)))
    return out


def token_mean(x, *, stream=None):
    """[B, ..., C] bfloat16 -> [B, C]: the mean over the tokens of each image."""
    import torch

    B, C = x.shape[0], x.shape[-1]
    n = x.numel() // (B * C)
    out = torch.empty((B, C), dtype=x.dtype, device=x.device)
    _check(load_library().wattn_token_mean(_ptr(x), _ptr(out), B, n, C, _stream(x, stream)))
    return out


def swin_block_workspace(B: int, Hg: int, Wg: int, C: int) -> int:
    return int(load_library().wattn_swin_block_workspace(B, Hg, Wg, C))


def swin_block(x, params: dict, *, H: int, M: int, shift: int = 0, workspace=None, stream=None):
    """One pre-norm block in place on x [B, Hg, Wg, C] (bfloat16, C = 32 H).  ``params`` maps
    the wattn_block_params_t field names to device tensors (biases and theta may be None)."""
    import torch

    B, Hg, Wg, C = x.shape
    need = swin_block_workspace(B, Hg, Wg, C)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    bp = BlockParams(*[None if params.get(name) is None else params[name].data_ptr()
                       for name, _ in BlockParams._fields_])
    _check(load_library().wattn_swin_block(_ptr(x), ctypes.byref(bp), _ptr(workspace), workspace.numel(), B, Hg, Wg,
                                           C, H, M, shift, _stream(x, stream)))
    return x
