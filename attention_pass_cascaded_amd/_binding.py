"""ctypes binding to librfattn.so, with the same entry points as include/rf_attn.h.

This layer only marshals arguments: it checks the placement, dtype, shape and
contiguity of every tensor it hands over (inputs and caller-provided output
buffers alike, so that no kernel writes past a buffer that is too small),
allocates the outputs the caller does not provide with torch on the input's
device, and passes raw device pointers plus the current HIP stream.  Every step of the computation
runs in the HIP kernels.  There is no fallback: if the library is missing or a
call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# RF_ATTN_LIB names another build of the same library (the sanitized host build)
LIB_PATH = os.environ.get("RF_ATTN_LIB") or os.path.join(_PKG, "librfattn.so")

RF_OK, RF_ERR_INVALID_ARG, RF_ERR_UNSUPPORTED, RF_ERR_HIP = 0, 1, 2, 3
_DTYPE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
_MASK = {"none": 0, "causal": 1, "sliding": 2}

EXPORTED = ("rf_attn_fwd", "rf_attn_splitkv_fwd", "rf_attn_fwd_alibi", "rf_attn_splitkv_fwd_alibi",
            "rf_splitkv_num_splits", "rf_splitkv_workspace_bytes", "rf_lse_merge", "rf_rope_rotate", "rf_attn_bwd",
            "rf_attn_bwd_workspace_bytes", "rf_attn_bwd_noalloc", "rf_layernorm_fwd", "rf_softmax_topk", "rf_status_string",
            "rf_last_error")


class RFError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"rf_attn status {status}: {msg}")
        self.status = status


_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load (once) and type the C ABI.  Raises if the built library is absent."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it with `python -m attention_pass_cascaded_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.rf_attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, f, i, vp]
    lib.rf_attn_fwd.restype = i
    lib.rf_attn_splitkv_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, f, i, i, vp]
    lib.rf_attn_splitkv_fwd.restype = i
    lib.rf_attn_fwd_alibi.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, f, vp, i, vp]
    lib.rf_attn_fwd_alibi.restype = i
    lib.rf_attn_splitkv_fwd_alibi.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, f, vp, i, i, vp]
    lib.rf_attn_splitkv_fwd_alibi.restype = i
    lib.rf_splitkv_num_splits.argtypes = [i, i, i, i]
    lib.rf_splitkv_num_splits.restype = i
    lib.rf_splitkv_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.rf_splitkv_workspace_bytes.restype = sz
    lib.rf_lse_merge.argtypes = [vp, vp, vp, vp, i, i, i, i, vp]
    lib.rf_lse_merge.restype = i
    lib.rf_rope_rotate.argtypes = [vp, vp, i, i, i, f, i, i, vp]
    lib.rf_rope_rotate.restype = i
    lib.rf_attn_bwd.argtypes = [vp] * 10 + [i, i, i, i, i, i, f, i, i, f, vp, i, vp]
    lib.rf_attn_bwd.restype = i
    lib.rf_attn_bwd_noalloc.argtypes = [vp] * 9 + [i, i, i, i, i, i, f, i, i, f, vp, i, vp]
    lib.rf_attn_bwd_noalloc.restype = i
    lib.rf_attn_bwd_workspace_bytes.argtypes = [i, i, i]
    lib.rf_attn_bwd_workspace_bytes.restype = sz
    lib.rf_layernorm_fwd.argtypes = [vp] * 6 + [i, i, f, i, vp]
    lib.rf_layernorm_fwd.restype = i
    lib.rf_softmax_topk.argtypes = [vp, vp, vp, i, i, i, i, vp]
    lib.rf_softmax_topk.restype = i
    lib.rf_status_string.argtypes = [i]
    lib.rf_status_string.restype = ctypes.c_char_p
    lib.rf_last_error.argtypes = []
    lib.rf_last_error.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _check(status: int):
    if status != RF_OK:
        lib = load_library()
        raise RFError(status, lib.rf_last_error().decode())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() else None


def _check_inputs(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, H, N, D] tensor")
        if t.dtype != q.dtype:
            raise ValueError("q, k and v must share one dtype")
    if q.dtype not in _DTYPE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    B, Hq, Nq, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("k and v must be [B, Hkv, Nk, D] matching q")
    return B, Hq, k.shape[1], Nq, k.shape[2], D


def _out(name, t, shape, dtype, device):
    """A caller-provided output buffer: allocate it when absent, else check that
    it is a contiguous tensor of exactly ``shape`` and ``dtype`` on ``device``."""
    shape = tuple(int(x) for x in shape)
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.device != torch.device(device):  # the inputs it goes with are already on the GPU
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != shape:
        raise ValueError(f"{name} must have shape {list(shape)}, got {list(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _scale(scale, D):
    return 1.0 / math.sqrt(D) if scale is None else float(scale)


def _slopes(alibi_slopes, Hq, device):
    """ALiBi slopes as a device float32 [Hq] tensor (kept alive by the caller frame)."""
    if alibi_slopes is None:
        return None
    t = torch.as_tensor(alibi_slopes, dtype=torch.float32).to(device).contiguous()
    if t.shape != (Hq,):
        raise ValueError(f"alibi_slopes must have Hq={Hq} entries")
    return t


# Rotation Calculus on MI355X: causal fp16 B=4 H=12 D=64 with RoPE, fused vs
# rotate-first; the fused kernel wins up to this key length (the crossover N*
# of the measured sweep, `bench.py --rotation-sweep`; repeated sweeps put it
# between ~2760 and ~3150, where the two modes are within a few percent).
ROPE_FUSED_MAX_N = 3150


def fwd(q, k, v, scale=None, mask="none", window=0, rope_base=0.0, out=None, lse=None,
        alibi_slopes=None, rope_mode="fused"):
    """Fused forward.  Returns (o [B,Hq,Nq,D] in q.dtype, lse [B,Hq,Nq] float32).

    alibi_slopes: optional per-query-head slopes (sequence or tensor of Hq floats).
    rope_mode: "fused" rotates inside the attention kernel; "rotate_first" runs
    rf_rope_rotate on q and k first; "auto" picks rotate-first for Nk above the
    measured crossover when the inputs are not bfloat16 (rotating into bf16
    would round the rotated operands, which the fused kernel avoids).
    """
    if rope_base and rope_base > 0 and rope_mode != "fused":
        if rope_mode not in ("auto", "rotate_first"):
            raise ValueError(f"unknown rope_mode {rope_mode!r}")
        if rope_mode == "rotate_first" or (k.shape[2] > ROPE_FUSED_MAX_N and q.dtype != torch.bfloat16):
            return fwd_prerotated(q, k, v, rope_base, scale=scale, mask=mask, window=window, out=out,
                                  lse=lse, alibi_slopes=alibi_slopes)
    B, Hq, Hkv, Nq, Nk, D = _check_inputs(q, k, v)
    out = _out("out", out, q.shape, q.dtype, q.device)
    lse = _out("lse", lse, (B, Hq, Nq), torch.float32, q.device)
    slopes = _slopes(alibi_slopes, Hq, q.device)
    lib = load_library()
    _check(lib.rf_attn_fwd_alibi(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Nq, Nk, D,
                                 _scale(scale, D), _MASK[mask], int(window), float(rope_base), _ptr(slopes),
                                 _DTYPE[q.dtype], _stream(q)))
    return out, lse


def num_splits_for(q, k, cu_count: int = 0) -> int:
    """The library's chunk count (rf_splitkv_num_splits) for q [B,Hq,Nq,D]
    against k [B,Hkv,Nk,D]; cu_count 0 asks the current device."""
    n = int(load_library().rf_splitkv_num_splits(k.shape[0], k.shape[1], k.shape[2], int(cu_count)))
    if n < 1:
        raise ValueError("invalid sizes for a split-KV call")
    return n


def workspace_bytes(B, Hq, Nq, D, num_splits) -> int:
    return int(load_library().rf_splitkv_workspace_bytes(B, Hq, Nq, D, num_splits))


def splitkv_fwd(q, k, v, num_splits, scale=None, mask="none", window=0, rope_base=0.0,
                o_part=None, lse_part=None, alibi_slopes=None):
    """Split-KV partials: (o_part [B,Hq,Nq,S,D] float32, lse_part [B,Hq,Nq,S] float32)."""
    B, Hq, Hkv, Nq, Nk, D = _check_inputs(q, k, v)
    S = int(num_splits)
    o_part = _out("o_part", o_part, (B, Hq, Nq, S, D), torch.float32, q.device)
    lse_part = _out("lse_part", lse_part, (B, Hq, Nq, S), torch.float32, q.device)
    slopes = _slopes(alibi_slopes, Hq, q.device)
    lib = load_library()
    _check(lib.rf_attn_splitkv_fwd_alibi(_ptr(q), _ptr(k), _ptr(v), _ptr(o_part), _ptr(lse_part),
                                         B, Hq, Hkv, Nq, Nk, D, _scale(scale, D), _MASK[mask], int(window),
                                         float(rope_base), _ptr(slopes), S, _DTYPE[q.dtype], _stream(q)))
    return o_part, lse_part


def lse_merge(o_part, lse_part, out_dtype=torch.float32, out=None, lse=None):
    """Merge partials along the chunk axis: o_part [..., S, D], lse_part [..., S]."""
    if not (o_part.is_cuda and lse_part.is_cuda and o_part.is_contiguous() and lse_part.is_contiguous()):
        raise ValueError("o_part and lse_part must be contiguous GPU tensors")
    if o_part.dtype != torch.float32 or lse_part.dtype != torch.float32:
        raise ValueError("partials are float32")
    S, D = o_part.shape[-2], o_part.shape[-1]
    lead = tuple(o_part.shape[:-2])
    if tuple(lse_part.shape) != lead + (S,):
        raise ValueError("lse_part must be o_part.shape[:-1]")
    rows = math.prod(lead)
    if lse_part.device != o_part.device:
        raise ValueError("o_part and lse_part must be on one device")
    if out is not None:
        out_dtype = out.dtype
    if out_dtype not in _DTYPE:
        raise ValueError(f"unsupported output dtype {out_dtype}")
    out = _out("out", out, lead + (D,), out_dtype, o_part.device)
    lse = _out("lse", lse, lead, torch.float32, o_part.device)
    lib = load_library()
    _check(lib.rf_lse_merge(_ptr(o_part), _ptr(lse_part), _ptr(out), _ptr(lse), rows, S, D,
                            _DTYPE[out.dtype], _stream(o_part)))
    return out, lse


def rope_rotate(x, base, pos_offset=0, out=None):
    """Rotary embedding of x [B, H, N, D] at positions pos_offset + n (out may be x)."""
    if not x.is_cuda or x.dim() != 4 or not x.is_contiguous() or x.dtype not in _DTYPE:
        raise ValueError("x must be a contiguous [B, H, N, D] GPU tensor of float32/float16/bfloat16")
    out = _out("out", out, x.shape, x.dtype, x.device)
    B, H, N, D = x.shape
    _check(load_library().rf_rope_rotate(_ptr(x), _ptr(out), B * H, N, D, float(base), int(pos_offset),
                                         _DTYPE[x.dtype], _stream(x)))
    return out


def fwd_prerotated(q, k, v, rope_base, scale=None, mask="none", window=0, out=None, lse=None,
                   alibi_slopes=None):
    """RoPE attention as two passes: rotate q and k into temporaries, then the
    fused forward without rotation (the other side of the Rotation Calculus)."""
    qr = rope_rotate(q, rope_base, pos_offset=k.shape[2] - q.shape[2])
    kr = rope_rotate(k, rope_base, pos_offset=0)
    return fwd(qr, kr, v, scale=scale, mask=mask, window=window, rope_base=0.0, out=out, lse=lse,
               alibi_slopes=alibi_slopes)


def decode(q, k, v, num_splits=None, scale=None, mask="none", window=0, rope_base=0.0, alibi_slopes=None):
    """Split-KV attention: partials then log-sum-exp merge.  Returns (o, lse)
    like fwd.  num_splits None takes the library's rule (num_splits_for)."""
    if num_splits is None:
        num_splits = num_splits_for(q, k)
    op, lp = splitkv_fwd(q, k, v, num_splits, scale, mask, window, rope_base, alibi_slopes=alibi_slopes)
    return lse_merge(op, lp, out_dtype=q.dtype)


def bwd(q, k, v, o, lse, dout, scale=None, mask="none", window=0, rope_base=0.0, alibi_slopes=None,
        dq=None, dk=None, dv=None, workspace=None):
    """Gradients (dq, dk, dv) of fwd for the loss gradient dout, from the
    forward's o and lse (same arguments as the forward call)."""
    B, Hq, Hkv, Nq, Nk, D = _check_inputs(q, k, v)
    for name, t, shape in (("o", o, q.shape), ("dout", dout, q.shape)):
        if not t.is_cuda or t.dtype != q.dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor like q")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Nq) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, Hq, Nq] tensor")
    dq = _out("dq", dq, q.shape, q.dtype, q.device)
    dk = _out("dk", dk, k.shape, k.dtype, q.device)
    dv = _out("dv", dv, v.shape, v.dtype, q.device)
    lib = load_library()
    nbytes = int(lib.rf_attn_bwd_workspace_bytes(B, Hq, Nq))
    if workspace is None:
        workspace = torch.empty(max(nbytes // 4, 1), dtype=torch.float32, device=q.device)
    elif (not workspace.is_cuda or workspace.device != q.device or workspace.dtype != torch.float32
          or not workspace.is_contiguous() or workspace.numel() * 4 < nbytes):
        raise ValueError(f"workspace must be a contiguous float32 tensor on {q.device} of at least {nbytes} bytes")
    slopes = _slopes(alibi_slopes, Hq, q.device)
    _check(lib.rf_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                           _ptr(dv), _ptr(workspace), B, Hq, Hkv, Nq, Nk, D, _scale(scale, D), _MASK[mask],
                           int(window), float(rope_base), _ptr(slopes), _DTYPE[q.dtype], _stream(q)))
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, scale=None, mask="none", window=0, rope_base=0.0,
                alibi_slopes=None):
    """rf_attn_bwd_noalloc: the gradients into the caller's dq, dk, dv with
    the row terms in the library's static per-GPU array (no workspace; calls
    that overlap on one GPU race).  alibi_slopes must then be a float32 [Hq]
    GPU tensor (a sequence would be copied to a new device tensor)."""
    B, Hq, Hkv, Nq, Nk, D = _check_inputs(q, k, v)
    for name, t, shape in (("o", o, q.shape), ("dout", dout, q.shape)):
        if not t.is_cuda or t.dtype != q.dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor like q")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Nq) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, Hq, Nq] tensor")
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t is None:
            raise ValueError(f"{name} must be provided")
        _out(name, t, like.shape, like.dtype, q.device)
    if alibi_slopes is not None and not (isinstance(alibi_slopes, torch.Tensor) and alibi_slopes.is_cuda):
        raise ValueError("alibi_slopes must be a float32 [Hq] GPU tensor here")
    slopes = _slopes(alibi_slopes, Hq, q.device)
    _check(load_library().rf_attn_bwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), B, Hq, Hkv, Nq,
        Nk, D, _scale(scale, D), _MASK[mask], int(window), float(rope_base), _ptr(slopes), _DTYPE[q.dtype],
        _stream(q)))
    return dq, dk, dv


def layernorm(x, gamma, beta, eps=1e-5, y=None, mean=None, rstd=None):
    """LayerNorm over the last axis of x [..., H].  Returns (y, mean, rstd)."""
    if not x.is_cuda or not x.is_contiguous() or x.dtype not in _DTYPE:
        raise ValueError("x must be a contiguous GPU tensor of float32/float16/bfloat16")
    H = x.shape[-1]
    for name, t in (("gamma", gamma), ("beta", beta)):
        if not t.is_cuda or t.dtype != x.dtype or tuple(t.shape) != (H,) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [H] GPU tensor of x's dtype")
    rows = x.numel() // H if H else 0
    y = _out("y", y, x.shape, x.dtype, x.device)
    mean = _out("mean", mean, x.shape[:-1], torch.float32, x.device)
    rstd = _out("rstd", rstd, x.shape[:-1], torch.float32, x.device)
    _check(load_library().rf_layernorm_fwd(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), _ptr(mean), _ptr(rstd),
                                           rows, H, float(eps), _DTYPE[x.dtype], _stream(x)))
    return y, mean, rstd


def softmax_topk(x, k, values=None, indices=None):
    """Softmax over the last axis of x [..., E], then its k largest entries:
    (values float32 [..., k] in descending order, indices int32 [..., k])."""
    if not x.is_cuda or not x.is_contiguous() or x.dtype not in _DTYPE:
        raise ValueError("x must be a contiguous GPU tensor of float32/float16/bfloat16")
    E = x.shape[-1]
    rows = x.numel() // E if E else 0
    shape = tuple(x.shape[:-1]) + (int(k),)
    values = _out("values", values, shape, torch.float32, x.device)
    indices = _out("indices", indices, shape, torch.int32, x.device)
    _check(load_library().rf_softmax_topk(_ptr(x), _ptr(values), _ptr(indices), rows, E, int(k),
                                          _DTYPE[x.dtype], _stream(x)))
    return values, indices
